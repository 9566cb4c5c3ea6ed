"""The seeded input generator: determinism, shapes, and the load statistics
each named workload is meant to have (CPU only)."""
import numpy as np

import moe_synth
from moe_synth import WORKLOADS


def test_deterministic_and_shaped():
    sh = WORKLOADS["tiny_fp8"]
    a = moe_synth.make_inputs(sh)
    b = moe_synth.make_inputs(sh)
    for key in ("x", "x_sf", "w13", "w13_sf", "w2", "w2_sf", "topk_idx", "topk_weights", "logits"):
        assert np.array_equal(a[key], b[key]), key
    assert a["x"].shape == (64, 256) and a["x"].dtype == np.uint8
    assert a["x_sf"].shape == (64, 2) and a["x_sf"].dtype == np.float32
    assert a["w13"].shape == (8, 256, 256) and a["w13_sf"].shape == (8, 2, 2)
    assert a["w2"].shape == (8, 256, 128) and a["w2_sf"].shape == (8, 2, 1)
    assert a["topk_idx"].dtype == np.int64 and a["topk_weights"].dtype == np.float32


def test_mx_shapes():
    sh = WORKLOADS["w4a8_mx_logits"].with_(tokens=8, experts=2)
    a = moe_synth.make_inputs(sh)
    assert a["x"].shape == (8, 2880) and a["x_sf"].shape == (8, 90) and a["x_sf"].dtype == np.uint8
    assert a["w13"].shape == (2, 5760, 1440) and a["w13_sf"].shape == (2, 5760, 90)
    assert a["w2"].shape == (2, 2880, 1440) and a["w2_sf"].shape == (2, 2880, 90)
    assert "topk_idx" not in a


def test_prefill_zipf_load_is_skewed():
    sh = WORKLOADS["prefill_fp8_zipf"]
    a = moe_synth.make_inputs(sh, with_weights=False)
    counts = np.bincount(a["topk_idx"].reshape(-1), minlength=sh.experts)
    mean = sh.pairs / sh.experts
    assert counts.max() >= 3.5 * mean
    assert 2 <= int((counts == 0).sum()) <= 8


def test_decode_load_is_uniform():
    sh = WORKLOADS["decode_fp8"]
    a = moe_synth.make_inputs(sh, with_weights=False)
    counts = np.bincount(a["topk_idx"].reshape(-1), minlength=sh.experts)
    assert counts.min() > 0 and counts.max() < 2 * sh.pairs / sh.experts


def test_nvfp4_shapes_and_quantisation_error():
    from oracle import dequant_nvfp4
    sh = moe_synth.WORKLOADS["nvfp4_decode"].with_(tokens=16, hidden=256, inter=128, experts=3, topk=2)
    inp = moe_synth.make_inputs(sh)
    assert inp["x"].dtype == np.uint16 and inp["x_sf"] is None
    assert inp["w13"].shape == (3, 256, 128) and inp["w13_sf"].shape == (3, 256, 16)
    assert inp["w2"].shape == (3, 256, 64) and inp["w2_sf"].shape == (3, 256, 8)
    assert inp["w13_gs"].shape == (3,) and inp["w2_gs"].dtype == np.float32
    # the draws behind the codes: redraw expert 1's w13 and compare with its dequantisation
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([sh.seed, 3, 1])))
    w = rng.standard_normal((256, 256), dtype=np.float32) * np.float32(1.0 / 16.0)
    deq = dequant_nvfp4(inp["w13"][1], inp["w13_sf"][1], inp["w13_gs"][1])
    step = np.repeat(np.abs(w).reshape(256, 16, 16).max(axis=2) / 6.0, 16, axis=1)  # block amax / 6
    assert np.all(np.abs(deq - w) <= 1.07 * step + 1e-12)
