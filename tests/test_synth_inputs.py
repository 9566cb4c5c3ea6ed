"""The seeded input generator: determinism, shapes, and the load statistics
each named workload is meant to have (CPU only)."""
import numpy as np

import moe_synth
from moe_synth import CONFIGS


def test_deterministic_and_shaped():
    sh = CONFIGS["tiny_fp8"]
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
    sh = CONFIGS["w4a8_mx_logits"].with_(tokens=8, experts=2)
    a = moe_synth.make_inputs(sh)
    assert a["x"].shape == (8, 2880) and a["x_sf"].shape == (8, 90) and a["x_sf"].dtype == np.uint8
    assert a["w13"].shape == (2, 5760, 1440) and a["w13_sf"].shape == (2, 5760, 90)
    assert a["w2"].shape == (2, 2880, 1440) and a["w2_sf"].shape == (2, 2880, 90)
    assert "topk_idx" not in a


def test_prefill_zipf_load_is_skewed():
    sh = CONFIGS["prefill_fp8_zipf"]
    a = moe_synth.make_inputs(sh, with_weights=False)
    counts = np.bincount(a["topk_idx"].reshape(-1), minlength=sh.experts)
    mean = sh.pairs / sh.experts
    assert counts.max() >= 3.5 * mean
    assert 2 <= int((counts == 0).sum()) <= 8


def test_decode_load_is_uniform():
    sh = CONFIGS["decode_fp8"]
    a = moe_synth.make_inputs(sh, with_weights=False)
    counts = np.bincount(a["topk_idx"].reshape(-1), minlength=sh.experts)
    assert counts.min() > 0 and counts.max() < 2 * sh.pairs / sh.experts
