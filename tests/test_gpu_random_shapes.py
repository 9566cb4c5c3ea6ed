"""Parity over seeded random shapes: every format, both tile regimes forced, sizes
drawn so that rows, columns and K-steps end in ragged tiles (experts smaller and
larger than a tile, column counts that are not multiples of a tile, K tails for
the formats that allow them).  As for the fixed small cases: the FromLogits
routing (ids bit-exact, weights to 1e-5), the forward output against the pure
oracle (relative L2, and max-abs / RMS with the rounding-tie flips of the
requantised intermediate accounted for), and stage by stage."""
import numpy as np
import pytest

import moe_synth
import oracle
import torch

from gpu_util import (check_against_oracle, device_inputs, fwd_kwargs, geometry, make_moe, run_ffn_intermediates,
                      run_forward)

pytestmark = pytest.mark.gpu

# (H, I) granularity per format: the library's moe_create constraints
_GRAIN = {"fp8_block128": 128, "bf16": 64, "w4a8_mx": 32, "nvfp4_w4a16": 64, "nvfp4": 64}


def _shape(fmt, seed):
    rng = np.random.default_rng(seed)
    g = _GRAIN[fmt]
    H = int(rng.integers(2, 9)) * g + (g if fmt == "w4a8_mx" and rng.random() < 0.5 else 0)
    I = int(rng.integers(2, 9)) * g
    E = int(rng.integers(1, 17))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 300))
    routing = "from_logits" if fmt == "w4a8_mx" and rng.random() < 0.5 else "precomputed"
    return moe_synth.MoEShape(f"rand_{fmt}_{seed}", seed, T, H, I, E, k, fmt, routing)


@pytest.mark.parametrize("regime", ["decode", "prefill"])
@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("fmt", list(_GRAIN))
def test_random_shape_forward(fmt, seed, regime):
    sh = _shape(fmt, 1000 * seed + len(fmt))
    print(f"case {sh.name}: T={sh.tokens} H={sh.hidden} I={sh.inter} E={sh.experts} k={sh.topk} "
          f"{sh.routing} {regime}", flush=True)
    inp = moe_synth.make_inputs(sh)
    moe = make_moe(sh, tile_regime=regime)
    d = device_inputs(inp)
    out = run_forward(moe, d, sh.tokens)
    ids = d["topk_idx"].cpu().numpy()
    w = d["topk_weights"].cpu().numpy()
    if sh.routing == "from_logits":
        ref_ids, ref_w = oracle.route_from_logits(inp["logits"], sh.topk)
        assert np.array_equal(ids, ref_ids)
        np.testing.assert_allclose(w, ref_w, rtol=1e-5, atol=1e-7)
    ref = oracle.forward(geometry(sh), inp["x"], inp["x_sf"], inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"],
                         topk_idx=ids, topk_weights=w, **fwd_kwargs(inp))
    res = run_ffn_intermediates(moe, d, sh.tokens)
    assert torch.equal(res[0].view(torch.int16), out.view(torch.int16))
    check_against_oracle(sh, inp, out, ref, res, ids, w, sh.name)
