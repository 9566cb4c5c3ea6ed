"""GPU parity at the five named workloads' full sizes, in the launch
configuration the benchmark times (moe_forward, automatic tile regime).

The routing plan is compared in full (bit-exact).  Every row of the heaviest
and of the lightest active expert (the heaviest spans all of its m-tiles) is
compared against the pure oracle at its pair slot of y, within relative L2
<= 1e-2 and max-abs <= 5e-2 * RMS, and stage by stage (requantised intermediate
codes with rounding ties allowed; the down projection of the GPU's own
intermediate).  The combined output is compared on a seeded sample of tokens
that the oracle computes one by one, within the same two bounds against the
pure oracle."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import (c_scale, check_intermediate, check_y_rows, compare_out, device_inputs, fwd_kwargs, geometry,
                      gs_kwargs, make_moe, prepared)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

SAMPLE = 24


def _rows_of(h, hsf, rows, fmt):
    ridx = torch.as_tensor(rows, dtype=torch.int64, device="cuda")
    hc = h.index_select(0, ridx).cpu()
    hc = hc.view(torch.int16).numpy().view(np.uint16) if fmt in ("bf16", "nvfp4_w4a16", "nvfp4") else hc.numpy()
    hs = None if hsf is None else hsf.index_select(0, ridx).cpu().numpy()
    return hc, hs


def _check_whole_expert(sh, inp, geo, e, ref_plan, y, h, hsf):
    """Every row of expert e: y at the rows' pair slots against the pure oracle
    (both output bounds), and stage by stage.  Returns (rows, rel-L2, max-abs/RMS, flips)."""
    k, I = sh.topk, sh.inter
    r0, r1 = int(ref_plan["expert_start_indices"][e]), int(ref_plan["expert_start_indices"][e + 1])
    src = ref_plan["src_info"][r0:r1]
    toks = src // k
    X = oracle.dequant_activations(geo, inp["x"][toks], None if inp["x_sf"] is None else inp["x_sf"][toks])
    w13d, w2d = oracle.dequant_expert(geo, inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"], e, **gs_kwargs(inp))
    hx = oracle.swiglu_clamped(X @ w13d[:I].T, X @ w13d[I:].T, geo.clamp)
    del X
    y_pure = oracle.requant(geo, hx, c_scale(inp, e)) @ w2d.T
    y_gpu = y.index_select(0, torch.as_tensor(src, dtype=torch.int64, device="cuda")).float().cpu()
    rl2, mr = compare_out(y_gpu, y_pure)
    hc, hs = _rows_of(h, hsf, np.arange(r0, r1), sh.fmt)
    hg, flips = check_intermediate(sh.fmt, hx, hc, hs, I, c_scale(inp, e))
    check_y_rows(y_gpu.numpy().astype(np.float64), hg @ w2d.T)
    return r1 - r0, rl2, mr, flips


def _gather_intermediate(moe, d, T, rows):
    """moe_plan, moe_ffn_gate_up, moe_ffn_down; return (plan, y, h codes, h scales) of the
    given rows, and the whole h and h_sf buffers."""
    plan = moe.alloc_plan(T)
    ws = moe.alloc_workspace(T)
    if moe.route_mode == "precomputed":
        moe.plan(T, plan, topk_idx=d["topk_idx"], ws=ws)
    else:
        moe.plan(T, plan, routing_logits=d["logits"], topk_idx_out=d["topk_idx"], topk_weights_out=d["topk_weights"],
                 ws=ws)
    h, hsf = moe.alloc_intermediate(T)
    moe.ffn_gate_up(T, d["x"], d["x_sf"], prepared(moe, d), plan, h, hsf)
    y = torch.zeros((T * moe.topk, moe.hidden), dtype=torch.bfloat16, device="cuda")
    moe.ffn_down(T, h, hsf, prepared(moe, d), plan, y)
    torch.cuda.synchronize()
    hc, hs = _rows_of(h, hsf, rows, moe.fmt)
    return plan, y, hc, hs, h, hsf


@pytest.mark.parametrize("name", moe_synth.CONFIG_ORDER + ["nvfp4_decode", "nvfp4x4_decode"])
def test_named_workload_full_size(name):
    sh = moe_synth.WORKLOADS[name]
    print(f"[fullsize] {name}: generating inputs", flush=True)
    inp = moe_synth.make_inputs(sh)
    T, k, E, H, I = sh.tokens, sh.topk, sh.experts, sh.hidden, sh.inter
    moe = make_moe(sh)
    d = device_inputs(inp)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = moe.alloc_workspace(T)
    print(f"[fullsize] {name}: moe_forward T={T}", flush=True)
    moe.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], d["logits"], prepared(moe, d), out, ws)
    torch.cuda.synchronize()
    out_np = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out_np))

    # routing: FromLogits ids bit-exact, weights to 1e-5; the plan bit-exact
    if sh.routing == "from_logits":
        ids, w_ref = oracle.route_from_logits(inp["logits"], k)
        got_ids = d["topk_idx"].cpu().numpy()
        assert np.array_equal(got_ids, ids)
        np.testing.assert_allclose(d["topk_weights"].cpu().numpy(), w_ref, rtol=1e-5, atol=1e-7)
        w = d["topk_weights"].cpu().numpy().astype(np.float64)
    else:
        ids, w = inp["topk_idx"], inp["topk_weights"].astype(np.float64)
    ref_plan = oracle.build_plan(ids, E)

    # sampled tokens, stage by stage
    rng = np.random.default_rng(1234)
    toks = np.sort(rng.choice(T, size=min(SAMPLE, T), replace=False))
    pairs = [(t, j) for t in toks for j in range(k) if ref_plan["pair_row"][t * k + j] >= 0]
    rows = [int(ref_plan["pair_row"][t * k + j]) for t, j in pairs]
    plan, y, h_g, hsf_g, h_all, hsf_all = _gather_intermediate(moe, d, T, rows)
    for f, key in (("expert_counts", "expert_counts"), ("expert_start_indices", "expert_start_indices"),
                   ("expert_ids", "expert_ids"), ("pair_row", "pair_row")):
        assert np.array_equal(plan[f].cpu().numpy()[: ref_plan[key].size], ref_plan[key]), f
    nv = int(ref_plan["expert_start_indices"][-1])
    assert np.array_equal(plan["src_info"].cpu().numpy()[:nv], ref_plan["src_info"])

    geo = geometry(sh)
    xd = oracle.dequant_activations(geo, inp["x"][toks], None if inp["x_sf"] is None else inp["x_sf"][toks])
    tpos = {int(t): n for n, t in enumerate(toks)}
    by_e: dict = {}
    for n, (t, j) in enumerate(pairs):
        by_e.setdefault(int(ids[t, j]), []).append(n)
    y_ref2 = np.zeros((len(pairs), H))
    flips = 0
    for e, lst in by_e.items():
        w13d, w2d = oracle.dequant_expert(geo, inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"], e,
                                          **gs_kwargs(inp))
        X = xd[[tpos[pairs[n][0]] for n in lst]]
        hx = oracle.swiglu_clamped(X @ w13d[:I].T, X @ w13d[I:].T, geo.clamp)
        hg, f = check_intermediate(sh.fmt, hx, h_g[lst], None if hsf_g is None else hsf_g[lst], I, c_scale(inp, e))
        flips += f
        y_ref2[lst] = hg @ w2d.T
    # y rows at their pair slots
    check_y_rows(y.float().cpu().numpy()[[t * k + j for t, j in pairs]].astype(np.float64), y_ref2)
    # combined output of the sampled tokens
    out_ref2 = np.zeros((len(toks), H))
    for n, (t, j) in enumerate(pairs):
        out_ref2[tpos[t]] += w[t, j] * y_ref2[n]
    compare_out(torch.from_numpy(out_np[toks]), out_ref2)
    # and the pure oracle on the sample, relative L2
    ref = oracle.forward_tokens(geo, toks, inp["x"], inp["x_sf"], inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"],
                                ids, w, **fwd_kwargs(inp))
    rl2, mr = compare_out(torch.from_numpy(out_np[toks]), ref)
    print(f"[fullsize] {name}: sampled tokens: rel-L2 {rl2:.2e}, max-abs/RMS {mr:.2e} against the pure oracle "
          f"({len(pairs)} pairs, {flips} rounding-tie flips)", flush=True)

    # every row of the heaviest and of the lightest active expert
    counts = ref_plan["expert_counts"]
    act = np.flatnonzero(counts > 0)
    for e in sorted({int(act[np.argmax(counts[act])]), int(act[np.argmin(counts[act])])}):
        n, rl2, mr, fl = _check_whole_expert(sh, inp, geo, e, ref_plan, y, h_all, hsf_all)
        print(f"[fullsize] {name}: expert {e}, all {n} rows: rel-L2 {rl2:.2e}, max-abs/RMS {mr:.2e} against the "
              f"pure oracle ({fl} rounding-tie flips)", flush=True)
