"""GPU parity of the optional pieces around the routed path: bias-aware FromLogits
routing (moe_plan_ex), the combine's fused addends (moe_combine_ex: a shared
expert's output and a residual), and the whole path with all of them
(moe_forward_ex), each against the oracle; and the timed GEMM legs, whose
events carry the kernels' own start and end."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import compare_out, device_inputs, geometry, make_moe, prepared

pytestmark = pytest.mark.gpu


def small(name, seed, T, H, I, E, k, fmt, routing="precomputed"):
    return moe_synth.MoEShape(name, seed, T, H, I, E, k, fmt, routing)


def _bias(E, seed):
    rng = np.random.default_rng(seed)
    b = (rng.standard_normal(E) * 0.5).astype(np.float32)
    b[E // 3] = 8.0  # one expert the bias always selects
    return b


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (300, 128, 4), (37, 512, 8)])
def test_route_from_logits_biased(T, E, k):
    rng = np.random.default_rng(100 + T)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = _bias(E, T)
    lg[0, :] = 0.0                          # ties among the biased keys of equal bias
    bias_t = bias.copy()
    bias_t[: min(E, 6)] = 1.0               # ... e.g. experts 0..5 tie at key 1.0 on token 0
    sh = small("route_bias", 1, T, 256, 128, E, k, "fp8_block128", "from_logits")
    moe = make_moe(sh)
    plan = moe.alloc_plan(T)
    ws = moe.alloc_workspace(T)
    ids = torch.empty((T, k), dtype=torch.int64, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.plan(T, plan, routing_logits=torch.from_numpy(lg).cuda(), topk_idx_out=ids, topk_weights_out=w, ws=ws,
             routing_bias=torch.from_numpy(bias_t).cuda())
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route_from_logits(lg, k, bias_t)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-7)
    # the bias changed the selection somewhere (else the test proves nothing)
    assert not np.array_equal(ref_ids, oracle.route_from_logits(lg, k)[0])


def test_route_biased_nan_and_ragged_expert_count():
    """E not a multiple of the wave width; NaN logits and a NaN bias entry rank lowest."""
    T, E, k = 50, 100, 4
    rng = np.random.default_rng(77)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::5, 3] = np.nan
    lg[2, :10] = np.nan
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    bias[7] = np.nan
    bias[99] = 4.0
    sh = small("route_bias_nan", 1, T, 256, 128, E, k, "fp8_block128", "from_logits")
    moe = make_moe(sh)
    plan = moe.alloc_plan(T)
    ws = moe.alloc_workspace(T)
    ids = torch.empty((T, k), dtype=torch.int64, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.plan(T, plan, routing_logits=torch.from_numpy(lg).cuda(), topk_idx_out=ids, topk_weights_out=w, ws=ws,
             routing_bias=torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route_from_logits(lg, k, bias)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-7)
    assert not np.isin(ref_ids, [7]).any()  # the NaN-biased expert is never chosen


@pytest.mark.parametrize("with_bias", [False, True])
def test_route_nan_expert_selected(with_bias):
    """NaN logits among the k selected (a token with fewer non-NaN logits than k): a NaN
    logit reads as -inf, so the NaN expert is chosen last (lowest index among the
    tied) and gets weight 0; a token whose logits are all NaN gets NaN weights."""
    T, E, k = 40, 64, 4
    rng = np.random.default_rng(91)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[1, :] = np.nan
    lg[1, [5, 40]] = [0.25, 1.5]        # two real logits, k = 4: two NaN experts selected
    lg[3, :] = np.nan
    lg[3, 63] = -2.0                   # one real logit
    lg[6, :] = np.nan                  # all NaN: 0/0 weights
    lg[9, ::2] = np.nan                # half NaN: none selected
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32) if with_bias else None
    sh = small("route_nan_sel", 1, T, 256, 128, E, k, "fp8_block128", "from_logits")
    moe = make_moe(sh)
    plan = moe.alloc_plan(T)
    ws = moe.alloc_workspace(T)
    ids = torch.empty((T, k), dtype=torch.int64, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.plan(T, plan, routing_logits=torch.from_numpy(lg).cuda(), topk_idx_out=ids, topk_weights_out=w, ws=ws,
             routing_bias=None if bias is None else torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route_from_logits(lg, k, bias)
    got_ids, got_w = ids.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(got_ids, ref_ids)
    np.testing.assert_allclose(got_w, ref_w, rtol=1e-5, atol=1e-7, equal_nan=True)
    assert (ref_w[1, 2:] == 0).all() and (ref_w[3, 1:] == 0).all() and np.isnan(ref_w[6]).all()
    assert (got_w[1, 2:] == 0).all() and (got_w[3, 1:] == 0).all()


def test_combine_addends():
    rng = np.random.default_rng(9)
    T, k, E, H = 77, 3, 6, 4096
    ids = rng.integers(-1, E, size=(T, k))
    ids[5, :] = -1                                   # a token with no valid slot: the addends only
    w = rng.random((T, k)).astype(np.float32)
    sh = small("comb_add", 1, T, H, 128, E, k, "fp8_block128")
    moe = make_moe(sh)
    plan = moe.alloc_plan(T)
    ws = moe.alloc_workspace(T)
    moe.plan(T, plan, topk_idx=torch.from_numpy(ids).cuda(), ws=ws)
    y = torch.randn((T * k, H), device="cuda").to(torch.bfloat16)
    shared = torch.randn((T, H), device="cuda").to(torch.bfloat16)
    residual = torch.randn((T, H), device="cuda").to(torch.bfloat16)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.combine(T, y, torch.from_numpy(w).cuda(), plan, out, shared=shared, residual=residual)
    torch.cuda.synchronize()
    ref_plan = oracle.build_plan(ids, E)
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    ref = oracle.combine(f64(y), w, np.where(ref_plan["pair_row"] >= 0, np.arange(T * k), -1), H,
                         (f64(shared), f64(residual)))
    np.testing.assert_allclose(out.float().cpu().numpy(), ref, rtol=2 ** -7, atol=1e-5)


@pytest.mark.parametrize("fmt", ["fp8_block128", "bf16"])
def test_forward_with_bias_shared_expert_and_residual(fmt):
    T, H, I, E, k = 96, 512, 256, 8, 2
    sh = small("ext_" + fmt, 31, T, H, I, E, k, fmt, "from_logits")
    inp = moe_synth.make_inputs(sh)
    bias = _bias(E, 3)
    # the shared expert: one more expert of the same format that every token visits with weight 1
    sh1 = small("ext_shared_" + fmt, 32, T, H, I, 1, 1, fmt)
    inp1 = moe_synth.make_inputs(sh1)
    moe1 = make_moe(sh1)
    d1 = device_inputs(inp1, topk_idx=np.zeros((T, 1), np.int64), topk_weights=np.ones((T, 1), np.float32))
    d = device_inputs(inp)
    plan1 = moe1.alloc_plan(T)
    ws1 = moe1.alloc_workspace(T)
    moe1.plan(T, plan1, topk_idx=d1["topk_idx"], ws=ws1)
    y_shared = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")  # [T, 1, H]: token order
    moe1.ffn(T, d["x"], d["x_sf"], prepared(moe1, d1), plan1, y_shared, ws1)
    residual = torch.randn((T, H), device="cuda").to(torch.bfloat16)
    moe = make_moe(sh)
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = moe.alloc_workspace(T)
    moe.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], d["logits"], prepared(moe, d), out, ws,
                routing_bias=torch.from_numpy(bias).cuda(), shared=y_shared, residual=residual)
    torch.cuda.synchronize()
    geo1 = geometry(sh1)
    shared_ref = oracle.forward(geo1, inp["x"], inp["x_sf"], inp1["w13"], inp1["w13_sf"], inp1["w2"], inp1["w2_sf"],
                                topk_idx=np.zeros((T, 1), np.int64), topk_weights=np.ones((T, 1)))["y_rows"]
    ref = oracle.forward(geometry(sh), inp["x"], inp["x_sf"], inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"],
                         logits=inp["logits"], routing_bias=bias, shared=shared_ref,
                         residual=residual.float().cpu().numpy().astype(np.float64))
    assert np.array_equal(d["topk_idx"].cpu().numpy(), ref["topk_idx"])
    compare_out(out, ref["out"])


@pytest.mark.parametrize("fmt", ["fp8_block128", "w4a8_mx"])
def test_timed_legs_match_untimed(fmt):
    """moe_ffn_gate_up_timed / moe_ffn_down_timed write what the untimed legs write,
    and their events enclose a positive kernel time shorter than the two events
    recorded around the launch in the stream."""
    sh = small("timed_" + fmt, 51, 200, 512, 256, 8, 2, fmt)
    inp = moe_synth.make_inputs(sh)
    moe = make_moe(sh)
    d = device_inputs(inp)
    w = prepared(moe, d)
    T = sh.tokens
    plan = moe.alloc_plan(T)
    ws = moe.alloc_workspace(T)
    moe.plan(T, plan, topk_idx=d["topk_idx"], ws=ws)
    outs = []
    for timed in (False, True):
        h, hsf = moe.alloc_intermediate(T)
        y = torch.zeros((T * sh.topk, sh.hidden), dtype=torch.bfloat16, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)] if timed else None
        if timed:
            for e in ev[:4]:
                e.record()  # creates the events
            ev[4].record()
        moe.ffn_gate_up(T, d["x"], d["x_sf"], w, plan, h, hsf, events=ev[0:2] if timed else None)
        moe.ffn_down(T, h, hsf, w, plan, y, events=ev[2:4] if timed else None)
        if timed:
            ev[5].record()
        torch.cuda.synchronize()
        outs.append((h.clone(), y.clone()))
        if timed:
            g, dn, around = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3]), ev[4].elapsed_time(ev[5])
            assert 0 < g and 0 < dn and g + dn <= around, (g, dn, around)
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_out_fp32_combine():
    """moe_config.out_fp32: the combine writes its fp32 sum unrounded; rounding it to
    bf16 (RNE) gives the bf16 output bit for bit, and it meets the output contract
    against the oracle."""
    sh = small("out_f32", 41, 90, 512, 256, 8, 3, "fp8_block128")
    inp = moe_synth.make_inputs(sh)
    d = device_inputs(inp)
    m16 = make_moe(sh)
    m32 = make_moe(sh, out_fp32=True)
    w = prepared(m16, d)
    T = sh.tokens
    o16 = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty((T, sh.hidden), dtype=torch.float32, device="cuda")
    m16.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], None, w, o16, m16.alloc_workspace(T))
    m32.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], None, w, o32, m32.alloc_workspace(T))
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    ref = oracle.forward(geometry(sh), inp["x"], inp["x_sf"], inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"],
                         topk_idx=inp["topk_idx"], topk_weights=inp["topk_weights"])
    compare_out(o32, ref["out"])
