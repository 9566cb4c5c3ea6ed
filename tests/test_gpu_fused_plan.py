"""The routing plan built inside the gate_up launch (moe_plan_ffn_gate_up,
moe_config.fuse_plan): every workgroup of a weight-bound gate_up launch counts
the ids and gathers its own rows, and the launch writes the plan.  Plan buffers
and the intermediate must equal moe_plan + moe_ffn_gate_up bit for bit, and the
forward pass moe_forward's without it.  Covered: every format, int32 and int64
ids, masked / bad / duplicate ids and a token without a valid slot, routing
from logits, 1024 experts at the 8192-pair limit (fuse_plan = 2 forces the
in-launch form where the cost rule would keep the plan kernel), one token, repeated calls on
one set of plan buffers, the prefill regime (where the call launches the plan
kernel itself), the fused combine alongside, and the full decode and W4A8
workloads."""
import numpy as np
import pytest
import torch

import moe_synth
from gpu_util import device_inputs, make_moe, prepared

pytestmark = pytest.mark.gpu

SENTINEL = -7777
PLAN_KEYS = ("expert_counts", "expert_start_indices", "expert_ids", "num_active_experts", "src_info", "pair_row",
             "status", "combine_counters")

CASES = [
    ("fp8", dict(T=100, H=512, I=256, E=8, k=4, fmt="fp8_block128"), 64),
    ("fp8_ids32", dict(T=100, H=512, I=256, E=8, k=4, fmt="fp8_block128"), 32),
    ("bf16", dict(T=96, H=512, I=320, E=4, k=2, fmt="bf16"), 64),
    ("mx_logits", dict(T=80, H=576, I=352, E=6, k=3, fmt="w4a8_mx", routing="from_logits"), 64),
    ("nvfp4", dict(T=100, H=512, I=320, E=8, k=4, fmt="nvfp4_w4a16"), 64),
    ("nvfp4x4", dict(T=100, H=512, I=320, E=8, k=4, fmt="nvfp4"), 64),
    ("fp8_1024_experts", dict(T=1024, H=256, I=128, E=1024, k=8, fmt="fp8_block128"), 64),
    ("fp8_one_token", dict(T=1, H=256, I=128, E=8, k=4, fmt="fp8_block128"), 64),
]


def _shape(name, kw, seed=17):
    kw = dict(kw)
    return moe_synth.MoEShape(name, seed, kw.pop("T"), kw.pop("H"), kw.pop("I"), kw.pop("E"), kw.pop("k"),
                              kw.pop("fmt"), kw.pop("routing", "precomputed"))


def _odd_ids(inp, sh):
    """Masked slots, ids outside [0, E), a duplicate expert and a token with no valid slot."""
    ids = inp["topk_idx"].copy()
    if sh.tokens >= 12:
        ids[::9, 0] = -1
        ids[5, :] = -1
        ids[2, 1 % sh.topk] = sh.experts + 3  # bad: counted in status, masked
        ids[4, 0] = -5                        # bad
        ids[11, 1 % sh.topk] = ids[11, 0]     # duplicate within a token
    return ids


def _plan_buffers(m, T):
    plan = m.alloc_plan(T)
    for v in plan.values():
        v.fill_(SENTINEL)
    return plan


def _intermediate(m, T):
    h, hsf = m.alloc_intermediate(T)
    h.view(torch.uint8).fill_(0xA5)
    if hsf is not None:
        hsf.view(torch.uint8).fill_(0xA5)
    return h, hsf


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _run_both(sh, inp, d, m, regime_note=""):
    """(separate, in-launch) plan buffers, intermediates and routing outputs."""
    T = sh.tokens
    w = prepared(m, d)
    ws = m.alloc_workspace(T)
    res = []
    for fused in (False, True):
        plan = _plan_buffers(m, T)
        h, hsf = _intermediate(m, T)
        kw = {}
        if sh.routing == "precomputed":
            kw["topk_idx"] = d["topk_idx"]
        else:
            kw.update(routing_logits=d["logits"],
                      topk_idx_out=torch.full_like(d["topk_idx"], SENTINEL),
                      topk_weights_out=torch.full_like(d["topk_weights"], float("nan")))
        if fused:
            m.plan_ffn_gate_up(T, d["x"], d["x_sf"], w, plan, h, hsf, ws=ws, **kw)
        else:
            m.plan(T, plan, ws=ws, **kw)
            m.ffn_gate_up(T, d["x"], d["x_sf"], w, plan, h, hsf)
        torch.cuda.synchronize()
        res.append((plan, h, hsf, kw))
    return res


def _assert_equal(res, name):
    (p0, h0, s0, k0), (p1, h1, s1, k1) = res
    for key in PLAN_KEYS:
        assert torch.equal(p0[key], p1[key]), f"{name}: plan[{key}] differs"
    n = int(p1["expert_start_indices"][-1].item())  # rows of valid pairs; src_info past them is not written
    assert (p1["src_info"][:n] != SENTINEL).all() and (p1["pair_row"] != SENTINEL).all(), f"{name}: plan entries unwritten"
    assert _same(h0, h1), f"{name}: h differs"
    if s0 is not None:
        assert _same(s0, s1), f"{name}: h_sf differs"
    if "topk_idx_out" in k0:
        assert torch.equal(k0["topk_idx_out"], k1["topk_idx_out"])
        assert torch.equal(k0["topk_weights_out"], k1["topk_weights_out"])


@pytest.mark.parametrize("name,kw,bits", CASES, ids=[c[0] for c in CASES])
def test_plan_in_gate_up_equals_separate(name, kw, bits):
    sh = _shape(name, kw)
    print(f"[fused-plan] {name} ids{bits}", flush=True)
    inp = moe_synth.make_inputs(sh)
    ids = _odd_ids(inp, sh) if sh.routing == "precomputed" else None
    d = device_inputs(inp, topk_idx=ids, idx_dtype=torch.int64 if bits == 64 else torch.int32)
    m = make_moe(sh, tile_regime="decode", topk_idx_bits=bits, fuse_plan=2)  # in-launch wherever possible
    res = _run_both(sh, inp, d, m)
    _assert_equal(res, name)
    if ids is not None and sh.tokens >= 12:
        assert int(res[1][0]["status"].item()) == 2
        assert (res[1][0]["pair_row"].view(sh.tokens, sh.topk)[5] == -1).all()


def test_repeated_calls_on_one_plan():
    """Two calls on the same plan buffers, the second with different routing and
    fewer active experts: nothing of the first call's plan may survive."""
    sh = _shape("fused_plan_repeat", dict(T=120, H=512, I=256, E=12, k=3, fmt="fp8_block128"))
    inp = moe_synth.make_inputs(sh)
    T, k = sh.tokens, sh.topk
    m = make_moe(sh, tile_regime="decode", fuse_plan=2)
    d = device_inputs(inp)
    w = prepared(m, d)
    ws = m.alloc_workspace(T)
    pa, pb = _plan_buffers(m, T), _plan_buffers(m, T)
    ha, hsa = _intermediate(m, T)
    hb, hsb = _intermediate(m, T)
    rng = np.random.default_rng(9)
    for call in range(2):
        hi = sh.experts if call == 0 else 5
        ids = torch.from_numpy(rng.integers(-1, hi, size=(T, k))).cuda()
        m.plan(T, pa, topk_idx=ids, ws=ws)
        m.ffn_gate_up(T, d["x"], d["x_sf"], w, pa, ha, hsa)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in ev:
            e.record()
        m.plan_ffn_gate_up(T, d["x"], d["x_sf"], w, pb, hb, hsb, topk_idx=ids, ws=ws, events=ev if call else None)
        torch.cuda.synchronize()
        for key in PLAN_KEYS:
            assert torch.equal(pa[key], pb[key]), f"call {call}: plan[{key}]"
        n = int(pa["expert_start_indices"][-1].item())
        assert _same(ha[:n], hb[:n]) and _same(hsa[:n], hsb[:n]), f"call {call}: h"
    assert ev[0].elapsed_time(ev[1]) > 0


def test_prefill_regime_launches_the_plan_itself():
    """Outside the weight-bound regime the call is moe_plan then moe_ffn_gate_up."""
    sh = _shape("fused_plan_prefill", dict(T=300, H=896, I=384, E=4, k=2, fmt="fp8_block128"))
    inp = moe_synth.make_inputs(sh)
    d = device_inputs(inp, topk_idx=_odd_ids(inp, sh))
    m = make_moe(sh, tile_regime="prefill", fuse_plan=2)
    _assert_equal(_run_both(sh, inp, d, m), "prefill")


CFG = [("fp8", dict(T=100, H=512, I=256, E=8, k=4, fmt="fp8_block128")),
       ("mx_logits", dict(T=80, H=576, I=352, E=6, k=3, fmt="w4a8_mx", routing="from_logits")),
       ("nvfp4x4", dict(T=100, H=512, I=320, E=8, k=4, fmt="nvfp4"))]


@pytest.mark.parametrize("name,kw", CFG, ids=[c[0] for c in CFG])
@pytest.mark.parametrize("fuse_combine", [False, True])
def test_forward_with_fuse_plan(name, kw, fuse_combine):
    """moe_forward with fuse_plan (and optionally fuse_combine: two launches in all
    for precomputed routing) against moe_forward without either."""
    sh = _shape(name, kw)
    print(f"[fused-plan] forward {name} fuse_combine={fuse_combine}", flush=True)
    inp = moe_synth.make_inputs(sh)
    ids = _odd_ids(inp, sh) if sh.routing == "precomputed" else None
    T, H = sh.tokens, sh.hidden
    outs = []
    for fp, fc in ((0, False), (2, fuse_combine)):
        d = device_inputs(inp, topk_idx=ids)
        m = make_moe(sh, tile_regime="decode", fuse_combine=fc, fuse_plan=fp)
        w = prepared(m, d)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        m.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], d["logits"], w, out, m.alloc_workspace(T))
        torch.cuda.synchronize()
        outs.append((out, d["topk_idx"].clone(), d["topk_weights"].clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])


@pytest.mark.parametrize("workload", ["decode_fp8", "w4a8_mx_logits", "nvfp4x4_decode"])
def test_full_size_workloads(workload):
    """The full decode-scale workloads: plan and intermediate bit for bit, and the
    forward output of moe_forward with fuse_plan against without."""
    sh = moe_synth.WORKLOADS[workload]
    print(f"[fused-plan] {workload}: generating inputs", flush=True)
    inp = moe_synth.make_inputs(sh)
    d = device_inputs(inp)
    m = make_moe(sh, fuse_plan=2)  # in the gate_up launch even where the cost rule would not (W4A8)
    _assert_equal(_run_both(sh, inp, d, m), workload)
    T, H = sh.tokens, sh.hidden
    outs = []
    for fp in (0, 2):
        m2 = make_moe(sh, fuse_plan=fp)
        w = prepared(m2, d)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        m2.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], d["logits"], w, out,
                   m2.alloc_workspace(T))
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.isfinite(outs[1].float()).all()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("fill", [-1, 1000])
def test_no_valid_pair(fill):
    """Every slot masked (-1) or out of range: the in-launch plan has no tile to run,
    and workgroup 0 alone must still write counts, offsets, the active list, status
    and every pair_row; the forward output is zero."""
    sh = _shape("fused_plan_empty", dict(T=16, H=256, I=128, E=8, k=4, fmt="fp8_block128"))
    inp = moe_synth.make_inputs(sh)
    ids = np.full((sh.tokens, sh.topk), fill, dtype=np.int64)
    d = device_inputs(inp, topk_idx=ids)
    m = make_moe(sh, tile_regime="decode", fuse_plan=2)
    res = _run_both(sh, inp, d, m)
    _assert_equal(res, f"fill {fill}")
    plan = res[1][0]
    assert int(plan["num_active_experts"].item()) == 0 and (plan["expert_ids"] == -1).all()
    assert int(plan["status"].item()) == (0 if fill == -1 else sh.tokens * sh.topk)
    assert (plan["pair_row"] == -1).all()
    T, H = sh.tokens, sh.hidden
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    m.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], d["logits"], prepared(m, d), out,
              m.alloc_workspace(T))
    torch.cuda.synchronize()
    assert (out.float() == 0).all()
