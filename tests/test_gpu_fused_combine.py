"""The combine fused into the down GEMM's epilogue (moe_config.fuse_combine,
moe_ffn_down_combine): the tile that completes a token's valid slots reduces
that token's column block, in slot order, so the output must equal the separate
combine's bit for bit.  Covered: every format and both tile regimes, masked
slots and tokens without any valid slot, duplicate experts in a token, the
shared-expert and residual addends, fp32 output, the split entry points,
repeated calls on one plan (the plan zeroes the arrival counters each call), and
down tiles split over K (the split tail), at small sizes and the full Mixtral shape."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import compare_out, device_inputs, fwd_kwargs, geometry, make_moe, prepared

pytestmark = pytest.mark.gpu

CASES = [
    ("fp8_decode", dict(T=100, H=512, I=256, E=8, k=4, fmt="fp8_block128"), "decode"),
    ("fp8_prefill", dict(T=300, H=896, I=384, E=4, k=2, fmt="fp8_block128"), "prefill"),
    ("bf16_decode", dict(T=96, H=512, I=320, E=4, k=2, fmt="bf16"), "decode"),
    ("bf16_prefill", dict(T=200, H=448, I=256, E=3, k=2, fmt="bf16"), "prefill"),
    ("mx_logits", dict(T=80, H=576, I=352, E=6, k=3, fmt="w4a8_mx", routing="from_logits"), "decode"),
    ("nvfp4", dict(T=100, H=512, I=320, E=8, k=4, fmt="nvfp4_w4a16"), "decode"),
    ("nvfp4x4", dict(T=100, H=512, I=320, E=8, k=4, fmt="nvfp4"), "prefill"),
    # down tiles in a partial last round split over K (the split tail): the
    # completing piece's epilogue runs the fused combine
    ("fp8_prefill_split", dict(T=256, H=896, I=1152, E=4, k=2, fmt="fp8_block128"), "prefill"),
    ("bf16_prefill_split", dict(T=200, H=448, I=1088, E=3, k=2, fmt="bf16"), "prefill"),
]


def _shape(name, kw):
    kw = dict(kw)
    return moe_synth.MoEShape(name, 13, kw.pop("T"), kw.pop("H"), kw.pop("I"), kw.pop("E"), kw.pop("k"),
                              kw.pop("fmt"), kw.pop("routing", "precomputed"))


def _masked_ids(inp, sh):
    ids = inp["topk_idx"].copy()
    ids[::9, 0] = -1          # masked slots
    ids[5, :] = -1            # a token with no valid slot
    ids[7, :] = -1
    ids[11, 1 % sh.topk] = ids[11, 0]  # a duplicate expert within a token
    return ids


@pytest.mark.parametrize("name,kw,regime", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("addends", [False, True])
def test_fused_forward_equals_separate(name, kw, regime, addends):
    sh = _shape(name, kw)
    print(f"[fused] {name} {regime} addends={addends}", flush=True)
    inp = moe_synth.make_inputs(sh)
    ids = _masked_ids(inp, sh) if sh.routing == "precomputed" else None
    d = device_inputs(inp, topk_idx=ids)
    m0 = make_moe(sh, tile_regime=regime)
    m1 = make_moe(sh, tile_regime=regime, fuse_combine=True)
    w = prepared(m0, d)
    T, H = sh.tokens, sh.hidden
    g = torch.Generator(device="cpu").manual_seed(3)
    shared = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda() if addends else None
    residual = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda() if addends else None
    outs = []
    for m in (m0, m1):
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        m.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], d["logits"], w, out, m.alloc_workspace(T),
                  shared=shared, residual=residual)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.isfinite(outs[1].float()).all()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    if sh.routing == "precomputed":
        ref = oracle.forward(geometry(sh), inp["x"], inp["x_sf"], inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"],
                             topk_idx=ids, topk_weights=inp["topk_weights"], shared=None if shared is None else
                             shared.float().cpu().numpy(), residual=None if residual is None else
                             residual.float().cpu().numpy(), **fwd_kwargs(inp))
        if not addends:
            assert np.all(outs[1][5].float().cpu().numpy() == 0)
        compare_out(outs[1], ref["out"], max_rms=np.inf)


@pytest.mark.parametrize("regime", ["decode", "prefill"])
def test_fused_split_entry_points_and_repeated_calls(regime):
    """plan -> gate_up -> down_combine (timed and untimed) against plan -> gate_up ->
    down -> combine_ex, twice on the same plan buffers with different routing, and
    an fp32 output."""
    sh = _shape("fused_split", dict(T=160, H=512, I=256, E=6, k=3, fmt="fp8_block128"))
    inp = moe_synth.make_inputs(sh)
    T, H, k = sh.tokens, sh.hidden, sh.topk
    for out_f32 in (False, True):
        m = make_moe(sh, tile_regime=regime, out_fp32=out_f32)
        d = device_inputs(inp)
        w = prepared(m, d)
        plan = m.alloc_plan(T)
        ws = m.alloc_workspace(T)
        h, hsf = m.alloc_intermediate(T)
        y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
        odt = torch.float32 if out_f32 else torch.bfloat16
        rng = np.random.default_rng(5)
        for call in range(2):
            ids = rng.integers(-1, sh.experts, size=(T, k))
            ids[3, :] = -1
            idt = torch.from_numpy(ids).cuda()
            m.plan(T, plan, topk_idx=idt, ws=ws)
            m.ffn_gate_up(T, d["x"], d["x_sf"], w, plan, h, hsf)
            a = torch.full((T, H), float("nan"), dtype=odt, device="cuda")
            b = torch.full((T, H), float("nan"), dtype=odt, device="cuda")
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            for e in ev:
                e.record()
            m.ffn_down_combine(T, h, hsf, w, plan, d["topk_weights"], y, a, events=ev if call else None)
            m.ffn_down(T, h, hsf, w, plan, y)
            m.combine(T, y, d["topk_weights"], plan, b)
            torch.cuda.synchronize()
            va = a.view(torch.int32) if out_f32 else a.view(torch.int16)
            vb = b.view(torch.int32) if out_f32 else b.view(torch.int16)
            assert torch.equal(va, vb), f"call {call} out_f32={out_f32}"
            assert (a[3] == 0).all()
            assert ev[0].elapsed_time(ev[1]) > 0


def test_fused_full_mixtral_split_tail():
    """The Mixtral-shaped BF16 workload at full size: its down leg leaves 24 tiles
    for a last round of 256 slots, which split over K; the completing piece's
    epilogue runs the fused combine.  Fused and separate outputs bit for bit."""
    sh = moe_synth.WORKLOADS["mixtral_bf16"]
    print(f"[fused] {sh.name} full size", flush=True)
    inp = moe_synth.make_inputs(sh)
    d = device_inputs(inp)
    m0 = make_moe(sh)
    m1 = make_moe(sh, fuse_combine=True)
    w = prepared(m0, d)
    T, H = sh.tokens, sh.hidden
    outs = []
    for m in (m0, m1):
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        m.forward(T, d["x"], d["x_sf"], d["topk_idx"], d["topk_weights"], d["logits"], w, out, m.alloc_workspace(T))
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.isfinite(outs[1].float()).all()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
