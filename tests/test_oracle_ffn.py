"""Pins of the oracle's FFN arithmetic: hand-worked closed forms, a dense
no-routing equivalence, E=1 against an independent torch float64 chain,
routing invariances and requantisation properties (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import moe_synth
from oracle import (Geometry, build_plan, combine, expert_rows, forward, forward_tokens, mx_exponent,
                    requant_fp8_block128, requant_mx, requant_nvfp4, silu, swiglu_clamped)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def test_silu_anchor_values():
    for z, v in GOLD["silu"]["points"]:
        assert abs(silu(np.array([z]))[0] - v) <= 1e-15 * max(1.0, abs(v))
    z = np.array([-800.0, -50.0, 50.0, 800.0])
    s = silu(z)
    assert np.all(np.isfinite(s))
    assert np.allclose(silu(z) - silu(-z), z, rtol=1e-15, atol=0)  # silu(z) - silu(-z) = z


def test_swiglu_clamp_sides():
    g = np.array([20.0, -20.0, 3.0])
    u = np.array([-30.0, 30.0, 2.0])
    h = swiglu_clamped(g, u, 10.0)
    # gate is clamped above only, up on both sides
    assert h[0] == silu(np.array([10.0]))[0] * -10.0
    assert h[1] == silu(np.array([-20.0]))[0] * 10.0
    assert h[2] == silu(np.array([3.0]))[0] * 2.0


def _unit_case(fmt, gate=1.0, up=1.0):
    H, I, E = 256, 128, 2
    geo = Geometry(H, I, E, 1, fmt)
    if fmt == "fp8_block128":
        one = 0x38  # E4M3 1.0
        x = np.zeros((1, H), np.uint8)
        x[0, 0] = one
        x_sf = np.ones((1, H // 128), np.float32)
        w13 = np.zeros((E, 2 * I, H), np.uint8)
        w13_sf = np.ones((E, 2, 2), np.float32)
        w2 = np.zeros((E, H, I), np.uint8)
        w2_sf = np.ones((E, 2, 1), np.float32)
        # E4M3 codes of the gate/up entries (exactly representable values)
        enc = {1.0: 0x38, 20.0: 0x5A, -30.0: 0xDF}
        w13[0, 0, 0] = enc[gate]
        w13[0, I, 0] = enc[up]
        w2[0, 5, 0] = one
    elif fmt == "bf16":
        x = np.zeros((1, H), np.uint16)
        x[0, 0] = 0x3F80
        x_sf = w13_sf = w2_sf = None
        w13 = np.zeros((E, 2 * I, H), np.uint16)
        w13[0, 0, 0] = w13[0, I, 0] = 0x3F80
        w2 = np.zeros((E, H, I), np.uint16)
        w2[0, 5, 0] = 0x3F80
    else:  # w4a8_mx
        x = np.zeros((1, H), np.uint8)
        x[0, 0] = 0x38
        x_sf = np.full((1, H // 32), 127, np.uint8)
        w13 = np.zeros((E, 2 * I, H // 2), np.uint8)
        w13[0, 0, 0] = w13[0, I, 0] = 0x02  # E2M1 1.0 in the low nibble = element 0
        w13_sf = np.full((E, 2 * I, H // 32), 127, np.uint8)
        w2 = np.zeros((E, H, I // 2), np.uint8)
        w2[0, 5, 0] = 0x02
        w2_sf = np.full((E, H, I // 32), 127, np.uint8)
    ids = np.array([[0]])
    w = np.array([[1.0]], np.float32)
    return geo, (x, x_sf, w13, w13_sf, w2, w2_sf), ids, w


def test_e4m3_codes_used_by_hand_cases():
    from oracle import e4m3_decode
    assert e4m3_decode(np.array([0x38, 0x5A, 0xDF], np.uint8)).tolist() == [1.0, 20.0, -30.0]


@pytest.mark.parametrize("key,gate,up", [("unit_path_fp8", 1.0, 1.0), ("clamp_path_fp8", 20.0, -30.0)])
def test_hand_case_fp8(key, gate, up):
    gold = GOLD[key]
    geo, ops, ids, w = _unit_case("fp8_block128", gate, up)
    res = forward(geo, *ops, topk_idx=ids, topk_weights=w)
    out = res["out"]
    assert out[0, 5] == pytest.approx(gold["out_0_5"], rel=1e-15, abs=0)
    assert np.count_nonzero(out) == 1
    h = swiglu_clamped(np.array([[gate] + [0.0] * 127]), np.array([[up] + [0.0] * 127]), 10.0)
    assert h[0, 0] == pytest.approx(gold["h0"], rel=1e-15)
    _, s = requant_fp8_block128(h)
    assert s[0, 0] == gold["scale0"]


def test_hand_case_bf16():
    geo, ops, ids, w = _unit_case("bf16")
    out = forward(geo, *ops, topk_idx=ids, topk_weights=w)["out"]
    assert out[0, 5] == GOLD["unit_path_bf16"]["out_0_5"]
    assert np.count_nonzero(out) == 1


def test_hand_case_mx():
    geo, ops, ids, w = _unit_case("w4a8_mx")
    out = forward(geo, *ops, topk_idx=ids, topk_weights=w)["out"]
    assert out[0, 5] == GOLD["unit_path_mx"]["out_0_5"]
    assert np.count_nonzero(out) == 1
    h = np.zeros((1, 128))
    h[0, 0] = silu(np.array([1.0]))[0]
    _, b = requant_mx(h)
    assert b[0, 0] == GOLD["unit_path_mx"]["scale_byte0"]


def test_mx_exponent_brute_force():
    rng = np.random.default_rng(3)
    a = np.concatenate([np.exp(rng.uniform(-90, 90, 3000)), 448.0 * 2.0 ** np.arange(-20, 20),
                        np.nextafter(448.0 * 2.0 ** np.arange(-20, 20), 0), [0.0, 1e-45, 3e38]])
    got = mx_exponent(a)
    for v, e in zip(a, got):
        if v == 0:
            assert e == -127
            continue
        cand = [x for x in range(-127, 128) if 448.0 * 2.0 ** x >= v]
        assert e == (min(cand) if cand else 127)


def test_requant_fp8_idempotent_on_grid():
    rng = np.random.default_rng(4)
    grid = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    grid = grid[~np.isnan(grid)]
    q = rng.choice(grid, size=(5, 256))
    q[:, 0], q[:, 128] = 448.0, -448.0  # each block's amax is 448 so that s is the block scale exactly
    s = np.array([2.0 ** -7, 0.75, 3.0, 1.0, 0.125])
    h = q * s[:, None]
    hd, sc = requant_fp8_block128(h)
    assert np.array_equal(hd, h)
    assert np.array_equal(sc, np.repeat(s[:, None], 2, axis=1))


def test_requant_zero_block():
    h = np.zeros((2, 256))
    h[1, 130] = 1.0
    hd, s = requant_fp8_block128(h)
    assert s[0].tolist() == [1.0, 1.0] and s[1, 0] == 1.0
    assert hd[1, 130] == pytest.approx(1.0, rel=2 ** -4)
    hd2, b = requant_mx(h)
    assert b[0, 0] == 0 and np.all(hd2[0] == 0)


def _small_inputs(fmt, T=24, H=256, I=128, E=4, k=2, seed=7, x_scale=1.0):
    routing = "from_logits" if fmt == "w4a8_mx" else "precomputed"
    sh = moe_synth.MoEShape("t", seed, T, H, I, E, k, fmt, routing, x_scale=x_scale)
    return sh, moe_synth.make_inputs(sh)


def _ops(inp):
    return inp["x"], inp["x_sf"], inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"]


def _gs(inp):
    """The NVFP4 per-expert global scales as forward()/dequant_expert() keywords."""
    return {"w13_gs": inp["w13_gs"], "w2_gs": inp["w2_gs"]} if "w13_gs" in inp else {}


def _cs(inp, e=None):
    """NVFP4 x NVFP4: the per-expert input scales of the intermediate (all, or expert e's)."""
    if "c_scales" not in inp:
        return None
    return inp["c_scales"] if e is None else inp["c_scales"][e]


@pytest.mark.parametrize("fmt", ["fp8_block128", "bf16", "w4a8_mx", "nvfp4_w4a16", "nvfp4"])
def test_dense_equivalence_topk_equals_E(fmt):
    sh, inp = _small_inputs(fmt, E=3, k=3)
    geo = Geometry(sh.hidden, sh.inter, sh.experts, sh.topk, fmt)
    T = sh.tokens
    ids = np.tile(np.arange(3), (T, 1))
    w = np.full((T, 3), 1.0 / 3)
    res = forward(geo, *_ops(inp), topk_idx=ids, topk_weights=w, c_scales=_cs(inp), **_gs(inp))
    # no routing code: every expert over every token, averaged
    from oracle import dequant_activations, dequant_expert
    xd = dequant_activations(geo, inp["x"], inp["x_sf"])
    dense = np.zeros((T, sh.hidden))
    for e in range(3):
        w13d, w2d = dequant_expert(geo, inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"], e, **_gs(inp))
        dense += expert_rows(geo, xd, w13d, w2d, _cs(inp, e)) / 3
    assert np.allclose(res["out"], dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


# ---- independent torch float64 chain for E = 1, k = 1 (the textbook dense FFN)
_E2M1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
                     dtype=torch.float64)


def _torch_deq(fmt, codes, scales, br=1, bc=128, fp4=False):
    c = torch.from_numpy(np.ascontiguousarray(codes))
    if fmt == "bf16":
        return c.view(torch.bfloat16).to(torch.float64)
    if fmt == "fp8_block128":
        v = c.view(torch.float8_e4m3fn).to(torch.float64)
        s = torch.from_numpy(scales).to(torch.float64)
        return v * s.repeat_interleave(br, 0).repeat_interleave(bc, 1)
    if fp4:
        v = torch.stack([_E2M1[(c & 15).long()], _E2M1[(c >> 4).long()]], dim=-1).reshape(c.shape[0], -1)
    else:
        v = c.view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64)
    return v * s.repeat_interleave(32, 1)


def _torch_nvfp4(packed, block_scales, gs):
    c = torch.from_numpy(np.ascontiguousarray(packed))
    v = torch.stack([_E2M1[(c & 15).long()], _E2M1[(c >> 4).long()]], dim=-1).reshape(c.shape[0], -1)
    s = torch.from_numpy(np.ascontiguousarray(block_scales)).view(torch.float8_e4m3fn).to(torch.float64)
    return v * s.repeat_interleave(16, 1) * float(gs)


def _torch_e2m1_round(v):
    """Nearest signed E2M1 value, ties to the even code, saturated at 6 (torch)."""
    mags = _E2M1[:8]
    a = v.abs().clamp(max=6.0)
    d = (a.unsqueeze(-1) - mags).abs()
    best = d.min(-1, keepdim=True).values
    cand = d == best
    code = torch.where(cand.sum(-1) > 1, torch.argmax((cand & (torch.arange(8) % 2 == 0)).to(torch.int64), -1),
                       torch.argmax(cand.to(torch.int64), -1))
    return torch.copysign(mags[code], v)


def _torch_requant(fmt, h, c=None):
    if fmt in ("bf16", "nvfp4_w4a16"):
        return h.to(torch.bfloat16).to(torch.float64)
    if fmt == "nvfp4":  # per 16: E4M3 block scale of amax / (6 c), E2M1 codes of h / (s c); returns codes * s
        R, C = h.shape
        hb = h.reshape(R, C // 16, 16)
        s = (hb.abs().amax(-1, keepdim=True) / (6 * c)).clamp(max=448).to(torch.float32).to(
            torch.float8_e4m3fn).to(torch.float64)
        den = s * c
        q = torch.where(den > 0, _torch_e2m1_round(hb / torch.where(den > 0, den, torch.ones_like(den))),
                        torch.zeros_like(hb))
        return (q * s).reshape(R, C)
    R, C = h.shape
    if fmt == "fp8_block128":
        hb = h.reshape(R, C // 128, 128)
        a = hb.abs().amax(-1, keepdim=True)
        s = (a / 448).to(torch.float32).to(torch.float64)
        s = torch.where(a == 0, torch.ones_like(s), s)
    else:
        hb = h.reshape(R, C // 32, 32)
        a = hb.abs().amax(-1, keepdim=True)
        e = torch.ceil(torch.log2(a / 448)).clamp(-127, 127)
        e = torch.where(448 * torch.exp2(e - 1) >= a, e - 1, e)  # guard log2 rounding up
        e = torch.where(448 * torch.exp2(e) < a, e + 1, e)  # guard log2 rounding down
        s = torch.where(a == 0, torch.full_like(a, 2.0 ** -127), torch.exp2(e))
    q = (hb / s).clamp(-448, 448).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * s).reshape(R, C)


@pytest.mark.parametrize("fmt,x_scale", [("fp8_block128", 1.0), ("fp8_block128", 20.0), ("bf16", 1.0),
                                         ("bf16", 20.0), ("w4a8_mx", 1.0), ("w4a8_mx", 20.0), ("nvfp4_w4a16", 1.0),
                                         ("nvfp4_w4a16", 20.0), ("nvfp4", 1.0), ("nvfp4", 20.0)])
def test_single_expert_matches_torch_chain(fmt, x_scale):
    sh, inp = _small_inputs(fmt, T=16, E=1, k=1, x_scale=x_scale, H=256, I=256)
    geo = Geometry(sh.hidden, sh.inter, 1, 1, fmt)
    ids = np.zeros((sh.tokens, 1), np.int64)
    w = np.ones((sh.tokens, 1), np.float32)
    out = forward(geo, *_ops(inp), topk_idx=ids, topk_weights=w, c_scales=_cs(inp), **_gs(inp))["out"]
    H, I = sh.hidden, sh.inter
    if fmt == "nvfp4":  # both operands E2M1 x E4M3 per 16; each leg times its per-expert output scale
        x = _torch_nvfp4(inp["x"], inp["x_sf"], 1.0)
        w13 = _torch_nvfp4(inp["w13"][0], inp["w13_sf"][0], 1.0) * float(inp["w13_gs"][0])
        w2 = _torch_nvfp4(inp["w2"][0], inp["w2_sf"][0], 1.0) * float(inp["w2_gs"][0])
    elif fmt == "nvfp4_w4a16":
        x = _torch_deq("bf16", inp["x"], None)
        w13 = _torch_nvfp4(inp["w13"][0], inp["w13_sf"][0], inp["w13_gs"][0])
        w2 = _torch_nvfp4(inp["w2"][0], inp["w2_sf"][0], inp["w2_gs"][0])
    elif fmt == "w4a8_mx":
        x = _torch_deq(fmt, inp["x"], inp["x_sf"])
        w13 = _torch_deq(fmt, inp["w13"][0], inp["w13_sf"][0], fp4=True)
        w2 = _torch_deq(fmt, inp["w2"][0], inp["w2_sf"][0], fp4=True)
    else:
        x = _torch_deq(fmt, inp["x"], inp["x_sf"], 1, 128)
        w13 = _torch_deq(fmt, inp["w13"][0], None if inp["w13_sf"] is None else inp["w13_sf"][0], 128, 128)
        w2 = _torch_deq(fmt, inp["w2"][0], None if inp["w2_sf"] is None else inp["w2_sf"][0], 128, 128)
    g = x @ w13[:I].T
    u = x @ w13[I:].T
    if x_scale > 1:
        assert (g > 10).any() and (u.abs() > 10).any()  # the clamp fires
    h = torch.nn.functional.silu(torch.clamp(g, max=10.0)) * torch.clamp(u, -10.0, 10.0)
    ref = (_torch_requant(fmt, h, None if fmt != "nvfp4" else float(inp["c_scales"][0])) @ w2.T).numpy()
    err = np.abs(out - ref).max() / np.abs(ref).max()
    assert err < 1e-9, err


def test_invariances():
    sh, inp = _small_inputs("fp8_block128", T=20, E=5, k=3, seed=9)
    geo = Geometry(sh.hidden, sh.inter, sh.experts, sh.topk, sh.fmt)
    ops = _ops(inp)
    ids, w = inp["topk_idx"].copy(), inp["topk_weights"].astype(np.float64)
    ids[2, 1] = -1  # a masked slot
    base = forward(geo, *ops, topk_idx=ids, topk_weights=w)["out"]
    # token permutation permutes rows exactly
    perm = np.random.default_rng(0).permutation(sh.tokens)
    xs = (ops[0][perm], ops[1][perm]) + ops[2:]
    o = forward(geo, *xs, topk_idx=ids[perm], topk_weights=w[perm])["out"]
    assert np.allclose(o, base[perm], rtol=1e-12, atol=1e-12)  # BLAS blocking may reorder sums
    # slot permutation: same sum up to float order
    sp = [2, 0, 1]
    o = forward(geo, *ops, topk_idx=ids[:, sp], topk_weights=w[:, sp])["out"]
    assert np.allclose(o, base, rtol=1e-13, atol=1e-13)
    # relabelling experts together with their weights leaves the output unchanged
    rl = np.array([3, 0, 4, 1, 2])  # expert e -> rl[e]
    inv = np.argsort(rl)
    w13, w13s, w2, w2s = ops[2][inv], ops[3][inv], ops[4][inv], ops[5][inv]
    ids2 = np.where(ids >= 0, rl[np.maximum(ids, 0)], -1)
    o = forward(geo, ops[0], ops[1], w13, w13s, w2, w2s, topk_idx=ids2, topk_weights=w)["out"]
    assert np.array_equal(o, base)
    # linear in the router weights (x2 is exact)
    o = forward(geo, *ops, topk_idx=ids, topk_weights=2 * w)["out"]
    assert np.array_equal(o, 2 * base)
    # duplicate tokens give identical rows
    xs = (ops[0][[4, 4]], ops[1][[4, 4]]) + ops[2:]
    o = forward(geo, *xs, topk_idx=ids[[4, 4]], topk_weights=w[[4, 4]])["out"]
    assert np.array_equal(o[0], o[1]) and np.allclose(o[0], base[4], rtol=1e-12, atol=1e-12)


def test_forward_tokens_matches_forward():
    for fmt in ("fp8_block128", "bf16", "w4a8_mx"):
        sh, inp = _small_inputs(fmt, T=12, E=4, k=2, seed=12)
        geo = Geometry(sh.hidden, sh.inter, sh.experts, sh.topk, fmt)
        res = forward(geo, *_ops(inp), topk_idx=inp.get("topk_idx"), topk_weights=inp.get("topk_weights"),
                      logits=inp["logits"])
        toks = [0, 5, 11, 3]
        part = forward_tokens(geo, toks, *_ops(inp), res["topk_idx"], res["topk_weights"])
        assert np.allclose(part, res["out"][toks], rtol=1e-12, atol=1e-12)


def test_combine_masked_token_is_zero():
    y = np.arange(12.0).reshape(3, 4)
    pr = np.array([0, -1, -1, -1, 2, 1])
    out = combine(y, np.array([[0.5, 9.0], [1.0, 1.0], [0.25, 2.0]]), pr, 4)
    assert out[1].tolist() == [0, 0, 0, 0]
    assert np.allclose(out[0], 0.5 * y[0])
    assert np.allclose(out[2], 0.25 * y[2] + 2.0 * y[1])


def test_combine_addends_hand_case():
    # out[t] = sum of the weighted slot rows, then + shared[t] + residual[t]
    y = np.arange(12.0).reshape(3, 4)
    pr = np.array([0, -1, -1, -1, 2, 1])
    w = np.array([[0.5, 9.0], [1.0, 1.0], [0.25, 2.0]])
    shared = np.array([[1.0, 0, 0, 0], [0, 2.0, 0, 0], [0, 0, 3.0, 0]])
    residual = np.full((3, 4), -0.5)
    out = combine(y, w, pr, 4, (shared, residual))
    assert out[1].tolist() == [-0.5, 1.5, -0.5, -0.5]   # masked token: the addends only
    assert out[0].tolist() == (0.5 * y[0] + shared[0] - 0.5).tolist()
    assert out[2].tolist() == (0.25 * y[2] + 2.0 * y[1] + shared[2] - 0.5).tolist()
    assert np.array_equal(combine(y, w, pr, 4, (None, None)), combine(y, w, pr, 4))


# ---- NVFP4 (E2M1 values, E4M3 scale per 16 along K, fp32 global scale per expert)
def test_nvfp4_dequant_hand_values():
    from oracle import dequant_nvfp4
    # one row of 32 elements: bytes 0x21, 0xF7 then zeros; block scales 1.5 (E4M3 0x3C) and 0.25 (0x28)
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 0], packed[0, 1] = 0x21, 0xF7   # nibbles 1, 2, 7, 15 -> 0.5, 1.0, 6.0, -6.0
    packed[0, 8] = 0x3B                       # elements 16, 17: nibbles 11, 3 -> -1.5, 1.5
    scales = np.array([[0x3C, 0x28]], np.uint8)
    v = dequant_nvfp4(packed, scales, 0.5)
    want = np.zeros(32)
    want[:4] = np.array([0.5, 1.0, 6.0, -6.0]) * 1.5 * 0.5
    want[16:18] = np.array([-1.5, 1.5]) * 0.25 * 0.5
    assert np.array_equal(v[0], want)


def test_nvfp4_forward_equals_bf16_forward_on_exact_weights():
    """With a power-of-two global scale every NVFP4 weight is a bf16 value; the
    NVFP4 path must then give exactly the BF16 path's result on those weights."""
    from oracle import dequant_nvfp4
    sh, inp = _small_inputs("nvfp4_w4a16", E=3, k=2)
    inp["w13_gs"] = np.full(3, 2.0 ** -5, np.float32)
    inp["w2_gs"] = np.full(3, 2.0 ** -4, np.float32)
    to_bf16 = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w13b = np.stack([to_bf16(dequant_nvfp4(inp["w13"][e], inp["w13_sf"][e], inp["w13_gs"][e])) for e in range(3)])
    w2b = np.stack([to_bf16(dequant_nvfp4(inp["w2"][e], inp["w2_sf"][e], inp["w2_gs"][e])) for e in range(3)])
    geo_n = Geometry(sh.hidden, sh.inter, 3, 2, "nvfp4_w4a16")
    geo_b = Geometry(sh.hidden, sh.inter, 3, 2, "bf16")
    a = forward(geo_n, *_ops(inp), topk_idx=inp["topk_idx"], topk_weights=inp["topk_weights"], **_gs(inp))["out"]
    b = forward(geo_b, inp["x"], None, w13b, None, w2b, None, topk_idx=inp["topk_idx"],
                topk_weights=inp["topk_weights"])["out"]
    assert np.array_equal(a, b)


def test_nvfp4_down_global_scale_is_linear():
    sh, inp = _small_inputs("nvfp4_w4a16", E=3, k=2)
    geo = Geometry(sh.hidden, sh.inter, 3, 2, "nvfp4_w4a16")
    kw = dict(topk_idx=inp["topk_idx"], topk_weights=inp["topk_weights"])
    a = forward(geo, *_ops(inp), w13_gs=inp["w13_gs"], w2_gs=inp["w2_gs"], **kw)["out"]
    b = forward(geo, *_ops(inp), w13_gs=inp["w13_gs"], w2_gs=inp["w2_gs"] * 4, **kw)["out"]
    assert np.array_equal(b, 4 * a)


# ---- NVFP4 x NVFP4: E2M1 rounding and the requantisation against c_input_scales
def test_round_e2m1_brute_force():
    """RNE onto the signed E2M1 values with saturation, against a nearest-value
    search that breaks ties toward the even code (mantissa bit 0)."""
    from oracle import round_e2m1_sat
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # codes 0..7; the mantissa bit is the code's low bit
    rng = np.random.default_rng(8)
    vals = np.concatenate([rng.uniform(-8, 8, 4000), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 100.0],
                           -np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])])
    got = round_e2m1_sat(vals)
    for v, g in zip(vals, got):
        a = min(abs(v), 6.0)
        d = [abs(a - m) for m in mags]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert g == np.copysign(mags[c], v), (v, g)


def test_requant_nvfp4_hand_case():
    gold = GOLD["requant_nvfp4_block"]
    h = np.array([gold["h"] + [0.0] * 16])  # two blocks: the hand block and an all-zero block
    hq, s = requant_nvfp4(h, gold["c"])
    assert s[0, 0] == gold["scale"] and s[0, 1] == 0.0
    assert hq[0, :16].tolist() == gold["q_times_s"]
    assert np.all(hq[0, 16:] == 0)


def test_requant_nvfp4_grid_saturation_and_underflow():
    from oracle import e4m3_decode
    rng = np.random.default_rng(9)
    c = 0.01
    # values already on the grid (E2M1 codes times an E4M3 block scale whose block
    # reaches 6 * s * c) come back unchanged
    e4 = e4m3_decode(np.arange(0x08, 0x78, dtype=np.uint8))  # normal E4M3 values 2^-6 .. 240
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    for _ in range(20):
        s = rng.choice(e4)
        q = rng.choice(mags, 16) * rng.choice([-1, 1], 16)
        q[rng.integers(16)] = 6.0
        hq, sc = requant_nvfp4((q * s * c)[None, :], c)
        assert sc[0, 0] == s and np.array_equal(hq[0], q * s)
    # a block whose scale would exceed 448 saturates the scale at 448 and the codes at 6
    h = np.full((1, 16), 6.0 * 1000.0 * c)
    hq, sc = requant_nvfp4(h, c)
    assert sc[0, 0] == 448.0 and np.all(hq == 6.0 * 448.0)
    # a block too small for the smallest E4M3 scale becomes zero
    hq, sc = requant_nvfp4(np.full((1, 16), 1e-9), c)
    assert sc[0, 0] == 0.0 and np.all(hq == 0)
