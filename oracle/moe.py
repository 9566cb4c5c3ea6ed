"""Plain fp64 CPU oracle of the routed MoE expert-FFN path.

TEST INFRASTRUCTURE ONLY.  Imported by tests/, by ``__graft_entry__.smoke()``
and by the benchmark's CPU-baseline leg; the GPU path never imports, links or
calls it, and it shares no code with the GPU path.

It computes, one expert at a time, in float64:

1. exact dequantisation of the block-scaled operands  (``dequant_*``)
2. routing: the caller's precomputed top-k, or top-k from router logits
   (optionally ranked with a per-expert routing bias) followed by a softmax
   over the selected k                                      (``route_from_logits``)
3. the routing plan: per-expert counts, prefix-sum start offsets, the active
   expert list, and the stable (token, slot) -> row permutation  (``build_plan``)
4. the gate/up projection of each expert's rows             (``expert_rows``)
5. the clamped SwiGLU                                        (``swiglu_clamped``)
6. the intermediate requantisation, by the same stated rule as the GPU path
                                                             (``requant_*``)
7. the down projection
8. the router-weighted combine back into token order, plus optional
   addends (a shared expert's output, a residual)            (``combine``)

Sources, by page (the pages are API documentation; none prints formulas or
values, so each step states which reading it takes):

* flashinfer.megamoe.MegaMoESymmBuffer: geometry (hidden, intermediate_hidden,
  num_experts, num_topk), ``activation_clamp`` (default 10.0), and the staging
  views ``x`` (E4M3 [capacity, hidden]), ``x_sf`` (FP32 [capacity,
  hidden // 128]), ``topk_idx`` (INT64 [capacity, num_topk]) and
  ``topk_weights`` (FP32 [capacity, num_topk]).
* Struct_mega_ffn_ep_combine_send (max mega_ffn): the fused FFN's arguments —
  ``gate_up_weight`` (E, N1, K1), ``down_weight`` (E, N2, moe_dim),
  ``expert_start_indices`` (per-expert prefix-sum token offsets),
  ``expert_ids`` (active local expert ids, -1 = masked), ``src_info`` (per-row
  dispatch metadata), ``num_active_experts``, and ``clamp_activation``
  (selects the clamped L1 activation).
* flashinfer.fused_moe.MoEActivationPack: the operand encodings (DeepSeek FP8,
  MXFP8, MXFP4 x MXFP8, BF16, NVFP4 x BF16) and the routing input modes (precomputed
  ``topk_ids``/``topk_weights``; ``FromLogits`` with in-kernel top-k).
* DistributedEPCombine (max ep): ``router_weights`` scale each expert's
  contribution; ``input_tokens`` are the expert outputs; ``src_info`` records
  the origin of each received row.

Readings taken where the pages are silent (all listed in the design notes):
W13 rows [0, I) are gate and [I, 2I) are up; the activation is
silu(min(g, c)) * clamp(u, -c, c); the FP8 intermediate is requantised per
(row, 128 columns) with scale fp32(amax / 448) (1.0 for an all-zero block) and
E4M3 round-to-nearest-even with saturation; the MX intermediate uses per
(row, 32 columns) the smallest power of two 2**e with 448 * 2**e >= amax;
the BF16 intermediate is rounded to bf16; an NVFP4 weight is e2m1 * e4m3 block
scale (one per 16 along K) * the expert's fp32 global scale (the per-expert
scales of the max mega_ffn arguments), and the NVFP4 x BF16 intermediate is
rounded to bf16 like BF16's; NVFP4 x NVFP4 takes E2M1 activations with E4M3
block scales per 16, multiplies each leg by its per-expert output scale, and
requantises the intermediate per (row, 16 columns) to E2M1 with an E4M3 block
scale chosen against the expert's c_input_scales entry; rows inside an expert keep pair order
p = t * k + j; ``src_info[row] = p``; the combine sums valid slots in slot order;
ids outside [0, E) are masked slots that contribute nothing.

Parity pins (tests/test_oracle_*.py): codecs against torch's dtype tables;
hand-worked closed-form cases (tests/golden/); dense no-routing equivalence
(k = E, uniform weights); E = 1 against an independent float64 matmul chain;
brute-force routing and permutation invariants; requantisation idempotence.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .codecs import (bf16_decode, e2m1_decode_nibbles, e2m1_unpack, e4m3_decode, round_bf16, round_e2m1_sat,
                     round_e4m3_sat, ue8m0_decode)

FP8_BLOCK128 = "fp8_block128"
BF16 = "bf16"
W4A8_MX = "w4a8_mx"
NVFP4_W4A16 = "nvfp4_w4a16"
NVFP4 = "nvfp4"  # NVFP4 weights x NVFP4 activations


@dataclass(frozen=True)
class Geometry:
    """The problem statement of the MegaMoESymmBuffer page: hidden (H),
    intermediate_hidden (I), num_experts (E, local), num_topk (k)."""

    hidden: int
    inter: int
    experts: int
    topk: int
    fmt: str
    clamp: float = 10.0


# ------------------------------------------------------------------ dequant
def dequant_fp8_block(codes: np.ndarray, scales: np.ndarray, br: int, bc: int) -> np.ndarray:
    """E4M3 codes [R, C] with fp32 scales [R/br, C/bc] -> float64 values.
    (MoEActivationPack page, "DeepSeek FP8": E4M3 values with fp32 block scales;
    MegaMoESymmBuffer page: ``x_sf`` is one scale per token per 128 hidden columns.)"""
    v = e4m3_decode(codes)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), br, axis=0), bc, axis=1)
    return v * s


def dequant_mx(values: np.ndarray, scale_bytes: np.ndarray, is_fp4: bool) -> np.ndarray:
    """MX operand [R, K] (E4M3 codes, or packed E2M1 [R, K/2]) with UE8M0 bytes
    [R, K/32] -> float64 values; one power-of-two scale per 32 consecutive K.
    (MoEActivationPack page, "MXFP8" and "MXFP4 x MXFP8 (W4A8)".)"""
    if is_fp4:
        v = e2m1_decode_nibbles(e2m1_unpack(values))
    else:
        v = e4m3_decode(values)
    s = np.repeat(ue8m0_decode(scale_bytes), 32, axis=-1)
    return v * s


def dequant_nvfp4(values: np.ndarray, block_scales: np.ndarray, global_scale: float) -> np.ndarray:
    """NVFP4 operand: packed E2M1 [R, K/2] with E4M3 block scales [R, K/16] and one
    fp32 global scale -> float64 values (MoEActivationPack page, "NVFP4": packed
    uint8 values with float8_e4m3fn [., K/16] block scales; the max mega_ffn
    arguments carry one fp32 scale per expert)."""
    v = e2m1_decode_nibbles(e2m1_unpack(values))
    s = np.repeat(e4m3_decode(block_scales), 16, axis=-1)
    return v * s * float(global_scale)


def dequant_activations(geo: Geometry, x: np.ndarray, x_sf) -> np.ndarray:
    """Activations in float64.  NVFP4: codes times their E4M3 block scales; the
    activations' own global scale is not an operand of the FFN (it is part of the
    gate_up leg's per-expert output scale, the gate_up_expert_scales argument of the
    max mega_ffn page)."""
    if geo.fmt == FP8_BLOCK128:
        return dequant_fp8_block(x, x_sf, 1, 128)
    if geo.fmt == NVFP4:
        return dequant_nvfp4(x, x_sf, 1.0)
    if geo.fmt in (BF16, NVFP4_W4A16):
        return bf16_decode(x)
    if geo.fmt == W4A8_MX:
        return dequant_mx(x, x_sf, is_fp4=False)
    raise ValueError(geo.fmt)


def dequant_expert(geo: Geometry, w13, w13_sf, w2, w2_sf, e: int, w13_gs=None, w2_gs=None):
    """Expert e's gate/up weights [2I, H] and down weights [H, I] in float64.
    ``w13_gs``/``w2_gs`` are the per-expert scales of the NVFP4 formats: the weights'
    global scales (NVFP4 x BF16), or the legs' per-expert output scales (NVFP4 x
    NVFP4: gate_up_expert_scales and down_expert_scales of the max mega_ffn page).
    Either way the scale multiplies every product of the leg, so it is applied to
    the weights here."""
    if geo.fmt == FP8_BLOCK128:
        return (dequant_fp8_block(w13[e], w13_sf[e], 128, 128),
                dequant_fp8_block(w2[e], w2_sf[e], 128, 128))
    if geo.fmt == BF16:
        return bf16_decode(w13[e]), bf16_decode(w2[e])
    if geo.fmt == W4A8_MX:
        return dequant_mx(w13[e], w13_sf[e], True), dequant_mx(w2[e], w2_sf[e], True)
    if geo.fmt in (NVFP4_W4A16, NVFP4):
        return dequant_nvfp4(w13[e], w13_sf[e], w13_gs[e]), dequant_nvfp4(w2[e], w2_sf[e], w2_gs[e])
    raise ValueError(geo.fmt)


# ------------------------------------------------------------------ routing
def _nan_as_neg_inf(v: np.ndarray) -> np.ndarray:
    """A NaN router logit (or NaN ranking key) reads as -inf: it ranks below every
    number, and inside the softmax over the selected logits its term exp(-inf - m)
    is 0, so a NaN expert that is selected (k larger than the token's non-NaN
    logits) gets weight 0.  If every selected logit is -inf the softmax is 0/0 and
    the weights are NaN."""
    return np.where(np.isnan(v), -np.inf, v).astype(v.dtype)


def _selection_keys(lg: np.ndarray, bias) -> np.ndarray:
    """Ranking keys of FromLogits routing: the logits, plus the per-expert
    routing_bias of bias-aware methods when given (the sum is formed in fp32,
    the logits' precision); NaN ranks lowest."""
    key = lg if bias is None else (lg + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    return _nan_as_neg_inf(key)


def _softmax_selected(sel: np.ndarray) -> np.ndarray:
    """Softmax over the last axis of the selected logits in float64, NaN read as -inf."""
    sel = _nan_as_neg_inf(np.asarray(sel, dtype=np.float64))
    with np.errstate(invalid="ignore"):
        ex = np.exp(sel - sel.max(axis=-1, keepdims=True))
        return ex / ex.sum(axis=-1, keepdims=True)


def route_from_logits(logits: np.ndarray, k: int, bias=None):
    """FromLogits routing (MoEActivationPack page, routing_input_mode): per token
    the k experts with the largest logit, ties to the lower expert index, in that
    order; weights are a softmax over the k selected logits (float64), a NaN
    logit reading as -inf in both steps.  With a
    routing_bias (bias-aware methods on the same page) the experts are ranked by
    logit + bias, and the weights still come from the unbiased logits."""
    lg = np.asarray(logits, dtype=np.float32)
    key = _selection_keys(lg, bias)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        chosen: list[int] = []
        for _ in range(k):
            best = -1
            for e in range(E):
                if e in chosen:
                    continue
                if best < 0 or key[t, e] > key[t, best]:
                    best = e
            chosen.append(best)
        idx[t] = chosen
        w[t] = _softmax_selected(lg[t, chosen])
    return idx, w


def route_from_logits_fast(logits: np.ndarray, k: int, bias=None):
    """Same selection as ``route_from_logits`` through a stable sort (for large T)."""
    lg = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-_selection_keys(lg, bias), axis=1, kind="stable")[:, :k]
    return order.astype(np.int64), _softmax_selected(np.take_along_axis(lg, order, axis=1))


def build_plan(topk_idx: np.ndarray, num_experts: int) -> dict:
    """Routing plan (Struct_mega_ffn_ep_combine_send page, Args):

    * ``expert_counts[e]``       valid pairs routed to expert e
    * ``expert_start_indices``   E+1 exclusive prefix sums of the counts
    * ``expert_ids``             active experts (count > 0) ascending, then -1
    * ``num_active``             number of active experts
    * ``src_info[row]``          pair p = t*k + j held by that row; rows of one
                                 expert keep ascending p
    * ``pair_row[p]``            row of pair p, -1 for a masked slot
    * ``status``                 number of ids outside [0, E) other than -1
    """
    ids = np.asarray(topk_idx).astype(np.int64).reshape(-1)
    npairs = ids.size
    valid = (ids >= 0) & (ids < num_experts)
    counts = np.zeros(num_experts, dtype=np.int64)
    for p in range(npairs):
        if valid[p]:
            counts[ids[p]] += 1
    start = np.zeros(num_experts + 1, dtype=np.int64)
    for e in range(num_experts):
        start[e + 1] = start[e] + counts[e]
    src_info = np.empty(int(start[-1]), dtype=np.int64)
    pair_row = np.full(npairs, -1, dtype=np.int64)
    fill = start[:-1].copy()
    for p in range(npairs):  # ascending p: rows of an expert keep pair order
        if valid[p]:
            r = fill[ids[p]]
            src_info[r] = p
            pair_row[p] = r
            fill[ids[p]] += 1
    active = [e for e in range(num_experts) if counts[e] > 0]
    expert_ids = np.full(num_experts, -1, dtype=np.int64)
    expert_ids[:len(active)] = active
    status = int(np.sum(~valid & (ids != -1)))
    return {"expert_counts": counts, "expert_start_indices": start, "expert_ids": expert_ids,
            "num_active": len(active), "src_info": src_info, "pair_row": pair_row, "status": status}


# ------------------------------------------------------------------ FFN pieces
def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z), written so that exp never overflows."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu_clamped(g: np.ndarray, u: np.ndarray, c: float) -> np.ndarray:
    """Clamped SwiGLU (MegaMoESymmBuffer page, ``activation_clamp``;
    Struct_mega_ffn_ep_combine_send page, ``clamp_activation``):
    silu(min(g, c)) * clamp(u, -c, c)."""
    return silu(np.minimum(g, c)) * np.clip(u, -c, c)


def requant_fp8_block128(h: np.ndarray):
    """E4M3 with one fp32 scale per (row, 128 columns): s = fp32(amax / 448),
    s = 1 for an all-zero block, q = E4M3 RNE-saturated(h / s).
    Returns (dequantised values q*s, scales [R, C/128])."""
    R, C = h.shape
    hb = h.reshape(R, C // 128, 128)
    amax = np.abs(hb).max(axis=2)
    s = (amax / 448.0).astype(np.float32).astype(np.float64)
    s[amax == 0] = 1.0
    q = round_e4m3_sat(hb / s[..., None])
    return (q * s[..., None]).reshape(R, C), s


def mx_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with 448 * 2**e >= amax, clipped to [-127, 127];
    -127 for amax = 0.  Found by stepping e, no logarithm."""
    a = np.asarray(amax, dtype=np.float64).reshape(-1)
    out = np.empty(a.size, dtype=np.int64)
    for i, v in enumerate(a):
        if v == 0:
            out[i] = -127
            continue
        _, ex = np.frexp(v)  # start near the answer, then step to the exact minimum
        e = int(ex) - 9
        while 448.0 * 2.0 ** e < v:
            e += 1
        while 448.0 * 2.0 ** (e - 1) >= v:
            e -= 1
        out[i] = min(max(e, -127), 127)
    return out.reshape(np.shape(amax))


def requant_mx(h: np.ndarray):
    """MXFP8 intermediate: per (row, 32 columns) e = mx_exponent(amax),
    q = E4M3 RNE-saturated(h / 2**e).  Returns (q * 2**e, UE8M0 bytes e + 127)."""
    R, C = h.shape
    hb = h.reshape(R, C // 32, 32)
    e = mx_exponent(np.abs(hb).max(axis=2))
    sc = np.ldexp(1.0, e.astype(np.int32))
    q = round_e4m3_sat(hb / sc[..., None])
    return (q * sc[..., None]).reshape(R, C), (e + 127).astype(np.uint8)


def requant_nvfp4(h: np.ndarray, c: float):
    """NVFP4 intermediate (the NVFP4 re-quant of the max mega_ffn page, with the
    expert's c_input_scales entry c as the global scale): per (row, 16 columns)
    a = amax, block scale s = E4M3 RNE-saturated(a / (6 c)), codes
    q = E2M1 RNE-saturated(h / (s c)) (all zero where s = 0).  Returns (q * s,
    block scales [R, C/16]): the values the down projection consumes; c itself
    reaches the output through the down leg's per-expert output scale
    (down_expert_scales)."""
    R, C = h.shape
    hb = h.reshape(R, C // 16, 16)
    a = np.abs(hb).max(axis=2)
    s = round_e4m3_sat(a / (6.0 * float(c)))
    den = (s * float(c))[..., None]
    q = np.where(den > 0, round_e2m1_sat(hb / np.where(den > 0, den, 1.0)), 0.0)
    return (q * s[..., None]).reshape(R, C), s


def requant(geo: Geometry, h: np.ndarray, c_scale=None) -> np.ndarray:
    """The intermediate after its requantisation (c_scale: NVFP4's per-expert
    input scale)."""
    if geo.fmt == FP8_BLOCK128:
        return requant_fp8_block128(h)[0]
    if geo.fmt in (BF16, NVFP4_W4A16):
        return round_bf16(h)
    if geo.fmt == W4A8_MX:
        return requant_mx(h)[0]
    if geo.fmt == NVFP4:
        return requant_nvfp4(h, c_scale)[0]
    raise ValueError(geo.fmt)


def expert_rows(geo: Geometry, xd_rows: np.ndarray, w13d: np.ndarray, w2d: np.ndarray, c_scale=None) -> np.ndarray:
    """One expert's FFN over its rows: gate/up projection, clamped SwiGLU,
    intermediate requantisation, down projection (float64)."""
    I = geo.inter
    g = xd_rows @ w13d[:I].T
    u = xd_rows @ w13d[I:].T
    h = swiglu_clamped(g, u, geo.clamp)
    hd = requant(geo, h, c_scale)
    return hd @ w2d.T


def combine(y_rows: np.ndarray, topk_weights: np.ndarray, pair_row: np.ndarray, hidden: int,
            addends=()) -> np.ndarray:
    """Router-weighted combine (DistributedEPCombine page, ``router_weights``):
    out[t] = sum over valid slots j, ascending, of w[t, j] * y[row of (t, j)],
    then + each [T, H] addend (a shared expert's output fused into the combine,
    fused_shared_expert; a downstream elementwise epilogue such as a residual,
    has_epilogue_fusion: MAX mega_ffn / EP pages)."""
    w = np.asarray(topk_weights, dtype=np.float64)
    T, k = w.shape
    out = np.zeros((T, hidden), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = pair_row[t * k + j]
            if r >= 0:
                out[t] += w[t, j] * y_rows[r]
    for a in addends:
        if a is not None:
            out += np.asarray(a, dtype=np.float64).reshape(T, hidden)
    return out


# ------------------------------------------------------------------ forward
def forward(geo: Geometry, x, x_sf, w13, w13_sf, w2, w2_sf, topk_idx=None, topk_weights=None,
            logits=None, w13_gs=None, w2_gs=None, routing_bias=None, shared=None, residual=None,
            c_scales=None) -> dict:
    """Whole path over all tokens.  Routing is taken from ``topk_idx``/``topk_weights``
    when given, else computed from ``logits`` (and ``routing_bias``).  ``shared`` and
    ``residual`` ([T, H]) are added after the routed experts' weighted sum."""
    if topk_idx is None:
        topk_idx, topk_weights = route_from_logits_fast(logits, geo.topk, routing_bias)
    plan = build_plan(topk_idx, geo.experts)
    xd = dequant_activations(geo, x, x_sf)
    start, src = plan["expert_start_indices"], plan["src_info"]
    y = np.zeros((src.size, geo.hidden), dtype=np.float64)
    for e in range(geo.experts):
        r0, r1 = int(start[e]), int(start[e + 1])
        if r1 == r0:
            continue
        w13d, w2d = dequant_expert(geo, w13, w13_sf, w2, w2_sf, e, w13_gs, w2_gs)
        y[r0:r1] = expert_rows(geo, xd[src[r0:r1] // geo.topk], w13d, w2d, None if c_scales is None else c_scales[e])
    out = combine(y, topk_weights, plan["pair_row"], geo.hidden, (shared, residual))
    return {"out": out, "plan": plan, "y_rows": y, "topk_idx": np.asarray(topk_idx),
            "topk_weights": np.asarray(topk_weights, dtype=np.float64)}


def forward_tokens(geo: Geometry, tokens, x, x_sf, w13, w13_sf, w2, w2_sf, topk_idx, topk_weights,
                   w13_gs=None, w2_gs=None, c_scales=None) -> np.ndarray:
    """Outputs of selected tokens only, each computed on its own (the requantisation
    blocks lie inside one row, so a pair's result depends only on its token and
    expert).  Used to check full-size runs on a sample of tokens."""
    tokens = list(tokens)
    ids = np.asarray(topk_idx).astype(np.int64)
    w = np.asarray(topk_weights, dtype=np.float64)
    need: dict[int, list[tuple[int, int]]] = {}
    for n, t in enumerate(tokens):
        for j in range(geo.topk):
            e = int(ids[t, j])
            if 0 <= e < geo.experts:
                need.setdefault(e, []).append((n, j))
    xd = dequant_activations(geo, x[tokens], None if x_sf is None else x_sf[tokens])
    out = np.zeros((len(tokens), geo.hidden), dtype=np.float64)
    contrib = np.zeros((len(tokens), geo.topk, geo.hidden), dtype=np.float64)
    for e, lst in need.items():
        w13d, w2d = dequant_expert(geo, w13, w13_sf, w2, w2_sf, e, w13_gs, w2_gs)
        rows = np.array([n for n, _ in lst])
        y = expert_rows(geo, xd[rows], w13d, w2d, None if c_scales is None else c_scales[e])
        for (n, j), yr in zip(lst, y):
            contrib[n, j] = w[tokens[n], j] * yr
    for j in range(geo.topk):  # slot order
        out += contrib[:, j]
    return out
