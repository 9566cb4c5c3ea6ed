"""Seeded synthetic inputs for the routed MoE expert-FFN path.

This module only *produces* inputs: seeded random draws and their encoding
into the operand formats the path consumes.  It holds none of the path's own
arithmetic (no routing plan, no projection, no activation, no intermediate
requantisation, no combine).  Encodings into FP8 use torch's own dtype casts;
the E2M1 weight encoder below is a plain nearest-value search over the eight
E2M1 magnitudes.  Both the CPU oracle's tests and the GPU tests/benchmark draw
their inputs from here, so the two sides see identical bytes.

Operand formats (the encodings listed on the flashinfer.fused_moe
MoEActivationPack page and the staging views of the flashinfer.megamoe
MegaMoESymmBuffer page):

* ``fp8_block128``  x: E4M3 codes [T, H] + fp32 scales [T, H/128] (token-major);
  w13: E4M3 [E, 2I, H] + fp32 [E, 2I/128, H/128]; w2: E4M3 [E, H, I] +
  fp32 [E, H/128, I/128].
* ``bf16``          x [T, H], w13 [E, 2I, H], w2 [E, H, I] as bf16 bit patterns
  (uint16), no scales.
* ``w4a8_mx``       x: E4M3 [T, H] + UE8M0 bytes [T, H/32]; w13: packed E2M1
  [E, 2I, H/2] (element 2i in the low nibble of byte i) + UE8M0 [E, 2I, H/32];
  w2: packed E2M1 [E, H, I/2] + UE8M0 [E, H, I/32].
* ``nvfp4_w4a16``   x [T, H] bf16 bit patterns, no scale (the page's NVFP4 x BF16
  W4A16 pair); w13: packed E2M1 [E, 2I, H/2] + E4M3 block scales [E, 2I, H/16]
  + one fp32 global scale per expert ``w13_gs`` [E]; w2: packed E2M1
  [E, H, I/2] + E4M3 [E, H, I/16] + ``w2_gs`` [E].  A weight is
  e2m1 * e4m3 block scale * global scale.
* ``nvfp4``         x: packed E2M1 [T, H/2] + E4M3 block scales [T, H/16] (the
  page's NVFP4 x NVFP4 activations) against one global scale for the whole
  tensor; weights as ``nvfp4_w4a16``.  The per-expert scales handed to the FFN
  are those of the max mega_ffn arguments: ``w13_gs`` = gate_up_expert_scales
  (the activations' global scale times the gate_up weight's), ``c_scales`` =
  c_input_scales (the global scale the intermediate is requantised against: a
  static calibration value, drawn here around 16 / (6 * 448) per expert) and
  ``w2_gs`` = down_expert_scales (that input scale times the down weight's
  global scale).

Routing inputs: ``logits`` f32 [T, E] always; for precomputed routing the
caller-side ``topk_idx`` (int64 [T, k]) and ``topk_weights`` (f32 [T, k]) are
produced here, as a host router would produce them.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

FP8_BLOCK128 = "fp8_block128"
BF16 = "bf16"
W4A8_MX = "w4a8_mx"
NVFP4_W4A16 = "nvfp4_w4a16"
NVFP4 = "nvfp4"  # NVFP4 weights x NVFP4 activations

PRECOMPUTED = "precomputed"
FROM_LOGITS = "from_logits"

# generator stream ids
_S_LOGITS, _S_RANKS, _S_X, _S_W13, _S_W2, _S_CSCALE = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class MoEShape:
    """One workload: sizes, operand format and routing mode."""

    name: str
    seed: int
    tokens: int
    hidden: int
    inter: int
    experts: int
    topk: int
    fmt: str
    routing: str
    zipf_bias: bool = False  # per-expert logit bias -beta*s*ln(rank)
    zipf_s: float = 1.1
    zipf_beta: float = 3.0
    clamp: float = 10.0
    x_scale: float = 1.0  # multiplies the N(0,1) activations (clamp coverage)

    @property
    def pairs(self) -> int:
        return self.tokens * self.topk

    def with_(self, **kw) -> "MoEShape":
        return replace(self, **kw)


# The five named workloads.  Sizes follow the problem statement of the
# MegaMoESymmBuffer page (hidden, intermediate_hidden, num_experts, num_topk)
# at the shapes of common MoE layers.
WORKLOADS = {
    "tiny_fp8": MoEShape("tiny_fp8", 1, 64, 256, 128, 8, 2, FP8_BLOCK128, PRECOMPUTED),
    "decode_fp8": MoEShape("decode_fp8", 2, 256, 7168, 2048, 32, 8, FP8_BLOCK128, PRECOMPUTED),
    "prefill_fp8_zipf": MoEShape("prefill_fp8_zipf", 3, 8192, 7168, 2048, 32, 8, FP8_BLOCK128,
                                 PRECOMPUTED, zipf_bias=True),
    "mixtral_bf16": MoEShape("mixtral_bf16", 4, 4096, 4096, 14336, 8, 2, BF16, PRECOMPUTED),
    "w4a8_mx_logits": MoEShape("w4a8_mx_logits", 5, 2048, 2880, 2880, 128, 4, W4A8_MX, FROM_LOGITS),
}
CONFIG_ORDER = ["tiny_fp8", "decode_fp8", "prefill_fp8_zipf", "mixtral_bf16", "w4a8_mx_logits"]
# The NVFP4 weight x BF16 activation variant at the decode shape (not one of the
# five named workloads).
WORKLOADS["nvfp4_decode"] = MoEShape("nvfp4_decode", 6, 256, 7168, 2048, 32, 8, NVFP4_W4A16, PRECOMPUTED)
# NVFP4 weights x NVFP4 activations at the decode shape
WORKLOADS["nvfp4x4_decode"] = MoEShape("nvfp4x4_decode", 7, 256, 7168, 2048, 32, 8, NVFP4, PRECOMPUTED)


def _rng(seed: int, stream: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, expert])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- encoders
def _to_e4m3_codes(v: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN codes (torch cast, round-to-nearest-even), saturated."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _to_bf16_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# midpoints between consecutive E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
_E2M1_MID_UP = np.array([0.75, 1.75, 3.5], dtype=np.float32)  # ties whose upper neighbour has the even code


def _to_e2m1_codes(v: np.ndarray) -> np.ndarray:
    """float32 -> 4-bit E2M1 codes: nearest magnitude, ties to the even code, saturated at 6."""
    a = np.abs(v)
    code = np.searchsorted(_E2M1_MID, a, side="left").astype(np.uint8)
    code += np.isin(a, _E2M1_MID_UP).astype(np.uint8)
    return code | (((v < 0) & (code != 0)).astype(np.uint8) << 3)


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _block_amax(v: np.ndarray, br: int, bc: int) -> np.ndarray:
    r, c = v.shape
    return np.abs(v.reshape(r // br, br, c // bc, bc)).max(axis=(1, 3))


def quant_fp8_block(v: np.ndarray, br: int, bc: int):
    """float32 [R, C] -> (E4M3 codes [R, C], fp32 scales [R/br, C/bc]); scale = amax/448."""
    amax = _block_amax(v, br, bc)
    s = (amax.astype(np.float64) / 448.0).astype(np.float32)
    s[amax == 0] = 1.0
    full = np.repeat(np.repeat(s, br, axis=0), bc, axis=1)
    return _to_e4m3_codes(v / full), s


def _pow2_exponent_at_least(amax: np.ndarray, top: float) -> np.ndarray:
    """Smallest integer e with top * 2**e >= amax (amax > 0), clipped to [-127, 127]."""
    m, ex = np.frexp(amax.astype(np.float64) / top)  # amax/top = m * 2**ex, m in [0.5, 1)
    e = np.where(m == 0.5, ex - 1, ex)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int32)


def quant_mx_act(v: np.ndarray):
    """float32 [R, C] -> (E4M3 codes, UE8M0 bytes [R, C/32])."""
    r, c = v.shape
    amax = np.abs(v.reshape(r, c // 32, 32)).max(axis=2)
    e = _pow2_exponent_at_least(amax, 448.0)
    scale = np.ldexp(np.ones_like(amax, dtype=np.float64), e)
    q = _to_e4m3_codes((v.reshape(r, c // 32, 32) / scale[..., None]).reshape(r, c).astype(np.float32))
    return q, (e + 127).astype(np.uint8)


def quant_mx_weight(v: np.ndarray):
    """float32 [R, C] -> (packed E2M1 [R, C/2], UE8M0 bytes [R, C/32])."""
    r, c = v.shape
    amax = np.abs(v.reshape(r, c // 32, 32)).max(axis=2)
    e = _pow2_exponent_at_least(amax, 6.0)
    scale = np.ldexp(np.ones_like(amax, dtype=np.float64), e)
    codes = _to_e2m1_codes((v.reshape(r, c // 32, 32) / scale[..., None]).reshape(r, c).astype(np.float32))
    return _pack_nibbles(codes), (e + 127).astype(np.uint8)


def quant_nvfp4_weight(v: np.ndarray):
    """float32 [R, C] -> (packed E2M1 [R, C/2], E4M3 block scales [R, C/16], fp32 global scale).
    The global scale puts the largest block scale at the E4M3 maximum; each block's
    scale is its amax / 6 over the global scale, rounded to E4M3; the values are
    the nearest E2M1 codes of v over (block scale * global scale)."""
    r, c = v.shape
    amax = float(np.abs(v).max())
    gs = np.float32(amax / (6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    bamax = np.abs(v.reshape(r, c // 16, 16)).max(axis=2)
    sc = _to_e4m3_codes((bamax / (6.0 * float(gs))).astype(np.float32))
    sdec = torch.from_numpy(sc).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    denom = (sdec.astype(np.float64) * float(gs))[..., None]
    q = np.where(denom > 0, v.reshape(r, c // 16, 16) / np.where(denom > 0, denom, 1.0), 0.0)
    codes = _to_e2m1_codes(q.reshape(r, c).astype(np.float32))
    return _pack_nibbles(codes), sc, gs


# ---------------------------------------------------------------- draws
def draw_logits(shape: MoEShape) -> np.ndarray:
    lg = _rng(shape.seed, _S_LOGITS).standard_normal((shape.tokens, shape.experts), dtype=np.float32)
    if shape.zipf_bias:
        ranks = _rng(shape.seed, _S_RANKS).permutation(shape.experts) + 1
        bias = (-shape.zipf_beta * shape.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)
        lg = lg + bias[None, :]
    return lg


def host_router(logits: np.ndarray, k: int):
    """What a host-side router hands to a precomputed-routing call: the k largest
    logits per token (ties to the lower expert index) and a softmax over them."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int64), w.astype(np.float32)


def _weights_for_expert(shape: MoEShape, e: int):
    H, I = shape.hidden, shape.inter
    w13 = _rng(shape.seed, _S_W13, e).standard_normal((2 * I, H), dtype=np.float32) * np.float32(1.0 / math.sqrt(H))
    w2 = _rng(shape.seed, _S_W2, e).standard_normal((H, I), dtype=np.float32) * np.float32(1.0 / math.sqrt(I))
    if shape.fmt == FP8_BLOCK128:
        return quant_fp8_block(w13, 128, 128) + quant_fp8_block(w2, 128, 128)
    if shape.fmt == BF16:
        return _to_bf16_bits(w13), None, _to_bf16_bits(w2), None
    if shape.fmt == W4A8_MX:
        return quant_mx_weight(w13) + quant_mx_weight(w2)
    if shape.fmt in (NVFP4_W4A16, NVFP4):
        return quant_nvfp4_weight(w13) + quant_nvfp4_weight(w2)
    raise ValueError(shape.fmt)


def make_inputs(shape: MoEShape, with_weights: bool = True) -> dict:
    """All inputs of one workload as numpy arrays of raw encodings."""
    T, H, I, E, k = shape.tokens, shape.hidden, shape.inter, shape.experts, shape.topk
    out = {"shape": shape}
    logits = draw_logits(shape)
    out["logits"] = logits
    if shape.routing == PRECOMPUTED:
        out["topk_idx"], out["topk_weights"] = host_router(logits, k)
    x = _rng(shape.seed, _S_X).standard_normal((T, H), dtype=np.float32)
    if shape.x_scale != 1.0:
        x = x * np.float32(shape.x_scale)
    if shape.fmt == FP8_BLOCK128:
        out["x"], out["x_sf"] = quant_fp8_block(x, 1, 128)
    elif shape.fmt in (BF16, NVFP4_W4A16):
        out["x"], out["x_sf"] = _to_bf16_bits(x), None
    elif shape.fmt == NVFP4:
        out["x"], out["x_sf"], out["x_gs"] = quant_nvfp4_weight(x)
    else:
        out["x"], out["x_sf"] = quant_mx_act(x)
    if not with_weights:
        return out
    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda e: _weights_for_expert(shape, e), range(E)))
    if shape.fmt == NVFP4_W4A16:  # (w13, sf, gs, w2, sf, gs) per expert
        out["w13_gs"] = np.array([p[2] for p in parts], dtype=np.float32)
        out["w2_gs"] = np.array([p[5] for p in parts], dtype=np.float32)
        parts = [(p[0], p[1], p[3], p[4]) for p in parts]
    elif shape.fmt == NVFP4:
        # the legs' per-expert output scales and the intermediate's per-expert input scale
        c = (shape.x_scale * (12.0 + 8.0 * _rng(shape.seed, _S_CSCALE).random(E)) / (6.0 * 448.0)).astype(np.float32)
        out["c_scales"] = c
        out["w13_gs"] = (np.float32(out["x_gs"]) * np.array([p[2] for p in parts], dtype=np.float32)).astype(np.float32)
        out["w2_gs"] = (c * np.array([p[5] for p in parts], dtype=np.float32)).astype(np.float32)
        parts = [(p[0], p[1], p[3], p[4]) for p in parts]
    out["w13"] = np.stack([p[0] for p in parts])
    out["w13_sf"] = None if parts[0][1] is None else np.stack([p[1] for p in parts])
    out["w2"] = np.stack([p[2] for p in parts])
    out["w2_sf"] = None if parts[0][3] is None else np.stack([p[3] for p in parts])
    return out
