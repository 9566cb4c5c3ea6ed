"""Number-format codecs of the CPU oracle, written from the formats' definitions.

TEST INFRASTRUCTURE ONLY.  Part of the CPU oracle: imported by tests/, by
``__graft_entry__.smoke()`` and by the benchmark's CPU-baseline leg, never by
the GPU path.

Every function works on numpy arrays and returns float64 values (decoders) or
float64 values already rounded onto the target grid (rounders).  Nothing here
is shared with the GPU code.

Formats (operand encodings of the flashinfer.fused_moe MoEActivationPack page:
"DeepSeek FP8", "MXFP8", "MXFP4 x MXFP8 (W4A8)", "BF16", "NVFP4"):

* E4M3 (float8_e4m3fn): sign, 4 exponent bits (bias 7), 3 mantissa bits.
  Exponent field 0 is subnormal (m/8 * 2**-6); field 15 with mantissa 7 is
  NaN; there is no infinity, so the largest finite magnitude is 448.
* E2M1 (MXFP4 / NVFP4 element): sign, 2 exponent bits (bias 1), 1 mantissa bit.
  Exponent field 0 is subnormal (m/2 * 2**0).  Magnitudes 0 .. 6.
* UE8M0 (MX block scale): unsigned 8-bit exponent, value 2**(b - 127); the
  byte 255 is NaN.
* BF16: the upper 16 bits of an IEEE binary32.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    ef = (b >> 3) & 0xF
    mf = b & 0x7
    normal = (1.0 + mf / 8.0) * np.ldexp(1.0, (ef - 7).astype(np.int32))
    sub = (mf / 8.0) * 2.0 ** -6
    val = np.where(ef == 0, sub, normal)
    val = np.where((ef == 15) & (mf == 7), np.nan, val)
    return sign * val


def e2m1_decode_nibbles(nib: np.ndarray) -> np.ndarray:
    n = np.asarray(nib, dtype=np.uint8).astype(np.int64)
    sign = np.where(n & 0x8, -1.0, 1.0)
    ef = (n >> 1) & 0x3
    mf = n & 0x1
    normal = (1.0 + mf / 2.0) * np.ldexp(1.0, (ef - 1).astype(np.int32))
    sub = mf / 2.0
    return sign * np.where(ef == 0, sub, normal)


def e2m1_unpack(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., K/2] -> nibbles [..., K]; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def ue8m0_decode(b: np.ndarray) -> np.ndarray:
    bi = np.asarray(b, dtype=np.uint8).astype(np.int32)
    v = np.ldexp(1.0, bi - 127)
    return np.where(bi == 255, np.nan, v)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_to_grid(v: np.ndarray, mant_bits: int, emin: int, maxval: float, saturate: bool) -> np.ndarray:
    """Round float64 values to the nearest value of a binary floating-point format
    with ``mant_bits`` stored mantissa bits and minimum normal exponent ``emin``
    (subnormals below 2**emin), ties to even.  Beyond ``maxval`` the result is
    +-maxval when ``saturate`` is set, else +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)  # a = m * 2**ex, m in [0.5, 1)  -> exponent of a is ex - 1
    e = np.maximum(ex - 1, emin)
    quantum = np.ldexp(1.0, (e - mant_bits).astype(np.int32))
    r = np.rint(a / quantum) * quantum  # a / quantum is exact (power-of-two divide); rint = ties-to-even
    if saturate:
        r = np.minimum(r, maxval)
    else:
        r = np.where(r > maxval, np.inf, r)
    r = np.where(np.isnan(v), np.nan, r)
    return np.copysign(r, v)


def round_e4m3_sat(v: np.ndarray) -> np.ndarray:
    """Value of E4M3FN round-to-nearest-even with saturation to +-448."""
    return round_to_grid(v, 3, -6, E4M3_MAX, saturate=True)


def round_e2m1_sat(v: np.ndarray) -> np.ndarray:
    """Value of E2M1 round-to-nearest-even with saturation to +-6 (1 mantissa bit,
    minimum normal exponent 0, subnormal step 0.5)."""
    return round_to_grid(v, 1, 0, 6.0, saturate=True)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Value of bf16 round-to-nearest-even (8 exponent bits, 7 mantissa bits)."""
    return round_to_grid(v, 7, -126, float(np.ldexp(2.0 - 2.0 ** -7, 127)), saturate=False)
