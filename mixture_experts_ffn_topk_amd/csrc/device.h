// Device-side helpers shared by the gfx950 kernels of the MoE FFN library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define MOE_DEV __device__ __forceinline__
#define MOE_HOST_DEV __host__ __device__

MOE_DEV int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- conversions
// Two fp32 -> two bf16 (a in the low half), round to nearest even; a NaN stays a
// NaN.  One v_cvt_pk_bf16_f32 (gfx950's conversion) instead of the six or so VALU
// operations per value of rounding the bits by hand.
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
MOE_DEV uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_cvt{a, b}, bf16x2_cvt));
}
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 -> two E4M3FN codes (round to nearest even), saturated to +-448
// before the hardware conversion so that no code becomes NaN.  Returns the
// codes in the low 16 bits (a in byte 0, b in byte 1).
MOE_DEV uint32_t f32x2_to_e4m3_sat(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, 448.0f, -448.0f);
  b = __builtin_amdgcn_fmed3f(b, 448.0f, -448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// fp32 -> the nearest E2M1 value (0, .5, 1, 1.5, 2, 3, 4, 6 and negatives), ties to
// the even code, saturated at +-6: E2M1 steps by 0.5 below 2, by 1 in [2, 4) and
// by 2 from 4, and rintf rounds half to even, which is the even code on each grid.
MOE_DEV float e2m1_rne_sat(float v) {
  const float a = fminf(fabsf(v), 6.0f);
  float r;
  if (a < 2.0f)
    r = __builtin_rintf(a * 2.0f) * 0.5f;
  else if (a < 4.0f)
    r = __builtin_rintf(a);
  else
    r = __builtin_rintf(a * 0.5f) * 2.0f;
  return __builtin_copysignf(r, v);
}

// ---------------------------------------------------------------- activation
// x * sigmoid(x).  fast: hardware exp2 and reciprocal; else IEEE expf / divide.
template <bool FAST>
MOE_DEV float silu_f32(float x) {
  if (FAST) {
    float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);  // exp(-x)
    return x * __builtin_amdgcn_rcpf(1.0f + e);
  } else {
    return x / (1.0f + expf(-x));
  }
}

// Clamped SwiGLU: silu(min(g, c)) * clamp(u, -c, c).
template <bool FAST>
MOE_DEV float swiglu_clamped(float g, float u, float c) {
  g = fminf(g, c);
  u = fminf(fmaxf(u, -c), c);
  return silu_f32<FAST>(g) * u;
}

// Smallest integer e with 448 * 2^e >= a (a >= 0 finite), clipped to [-127, 127];
// -127 for a == 0.  Exact: a = m * 2^E with m in [1, 2); 448 = 1.75 * 2^8, so
// e = E - 8 when m <= 1.75 and E - 7 otherwise.
MOE_DEV int mx_exponent_for_amax(float a) {
  uint32_t u = __float_as_uint(a);
  if (u == 0) return -127;
  int ef = (int)(u >> 23);
  uint32_t man = u & 0x7FFFFFu;
  int e;
  if (ef == 0) {
    e = -127;  // subnormal amax: 448 * 2^-127 already covers it
  } else {
    e = ef - 127 - 8 + (man > 0x600000u ? 1 : 0);
  }
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^e as float for e in [-127, 127] (2^-127 is a subnormal).
MOE_DEV float exp2i(int e) {
  if (e >= -126) return __uint_as_float((uint32_t)(e + 127) << 23);
  return __uint_as_float(0x00400000u);  // 2^-127
}

// ---------------------------------------------------------------- wave helpers
MOE_DEV float wave_max_xor(float v, int width_mask_start, int width_mask_end) {
  for (int m = width_mask_start; m <= width_mask_end; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
