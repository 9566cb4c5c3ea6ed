// Router-weighted combine: out[t, :] = sum over valid slots j (ascending) of
// w[t, j] * y[t, j, :] (DistributedEPCombine page: router_weights scale each
// expert's contribution; the per-pair rows y are the expert outputs), then,
// when given, + shared[t, :] (a shared expert's output fused into the combine:
// the fused_shared_expert option of the MAX mega_ffn / EP pages) and
// + residual[t, :] (a downstream elementwise epilogue: has_epilogue_fusion).
// HBM-bound gather-reduce: each thread owns 8 consecutive bf16 columns of one
// token (the threads of the launch cover the [T, H/8] chunks in order, so no
// lane idles at a row's end) and reads the k slot rows with 16-byte loads, G at
// a time (G = k rounded up to 2, 4 or 8: Mixtral's k = 2 read 8 rows per group,
// six of them dummies, when G was always 8); fp32 accumulation; one bf16 rounding
// at the store, or an fp32 store (the combine dtype is a choice on the EPConfig
// and DistributedEPCombine pages).
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace moe {

constexpr int kCombineThreads = 256;

// WAVE_TOKEN: every wave's 64 chunks lie in one token (H a multiple of 512), so
// the token, its pair rows and weights are wave-uniform: scalar loads (decode
// 8.5 against 6.5 us when they were per-lane vector loads).
template <bool OUT_F32, int G, bool WAVE_TOKEN>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                                  const float* __restrict__ w,
                                                                  const int* __restrict__ pair_row, int T, int topk,
                                                                  int H, const uint16_t* __restrict__ shared,
                                                                  const uint16_t* __restrict__ residual,
                                                                  void* __restrict__ out) {
  const int cpt = H / 8;  // 8-column chunks per token
  const long long c = (long long)blockIdx.x * kCombineThreads + threadIdx.x;
  if (c >= (long long)T * cpt) return;
  const int tl = (int)(c / cpt);
  const int t = WAVE_TOKEN ? __builtin_amdgcn_readfirstlane(tl) : tl;
  const int col = (int)(c - (long long)t * cpt) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const long long p0 = (long long)t * topk;
  // Slots in groups of G with every row load issued before the first is used (a
  // masked slot's row, never written, is read but not added).  The rows are read
  // once: non-temporal loads.
  for (int j0 = 0; j0 < topk; j0 += G) {
    i32x4 v[G];
    bool ok[G];
    float wj[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = j0 + u;
      ok[u] = j < topk && pair_row[p0 + j] >= 0;
      wj[u] = ok[u] ? w[p0 + j] : 0.f;
      const long long row = p0 + (j < topk ? j : 0);
      v[u] = __builtin_bit_cast(i32x4, __builtin_nontemporal_load((const i32x4*)(y + row * H + col)));
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (!ok[u]) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t e = (uint32_t)v[u][q];
        acc[2 * q] = fmaf(wj[u], bf16_to_f32((uint16_t)(e & 0xFFFFu)), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wj[u], bf16_to_f32((uint16_t)(e >> 16)), acc[2 * q + 1]);
      }
    }
  }
  // the addends, in this order, after the slots
  const uint16_t* add[2] = {shared, residual};
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (add[a] == nullptr) continue;  // uniform
    const i32x4 v = *(const i32x4*)(add[a] + (long long)t * H + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t e = (uint32_t)v[q];
      acc[2 * q] += bf16_to_f32((uint16_t)(e & 0xFFFFu));
      acc[2 * q + 1] += bf16_to_f32((uint16_t)(e >> 16));
    }
  }
  if constexpr (OUT_F32) {
    f32x4* o = (f32x4*)((float*)out + (long long)t * H + col);
    o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    i32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (int)bf16x2_rne(acc[2 * q], acc[2 * q + 1]);
    *(i32x4*)((uint16_t*)out + (long long)t * H + col) = o;
  }
}

hipError_t launch_combine(const void* y, const float* w, const int* pair_row, int T, int topk, int H,
                          const void* shared, const void* residual, void* out, bool out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const long long chunks = (long long)T * (H / 8);
  const dim3 grid((unsigned)((chunks + kCombineThreads - 1) / kCombineThreads));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kCombineThreads), 0, s, (const uint16_t*)y, w, pair_row, T, topk, H,
                       (const uint16_t*)shared, (const uint16_t*)residual, out);
  };
  auto by_k = [&](auto out32, auto wave_token) {
    constexpr bool O = decltype(out32)::value, W = decltype(wave_token)::value;
    if (topk <= 2) go(combine_kernel<O, 2, W>);
    else if (topk <= 4) go(combine_kernel<O, 4, W>);
    else go(combine_kernel<O, 8, W>);
  };
  const bool wave_token = (H / 8) % 64 == 0;
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (out_f32) wave_token ? by_k(T_{}, T_{}) : by_k(T_{}, F_{});
  else wave_token ? by_k(F_{}, T_{}) : by_k(F_{}, F_{});
  return hipGetLastError();
}

}  // namespace moe
