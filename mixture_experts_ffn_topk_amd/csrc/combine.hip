// Router-weighted combine: out[t, :] = sum over valid slots j (ascending) of
// w[t, j] * y[t, j, :] (DistributedEPCombine page: router_weights scale each
// expert's contribution; the per-pair rows y are the expert outputs), then,
// when given, + shared[t, :] (a shared expert's output fused into the combine:
// the fused_shared_expert option of the MAX mega_ffn / EP pages) and
// + residual[t, :] (a downstream elementwise epilogue: has_epilogue_fusion).
// HBM-bound gather-reduce: each thread owns 8 consecutive bf16 columns and reads
// the k slot rows with 16-byte loads; fp32 accumulation; bf16 store.
#include "device.h"
#include "launch.h"

namespace moe {

constexpr int kCombineThreads = 256;
constexpr int kCombineCols = kCombineThreads * 8;  // columns per workgroup

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                                  const float* __restrict__ w,
                                                                  const int* __restrict__ pair_row, int topk, int H,
                                                                  const uint16_t* __restrict__ shared,
                                                                  const uint16_t* __restrict__ residual,
                                                                  uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int col = blockIdx.y * kCombineCols + threadIdx.x * 8;
  if (col >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const long long p0 = (long long)t * topk;
  // Slots in groups of 8 with every row load issued before the first is used (a
  // masked slot's row, never written, is read but not added).  The rows are read
  // once: non-temporal loads.
  for (int j0 = 0; j0 < topk; j0 += 8) {
    i32x4 v[8];
    bool ok[8];
    float wj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      ok[u] = j < topk && pair_row[p0 + j] >= 0;
      wj[u] = ok[u] ? w[p0 + j] : 0.f;
      const long long row = p0 + (j < topk ? j : 0);
      v[u] = __builtin_bit_cast(i32x4, __builtin_nontemporal_load((const i32x4*)(y + row * H + col)));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
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
  i32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = (int)((uint32_t)f32_to_bf16_rne(acc[2 * q]) | ((uint32_t)f32_to_bf16_rne(acc[2 * q + 1]) << 16));
  *(i32x4*)(out + (long long)t * H + col) = o;
}

hipError_t launch_combine(const void* y, const float* w, const int* pair_row, int T, int topk, int H,
                          const void* shared, const void* residual, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid(T, (H + kCombineCols - 1) / kCombineCols);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombineThreads), 0, s, (const uint16_t*)y, w, pair_row, topk, H,
                     (const uint16_t*)shared, (const uint16_t*)residual, (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace moe
