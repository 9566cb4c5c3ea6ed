// One-time relayout of expert weights into the tiles the grouped GEMMs stream
// (the Struct_mega_ffn_ep_combine_send page takes its gate_up weight
// pre-permuted; here every weight matrix is).
//
// A weight matrix of R rows (R a multiple of 16) and K elements per row is cut
// into tiles of 16 rows x one K-step (128 elements; 64 for BF16).  Tiles are
// stored expert-major, then by row block rb = row / 16, then by K-step ks, each
// tile contiguous in the lane order of the 16x16 MFMA operand (lane l = 16*g + r
// holds row 16*rb + r):
//   FP8, BF16: 2048 bytes; byte half*1024 + 16*l + b <- row byte ks*128 + 64*half + 16*g + b
//   MX (E2M1): 1024 bytes; byte 16*l + b <- row byte ks*64 + 16*g + b (zero past the row's end)
//   MX scales: 64 bytes;   byte l <- UE8M0 of K-block 4*ks + g (zero past the row's end)
// FP8 block scales keep their layout.
#include "device.h"
#include "launch.h"

namespace moe {

size_t prepared_tile_bytes(Fmt f) { return f == Fmt::MX ? 1024 : 2048; }
int prepared_ksteps(Fmt f, int K) {
  const int step = f == Fmt::BF16 ? 64 : 128;
  return (K + step - 1) / step;
}
size_t prepared_expert_bytes(Fmt f, int rows, int K) {
  return (size_t)(rows / 16) * prepared_ksteps(f, K) * prepared_tile_bytes(f);
}
size_t prepared_scale_expert_bytes(Fmt f, int rows, int K) {
  return f == Fmt::MX ? (size_t)(rows / 16) * prepared_ksteps(f, K) * 64 : 0;
}

// One thread per 16-byte chunk of the prepared tensor.
__global__ __launch_bounds__(256) void prepare_weight_tiles(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                            int rows, int row_bytes, int seg, int ksteps,
                                                            int tile_chunks, size_t total_chunks) {
  const size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total_chunks) return;
  const int q = (int)(c % tile_chunks);
  const size_t t = c / tile_chunks;
  const int ks = (int)(t % ksteps);
  const size_t t2 = t / ksteps;
  const int rblocks = rows / 16;
  const int rb = (int)(t2 % rblocks);
  const size_t e = t2 / rblocks;
  const int half = q / 64, l = q % 64, g = l / 16, r = l % 16;
  const int byte = ks * seg + half * 64 + g * 16;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (byte < row_bytes) v = *(const uint4*)(src + (e * rows + (size_t)(rb * 16 + r)) * row_bytes + byte);
  *(uint4*)(dst + c * 16) = v;
}

// One thread per byte of the prepared MX scale tensor.
__global__ __launch_bounds__(256) void prepare_mx_scales(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                         int rows, int kblocks, int ksteps, size_t total) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int l = (int)(i % 64);
  const size_t t = i / 64;
  const int ks = (int)(t % ksteps);
  const size_t t2 = t / ksteps;
  const int rblocks = rows / 16;
  const int rb = (int)(t2 % rblocks);
  const size_t e = t2 / rblocks;
  const int kb = ks * 4 + l / 16;
  dst[i] = kb < kblocks ? src[(e * rows + (size_t)(rb * 16 + l % 16)) * kblocks + kb] : (uint8_t)0;
}

hipError_t launch_prepare(Fmt f, int E, int rows, int K, const void* w, const void* w_sf, void* out, void* out_sf,
                          hipStream_t s) {
  const int ks = prepared_ksteps(f, K);
  const int row_bytes = f == Fmt::BF16 ? 2 * K : (f == Fmt::MX ? K / 2 : K);
  const int seg = f == Fmt::MX ? 64 : 128;
  const int tile_chunks = (int)(prepared_tile_bytes(f) / 16);
  const size_t chunks = (size_t)E * prepared_expert_bytes(f, rows, K) / 16;
  if (chunks > 0) {
    const size_t blocks = (chunks + 255) / 256;
    hipLaunchKernelGGL(prepare_weight_tiles, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)w,
                       (uint8_t*)out, rows, row_bytes, seg, ks, tile_chunks, chunks);
  }
  if (f == Fmt::MX) {
    const size_t total = (size_t)E * prepared_scale_expert_bytes(f, rows, K);
    if (total > 0) {
      const size_t blocks = (total + 255) / 256;
      hipLaunchKernelGGL(prepare_mx_scales, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)w_sf,
                         (uint8_t*)out_sf, rows, K / 32, ks, total);
    }
  } else if (f == Fmt::FP8 && out_sf != w_sf) {
    const size_t bytes = (size_t)E * (rows / 128) * (K / 128) * 4;
    hipError_t e = hipMemcpyAsync(out_sf, w_sf, bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace moe
