// One-time relayout of expert weights into the tiles the grouped GEMMs stream
// (the Struct_mega_ffn_ep_combine_send page takes its gate_up weight
// pre-permuted; here every weight matrix is).
//
// A weight matrix of R rows and K elements per row is cut into tiles of RT rows
// x one K-step, stored expert-major, then by row block rb = row / RT, then by
// K-step ks, each tile contiguous in the lane order of the MFMA operand:
//   FP8 (RT 16, K-step 128): 2048 bytes; byte 1024*piece + 16*l + b, l = 16*g + r,
//        <- row 16*rb + r, byte ks*128 + 64*piece + 16*g + b   (16x16x128 operand)
//   MX  (RT 16, K-step 128): 1024 bytes; byte 16*l + b, l = 16*g + r,
//        <- row 16*rb + r, byte ks*64 + 16*g + b, zero past the row's end
//   MX scales: 64 bytes per tile; byte l <- UE8M0 of K-block 4*ks + g, zero past the end
//   BF16 (RT 32, K-step 64): 4096 bytes; byte 1024*sub + 16*l + b, l = 32*h + r,
//        <- row 32*rb + r, byte ks*128 + 32*sub + 16*h + b      (32x32x16 operand)
//   NV4 (RT 32, K-step 64 elements = 32 packed bytes): 1024 bytes; byte 16*l + 4*sub + b,
//        l = 32*h + r, <- row 32*rb + r, byte ks*32 + 8*sub + 4*h + b: the E2M1 nibbles of
//        the 32x32x16 operand's sub-step sub (K elements 16*sub + 8*h ... + 7), zero past the end
//   NV4 scales: 128 bytes per tile; byte 4*r + sub <- E4M3 scale of K-block 4*ks + sub
// For BF16 and NV4 the rows of the gate_up weight are also interleaved: tile row
// 32*j + q is gate row 16*j + q for q < 16 and up row 16*j + q - 16 otherwise, so
// that a 32x32 output tile holds each gate column next to its up column.
// FP8 block scales keep their layout.
#include "device.h"
#include "launch.h"

namespace moe {

size_t prepared_tile_bytes(Fmt f) { return f == Fmt::BF16 ? 4096 : (f == Fmt::FP8 ? 2048 : 1024); }
static int tile_rows(Fmt f) { return f == Fmt::BF16 || f == Fmt::NV4 ? 32 : 16; }
int prepared_ksteps(Fmt f, int K) {
  const int step = f == Fmt::BF16 || f == Fmt::NV4 ? 64 : 128;
  return (K + step - 1) / step;
}
size_t prepared_expert_bytes(Fmt f, int rows, int K) {
  return (size_t)(rows / tile_rows(f)) * prepared_ksteps(f, K) * prepared_tile_bytes(f);
}
size_t prepared_scale_expert_bytes(Fmt f, int rows, int K) {
  if (f == Fmt::MX) return (size_t)(rows / 16) * prepared_ksteps(f, K) * 64;
  if (f == Fmt::NV4) return (size_t)(rows / 32) * prepared_ksteps(f, K) * 128;
  return 0;
}

// NV4 source row of tile row r in row block rb (gate_up rows interleaved)
__device__ __forceinline__ int nv4_row(int rb, int r, int gu_half) {
  if (gu_half > 0) return r < 16 ? 16 * rb + r : gu_half + 16 * rb + (r - 16);
  return 32 * rb + r;
}

// NV4 weights: one thread per 4-byte piece of the prepared tensor.
__global__ __launch_bounds__(256) void prepare_nv4_tiles(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                         int rows, int row_bytes, int ksteps, int gu_half,
                                                         size_t total_pieces) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total_pieces) return;
  const int q = (int)(i % 256);  // piece in the 1 KB tile: lane l = q / 4, sub-step q % 4
  const size_t t = i / 256;
  const int ks = (int)(t % ksteps);
  const size_t t2 = t / ksteps;
  const int rblocks = rows / 32;
  const int rb = (int)(t2 % rblocks);
  const size_t e = t2 / rblocks;
  const int l = q / 4, sub = q % 4, h = l / 32, r = l % 32;
  const int byte = ks * 32 + 8 * sub + 4 * h;
  uint32_t v = 0;
  if (byte < row_bytes) v = *(const uint32_t*)(src + (e * rows + (size_t)nv4_row(rb, r, gu_half)) * row_bytes + byte);
  ((uint32_t*)dst)[i] = v;
}

// NV4 block scales: one thread per byte of the prepared scale tensor.
__global__ __launch_bounds__(256) void prepare_nv4_scales(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int rows, int kblocks, int ksteps, int gu_half,
                                                          size_t total) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int j = (int)(i % 128);
  const size_t t = i / 128;
  const int ks = (int)(t % ksteps);
  const size_t t2 = t / ksteps;
  const int rblocks = rows / 32;
  const int rb = (int)(t2 % rblocks);
  const size_t e = t2 / rblocks;
  const int r = j / 4, kb = 4 * ks + j % 4;
  dst[i] = kb < kblocks ? src[(e * rows + (size_t)nv4_row(rb, r, gu_half)) * kblocks + kb] : (uint8_t)0;
}

// One thread per 16-byte chunk of the prepared tensor.  rt: tile rows; seg: row
// bytes per K-step; piece: row bytes per 1 KB piece of a tile; gu_half: for the
// interleaved BF16 gate_up weight, the row offset of the up half (else 0).
__global__ __launch_bounds__(256) void prepare_weight_tiles(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                            int rows, int row_bytes, int rt, int seg, int piece,
                                                            int ksteps, int tile_chunks, int gu_half,
                                                            size_t total_chunks) {
  const size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total_chunks) return;
  const int q = (int)(c % tile_chunks);
  const size_t t = c / tile_chunks;
  const int ks = (int)(t % ksteps);
  const size_t t2 = t / ksteps;
  const int rblocks = rows / rt;
  const int rb = (int)(t2 % rblocks);
  const size_t e = t2 / rblocks;
  const int pc = q / 64, l = q % 64, g = l / rt, r = l % rt;
  int row = rb * rt + r;
  if (gu_half > 0) row = r < 16 ? 16 * rb + r : gu_half + 16 * rb + (r - 16);
  const int byte = ks * seg + pc * piece + g * 16;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (byte < row_bytes) v = *(const uint4*)(src + (e * rows + (size_t)row) * row_bytes + byte);
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

hipError_t launch_prepare(Fmt f, int E, int rows, int K, bool gate_up, const void* w, const void* w_sf, void* out,
                          void* out_sf, hipStream_t s) {
  const int ks = prepared_ksteps(f, K);
  if (f == Fmt::NV4) {
    const int gu_half = gate_up ? rows / 2 : 0;
    const size_t pieces = (size_t)E * prepared_expert_bytes(f, rows, K) / 4;
    if (pieces > 0)
      hipLaunchKernelGGL(prepare_nv4_tiles, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s,
                         (const uint8_t*)w, (uint8_t*)out, rows, K / 2, ks, gu_half, pieces);
    const size_t total = (size_t)E * prepared_scale_expert_bytes(f, rows, K);
    if (total > 0)
      hipLaunchKernelGGL(prepare_nv4_scales, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                         (const uint8_t*)w_sf, (uint8_t*)out_sf, rows, K / 16, ks, gu_half, total);
    return hipGetLastError();
  }
  const int row_bytes = f == Fmt::BF16 ? 2 * K : (f == Fmt::MX ? K / 2 : K);
  const int seg = f == Fmt::MX ? 64 : 128;
  const int piece = f == Fmt::BF16 ? 32 : 64;
  const int gu_half = (f == Fmt::BF16 && gate_up) ? rows / 2 : 0;
  const int tile_chunks = (int)(prepared_tile_bytes(f) / 16);
  const size_t chunks = (size_t)E * prepared_expert_bytes(f, rows, K) / 16;
  if (chunks > 0) {
    const size_t blocks = (chunks + 255) / 256;
    hipLaunchKernelGGL(prepare_weight_tiles, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)w,
                       (uint8_t*)out, rows, row_bytes, tile_rows(f), seg, piece, ks, tile_chunks, gu_half, chunks);
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
