// Helpers shared by the grouped-GEMM kernels: the launch parameters, buffer
// resources and loads (plain, non-temporal, direct-to-LDS), wait-count encoding
// and the XCD-aware workgroup mapping.  Internal to the library.
#pragma once
#include "device.h"
#include "launch.h"

namespace moe {

#define LDS3 __attribute__((address_space(3)))  // LDS pointers of the direct-to-LDS loads
constexpr uint32_t kOOB = 0x80000000u;  // lane offset that reads zeros
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// kOOB if dead, else 0: OR-ed into a lane offset below 2^31 it turns the load
// into one that reads zeros, without a branch or a select (a uniform condition
// would otherwise become a branch around the load)
MOE_DEV uint32_t oob_if(bool dead) { return (uint32_t)dead << 31; }

// Direct-to-LDS buffer loads: lane l's 16 (4) bytes land at lds + 16 l (4 l).
// (Kept out of the kernel body: inline there, the host pass drops the kernel's
// launch stub.)
MOE_DEV void lds_load16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS3 void*)lds, 16, voff, soff, 0, 0);
}
MOE_DEV void lds_load4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS3 void*)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding): VMEM count <= vm, LDS / scalar count 0,
// export count not waited on.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 0xF) | ((vm >> 4) & 3) << 14 | 7 << 4; }

struct GemmParams {
  const int* start;     // expert_start_indices [E+1]
  const int* src_info;  // [npairs]
  int E, topk;
  int m_tiles_max, n_tiles;
  int K;       // reduction length in elements
  int ksteps;  // K-steps of 128 (FP8, MX) or 64 (BF16) elements
  int N;       // output columns: I (gate_up) or H (down)
  int n_rows;  // weight rows per expert: 2I (gate_up) or H (down)
  const uint8_t* A;
  uint32_t a_bytes;  // size of the A tensor
  uint32_t a_row_bytes;
  const void* A_sf;
  uint32_t a_sf_bytes;
  int a_sf_row;  // FP8: floats per row; MX: bytes per row
  const uint8_t* B;
  uint32_t b_tile;          // bytes of one prepared weight tile (16 rows x one K-step)
  uint32_t b_expert_bytes;  // prepared weight bytes per expert
  uint32_t bsc_expert_bytes;  // MX: prepared scale bytes per expert
  const void* B_sf;
  int b_sf_row;  // FP8: K/128 floats per 128-row block
  const float* B_gs;  // NV4, NVF4: the leg's per-expert output scale (the weights' global scale)
  const float* C_gs;  // NVF4 gate_up: per-expert global scale the intermediate is requantised against
  void* C;
  long long c_row_bytes;
  void* C_sf;
  int c_sf_row;
  float clamp;
  // down leg with the combine fused into its epilogue (fuse != 0): the tile that
  // stores the last valid slot of a token's column block reduces that block
  int fuse;
  int T;
  const int* pair_row;    // [T*k] pair -> row, -1 for a masked slot
  const float* topk_w;    // [T, k] router weights
  int* counters;          // [T, cnt_stride] arrivals per (token, column tile), zero on entry
  int cnt_stride;
  void* out;              // [T, N] bf16 (fp32 if out_f32)
  const uint16_t* shared;    // optional bf16 [T, N] addends
  const uint16_t* residual;
  int out_f32;
  int m_grid;             // GEMM workgroups of the grid; those past it write the tokens without a valid slot
  uint32_t y_bytes;       // size of y (fused combine: y is addressed through a buffer resource)
  // down leg, MFMA-bound tiles: the split tail's buffers (split_slots 0: no split)
  int* split_cnt;      // [split_slots] arrival counters, zero on entry, left zero
  float* split_part;   // [split_slots] fp32 partial tiles
  int split_slots;     // workgroups the part runs at once (at most kSplitMaxSlots)
  // gate_up leg that builds the routing plan itself (plan_ids != nullptr): every
  // workgroup histograms the ids into LDS and gathers its own rows; workgroup 0
  // writes the counts, offsets, active list and status, the workgroups of column
  // tile 0 their rows' src_info and pair_row (start / src_info above are then
  // outputs of this launch, read by the down leg and the combine)
  const void* plan_ids;   // [npairs] int64 (ids64) or int32 expert ids
  int ids64;
  int npairs;
  PlanPtrs plan_out;
};

// Cache-policy bits of buffer loads and stores (gfx950): device-scope coherence
// (stores write through to the level all XCDs share; loads do not hit lines that
// another XCD may have changed), and the non-temporal hint.
constexpr int kCpolDevice = 16;
constexpr int kCpolNt = 2;

MOE_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
MOE_DEV i32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// The same load with the non-temporal cache policy (nt): its lines go first when
// the L2 and the memory-side cache evict, so a stream read once does not push out
// data that is read again.
MOE_DEV i32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}

MOE_DEV int xcd_remap(int bid, int G) {
  // Work-groups are dealt round-robin over the 8 XCDs; give each XCD a
  // contiguous range of logical tiles so neighbours share its L2.
  const int q = G >> 3, r = G & 7, x = bid & 7, i = bid >> 3;
  return x * q + min(x, r) + i;
}

}  // namespace moe
