// Internal launcher interface between the host runtime (api.cpp) and the
// gfx950 kernels.  Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// NV4: NVFP4 weights x bf16 activations; NVF4: NVFP4 weights x NVFP4 activations (its gate_up
// leg decodes the activations while staging them; its down leg is NV4's on the bf16
// intermediate that holds the requantised codes times their block scales)
enum class Fmt : int { FP8 = 0, BF16 = 1, MX = 2, NV4 = 3, NVF4 = 4 };

struct PlanPtrs {
  int* expert_counts;
  int* expert_start_indices;
  int* expert_ids;
  int* num_active;
  int* src_info;
  int* pair_row;
  int* status;
  int* counters;   // fused-combine arrival counters to zero, or nullptr
  int n_counters;
  int* split_counters;  // the down leg's split-tail arrival counters to zero, or nullptr
  int n_split;
};

// Routing plan built inside the gate_up launch: at most this many pairs.
constexpr int kPlanFusedMaxPairs = 8192;
// The plan's own kernels: one block up to kPlanSingleBlockMaxPairs pairs, else
// a count and a scatter launch over blocks of plan_pairs_per_block(npairs) pairs: 1024
// to 4096 (a multiple of 1024), as few blocks as keep 16 busy (measured: 8192
// pairs over 8 blocks 7 us faster than in one; 65536 over 16 of 4096 faster than
// over 64 of 1024: more blocks, more per-block counts to sum per expert).
constexpr int kPlanSingleBlockMaxPairs = 2048;
constexpr int kPlanMaxPairsPerBlock = 4096;
int plan_pairs_per_block(int npairs);

int plan_num_blocks(int npairs);
size_t plan_workspace_bytes(int npairs, int E);
hipError_t launch_plan(const void* ids, bool idx64, int npairs, int E, const PlanPtrs& out, int* ws,
                       hipStream_t s);
// bias: per-expert selection bias [E] or nullptr
hipError_t launch_route_logits_topk(const float* logits, const float* bias, int T, int E, int k, void* idx_out,
                                    bool idx64, float* w_out, bool fast, hipStream_t s);

// Prepared weight layout: tiles of 16 rows x one K-step in MFMA lane order.
size_t prepared_tile_bytes(Fmt f);                           // 2048 (FP8), 4096 (BF16), 1024 (MX, NV4)
int prepared_ksteps(Fmt f, int K);                           // K-steps of 128 (64 for BF16, NV4) elements
size_t prepared_expert_bytes(Fmt f, int rows, int K);        // one expert's weight tiles
size_t prepared_scale_expert_bytes(Fmt f, int rows, int K);  // MX, NV4: one expert's scale tiles; else 0
// Relayout E experts' [rows, K] weights (and MX / NV4 scales; FP8 scales are copied).
// gate_up: the matrix is the gate_up weight (BF16 and NV4 interleave its gate and up rows).
hipError_t launch_prepare(Fmt f, int E, int rows, int K, bool gate_up, const void* w, const void* w_sf, void* out,
                          void* out_sf, hipStream_t s);

// Grouped GEMMs over prepared weights.  Tile rows per workgroup (BM) by regime.
struct FfnArgs {
  Fmt fmt;
  int T, E, topk, H, I;
  float clamp;
  bool fast;
  int bm;  // 80 (weight-bound tiles; 96 for bf16 operands) or 128 (MFMA-bound tiles)
  const int* start;     // expert_start_indices [E+1]
  const int* src_info;  // [T*k]
  const void* x;
  const void* x_sf;
  const void* w13;  // prepared layout
  const void* w13_sf;
  const void* w2;
  const void* w2_sf;
  const float* w13_gs;  // NV4: fp32 global scale per expert [E]; NVF4: the legs' per-expert output scales
  const float* w2_gs;
  const float* c_scales;  // NVF4: per-expert global scale of the requantised intermediate [E]
  void* h;     // intermediate [T*k, I] (E4M3 or bf16)
  void* h_sf;  // its scales: fp32 [T*k, I/128] (FP8) or UE8M0 [T*k, I/32] (MX)
  void* y;     // [T*k, H] bf16, row p = src_info[row]
  // optional timing events (hipEvent_t or null) carried by the launch of each leg's
  // kernel: gate_up start/stop, down start/stop
  hipEvent_t ev[4];
  // combine fused into the down leg (fuse_combine): out = sum_j w[t,j] y[t,j] (+ addends)
  bool fuse_combine;
  const int* pair_row;
  const float* topk_w;
  int* counters;  // [T, combine_counter_stride(H)] zeroed by the plan
  // the down leg's split tail (MFMA-bound tiles): ffn_split_bytes(fmt) bytes, its
  // counters zeroed by the plan; nullptr: no split
  void* split;
  void* out;
  const void* shared;
  const void* residual;
  bool out_f32;
  // routing plan built inside the gate_up launch (plan_ids != nullptr; weight-bound
  // tiles, npairs <= kPlanFusedMaxPairs): `plan` receives what launch_plan writes
  const void* plan_ids;
  bool ids64;
  PlanPtrs plan;
};
// Whether the gate_up launch can build the routing plan itself: weight-bound tiles
// and at most kPlanFusedMaxPairs pairs.  `pays` adds the cost rule: every workgroup
// of the launch reads and counts all the ids, so the pairs times the rounds of
// workgroups a CU runs must stay small (decode: 2048 pairs, 2 rounds of the
// worst-case grid; the W4A8 shape, 8192 pairs over ~11 rounds, is not).  The host
// API decides; the launcher builds the plan in the launch when handed the ids.
bool ffn_plan_fusable(Fmt f, int bm, int npairs, int E, int I, bool pays);
// int32 arrival counters per token that the fused combine needs: one per column
// tile of the down leg, at most ceil(H / 128)
inline int combine_counter_stride(int H) { return (H + 127) / 128; }
// Split tail of the MFMA-bound down leg: at most this many workgroups at once
// (partial tiles and counters) and pieces per tile.  The buffer holds the
// kSplitMaxSlots counters (ffn_split_counter_bytes), then the partial tiles;
// ffn_split_bytes is 0 for formats whose down leg never splits.
constexpr int kSplitMaxSlots = 256;
constexpr int kSplitMaxPieces = 8;
constexpr size_t ffn_split_counter_bytes() { return (size_t)kSplitMaxSlots * 4; }
size_t ffn_split_bytes(Fmt f);
size_t ffn_h_bytes(Fmt f, int rows, int I);
size_t ffn_hsf_bytes(Fmt f, int rows, int I);
int ffn_max_m_tiles(int npairs, int E, int bm);
// stage: 0 = both legs, 1 = gate_up only, 2 = down only
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s, int stage = 0);

// shared, residual: bf16 [T,H] addends or nullptr; out: bf16 [T,H], or fp32 when out_f32
hipError_t launch_combine(const void* y, const float* w, const int* pair_row, int T, int topk, int H,
                          const void* shared, const void* residual, void* out, bool out_f32, hipStream_t s);

}  // namespace moe
