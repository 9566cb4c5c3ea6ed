// Internal launcher interface between the host runtime (api.cpp) and the
// gfx950 kernels.  Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum class Fmt : int { FP8 = 0, BF16 = 1, MX = 2, NV4 = 3 };  // NV4: NVFP4 weights x bf16 activations

struct PlanPtrs {
  int* expert_counts;
  int* expert_start_indices;
  int* expert_ids;
  int* num_active;
  int* src_info;
  int* pair_row;
  int* status;
};

// Routing plan: one fused block up to this many pairs, else count/scan/scatter
// over blocks of kPlanPairsPerBlock pairs.
constexpr int kPlanFusedMaxPairs = 8192;
constexpr int kPlanPairsPerBlock = 4096;

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
  const float* w13_gs;  // NV4: fp32 global scale per expert [E]
  const float* w2_gs;
  void* h;     // intermediate [T*k, I] (E4M3 or bf16)
  void* h_sf;  // its scales: fp32 [T*k, I/128] (FP8) or UE8M0 [T*k, I/32] (MX)
  void* y;     // [T*k, H] bf16, row p = src_info[row]
  // optional timing events (hipEvent_t or null) carried by the launch of each leg's
  // kernel: gate_up start/stop, down start/stop
  hipEvent_t ev[4];
};
size_t ffn_h_bytes(Fmt f, int rows, int I);
size_t ffn_hsf_bytes(Fmt f, int rows, int I);
int ffn_max_m_tiles(int npairs, int E, int bm);
// stage: 0 = both legs, 1 = gate_up only, 2 = down only
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s, int stage = 0);

// shared, residual: bf16 [T,H] addends or nullptr
hipError_t launch_combine(const void* y, const float* w, const int* pair_row, int T, int topk, int H,
                          const void* shared, const void* residual, void* out, hipStream_t s);

}  // namespace moe
