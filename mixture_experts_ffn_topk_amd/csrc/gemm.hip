// Grouped (per-expert, variable-M) GEMMs of the expert FFN on gfx950 MFMA.
//
//   gate_up:  [rows of expert e] x W13[e]^T -> g, u  -> clamped SwiGLU -> requant -> h
//   down:     h[rows of expert e] x W2[e]^T          -> y[src_info[row]] (bf16)
//
// Both legs walk one shared expert list (Struct_mega_ffn_ep_combine_send page:
// num_active_experts / expert_start_indices); each workgroup finds its tile
// from the per-expert prefix sums, so no device-side tile list is needed.  A
// weight-bound gate_up launch can also build that plan itself (plan_ids set):
// every workgroup counts the ids into LDS, finds its tile there, and ranks its
// own expert's pairs while its weight ring is in flight; the launch writes the
// plan for the down leg and the combine (the plan kernel then leaves the step).
//
// Workgroup: WAVES wavefronts, BM rows x BN = WAVES*16*NT weight rows per tile.
//   * A (activation rows, gathered through src_info for gate_up) is staged in
//     LDS, KSG K-steps per stage, rows XOR-swizzled in 16-byte chunks; MFMA-bound
//     FP8 / bf16-operand tiles load it with direct-to-LDS buffer loads.
//   * B (weights) streams from HBM straight into VGPRs from the prepared tiles
//     (MFMA operand order, one 1 KB run per wave load), DEPTH K-steps deep,
//     each wave owning 16*NT weight rows.  Every weight byte of a tile is read
//     once; weight-bound tiles stream it with the non-temporal cache policy.
// Tiles map to the 8 XCDs in contiguous ranges: column-tile major for the
// MFMA-bound regime (an XCD's tiles share an expert's weights in its L2),
// expert major for the weight-bound one (an expert's activation rows stay in L2).
// All global loads are buffer loads: a uniform base, a loop-invariant 32-bit
// lane offset and the K-step offset in a scalar register; a lane offset past
// the end of the resource reads zeros, which masks rows and columns outside
// the problem.
// MFMA per format, weights as the first operand and activations as the second:
//   FP8 block-128: v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales per
//                  K-step of 128 into a partial, then acc += (sa[token] * sb) *
//                  partial with the fp32 block scales of the DeepSeek FP8 encoding.
//   BF16:          v_mfma_f32_32x32x16_bf16, four per 32-row tile and K-step of 64.
//   NV4 (NVFP4 x BF16): the same bf16 MFMAs on weights decoded in registers:
//                  E2M1 -> fp32 (exact) times the E4M3 block scale of its 16
//                  elements (exact in bf16); the expert's global scale
//                  multiplies the accumulators in the epilogue.
//   MX (W4A8):     v_mfma_scale_f32_16x16x128_f8f6f4, weights E2M1 + UE8M0,
//                  activations E4M3 + UE8M0, the block scales applied by the hardware.
// 16x16 output tiles hold 4 f32 per lane (token l%16, weight rows 4*(l/16)+i);
// 32x32 tiles 16 (token l%32, weight rows 8*(i/4)+4*(l/32)+i%4).
// Operand lane layout (lane l, g = l/16): an FP8 row segment of 128 bytes is fed
// as bytes [16g, 16g+16) and [64+16g, 64+16g+16); an E2M1 segment of 64 bytes
// as bytes [16g, 16g+16); the scale byte of lane l belongs to K-block g (32
// elements) of row l%16; a bf16 32x32x16 operand gives lane l = 32h + r the
// K elements [8h, 8h+8) of its 16-element sub-step, row r.
#include <hip/hip_ext.h>

#include <type_traits>

#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe {

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

// Formats whose MFMA runs on bf16 operands (32x32x16): BF16, and NV4, whose
// E2M1 weights are decoded to bf16 in registers.  Both take bf16 activations.
constexpr bool bf16_mma(Fmt f) { return f == Fmt::BF16 || f == Fmt::NV4 || f == Fmt::NVF4; }
// Formats whose weights are NVFP4, decoded to bf16 in registers.
constexpr bool nv4w(Fmt f) { return f == Fmt::NV4 || f == Fmt::NVF4; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// Two fp32 values -> packed bf16 (round to nearest even; NV4 products are exact in bf16)
MOE_DEV int pack_bf16x2(f32x2 v) { return __builtin_bit_cast(int, __builtin_convertvector(v, bf16x2v)); }
// NV4: 8 E2M1 values (a 32-bit word, element 2i in the low nibble of byte i) times
// their E4M3 block scale s, as 8 bf16.  The product of a 2-bit and a 4-bit
// significand is exact in bf16; the hardware conversion is exact (unit scale).
MOE_DEV i32x4 nv4_bf16x8(uint32_t d, float s) {
  i32x4 r;
  r[0] = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0) * s);
  r[1] = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1) * s);
  r[2] = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2) * s);
  r[3] = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3) * s);
  return r;
}


template <Fmt F, int NT>
struct BFrag {
  // 16-byte pieces of the lane's weight K-step segment: FP8 / BF16 use bytes
  // [16g, 16g+16) (lo) and [64+16g, 64+16g+16) (hi); MX uses lo (32 E2M1 values)
  // and a scale byte; NV4 uses lo[t] (32 E2M1 values of 32-row tile t) and sc[t]
  // (its four E4M3 block scales).  Kept as separate 4-register values so that each load
  // lands in the registers the MFMA reads.
  i32x4 lo[NT], hi[NT];
  int sc[NT];
};


template <Fmt F, bool GATEUP, int BM, int WAVES, int NT, int KSG>
struct Tile {
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int BN = WAVES * 16 * NT;  // weight rows per workgroup tile
  static constexpr int MT = BM / 16;
  // A is staged per K-step as kARows rows of 128 bytes, the 16-byte chunk c of
  // row r stored at chunk c ^ swz(r) (r & 7, below), so that the rows of an MFMA fragment read
  // spread over all LDS banks (a padded row stride still halves the read rate).
  // Weight-bound BF16 tiles keep a padded 144-byte row instead: the swizzle's
  // per-sub-step offsets do not fit their register budget.
  // direct-to-LDS staging (below); NVFP4 activations are decoded on the way to LDS.
  // Weight-bound MX tiles take their activation scales from a per-tile table
  // (kSfTab), so their activations can go direct-to-LDS too (W4A8 gate_up -1.5 %).
  static constexpr bool kDma = (F != Fmt::MX && F != Fmt::NVF4 && BM > 96) || (F == Fmt::MX && BM <= 96);
  // MFMA-bound FP8 and BF16 down tiles may split a last partial round over K (the
  // split tail; NVFP4 x BF16's would spill registers)
  static constexpr bool kSplit = !GATEUP && BM > 96 && kDma && (F == Fmt::FP8 || F == Fmt::BF16);
  static constexpr int kSwz = bf16_mma(F) && !kDma ? 0 : 7;
  // By the bank-conflict counter, the LDS serves a 128-bit read to lanes 0-7 and
  // 16-23 (8-15 and 24-31, ...) together.  A 32x32 BF16 fragment puts rows r and
  // r + 16 in lanes r and r + 16, and rows 16 x 128 bytes apart share banks, so the
  // swizzle of those tiles also flips chunk bit 0 with row bit 4 (Mixtral gate_up:
  // 125 M conflict cycles per launch to 2 M, -0.5 % time; 16x16 FP8 / MX
  // fragments put one row in lanes r and r + 16, which the XOR already spreads).
  static constexpr bool kSwz16 = bf16_mma(F) && kDma;
  MOE_HOST_DEV static constexpr int swz(int r) { return (r & kSwz) ^ (kSwz16 ? (r >> 4) & 1 : 0); }
  static constexpr int kARowBytes = bf16_mma(F) && !kDma ? 144 : 128;
  static constexpr int kAChunks = (BM * 8 + kThreads - 1) / kThreads;  // 16-byte A chunks per thread and K-step
  // A buffer rows: BM rounded up so that every thread stores every chunk it loads
  // (chunks past BM rows are zeros landing in spare rows): no divergent stores in the loop
  static constexpr int kARows = kAChunks * kThreads / 8;
  static constexpr int kOutRowBytes = GATEUP ? (BN / 2) * (bf16_mma(F) ? 2 : 1) : BN * 2;
  static constexpr int kOutStride = kOutRowBytes + 16;
  static constexpr int kAStepBytes = kARows * kARowBytes;
  // MFMA-bound FP8 / BF16 tiles and weight-bound MX tiles stage A with
  // direct-to-LDS loads, two stages ahead, into four buffers (at least three: the
  // load two stages ahead cannot land in the buffer being read; four keep the
  // unrolled K loop a divisor of the usual K-step counts, so that it runs no
  // padding steps): no staging registers, which also leaves BF16 room for the
  // swizzled layout.  The others load A into registers and store it,
  // double-buffered (measured faster for the weight-bound FP8 and BF16 tiles,
  // whose weight stream then starts before the activation addresses are known).
  static constexpr int kABufs = kDma ? 4 : 2;
  // Weight-bound MX tiles stage their rows' whole UE8M0 scale rows in LDS once per
  // tile (dynamic LDS) instead of four bytes per row and K-step: one cache line per
  // row and K-step was as many L2 requests as the weights' own.
  static constexpr bool kSfTab = F == Fmt::MX && BM <= 96;
  static constexpr int kABytes = kABufs * KSG * kAStepBytes;
  static constexpr int kOutBytes = BM * kOutStride;
  static constexpr int kUnion = kABytes > kOutBytes ? kABytes : kOutBytes;
  static constexpr int kSA = kThreads > BM ? kThreads : BM;  // A-scale slots per buffer (one per thread)
  static constexpr int kMaxKSteps = 256;  // FP8 weight scales of up to 256 K-steps staged in LDS
  // FP8 weight-scale blocks (128 rows) a tile touches: gate and up block, or a down window of BN rows
  static constexpr int kHB = BN / 2 / 128;  // gate_up: 128-column h blocks per tile
  static constexpr int kNB = GATEUP ? 2 * kHB : BN / 128 + 1;
  // a down tile starts at a multiple of BN: with BN a multiple of 64 it starts 0 or
  // 64 rows into a block, so BN / 128 + 1 blocks cover it
  static_assert(F != Fmt::FP8 || GATEUP || BN % 64 == 0, "FP8 down tiles cover whole 64-row halves of scale blocks");
  static constexpr int kLds = kUnion + kABufs * KSG * kSA * 4 + WAVES * BM * 4 + (F == Fmt::FP8 ? kNB * kMaxKSteps * 4 : 0);
};

// out[t, col .. col+8) = the sum over token t's valid slots j, in ascending order,
// of w[t,j] * y[t,j, col .. col+8) in fp32, then + shared + residual, rounded once
// to bf16 (or stored as fp32): the arithmetic of the separate combine kernel.
// The y rows are read with device-scope coherent loads (they were stored by
// other workgroups, possibly on other XCDs, with device-scope stores), all of a
// group of 8 slots issued before the first is used (a masked slot's row is read
// but not added).
MOE_DEV void combine_chunk8(const GemmParams& p, __amdgpu_buffer_rsrc_t y_rs, int t, int col) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const long long p0 = (long long)t * p.topk;
  for (int j0 = 0; j0 < p.topk; j0 += 8) {
    i32x4 v[8];
    bool ok[8];
    float wj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      const bool in = j < p.topk;
      ok[u] = in && p.pair_row[p0 + (in ? j : 0)] >= 0;
      wj[u] = p.topk_w[p0 + (in ? j : 0)];
      v[u] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     y_rs, (uint32_t)((p0 + (in ? j : 0)) * p.c_row_bytes + (long long)col * 2), 0, kCpolDevice));
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
  const uint16_t* add[2] = {p.shared, p.residual};
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (add[a] == nullptr) continue;
    const i32x4 v = *(const i32x4*)(add[a] + (long long)t * p.N + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t e = (uint32_t)v[q];
      acc[2 * q] += bf16_to_f32((uint16_t)(e & 0xFFFFu));
      acc[2 * q + 1] += bf16_to_f32((uint16_t)(e >> 16));
    }
  }
  if (p.out_f32) {
    f32x4* o = (f32x4*)((float*)p.out + (long long)t * p.N + col);
    o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    i32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (int)bf16x2_rne(acc[2 * q], acc[2 * q + 1]);
    *(i32x4*)((uint16_t*)p.out + (long long)t * p.N + col) = o;
  }
}
constexpr int kZeroSlotTokens = 64;  // tokens per workgroup that looks for tokens without a valid slot

// WAVES waves per workgroup and room for WGS workgroups per CU: the second
// launch bound is the minimum number of waves per SIMD, which caps a wave's
// registers at 512 / that number.
// ---------------------------------------------------------------- routing plan inside the gate_up launch
// (the plan of the Struct_mega_ffn_ep_combine_send page's operands: expert_start_indices,
// expert_ids, num_active_experts, src_info; pair_row is its inverse).  Every
// workgroup of a weight-bound gate_up launch builds what it needs in LDS -- the
// per-expert counts and offsets, and its own rows' pair indices -- so that no
// separate launch precedes it; the results equal launch_plan's bit for bit (rows
// of an expert in pair order, masked and bad ids as there).
struct PlanLds {
  int* cnt;    // [E]
  int* st;     // [E+1] exclusive offsets
  int* misc;   // [4]: bad-id count
  int* wc;     // [nch * waves] matches per (chunk, wave), then their exclusive offsets
  int* srcl;   // [BM] pair index of each of the tile's rows
  short* ex;   // [npairs] expert of each pair, -1 if masked
};
MOE_HOST_DEV inline size_t plan_lds_ints(int E, int npairs, int threads, int bm) {
  const int nch = (npairs + threads - 1) / threads;
  return ((size_t)(2 * E + 1 + 4 + nch * (threads / 64) + bm) + 3) & ~(size_t)3;  // 16-byte multiple
}
MOE_HOST_DEV inline size_t plan_lds_bytes(int E, int npairs, int threads, int bm) {
  return plan_lds_ints(E, npairs, threads, bm) * 4 + (size_t)npairs * 2;
}
// MX scale table: a row of sf_row scale bytes padded to a multiple of 4 with an odd
// dword count (the 16 rows a K-step's lanes read then fall in distinct banks).
MOE_HOST_DEV inline int mx_table_stride(int sf_row) {
  const int s = (sf_row + 3) & ~3;
  return ((s >> 2) & 1) ? s : s + 4;
}
MOE_HOST_DEV inline size_t plan_region_bytes(bool plan, int E, int npairs, int threads, int bm) {
  return plan ? (plan_lds_bytes(E, npairs, threads, bm) + 15) & ~(size_t)15 : 0;
}
MOE_DEV PlanLds plan_lds_carve(int* base, int E, int npairs, int threads, int bm) {
  const int nch = (npairs + threads - 1) / threads;
  PlanLds L;
  L.cnt = base;
  L.st = base + E;
  L.misc = L.st + E + 1;
  L.wc = L.misc + 4;
  L.srcl = L.wc + nch * (threads / 64);
  L.ex = (short*)(base + plan_lds_ints(E, npairs, threads, bm));
  return L;
}

// Counts and exclusive offsets of every expert into LDS; workgroup 0 also writes
// the plan's counts, offsets, active list (ascending, then -1), status, the pair
// rows of masked slots (-1) and zeroes the fused combine's and the split tail's counters.
template <int kThreads>
MOE_DEV void plan_counts_in_lds(const GemmParams& p, const PlanLds& L) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6, E = p.E, np = p.npairs;
  for (int e = tid; e < E; e += kThreads) L.cnt[e] = 0;
  if (tid == 0) L.misc[0] = 0;
  __syncthreads();
  int bad = 0;
  for (int q = tid; q < np; q += kThreads) {
    const long long v = p.ids64 ? ((const long long*)p.plan_ids)[q] : (long long)((const int*)p.plan_ids)[q];
    int e = -1;
    if (v >= 0 && v < E) e = (int)v;
    else if (v != -1) ++bad;
    L.ex[q] = (short)e;
    if (e >= 0) atomicAdd(&L.cnt[e], 1);
  }
  if (bad) atomicAdd(&L.misc[0], bad);
  __syncthreads();
  const bool head = blockIdx.x == 0;
  if (wave == 0) {
    int carry = 0, acarry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? L.cnt[e] : 0;
      const int a = c > 0;
      int incl = c, ainc = a;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d), oa = __shfl_up(ainc, d);
        if (lane >= d) {
          incl += o;
          ainc += oa;
        }
      }
      if (e < E) {
        L.st[e] = carry + incl - c;
        if (head) {
          p.plan_out.expert_counts[e] = c;
          p.plan_out.expert_start_indices[e] = carry + incl - c;
          if (a) p.plan_out.expert_ids[acarry + ainc - a] = e;
        }
      }
      carry += __shfl(incl, 63);
      acarry += __shfl(ainc, 63);
    }
    if (lane == 0) L.st[E] = carry;
    if (head) {
      if (lane == 0) {
        p.plan_out.expert_start_indices[E] = carry;
        *p.plan_out.num_active = acarry;
        *p.plan_out.status = L.misc[0];
      }
      for (int e = acarry + lane; e < E; e += 64) p.plan_out.expert_ids[e] = -1;
    }
  }
  if (head) {
    for (int q = tid; q < np; q += kThreads)
      if (L.ex[q] < 0) p.plan_out.pair_row[q] = -1;
    if (p.plan_out.counters != nullptr)
      for (int i = tid; i < p.plan_out.n_counters; i += kThreads) p.plan_out.counters[i] = 0;
    if (p.plan_out.split_counters != nullptr)
      for (int i = tid; i < p.plan_out.n_split; i += kThreads) p.plan_out.split_counters[i] = 0;
  }
  __syncthreads();
}

// A workgroup barrier that waits for this wave's LDS accesses only (outstanding
// global loads, such as a weight ring already in flight, keep flying).
MOE_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The pair indices of rows [lo, lo + rows) of `expert` (its pairs in pair order)
// into L.srcl (the workgroups of column tile 0 store them as the plan's src_info
// and pair_row at the end of the kernel).  Pair q = c * kThreads + tid is visited
// in (chunk c, wave, lane) order, which is pair order.
template <int kThreads>
MOE_DEV void plan_rows_in_lds(const GemmParams& p, const PlanLds& L, int expert, int lo, int rows) {
  constexpr int W = kThreads / 64;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6, np = p.npairs;
  const int nch = (np + kThreads - 1) / kThreads;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int c = 0; c < nch; ++c) {
    const int q = c * kThreads + tid;
    const uint64_t bal = __ballot(q < np && L.ex[q] == expert);
    if (lane == 0) L.wc[c * W + wave] = (int)__popcll(bal);
  }
  lds_barrier();
  if (wave == 0) {
    int carry = 0;
    for (int i0 = 0; i0 < nch * W; i0 += 64) {
      const int i = i0 + lane;
      const int v = i < nch * W ? L.wc[i] : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      if (i < nch * W) L.wc[i] = carry + incl - v;
      carry += __shfl(incl, 63);
    }
  }
  lds_barrier();
  for (int c = 0; c < nch; ++c) {
    const int q = c * kThreads + tid;
    const bool m = q < np && L.ex[q] == expert;
    const uint64_t bal = __ballot(m);
    if (m) {
      const int r = L.wc[c * W + wave] + (int)__popcll(bal & lt) - lo;
      if (r >= 0 && r < rows) L.srcl[r] = q;
    }
  }
  lds_barrier();
}

template <Fmt F, bool GATEUP, int BM, int WAVES, int NT, int DEPTH, int KSG, int WGS, bool FAST>
__global__ __launch_bounds__(64 * WAVES, (WAVES * WGS + 3) / 4) void ffn_gemm_kernel(GemmParams p) {
  using TL = Tile<F, GATEUP, BM, WAVES, NT, KSG>;
  constexpr int BN = TL::BN;
  constexpr int MT32 = BM / 32, NT32 = NT / 2;  // BF16: 32-row token slices and weight tiles
  static_assert(!bf16_mma(F) || BM % 32 == 0, "bf16-operand tiles hold whole 32-token slices");
  // Weight-bound BF16 tiles skip the 32-row token slices past the tile's rows
  // (experts smaller than the tile; measured faster).  The other K-steps compute
  // every slice (NVFP4: all but the last): a branch would split the
  // software-pipelined K-step into blocks the scheduler cannot interleave.
  constexpr bool kSkipSlices = bf16_mma(F);
  constexpr bool kPrio = BM > 96 && !bf16_mma(F);  // (measured: helps MFMA-bound FP8 / MX tiles only)
  static_assert(!GATEUP || NT % 2 == 0, "gate_up pairs a gate tile with an up tile");
  constexpr int HC = BN / 2;  // gate_up: h columns per tile (gate and up rows, NT/2 tiles each per wave)
  static_assert(!GATEUP || HC % 128 == 0, "a gate_up tile holds whole 128-column blocks of h");
  constexpr int MT = TL::MT;
  constexpr int kThreads = TL::kThreads;
  constexpr int HW = 8 * NT;  // gate_up: h columns per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds[TL::kLds];
  uint8_t* a_lds = lds;                                          // [kABufs][KSG][kARows][kARowBytes]
  uint8_t* out_lds = lds;                                        // aliases a_lds after the K loop
  uint32_t* sa_lds = (uint32_t*)(lds + TL::kUnion);              // [kABufs][KSG][kSA] (fp32 bits or 4 UE8M0 bytes)
  float* red_lds = (float*)(lds + TL::kUnion + TL::kABufs * KSG * TL::kSA * 4);  // [WAVES][BM]
  float* sb_lds = red_lds + WAVES * BM;                      // FP8: [kNB][kMaxKSteps] weight scales

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6, g = lane >> 4, r16 = lane & 15;

  // Fused combine: the workgroups past the GEMM grid write the output of the tokens
  // that have no valid slot (no tile will reduce them): the addends, or zeros.
  if (!GATEUP && p.fuse && (int)blockIdx.x >= p.m_grid) {
    const int t0 = ((int)blockIdx.x - p.m_grid) * kZeroSlotTokens;
    for (int t = t0; t < min(p.T, t0 + kZeroSlotTokens); ++t) {
      bool any = false;
      for (int j = 0; j < p.topk; ++j) any |= p.pair_row[(long long)t * p.topk + j] >= 0;
      if (any) continue;  // (uniform: every thread reads the same entries)
      for (int col = tid * 8; col < p.N; col += kThreads * 8) combine_chunk8(p, make_rsrc(p.C, p.y_bytes), t, col);
    }
    return;
  }

  // ---------------------------------------------------------------- routing plan (in-launch form)
  // Weight-bound gate_up launches may build the plan themselves (plan_ids set): the
  // offsets and the tile's row sources then come from LDS instead of the plan buffers.
  extern __shared__ __attribute__((aligned(16))) int plan_dyn[];  // dynamic LDS: the in-launch plan
  const int* st_p = p.start;
  PlanLds PL{};
  constexpr bool kPlanHere = GATEUP && BM <= 96;
  const bool plan_here = kPlanHere && p.plan_ids != nullptr;
  if constexpr (kPlanHere) {
    if (plan_here) {
      PL = plan_lds_carve(plan_dyn, p.E, p.npairs, kThreads, BM);
      plan_counts_in_lds<kThreads>(p, PL);
      st_p = PL.st;
    }
  }

  // ---------------------------------------------------------------- tile decode
  // The grid is sized for the worst case; the real m-tile count (per-expert tile
  // counts summed) sends the surplus workgroups home at once, so that the
  // XCD-aware mapping spreads real tiles only.
  int total_m = 0;
  for (int e0 = 0; e0 < p.E; e0 += 64) {
    const int e = e0 + lane;
    int t = e < p.E ? (st_p[e + 1] - st_p[e] + BM - 1) / BM : 0;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d);
    total_m += t;
  }
  total_m = __builtin_amdgcn_readfirstlane(total_m);
  const int G = total_m * p.n_tiles;
  // Split tail (MFMA-bound down tiles, split buffers given): when the tiles leave
  // a last partial round of at most half the slots (the workgroups the part runs
  // at once), each of those tail tiles is cut over K into S pieces of whole
  // K-loop trips, which run side by side after the whole tiles; each piece stores
  // its fp32 partial tile, and the last to arrive sums the partials in piece
  // order (the same result whichever arrives last) and runs the epilogue.
  constexpr bool kSplit = TL::kSplit;
  constexpr int U = lcm_c(TL::kABufs * KSG, DEPTH);  // K-steps per trip of the unrolled K loop
  int tail = 0, nparts = 1, piece = -1, tail_j = 0;
  if constexpr (kSplit) {
    if (p.split_slots > 0) {
      const int rem = G % p.split_slots;
      const int S = rem > 0 ? min(min(p.split_slots / rem, kSplitMaxPieces), (p.ksteps + U - 1) / U) : 1;
      if (S >= 2) tail = rem, nparts = S;
    }
  }
  const int Gw = G - tail;  // whole tiles
  int L;
  if ((int)blockIdx.x < Gw) {
    L = xcd_remap(blockIdx.x, Gw);
  } else {
    const int q = (int)blockIdx.x - Gw;
    if (q >= tail * nparts) return;
    tail_j = q / nparts;
    piece = q - tail_j * nparts;
    L = Gw + tail_j;
  }
  // this workgroup's K-steps [k0, k0 + KS)
  int k0 = 0, KS = p.ksteps;
  if (piece >= 0) {
    const int nu = (p.ksteps + U - 1) / U;
    k0 = piece * nu / nparts * U;
    KS = min(p.ksteps, (piece + 1) * nu / nparts * U) - k0;
  }
  // Weight-bound tiles (about one m-tile per expert: no weight reuse between
  // m-tiles) run expert-major, so that an expert's activation rows stay in the
  // XCD's L2 across its column tiles.  MFMA-bound tiles run column-tile-major, so
  // that an XCD's consecutive tiles share weights.
  const int m_tile = BM <= 96 ? L / p.n_tiles : L % total_m;
  const int n_tile = BM <= 96 ? L % p.n_tiles : L / total_m;
  int expert = -1, tile_in_e = 0, e_start = 0, e_count = 0;
  {
    int base = 0;
    for (int e0 = 0; e0 < p.E; e0 += 64) {
      const int e = e0 + lane;
      const int st_e = e < p.E ? st_p[e] : 0;
      const int cnt = e < p.E ? st_p[e + 1] - st_e : 0;
      const int tiles = (cnt + BM - 1) / BM;
      int incl = tiles;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      const int excl = incl - tiles;
      const bool hit = m_tile >= base + excl && m_tile < base + incl;
      const uint64_t bal = __ballot(hit);
      if (bal) {
        const int src = __ffsll((unsigned long long)bal) - 1;
        expert = e0 + src;
        tile_in_e = m_tile - base - __shfl(excl, src);
        e_start = __shfl(st_e, src);
        e_count = __shfl(cnt, src);
        break;
      }
      base += __shfl(incl, 63);
    }
  }
  expert = __builtin_amdgcn_readfirstlane(expert);
  tile_in_e = __builtin_amdgcn_readfirstlane(tile_in_e);
  if (expert < 0) return;  // (not reached: L < G)
  const int row0 = __builtin_amdgcn_readfirstlane(e_start) + tile_in_e * BM;
  const int rows = min(BM, __builtin_amdgcn_readfirstlane(e_count) - tile_in_e * BM);
  // the sources of the tile's rows: the plan's src_info, or (in-launch plan) LDS,
  // filled after the weight ring is issued (below)
  const int* src_p = p.src_info + row0;

  // ---------------------------------------------------------------- B (weight) addressing
  // Weights arrive in the prepared layout: per expert, tiles of 16 rows x one
  // K-step, row block major then K-step, each tile contiguous in MFMA lane order
  // (lane l's 16 bytes at 16*l, FP8/BF16 second halves 1 KB further), so one
  // load instruction of a wave reads 1 KB of consecutive bytes.
  // (a split piece's resources start at its first K-step: tile ks of a row block
  // lies ks tiles past the block's first)
  const __amdgpu_buffer_rsrc_t b_rs =
      make_rsrc(p.B + (size_t)expert * p.b_expert_bytes + (size_t)k0 * p.b_tile, p.b_expert_bytes - (uint32_t)k0 * p.b_tile);
  // FP8 weight scales of the tile, per thread (kNB rows of at most kMaxKSteps)
  constexpr int kSbPer = F == Fmt::FP8 ? (TL::kNB * TL::kMaxKSteps + kThreads - 1) / kThreads : 1;
  float sb_pre[kSbPer];
  __amdgpu_buffer_rsrc_t bsc_rs = b_rs;
  uint32_t b_off[NT], bsc_off[NT];
  // MX with four 16-row tiles per wave: the wave's 4 x 64 scale bytes of a K-step are
  // one dword per lane (lane l: dword l % 16 of tile l / 16), handed to the lanes
  // that use them with ds_bpermute: one load per K-step instead of one per tile.
  constexpr bool kMxDenseSc = F == Fmt::MX && NT == 4;
  uint32_t bsc_dense = kOOB;
  {
    if (F == Fmt::MX || nv4w(F))
      bsc_rs = make_rsrc((const uint8_t*)p.B_sf + (size_t)expert * p.bsc_expert_bytes, p.bsc_expert_bytes);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      int wrow0, col0;  // first weight row and first output column of the 16-row tile
      if (GATEUP) {
        col0 = n_tile * HC + wave * HW + 16 * (nt % (NT / 2));  // h column
        wrow0 = (nt < NT / 2 ? 0 : p.N) + col0;                      // gate rows, then up rows
      } else {
        col0 = n_tile * BN + wave * 16 * NT + 16 * nt;
        wrow0 = col0;
      }
      uint32_t tiles0 = (uint32_t)(wrow0 / 16) * (uint32_t)p.ksteps;  // first tile of the row block
      if (bf16_mma(F)) {
        // 32-row tiles: gate_up tile j holds gate rows [16j, 16j+16) then the
        // matching up rows; down tile j holds rows [32j, 32j+32)
        const int t = nt < NT32 ? nt : 0;
        col0 = GATEUP ? n_tile * HC + wave * HW + 16 * t : n_tile * BN + wave * 16 * NT + 32 * t;
        tiles0 = (uint32_t)(GATEUP ? col0 / 16 : col0 / 32) * (uint32_t)p.ksteps;
      }
      const bool ok = col0 < p.N;
      b_off[nt] = ok ? tiles0 * p.b_tile + (uint32_t)lane * 16u : kOOB;
      // MX: the lane's scale byte; NV4: the four scale bytes of the lane's tile row
      bsc_off[nt] = ok ? (nv4w(F) ? tiles0 * 128u + (uint32_t)(lane & 31) * 4u : tiles0 * 64u + (uint32_t)lane)
                       : kOOB;
      if (kMxDenseSc && (lane >> 4) == nt) bsc_dense = ok ? tiles0 * 64u + (uint32_t)(lane & 15) * 4u : kOOB;
    }
    if (F == Fmt::FP8) {
      // the tile's weight-scale rows, staged in LDS: gate_up [0, kHB) the gate
      // blocks, [kHB, 2 kHB) the up blocks; down: the kNB 128-row blocks from the
      // tile's first (blocks past the last stand in for dead columns).  Loaded
      // here, stored to LDS after the prologue's weight and activation loads are
      // issued, so that their round trip overlaps those loads.
      const float* sfe = (const float*)p.B_sf + (size_t)expert * (p.n_rows / 128) * p.b_sf_row + k0;
      const int nblk = p.n_rows / 128;
#pragma unroll
      for (int q = 0; q < kSbPer; ++q) {
        const int i = tid + q * kThreads;
        sb_pre[q] = 0.f;
        if (i < TL::kNB * KS) {
          const int j = i / KS, k = i - j * KS;
          const int hb = TL::kHB, hblk = p.N / 128;
          const int blk = GATEUP ? (j < hb ? min(n_tile * hb + j, hblk - 1) : hblk + min(n_tile * hb + j - hb, hblk - 1))
                                 : min(n_tile * BN / 128 + j, nblk - 1);
          sb_pre[q] = sfe[(size_t)blk * p.b_sf_row + k];
        }
      }
    }
  }
  // FP8: which staged scale row this wave's column tile nt uses
  auto sb_row = [&](int nt) {
    if (GATEUP) return (nt >= NT / 2 ? TL::kHB : 0) + (wave * HW + 16 * (nt % (NT / 2))) / 128;
    return ((n_tile * BN) % 128 + wave * 16 * NT + 16 * nt) / 128;
  };
  // Weight-bound tiles read each weight byte once in the whole launch: those loads
  // stream (non-temporal), which keeps the activation rows and the plan's tables
  // cached and, across launches, what the memory-side cache holds (decode gate_up
  // -10 %, down -6.5 %).  MFMA-bound tiles re-read an expert's weights from L2 in
  // every m-tile, so theirs stay cached.
  auto bload_w = [&](uint32_t voff, uint32_t soff) {
    return BM <= 96 ? bload16_nt(b_rs, voff, soff) : bload16(b_rs, voff, soff);
  };
  auto load_b = [&](BFrag<F, NT>& b, int ks) {
    const uint32_t dead = oob_if(ks >= KS);  // (the prepared layout is zero past a row's end)
    if constexpr (F == Fmt::BF16) {
      // 32-row tile t: four 1 KB sub-step pieces
#pragma unroll
      for (int t = 0; t < NT32; ++t) {
        const uint32_t o = b_off[t] | dead;
        b.lo[2 * t] = bload_w(o, (uint32_t)ks * p.b_tile);
        b.lo[2 * t + 1] = bload_w(o + 1024u, (uint32_t)ks * p.b_tile);
        b.hi[2 * t] = bload_w(o + 2048u, (uint32_t)ks * p.b_tile);
        b.hi[2 * t + 1] = bload_w(o + 3072u, (uint32_t)ks * p.b_tile);
      }
      return;
    }
    if constexpr (nv4w(F)) {
      // 32-row tile t: one 1 KB load of E2M1 data and the lanes' block scales
#pragma unroll
      for (int t = 0; t < NT32; ++t) {
        b.lo[t] = bload_w(b_off[t] | dead, (uint32_t)ks * p.b_tile);
        b.sc[t] = (int)__builtin_amdgcn_raw_buffer_load_b32(bsc_rs, bsc_off[t] | dead, (uint32_t)ks * 128u, 0);
      }
      return;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t o = b_off[nt] | dead;
      b.lo[nt] = bload_w(o, (uint32_t)ks * p.b_tile);
      if (F == Fmt::MX) {
        if constexpr (kMxDenseSc) {
          if (nt == 0) b.sc[0] = (int)__builtin_amdgcn_raw_buffer_load_b32(bsc_rs, bsc_dense | dead, (uint32_t)ks * 64u, 0);
        } else {
          b.sc[nt] = (int)__builtin_amdgcn_raw_buffer_load_b8(bsc_rs, bsc_off[nt] | dead, (uint32_t)ks * 64u, 0);
        }
      } else {
        b.hi[nt] = bload_w(o + 1024u, (uint32_t)ks * p.b_tile);
      }
    }
  };

  // ---------------------------------------------------------------- A (activation) addressing
  // A is staged KSG K-steps at a time.  For each K-step of a stage, thread tid
  // loads 16-byte chunks c = tid + threads*i of the BM x 128-byte tile: row c/8, chunk c%8.
  // The gathered rows' src_info entries are loaded here, without branches (rows
  // past the tile's read its last entry and are then masked), before the weight
  // ring is issued, and used after it: their round trip then overlaps the
  // weights' instead of preceding it.
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(p.A + (size_t)k0 * 128u, p.a_bytes - (uint32_t)k0 * 128u);
  int a_src[TL::kAChunks];
  auto gather_a_src = [&]() {
#pragma unroll
    for (int i = 0; i < TL::kAChunks; ++i)
      a_src[i] = GATEUP ? src_p[min((tid + kThreads * i) >> 3, rows - 1)] : 0;
  };
  if (!plan_here) gather_a_src();
  int asf_src = GATEUP && F == Fmt::FP8 && !plan_here ? src_p[min(tid, rows - 1)] : 0;
  // MX activation scales per stage: the BM x 4 UE8M0 bytes of each of its KSG
  // K-steps, loaded densely, one byte per lane and load (entry e: K-step e / (4 BM),
  // tile row (e % (4 BM)) / 4, K-block e % 4), so that a wave issues one or two
  // loads per stage instead of one per K-block (a scale row of H/32 bytes need not
  // be 4-byte aligned, so wider loads do not apply).
  constexpr int kSfTotal = BM * 4 * KSG;
  constexpr int kSfQ = F == Fmt::MX ? (kSfTotal + kThreads - 1) / kThreads : 1;
  constexpr int kSfN = F == Fmt::MX ? kSfQ : KSG;  // scale registers per stage
  // the K-step of entry tid + kThreads q, known at compile time for every MX tiling
  static_assert(F != Fmt::MX || KSG == 1 || (BM * 4) % kThreads == 0, "MX scale entries: K-step per load");
  auto sf_u = [](int q) { return KSG == 1 ? 0 : kThreads * q / (BM * 4); };
  int asf_srcq[kSfQ];
  auto gather_sf_src = [&]() {
#pragma unroll
    for (int q = 0; q < kSfQ; ++q) {
      const int row = ((tid + kThreads * q) % (BM * 4)) >> 2;
      asf_srcq[q] = GATEUP && F == Fmt::MX ? src_p[min(row, rows - 1)] : 0;
    }
  };
  if (!plan_here) gather_sf_src();
  // weight ring: DEPTH K-steps per wave, DEPTH-1 of them in flight while one is consumed.
  // Issued first, before the activation rows' addresses are known (direct-to-LDS
  // tiles: the first stage's K-steps here, the rest after the first activation stage).
  BFrag<F, NT> bq[DEPTH];
#pragma unroll
  for (int d = 0; d < (TL::kDma ? KSG : DEPTH); ++d) load_b(bq[d], d);
  __builtin_amdgcn_sched_barrier(0);
  // In-launch plan: the tile's rows are gathered while the weight ring is in flight
  // (its barriers wait for LDS traffic only, not for those loads).
  // (LDS reads through an LDS pointer: through a generic one they would be flat
  // loads, whose wait would also wait for the weight ring)
  if constexpr (kPlanHere) {
    if (plan_here) {
      plan_rows_in_lds<kThreads>(p, PL, expert, tile_in_e * BM, rows);
      const LDS3 int* sl = (const LDS3 int*)PL.srcl;
#pragma unroll
      for (int i = 0; i < TL::kAChunks; ++i) a_src[i] = sl[min((tid + kThreads * i) >> 3, rows - 1)];
#pragma unroll
      for (int q = 0; q < kSfQ; ++q)
        if (F == Fmt::MX) asf_srcq[q] = sl[min(((tid + kThreads * q) % (BM * 4)) >> 2, rows - 1)];
      if (F == Fmt::FP8) asf_src = sl[min(tid, rows - 1)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  uint32_t a_off[TL::kAChunks];
  uint32_t a_sfo[F == Fmt::NVF4 ? TL::kAChunks : 1];
#pragma unroll
  for (int i = 0; i < TL::kAChunks; ++i) {
    const int c = tid + kThreads * i;
    const int r = c >> 3;
    const uint32_t arow = GATEUP ? (uint32_t)(a_src[i] / p.topk) : (uint32_t)(row0 + r);
    // direct-to-LDS: slot c of the K-step block holds row r's chunk (c & 7) ^ swz(r)
    const uint32_t chunk = TL::kDma ? (uint32_t)((c & 7) ^ TL::swz(r)) : (uint32_t)(c & 7);
    // NVF4: a chunk of 8 activations is 4 packed bytes
    a_off[i] = r < rows ? arow * p.a_row_bytes + chunk * (F == Fmt::NVF4 ? 4u : 16u) : kOOB;
    // NVF4: the E4M3 scale of the chunk's 16-element block (elements 64 ks + 8 (c & 7) ..)
    if constexpr (F == Fmt::NVF4) a_sfo[i] = r < rows ? arow * (uint32_t)p.a_sf_row + ((c & 7) >> 1) : kOOB;
  }
  // FP8: the fp32 A scale of row tid per K-step; threads past the tile's rows load zeros
  const __amdgpu_buffer_rsrc_t asf_rs = F == Fmt::FP8 ? make_rsrc((const uint8_t*)p.A_sf + (size_t)k0 * 4u, p.a_sf_bytes - (uint32_t)k0 * 4u)
                                                       : make_rsrc(p.A_sf, p.a_sf_bytes);
  const uint32_t asf_off =
      (F == Fmt::FP8 && tid < rows)
          ? (GATEUP ? (uint32_t)(asf_src / p.topk) : (uint32_t)(row0 + tid)) * (uint32_t)p.a_sf_row * (F == Fmt::FP8 ? 4u : 1u)
          : kOOB;
  uint32_t asf_offq[kSfQ];  // MX: entry tid + kThreads q
#pragma unroll
  for (int q = 0; q < kSfQ; ++q) {
    const int e = tid + kThreads * q, u = sf_u(q), rem = e - u * (BM * 4), row = rem >> 2;
    const uint32_t rt = GATEUP ? (uint32_t)(asf_srcq[q] / p.topk) : (uint32_t)(row0 + row);
    asf_offq[q] = (F == Fmt::MX && e < kSfTotal && row < rows) ? rt * (uint32_t)p.a_sf_row + (uint32_t)(4 * u + (rem & 3))
                                                                : kOOB;
  }

  // down: the pair slot of each tile row, for the epilogue's scatter (loaded early)
  const int pair_of_row = (!GATEUP && tid < rows) ? p.src_info[row0 + tid] : 0;

  // ---------------------------------------------------------------- main loop
  // FP8, MX: 16x16 tiles acc[token slice][weight tile]; BF16: 32x32 tiles
  // acc32[32-token slice][32-row weight tile] (v_mfma_f32_32x32x16_bf16)
  f32x4 acc[bf16_mma(F) ? 1 : MT][bf16_mma(F) ? 1 : NT];
  f32x16 acc32[bf16_mma(F) ? MT32 : 1][bf16_mma(F) ? NT32 : 1];
  if constexpr (bf16_mma(F)) {
#pragma unroll
    for (int mt = 0; mt < MT32; ++mt)
#pragma unroll
      for (int t = 0; t < NT32; ++t) acc32[mt][t] = f32x16{};
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Loads past the last K-step read zeros (no branch, so the register rings stay static).
  auto load_a = [&](i32x4 (&v)[KSG][TL::kAChunks], uint32_t (&s)[kSfN], int st) {
#pragma unroll
    for (int u = 0; u < KSG; ++u) {
      const int ks = st * KSG + u;
      const uint32_t dead = oob_if(ks >= KS);
#pragma unroll
      for (int i = 0; i < TL::kAChunks; ++i) {
        uint32_t o = a_off[i] | dead;
        if (F == Fmt::MX) o |= oob_if(ks * 128 + (((tid + kThreads * i) & 7) * 16) >= p.K);  // K tail
        if constexpr (F == Fmt::NVF4) {
          // 8 packed E2M1 values and their block's E4M3 scale, decoded in store_a
          v[u][i][0] = (int)__builtin_amdgcn_raw_buffer_load_b32(a_rs, o, (uint32_t)ks * 32u, 0);
          v[u][i][1] = (int)__builtin_amdgcn_raw_buffer_load_b8(asf_rs, a_sfo[i] | dead, (uint32_t)ks * 4u, 0);
        } else {
          v[u][i] = bload16(a_rs, o, (uint32_t)ks * 128u);
        }
      }
    }
    if constexpr (F == Fmt::FP8) {
#pragma unroll
      for (int u = 0; u < KSG; ++u) {
        const int ks = st * KSG + u;
        s[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(asf_rs, (asf_off + 4u * u) | oob_if(ks >= KS),
                                                              (uint32_t)st * (KSG * 4u), 0);
      }
    } else if constexpr (F == Fmt::MX && !TL::kSfTab) {
      // byte 4 ks + (e % 4) of the row; K-blocks past the row's end and entries past
      // the stage's read zeros (no branch in the main loop)
#pragma unroll
      for (int q = 0; q < kSfQ; ++q) {
        const uint32_t o = asf_offq[q] | oob_if(st * KSG * 4 + 4 * sf_u(q) + (tid & 3) >= p.a_sf_row);
        s[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(asf_rs, o, (uint32_t)st * (KSG * 4u), 0);
      }
    }
  };
  auto store_a = [&](const i32x4 (&v)[KSG][TL::kAChunks], const uint32_t (&s)[kSfN], int buf) {
#pragma unroll
    for (int u = 0; u < KSG; ++u) {
      uint8_t* base = a_lds + (buf * KSG + u) * TL::kAStepBytes;
#pragma unroll
      for (int i = 0; i < TL::kAChunks; ++i) {
        const int c = tid + kThreads * i, r = c >> 3;
        // NVF4: e2m1 x E4M3 block scale, exact in bf16
        const i32x4 val = F == Fmt::NVF4 ? nv4_bf16x8((uint32_t)v[u][i][0], __builtin_amdgcn_cvt_f32_fp8(v[u][i][1], 0))
                                         : v[u][i];
        *(i32x4*)(base + r * TL::kARowBytes + (((c & 7) ^ (r & TL::kSwz)) * 16)) = val;
      }
    }
    if constexpr (F == Fmt::FP8) {
#pragma unroll
      for (int u = 0; u < KSG; ++u) sa_lds[(buf * KSG + u) * TL::kSA + tid] = s[u];
    } else if constexpr (F == Fmt::MX && !TL::kSfTab) {
      // the four lanes of a quad hold the four bytes of one row's scale word (entry
      // e = 4 row + block): the quad's first lane gathers them (DPP quad
      // permutations) and stores the word
#pragma unroll
      for (int q = 0; q < kSfQ; ++q) {
        const int v = (int)s[q];
        const uint32_t w = (uint32_t)v | (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x55, 0xF, 0xF, false) << 8 |
                           (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0xAA, 0xF, 0xF, false) << 16 |
                           (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0xFF, 0xF, 0xF, false) << 24;
        const int e = tid + kThreads * q, u = sf_u(q);
        // every lane stores (a branch here costs registers across the main loop): the
        // other lanes write a spare slot past the tile's rows, which no K-step reads
        static_assert(F != Fmt::MX || TL::kSA > BM, "a spare scale slot");
        const int slot = ((tid & 3) == 0 && e < kSfTotal) ? (e - u * (BM * 4)) >> 2 : TL::kSA - 1;
        sa_lds[(buf * KSG + u) * TL::kSA + slot] = w;
      }
    }
  };

  // FP8: A(st) and its scales go straight from HBM into LDS buffer `buf`.  Lane l
  // of a wave's load lands at the instruction's LDS base + 16 l (4 l for the
  // scale), so the lane loads the chunk that slot holds (swizzle in a_off).
  auto dma_a = [&](int st, int buf) {
#pragma unroll
    for (int u = 0; u < KSG; ++u) {
      const int ks = st * KSG + u;
      const uint32_t dead = oob_if(ks >= KS);
      uint8_t* base = a_lds + (buf * KSG + u) * TL::kAStepBytes;
#pragma unroll
      for (int i = 0; i < TL::kAChunks; ++i) {
        uint32_t o = a_off[i] | dead;
        if constexpr (F == Fmt::MX) {
          // K tail (MX rows need only be a multiple of 32 long): the chunk this slot
          // holds, (c & 7) ^ swz(r), past the row's end reads zeros
          const int c = tid + kThreads * i;
          o |= oob_if(ks * 128 + (((c & 7) ^ TL::swz(c >> 3)) * 16) >= p.K);
        }
        lds_load16(a_rs, base + (i * kThreads + wave * 64) * 16, o, (uint32_t)ks * 128u);
      }
      if constexpr (F == Fmt::FP8)
        lds_load4(asf_rs, sa_lds + (buf * KSG + u) * TL::kSA + wave * 64, (asf_off + 4u * u) | dead,
                  (uint32_t)st * (KSG * 4u));
    }
  };
  // VMEM instructions per stage: the A loads (D) and the weight-ring refills (R)
  // (MX with dense weight scales: NT weight loads and one scale load per K-step)
  constexpr int kD = KSG * (TL::kAChunks + (F == Fmt::FP8 ? 1 : 0));
  constexpr int kR = KSG * (nv4w(F) ? NT : kMxDenseSc ? NT + 1 : NT * 2);

  i32x4 av[TL::kDma ? 1 : 2][KSG][TL::kAChunks];
  uint32_t as[TL::kDma ? 1 : 2][kSfN] = {};
  const LDS3 uint32_t* sft = nullptr;  // weight-bound MX: the tile's scale rows ([BM][sft_dw] dwords)
  int sft_dw = 0;
  if constexpr (TL::kDma) {
    // Ring K-steps of stage 0 (above), A(0), the ring K-steps of stage 1, A(1),
    // in this order (the scheduling barriers keep it).  When stage st waits for
    // A(st), the VMEM instructions issued after A(st) are first this stage's
    // ring loads (kR: the prologue's stage-1 loads, or the refills issued in
    // stage st - 2, since DEPTH = 2 KSG), then A(st + 1) and the later refills.
    // Waiting down to kR + kD outstanding therefore lands A(st) and this stage's
    // weights and nothing later: one wait count for every stage, no branches.
    static_assert(!TL::kDma || DEPTH == 2 * KSG, "the direct-to-LDS pipeline keeps two stages of weights in flight");
    __builtin_amdgcn_sched_barrier(0);
    dma_a(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = KSG; d < DEPTH; ++d) load_b(bq[d], d);
    __builtin_amdgcn_sched_barrier(0);
    dma_a(1, 1);
    __builtin_amdgcn_sched_barrier(0);
  } else {
    load_a(av[0], as[0], 0);
    load_a(av[1], as[1], 1);
    store_a(av[0], as[0], 0);
  }
  if constexpr (TL::kSfTab) {
    // (after the prologue's activation and ring loads: the fill waits for its own
    // loads, and so for every older one, before the first stage's wait counts apply)
    // the tile's scale rows: sf_row bytes per row (UE8M0 per 32 activations), rows
    // past the tile's and bytes past a row's end zero (so that every K-block of
    // the padded last K-step reads a finite scale), into the [BM][stride] table
    uint8_t* tb = (uint8_t*)plan_dyn + plan_region_bytes(plan_here, p.E, p.npairs, kThreads, BM);
    const int sfr = p.a_sf_row, stride = mx_table_stride(sfr);
    sft = (const LDS3 uint32_t*)tb;
    sft_dw = stride >> 2;
    int* rtok = (int*)red_lds;  // gate_up: the token of each tile row (the epilogue reuses the space)
    if (GATEUP) {
      if ((tid & 7) == 0) {
#pragma unroll
        for (int i = 0; i < TL::kAChunks; ++i) {
          const int r = (tid + kThreads * i) >> 3;
          if (r < BM) rtok[r] = r < rows ? a_src[i] / p.topk : -1;
        }
      }
      lds_barrier();
    }
    // entries i = tid + kThreads j of W bytes each (the widest the row length's
    // alignment allows: a scale row starts at a multiple of sf_row bytes), 16
    // loads in flight per thread
    auto fill = [&](auto wbytes) {
      constexpr int W = decltype(wbytes)::value;
      const int per_row = stride / W, n = BM * per_row;
      const int dr = kThreads / per_row, du = kThreads % per_row;
      for (int j0 = 0; j0 * kThreads < n; j0 += 16) {
        uint32_t v[16];
        int r = (j0 * kThreads + tid) / per_row, u = (j0 * kThreads + tid) % per_row;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int tok = r >= BM ? -1 : GATEUP ? rtok[r] : (r < rows ? row0 + r : -1);
          const uint32_t off =
              (tok >= 0 && u * W < sfr) ? (uint32_t)tok * (uint32_t)sfr + (uint32_t)(u * W) : kOOB;
          if constexpr (W == 4) v[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(asf_rs, off, 0, 0);
          else if constexpr (W == 2) v[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(asf_rs, off, 0, 0);
          else v[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(asf_rs, off, 0, 0);
          u += du;
          r += dr;
          if (u >= per_row) {
            u -= per_row;
            ++r;
          }
        }
        r = (j0 * kThreads + tid) / per_row;
        u = (j0 * kThreads + tid) % per_row;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (r < BM) {
            if constexpr (W == 4) *(uint32_t*)(tb + r * stride + u * 4) = v[j];
            else if constexpr (W == 2) *(uint16_t*)(tb + r * stride + u * 2) = (uint16_t)v[j];
            else tb[r * stride + u] = (uint8_t)v[j];
          }
          u += du;
          r += dr;
          if (u >= per_row) {
            u -= per_row;
            ++r;
          }
        }
      }
    };
    if ((sfr & 3) == 0) fill(std::integral_constant<int, 4>{});
    else if ((sfr & 1) == 0) fill(std::integral_constant<int, 2>{});
    else fill(std::integral_constant<int, 1>{});
  }
  if (F == Fmt::FP8) {
#pragma unroll
    for (int q = 0; q < kSbPer; ++q) {
      const int i = tid + q * kThreads;
      if (i < TL::kNB * KS) {
        const int j = i / KS;
        sb_lds[j * TL::kMaxKSteps + (i - j * KS)] = sb_pre[q];
      }
    }
  }

  // One K-step on the staged A of LDS buffer `buf` (K-step u of the stage) and B(ks) in `bq_`.
  // `issue` runs once inside the step: the direct-to-LDS stages pass the loads of
  // A two stages ahead (FP8: after MFMA kIssueAfter; the other formats: first).
  auto kstep = [&](const BFrag<F, NT>& bq_, int buf, int u, int ks, auto&& issue) {
    const uint8_t* abuf = a_lds + (buf * KSG + u) * TL::kAStepBytes;
    const uint32_t* sbuf = sa_lds + (buf * KSG + u) * TL::kSA;
    // activation fragment of token slice mt: token row mt*16 + r16, bytes [16g, 16g+16) and [64+16g, 64+16g+16)
    // (token row mt*16 + r16 has row & 7 == r16 & 7: the swizzled chunk offsets are per lane)
    const int lo_off = 16 * (g ^ (r16 & TL::kSwz)), hi_off = lo_off ^ 64;
    auto rd_lo = [&](int mt) { return *(const i32x4*)(abuf + (mt * 16 + r16) * TL::kARowBytes + lo_off); };
    auto rd_hi = [&](int mt) { return *(const i32x4*)(abuf + (mt * 16 + r16) * TL::kARowBytes + hi_off); };
    // The weights are the MFMA's first operand and the activations its second, so
    // a lane's outputs are 4 weight rows (16*nt + 4g + i) of one token (mt*16 + r16):
    // the activation scale of a lane is one value per token slice.
    if (F == Fmt::FP8) {
      // one 16x16x128 FP8 MFMA per K-step (unit hardware scales) into a fresh
      // partial, then acc += (sa[token] * sb[block]) * partial
      const int kc = min(ks, KS - 1);  // a step past the end multiplies zeros
      // A wave's weight rows of one kind lie in one 128-row scale block (gate_up: 8 NT
      // gate and as many up rows per wave, 32-aligned; down: 16 NT rows, 64-aligned),
      // so a token slice needs sa * sb once per kind, not once per tile.
      static_assert(!GATEUP || (8 * NT <= 128 && 128 % (8 * NT) == 0), "a wave's gate rows share a scale block");
      static_assert(GATEUP || (16 * NT <= 128 && 128 % (16 * NT) == 0), "a wave's down rows share a scale block");
      constexpr int kKinds = GATEUP ? 2 : 1;
      float sbk[kKinds];
#pragma unroll
      for (int j = 0; j < kKinds; ++j) sbk[j] = sb_lds[sb_row(j * (NT / kKinds)) * TL::kMaxKSteps + kc];
      // Software-pipelined: the scale update of MFMA i is issued after MFMA i+2
      // (three partials in flight: with two, the update read a partial the matrix
      // core was still writing, and the compiler padded every other MFMA with a
      // 7-cycle wait; prefill gate_up -3.5 %, down -3 %), and the activation
      // fragment of the next token slice is read one slice ahead, so that the
      // matrix core never waits on the VALU or on LDS within a wave.  Every token
      // slice is computed (slices past the tile's rows multiply zeros).
      auto rd8 = [&](int mt) { return (i32x8)__builtin_shufflevector(rd_lo(mt), rd_hi(mt), 0, 1, 2, 3, 4, 5, 6, 7); };
      auto rd_sa = [&](int mt) { return __builtin_bit_cast(float, sbuf[mt * 16 + r16]); };
      i32x8 a_cur = rd8(0), a_nxt = rd8(MT > 1 ? 1 : 0);
      float sa_cur = rd_sa(0), sa_nxt = rd_sa(MT > 1 ? 1 : 0);
      float ssb[kKinds];  // sa * sb of the current token slice, per kind
#pragma unroll
      for (int j = 0; j < kKinds; ++j) ssb[j] = sa_cur * sbk[j];
      f32x4 prev = {}, prev2 = {};
      float s_prev = 0.f, s_prev2 = 0.f;
#pragma unroll
      for (int i = 0; i < MT * NT; ++i) {
        const int mt = i / NT, nt = i % NT;
        const i32x8 b8 = __builtin_shufflevector(bq_.lo[nt], bq_.hi[nt], 0, 1, 2, 3, 4, 5, 6, 7);
        const f32x4 cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a_cur, f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                           0, 0, 127, 0, 127);
        const float s_cur = ssb[nt / (NT / kKinds)];
        if (i > 1) acc[(i - 2) / NT][(i - 2) % NT] += prev2 * s_prev2;
        prev2 = prev;
        s_prev2 = s_prev;
        if (nt == NT - 1 && mt + 1 < MT) {
          a_cur = a_nxt;
          sa_cur = sa_nxt;
#pragma unroll
          for (int j = 0; j < kKinds; ++j) ssb[j] = sa_cur * sbk[j];
          if (mt + 2 < MT) {
            a_nxt = rd8(mt + 2);
            sa_nxt = rd_sa(mt + 2);
          }
        }
        prev = cur;
        s_prev = s_cur;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // this MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then the scale update of the one before the previous
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // then the LDS reads of the slice after next
        __builtin_amdgcn_sched_barrier(0);
        // After the stage barrier the matrix core waits for the first MFMA; issuing
        // the next activation stage's direct-to-LDS loads a few MFMAs in, rather
        // than between the barrier and the first fragment reads, keeps them off
        // that path (bit-identical; prefill gate_up -2.1 %, down -1.5 %; after MFMA
        // 1: -1.4 %; after 11 or 19: no gain).
        constexpr int kIssueAfter = MT * NT > 5 ? 5 : 0;
        if (i == kIssueAfter) issue();
      }
      if (MT * NT > 1) acc[(MT * NT - 2) / NT][(MT * NT - 2) % NT] += prev2 * s_prev2;
      acc[MT - 1][NT - 1] += prev * s_prev;
    } else if constexpr (bf16_mma(F)) {
      issue();
      // 32x32x16 MFMAs: lane l = 32*h + r holds token mt*32 + r and bytes
      // [32*sub + 16*h, +16) of the K-step segment; weight sub-step fragments
      // are bq_.lo[2t], lo[2t+1], hi[2t], hi[2t+1] for sub = 0..3 (BF16), or
      // decoded from word sub of bq_.lo[t] with block scale byte sub of bq_.sc[t] (NV4)
      const int r32 = lane & 31, h32 = lane >> 5;
      auto rd_a = [&](int mt, int sub) {
        return *(const i32x4*)(abuf + (mt * 32 + r32) * TL::kARowBytes + 16 * ((2 * sub + h32) ^ TL::swz(r32)));
      };
      if constexpr (nv4w(F)) {
        // Sub-step outer: the weights of sub-step sub + 1 are decoded (VALU) while
        // the MFMAs of sub-step sub, issued just before, run on the matrix core.
        // Every token slice but the last is computed unconditionally (slices past
        // the tile's rows multiply zeros); the last only when it holds rows.
        float scf[NT32][4];  // the four E4M3 block scales of each tile row, as fp32
#pragma unroll
        for (int t = 0; t < NT32; ++t) {
          scf[t][0] = __builtin_amdgcn_cvt_f32_fp8(bq_.sc[t], 0);
          scf[t][1] = __builtin_amdgcn_cvt_f32_fp8(bq_.sc[t], 1);
          scf[t][2] = __builtin_amdgcn_cvt_f32_fp8(bq_.sc[t], 2);
          scf[t][3] = __builtin_amdgcn_cvt_f32_fp8(bq_.sc[t], 3);
        }
        auto dec = [&](int t, int sub) { return nv4_bf16x8((uint32_t)bq_.lo[t][sub], scf[t][sub]); };
        const bool last_live = (MT32 - 1) * 32 < rows;
        i32x4 cur[NT32];
#pragma unroll
        for (int t = 0; t < NT32; ++t) cur[t] = dec(t, 0);
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
          i32x4 nxt[NT32];
          if (sub < 3) {
#pragma unroll
            for (int t = 0; t < NT32; ++t) nxt[t] = dec(t, sub + 1);
          }
#pragma unroll
          for (int mt = 0; mt < MT32; ++mt) {
            if (mt == MT32 - 1 && !last_live) break;  // wave-uniform
            const i32x4 a = rd_a(mt, sub);
#pragma unroll
            for (int t = 0; t < NT32; ++t)
              acc32[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur[t]),
                                                                     __builtin_bit_cast(bf16x8, a), acc32[mt][t], 0, 0, 0);
          }
          if (sub < 3) {
#pragma unroll
            for (int t = 0; t < NT32; ++t) cur[t] = nxt[t];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else if constexpr (BM > 96) {
        // MFMA-bound BF16: (sub-step, token slice) pairs, sub-step outer, so that
        // consecutive MFMAs update different accumulators; every slice computed
        // (no branch), each activation fragment read from LDS one pair ahead.
        constexpr int NP = 4 * MT32;
        i32x4 a_cur = rd_a(0, 0), a_nxt = rd_a(NP > 1 ? 1 % MT32 : 0, NP > 1 ? 1 / MT32 : 0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int sub = i / MT32, mt = i % MT32;
#pragma unroll
          for (int t = 0; t < NT32; ++t) {
            const i32x4 b = sub < 2 ? bq_.lo[2 * t + sub] : bq_.hi[2 * t + sub - 2];
            acc32[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b),
                                                                   __builtin_bit_cast(bf16x8, a_cur), acc32[mt][t], 0, 0, 0);
          }
          a_cur = a_nxt;
          if (i + 2 < NP) a_nxt = rd_a((i + 2) % MT32, (i + 2) / MT32);
          __builtin_amdgcn_sched_group_barrier(0x008, NT32, 0);  // this pair's MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // then the read two pairs ahead
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MT32; ++mt) {
          if (kSkipSlices && mt * 32 >= rows) break;  // wave-uniform: no token rows left
#pragma unroll
          for (int sub = 0; sub < 4; ++sub) {
            const i32x4 a = rd_a(mt, sub);
#pragma unroll
            for (int t = 0; t < NT32; ++t) {
              const i32x4 b = sub < 2 ? bq_.lo[2 * t + sub] : bq_.hi[2 * t + sub - 2];
              acc32[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b),
                                                                     __builtin_bit_cast(bf16x8, a), acc32[mt][t], 0, 0, 0);
            }
          }
        }
      }
    } else {
      issue();
      // the lane's scale byte of each tile: byte l of the tile's 64 (dense: held by
      // lane 16 nt + l / 4, byte l % 4; the MFMA reads the operand's low byte)
      int scb[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        scb[nt] = kMxDenseSc ? __builtin_amdgcn_ds_bpermute((16 * nt + (lane >> 2)) * 4, bq_.sc[0]) >> (8 * (lane & 3))
                             : bq_.sc[nt];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i32x4 alo = rd_lo(mt), ahi = rd_hi(mt);
        {
          // weights E2M1 (first operand, format 4), activations E4M3 (format 0);
          // each lane's scale byte: its row (weight row / token) in K-block g
          const i32x8 a8 = __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7);
          const uint32_t sw = TL::kSfTab ? sft[(mt * 16 + r16) * sft_dw + min(ks, KS - 1)] : sbuf[mt * 16 + r16];
          const int sa = (int)((sw >> (8 * g)) & 0xFFu);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const i32x8 b8 = {bq_.lo[nt][0], bq_.lo[nt][1], bq_.lo[nt][2], bq_.lo[nt][3], 0, 0, 0, 0};
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, acc[mt][nt], 4, 0, 0, scb[nt], 0,
                                                                           sa);
          }
        }
      }
    }
  };

  // One stage of KSG K-steps: A(st) is in LDS buffer st&1 and A(st+1) in flight in
  // `an`; issues A(st+2) into `ap`, and refills each consumed weight-ring slot.
  auto stage = [&](int st, int su, i32x4 (&ap)[KSG][TL::kAChunks], uint32_t (&sp)[kSfN],
                   i32x4 (&an)[KSG][TL::kAChunks], uint32_t (&sn)[kSfN]) {
    load_a(ap, sp, st + 2);
    __syncthreads();
    // The MFMA section runs at raised wave priority, so that while one wave of a
    // SIMD feeds the matrix core the other's loads and LDS stores fill the gaps.
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int u = 0; u < KSG; ++u) {
      const int ks = st * KSG + u;
      BFrag<F, NT>& slot = bq[(su * KSG + u) % DEPTH];
      kstep(slot, su & 1, u, ks, [] {});
      // keep the next K-step's LDS reads from being hoisted over this one (register pressure)
      if (u + 1 < KSG) __builtin_amdgcn_sched_barrier(0);
      // The refill of this ring slot must not be hoisted above the MFMAs that read
      // its previous contents (the two values would then both be live): tie the
      // load's scalar offset to the step's last accumulator update.
      int ks_next = ks + DEPTH;
      if constexpr (bf16_mma(F))
        asm volatile("; ring refill after step" : "+s"(ks_next) : "v"(acc32[MT32 - 1][NT32 - 1][15]));
      else
        asm volatile("; ring refill after step" : "+s"(ks_next) : "v"(acc[MT - 1][NT - 1][3]));
      load_b(slot, ks_next);
    }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
    store_a(an, sn, (su + 1) & 1);
  };

  // Direct-to-LDS stage: A(st) was loaded into buffer st % kABufs two stages ago.  Each wave
  // waits for its own loads of A(st) and of this stage's weights (the VMEM
  // counter retires in order; see the prologue for the count), and its LDS
  // accesses; the barrier then publishes the buffer and frees buffer
  // (st + 2) % kABufs, last read in stage st - 2, for A(st + 2).  A plain
  // s_barrier: __syncthreads would wait for every outstanding load.
  auto stage_dma = [&](int st, int su) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kR + kD));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // A(st + 2), issued inside the first K-step: the same VMEM order (the A loads,
    // then the ring refills), so the wait count above still holds
    auto issue_a = [&] {
      dma_a(st + 2, (su + 2) % TL::kABufs);
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int u = 0; u < KSG; ++u) {
      const int ks = st * KSG + u;
      BFrag<F, NT>& slot = bq[(su * KSG + u) % DEPTH];
      if (u == 0) kstep(slot, su % TL::kABufs, u, ks, issue_a);
      else kstep(slot, su % TL::kABufs, u, ks, [] {});
      if (u + 1 < KSG) __builtin_amdgcn_sched_barrier(0);
      int ks_next = ks + DEPTH;
      if constexpr (bf16_mma(F))
        asm volatile("; ring refill after step" : "+s"(ks_next) : "v"(acc32[MT32 - 1][NT32 - 1][15]));
      else
        asm volatile("; ring refill after step" : "+s"(ks_next) : "v"(acc[MT - 1][NT - 1][3]));
      load_b(slot, ks_next);
    }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Unrolled so that both rings (DEPTH weight buffers, kABufs activation
  // buffers) index statically: U K-steps = SU stages per trip.  The trip count is rounded
  // up to the unroll: the extra steps load zeros and add zeros, and the loop has
  // no early exit (an exit per step would make the compiler drain every
  // outstanding load there).
  constexpr int SU = U / KSG;
  const int KS_PAD = (KS + U - 1) / U * U;
  if constexpr (TL::kDma) {
    for (int ks0 = 0; ks0 < KS_PAD; ks0 += U) {
#pragma unroll
      for (int su = 0; su < SU; ++su) stage_dma(ks0 / KSG + su, su);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the trailing loads (zeros) have landed before the LDS is reused
  } else {
    for (int ks0 = 0; ks0 < KS_PAD; ks0 += U) {
#pragma unroll
      for (int su = 0; su < SU; ++su)
        stage(ks0 / KSG + su, su, av[su & 1], as[su & 1], av[(su + 1) & 1], as[(su + 1) & 1]);
    }
  }
  __syncthreads();  // every wave is done with the A buffers; the output tile reuses them

  // ---------------------------------------------------------------- split tail
  if constexpr (kSplit) {
    if (piece >= 0) {
      // Partial tile of piece s of tail tile j in slot j * nparts + s, lane-major
      // (f32x4 v of thread tid at (v * threads + tid) * 16 bytes), stored at device
      // scope; once every thread's stores have completed, the workgroup arrives at
      // the tile's counter.  The piece that completes the count (it resets the
      // counter for the next launch) reads every partial at device scope and sums
      // them in piece order; the others are done.  No waiting, no data atomics.
      constexpr int kV = bf16_mma(F) ? MT32 * NT32 * 4 : MT * NT;  // f32x4 per lane
      const __amdgpu_buffer_rsrc_t ws = make_rsrc(p.split_part, (uint32_t)p.split_slots * kV * kThreads * 16u);
      auto off = [&](int slot, int v) { return (uint32_t)(((slot * kV + v) * kThreads + tid) * 16); };
      auto get = [&](int v) -> f32x4 {
        if constexpr (bf16_mma(F)) {
          const f32x16& a = acc32[v / (NT32 * 4)][(v / 4) % NT32];
          const int q = v % 4;
          return f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
        } else {
          return acc[v / NT][v % NT];
        }
      };
      auto put = [&](int v, f32x4 x) {
        if constexpr (bf16_mma(F)) {
          f32x16& a = acc32[v / (NT32 * 4)][(v / 4) % NT32];
          const int q = v % 4;
          a[4 * q] = x[0], a[4 * q + 1] = x[1], a[4 * q + 2] = x[2], a[4 * q + 3] = x[3];
        } else {
          acc[v / NT][v % NT] = x;
        }
      };
      const int slot0 = tail_j * nparts;
#pragma unroll
      for (int v = 0; v < kV; ++v)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, get(v)), ws, off(slot0 + piece, v), 0,
                                               kCpolDevice | kCpolNt);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      int* last_lds = (int*)red_lds;
      if (tid == 0) {
        const bool last = atomicAdd(p.split_cnt + tail_j, 1) == nparts - 1;
        if (last) atomicExch(p.split_cnt + tail_j, 0);
        *last_lds = last;
      }
      __syncthreads();
      const bool last = *last_lds != 0;
      __syncthreads();  // every wave has read the flag before the epilogue reuses the space
      if (!last) return;  // (uniform)
#pragma unroll
      for (int v = 0; v < kV; ++v) put(v, f32x4{0.f, 0.f, 0.f, 0.f});
      // kB loads in flight before the first add (one at a time, each would wait
      // out a full memory round trip)
      constexpr int kB = 16;
      static_assert(kV % kB == 0, "whole load batches");
      for (int sp = 0; sp < nparts; ++sp) {
#pragma unroll
        for (int v0 = 0; v0 < kV; v0 += kB) {
          f32x4 t[kB];
#pragma unroll
          for (int i = 0; i < kB; ++i)
            t[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ws, off(slot0 + sp, v0 + i), 0,
                                                                                   kCpolDevice));
#pragma unroll
          for (int i = 0; i < kB; ++i) put(v0 + i, get(v0 + i) + t[i]);
        }
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  // Lane (r16, g) holds, for token slice mt, token row mt*16 + r16 and the wave's
  // weight rows 16*nt + 4g + i (i < 4): four consecutive output columns.
  // BF16 (32x32 tiles): lane l = 32*h32 + r32 holds token mt*32 + r32 and the
  // tile's rows 8*(i/4) + 4*h32 + i%4 (i < 16); in a gate_up tile rows < 16 are
  // gate rows and row 16 + j the up row of gate row j, so acc32[..][i] pairs with [i + 8].
  const int r32 = lane & 31, h32 = lane >> 5;
  if constexpr (nv4w(F)) {
    // the expert's global weight scale multiplies every output of the leg
    const float gsc = p.B_gs[expert];
#pragma unroll
    for (int mt = 0; mt < MT32; ++mt)
#pragma unroll
      for (int t = 0; t < NT32; ++t) acc32[mt][t] *= gsc;
  }
  if (GATEUP) {
    constexpr int NJ = NT / 2;  // gate (and up) column tiles per wave
    const float c = p.clamp;
    if constexpr (F == Fmt::NVF4) {
      // NVFP4 requantisation of h against the expert's intermediate scale c_e (the
      // c_input_scales of the max mega_ffn page): per (row, 16 columns) block scale
      // s = E4M3_RNE_sat(amax / (6 c_e)) and codes E2M1_RNE_sat(h / (s c_e)).  The
      // intermediate stores the codes times their block scale, exact in bf16; the
      // down leg's output scale carries c_e.  A 32-row tile holds 16 h columns:
      // lanes l and l ^ 32 share a token and hold 8 columns each.
      const float ce = p.C_gs[expert];
      const float six_c = 6.0f * ce;
#pragma unroll
      for (int mt = 0; mt < MT32; ++mt)
#pragma unroll
        for (int t = 0; t < NT32; ++t) {
          float v[2][4];
          float m = 0.f;
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[q][i] = swiglu_clamped<FAST>(acc32[mt][t][4 * q + i], acc32[mt][t][4 * q + i + 8], c);
              m = fmaxf(m, fabsf(v[q][i]));
            }
          m = fmaxf(m, __shfl_xor(m, 32));
          const float sb = __builtin_amdgcn_cvt_f32_fp8((int)f32x2_to_e4m3_sat(m / six_c, 0.f), 0);
          const float den = sb * ce;
          const float inv = den > 0.f ? 1.0f / den : 0.f;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = e2m1_rne_sat(v[q][i] * inv) * sb;
            const uint32_t w0 = bf16x2_rne(o[0], o[1]);
            const uint32_t w1 = bf16x2_rne(o[2], o[3]);
            *(uint2*)(out_lds + (mt * 32 + r32) * TL::kOutStride + (wave * HW + 16 * t + 8 * q + 4 * h32) * 2) =
                uint2{w0, w1};
          }
        }
    } else if constexpr (bf16_mma(F)) {
#pragma unroll
      for (int mt = 0; mt < MT32; ++mt)
#pragma unroll
        for (int t = 0; t < NT32; ++t)
#pragma unroll
          for (int q = 0; q < 2; ++q) {  // gate rows 8q + 4*h32 + (0..3)
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = swiglu_clamped<FAST>(acc32[mt][t][4 * q + i], acc32[mt][t][4 * q + i + 8], c);
            const uint32_t w0 = bf16x2_rne(v[0], v[1]);
            const uint32_t w1 = bf16x2_rne(v[2], v[3]);
            *(uint2*)(out_lds + (mt * 32 + r32) * TL::kOutStride + (wave * HW + 16 * t + 8 * q + 4 * h32) * 2) =
                uint2{w0, w1};
          }
    } else {
      float h[MT][NJ][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) h[mt][j][i] = swiglu_clamped<FAST>(acc[mt][j][i], acc[mt][j + NJ][i], c);
      // per-row amax over this wave's HW columns (4 values x NJ tiles in a lane,
      // then the 4 lanes g of the row), then over the waves sharing a
      // requantisation block (128/HW of them for FP8's 128 columns, 32/HW of
      // them for MX's 32)
      constexpr int WPB = F == Fmt::FP8 ? 128 / HW : (32 / HW > 0 ? 32 / HW : 1);  // waves per block
      static_assert(!GATEUP || F != Fmt::FP8 || (128 % HW == 0 && WAVES % WPB == 0), "FP8 blocks span whole waves");
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(h[mt][j][i]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (g == 0) red_lds[wave * BM + mt * 16 + r16] = m;
      }
      __syncthreads();
      const int w0 = wave - wave % WPB;  // first wave of this wave's block
      const int hcol_blk = n_tile * HC + w0 * HW;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + r16;
        float a = red_lds[w0 * BM + r];
#pragma unroll
        for (int w = 1; w < WPB; ++w) a = fmaxf(a, red_lds[(w0 + w) * BM + r]);
        const bool writer = wave == w0 && g == 0 && r < rows && hcol_blk < p.N;
        float q;
        if (F == Fmt::FP8) {
          const float sc = a > 0.f ? a / 448.0f : 1.0f;
          q = 1.0f / sc;
          if (writer) ((float*)p.C_sf)[(long long)(row0 + r) * p.c_sf_row + hcol_blk / 128] = sc;
        } else {
          const int e = mx_exponent_for_amax(a);
          q = exp2i(-e);
          if (writer) ((uint8_t*)p.C_sf)[(long long)(row0 + r) * p.c_sf_row + hcol_blk / 32] = (uint8_t)(e + 127);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const uint32_t lo = f32x2_to_e4m3_sat(h[mt][j][0] * q, h[mt][j][1] * q);
          const uint32_t hi = f32x2_to_e4m3_sat(h[mt][j][2] * q, h[mt][j][3] * q);
          *(uint32_t*)(out_lds + r * TL::kOutStride + wave * HW + 16 * j + 4 * g) = lo | (hi << 16);
        }
      }
    }
    __syncthreads();
    // coalesced copy of the tile's h rows: 16-byte chunks
    constexpr int CPR = TL::kOutRowBytes / 16;  // chunks per row
    constexpr int elem = bf16_mma(F) ? 2 : 1;
    for (int c = tid; c < BM * CPR; c += kThreads) {
      const int r = c / CPR, cc = c % CPR;
      const int col = n_tile * HC + cc * 16 / elem;
      if (r < rows && col < p.N) {
        *(i32x4*)((uint8_t*)p.C + (long long)(row0 + r) * p.c_row_bytes + (long long)n_tile * HC * elem +
                  cc * 16) = *(const i32x4*)(out_lds + r * TL::kOutStride + cc * 16);
      }
    }
    // in-launch plan: the workgroups of column tile 0 store their rows' src_info and
    // pair_row (here, not in the prologue, where the stores would hold up the first
    // wait on the activation loads behind the weight ring)
    if constexpr (kPlanHere) {
      if (plan_here && n_tile == 0) {
        for (int r = tid; r < rows; r += kThreads) {
          const int q = PL.srcl[r];
          p.plan_out.src_info[row0 + r] = q;
          p.plan_out.pair_row[q] = row0 + r;
        }
      }
    }
  } else {
    // down: bf16 rows scattered to their pair slots y[src_info[row]]
    if constexpr (bf16_mma(F)) {
#pragma unroll
      for (int mt = 0; mt < MT32; ++mt)
#pragma unroll
        for (int t = 0; t < NT32; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {  // rows 8q + 4*h32 + (0..3) of the tile
            const f32x16& a = acc32[mt][t];
            const uint32_t w0 = bf16x2_rne(a[4 * q], a[4 * q + 1]);
            const uint32_t w1 = bf16x2_rne(a[4 * q + 2], a[4 * q + 3]);
            *(uint2*)(out_lds + (mt * 32 + r32) * TL::kOutStride + (wave * 16 * NT + 32 * t + 8 * q + 4 * h32) * 2) =
                uint2{w0, w1};
          }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint32_t w0 = bf16x2_rne(acc[mt][nt][0], acc[mt][nt][1]);
          const uint32_t w1 = bf16x2_rne(acc[mt][nt][2], acc[mt][nt][3]);
          *(uint2*)(out_lds + (mt * 16 + r16) * TL::kOutStride + (wave * 16 * NT + 16 * nt + 4 * g) * 2) = uint2{w0, w1};
        }
    }
    int* pair_lds = (int*)red_lds;  // [BM]
    if (tid < BM) pair_lds[tid] = pair_of_row;
    __syncthreads();
    constexpr int CPR = BN * 2 / 16;
    const __amdgpu_buffer_rsrc_t y_rs = make_rsrc(p.C, p.y_bytes);
    for (int c = tid; c < BM * CPR; c += kThreads) {
      const int r = c / CPR, cc = c % CPR;
      const int col = n_tile * BN + cc * 8;
      if (r < rows && col < p.N) {
        const long long pair = pair_lds[r];
        const i32x4 v = *(const i32x4*)(out_lds + r * TL::kOutStride + cc * 16);
        if (p.fuse) {
          // fused combine: a device-scope store, written through to the level that
          // every XCD reads coherently (another workgroup may reduce this row)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                                 y_rs, (uint32_t)(pair * p.c_row_bytes + (long long)col * 2), 0,
                                                 kCpolDevice | kCpolNt);
        } else {
          // y is read once, by the combine: a non-temporal store (decode down -6 %,
          // prefill down -4 %: the weights the tiles re-read stay cached)
          __builtin_nontemporal_store(v, (i32x4*)((uint8_t*)p.C + pair * p.c_row_bytes + (long long)col * 2));
        }
      }
    }
    if (p.fuse) {
      // Fused combine (the single-GPU form of the EPConfig page's fuse_ffn_combine_send;
      // per-destination arrival counts as in the mega_ffn page's arrival_count).
      // Each thread waits for its device-scope y stores to complete; then each tile
      // row arrives at its (token, column tile) counter.  The arrival that completes
      // a token's valid slots finds every other slot's row stored at device scope,
      // and its workgroup reduces that token's column block with device-scope loads,
      // in slot order: the result, bit for bit, of the separate combine, with no
      // data atomics, no cache-wide write-back or invalidation, and no waiting.
      __builtin_amdgcn_s_waitcnt(0);
      int* comp = pair_lds + BM;       // [BM] tokens this tile completed
      int* ncomp = pair_lds + 2 * BM;  // [1]
      static_assert(WAVES * BM >= 2 * BM + 1, "room for the completion list");
      if (tid == 0) *ncomp = 0;
      __syncthreads();
      if (tid < rows) {
        const int t = pair_lds[tid] / p.topk;
        int valid = 0;
        for (int j = 0; j < p.topk; ++j) valid += p.pair_row[(long long)t * p.topk + j] >= 0;
        const int old = atomicAdd(p.counters + (long long)t * p.cnt_stride + n_tile, 1);
        if (old + 1 == valid) comp[atomicAdd(ncomp, 1)] = t;
      }
      __syncthreads();
      const int nc = *ncomp;
      constexpr int C8 = BN / 8;  // 8-column chunks of the tile's columns
      for (int it = tid; it < nc * C8; it += kThreads) {
        const int col = n_tile * BN + (it % C8) * 8;
        if (col < p.N) combine_chunk8(p, y_rs, comp[it / C8], col);
      }
    }
  }
}

// ------------------------------------------------------------------ host side
size_t ffn_h_bytes(Fmt f, int rows, int I) { return (size_t)rows * I * (bf16_mma(f) ? 2 : 1); }
size_t ffn_hsf_bytes(Fmt f, int rows, int I) {
  if (f == Fmt::FP8) return (size_t)rows * (I / 128) * 4;
  if (f == Fmt::MX) return (size_t)rows * (I / 32);
  return 0;
}
int ffn_max_m_tiles(int npairs, int E, int bm) {
  const long long act = npairs < E ? npairs : E;
  return (int)(((long long)npairs + act * (bm - 1)) / bm);
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

// Split tail buffer: the counters, then one partial tile per slot (the
// MFMA-bound down tiles: 512 threads x 128 fp32 accumulators each).
constexpr size_t kSplitSlotBytes = (size_t)512 * 128 * 4;
size_t ffn_split_bytes(Fmt f) {
  if (f != Fmt::FP8 && f != Fmt::BF16) return 0;
  return ffn_split_counter_bytes() + (size_t)kSplitMaxSlots * kSplitSlotBytes;
}

template <Fmt F, bool GATEUP, int BM, int WAVES, int NT, int DEPTH, int KSG, int WGS>
// With timing events the launch carries them in its own dispatch, so they hold the
// kernel's start and end, not those of separate marker commands in the stream.
static void launch_one(const GemmParams& gp_in, bool fast, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  GemmParams gp = gp_in;
  using TL = Tile<F, GATEUP, BM, WAVES, NT, KSG>;
  // split tail: the workgroups the part runs at once, and room in the grid for the
  // pieces past the whole tiles (at most one per slot)
  // (a partial tile: BM x NT / 16 fp32 x 4 per thread)
  static_assert(!TL::kSplit || (size_t)64 * WAVES * BM * NT <= kSplitSlotBytes, "a partial tile fits its slot");
  const int slots = device_cus() * WGS;
  gp.split_slots = (TL::kSplit && gp.split_part != nullptr) ? (slots < kSplitMaxSlots ? slots : kSplitMaxSlots) : 0;
  gp.m_grid = gp.m_tiles_max * gp.n_tiles + gp.split_slots;
  int grid = gp.m_grid;
  // fused combine: workgroups for the tokens without a valid slot
  if (!GATEUP && gp.fuse) grid += (gp.T + kZeroSlotTokens - 1) / kZeroSlotTokens;
  if (grid <= 0) return;
  // dynamic LDS: the in-launch routing plan (weight-bound gate_up only), then the
  // weight-bound MX tiles' scale table
  const size_t dyn = plan_region_bytes(GATEUP && BM <= 96 && gp.plan_ids != nullptr, gp.E, gp.npairs, 64 * WAVES, BM) +
                     (TL::kSfTab ? (size_t)BM * mx_table_stride(gp.a_sf_row) : 0);
  if (fast)
    hipExtLaunchKernelGGL((ffn_gemm_kernel<F, GATEUP, BM, WAVES, NT, DEPTH, KSG, WGS, true>), dim3(grid),
                          dim3(64 * WAVES), dyn, s, e0, e1, 0, gp);
  else
    hipExtLaunchKernelGGL((ffn_gemm_kernel<F, GATEUP, BM, WAVES, NT, DEPTH, KSG, WGS, false>), dim3(grid),
                          dim3(64 * WAVES), dyn, s, e0, e1, 0, gp);
}

// Launch configuration per format, regime and leg: waves per workgroup, 16-row
// column tiles per wave, weight-ring depth (K-steps) and K-steps per LDS stage
// of the activations.  Chosen by measurement on the decode, prefill, Mixtral
// BF16 and W4A8 shapes (deeper rings and stages cost registers and spill).
struct LegConfig {
  int waves, nt, depth, ksg, wgs;  // wgs: workgroups per CU the registers must allow
};
template <Fmt F, bool GATEUP, int BM>
constexpr LegConfig leg_config() {
  if (BM <= 96) {  // weight-bound tiles
    if (GATEUP) return {4, 4, 2, 1, 2};  // 4 waves x 64 weight rows, two workgroups per CU
    if (F == Fmt::FP8) return {7, 4, 2, 1, 1};  // 448 columns: 7168 = 16 tiles (two even rounds of 256)
    if (F == Fmt::MX) return {4, 4, 2, 1, 2};   // 256 columns, two workgroups per CU
    return {8, 2, 2, 1, 1};
  }
  // MFMA-bound tiles
  if (F == Fmt::MX) return {8, 2, 6, 2, 1};
  if (bf16_mma(F)) return {8, 4, 2, 1, 1};  // 512 weight rows (gate_up: 256 h columns)
  if (F == Fmt::FP8) return {8, 4, 2, 1, 1};  // 512 weight rows (gate_up: 256 h columns)
  return {8, 2, 2, 2, 1};
}
template <Fmt F, bool GATEUP, int BM>
static void launch_leg(const GemmParams& gp, bool fast, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr LegConfig c = leg_config<F, GATEUP, BM>();
  launch_one<F, GATEUP, BM, c.waves, c.nt, c.depth, c.ksg, c.wgs>(gp, fast, s, e0, e1);
}

template <Fmt F, int BM>
static void launch_pair(const GemmParams& g1_in, const GemmParams& g2_in, bool fast, hipStream_t s, int stage,
                        const hipEvent_t (&ev)[4]) {
  if (stage != 2) {
    constexpr LegConfig c = leg_config<F, true, BM>();
    constexpr int hc = c.waves * 16 * c.nt / 2;  // h columns of a gate_up tile
    GemmParams g1 = g1_in;
    g1.n_tiles = (g1.N + hc - 1) / hc;
    launch_leg<F, true, BM>(g1, fast, s, ev[0], ev[1]);
  }
  if (stage != 1) {
    constexpr LegConfig c = leg_config<F, false, BM>();
    constexpr int bn = c.waves * 16 * c.nt;  // output columns of a down tile
    GemmParams g2 = g2_in;
    g2.n_tiles = (g2.N + bn - 1) / bn;
    launch_leg<F, false, BM>(g2, fast, s, ev[2], ev[3]);
  }
}

bool ffn_plan_fusable(Fmt f, int bm, int npairs, int E, int I, bool pays) {
  if (npairs <= 0 || npairs > kPlanFusedMaxPairs) return false;
  if (bf16_mma(f) && bm <= 96) bm = 96;
  if (bm > 96) return false;  // MFMA-bound tiles: thousands of workgroups
  if (!pays) return true;
  // weight-bound gate_up tiles: 4 waves x 64 weight rows (128 h columns), two workgroups per CU
  static_assert(leg_config<Fmt::FP8, true, 80>().waves == 4 && leg_config<Fmt::FP8, true, 80>().nt == 4 &&
                    leg_config<Fmt::MX, true, 80>().waves == 4 && leg_config<Fmt::BF16, true, 96>().waves == 4 &&
                    leg_config<Fmt::NV4, true, 96>().nt == 4,
                "the weight-bound gate_up tile the cost rule assumes");
  constexpr long long kSlots = 256LL * 2;  // CUs of the part x workgroups per CU
  const long long grid = (long long)ffn_max_m_tiles(npairs, E, bm) * ((I + 127) / 128);
  const long long rounds = (grid + kSlots - 1) / kSlots;
  return rounds * npairs <= 4096;
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s, int stage) {
  const int npairs = a.T * a.topk;
  if (npairs == 0) return hipSuccess;
  const int elem_k = bf16_mma(a.fmt) ? 64 : 128;
  const uint32_t esz = bf16_mma(a.fmt) ? 2 : 1;
  const int sf_div = a.fmt == Fmt::FP8 ? 128 : 32;
  const Fmt wf = a.fmt == Fmt::NVF4 ? Fmt::NV4 : a.fmt;  // the weights' encoding
  GemmParams g1{}, g2{};
  // gate_up: A = x rows gathered through src_info, B = w13 [E, 2I, H]
  g1.start = a.start;
  g1.src_info = a.src_info;
  g1.E = a.E;
  g1.topk = a.topk;
  // BF16 weight-bound tiles are 96 rows (whole 32-token slices of its 32x32 MFMA)
  const int bm = (bf16_mma(a.fmt) && a.bm <= 96) ? 96 : a.bm;
  g1.m_tiles_max = ffn_max_m_tiles(npairs, a.E, bm);
  g1.K = a.H;
  g1.ksteps = (a.H + elem_k - 1) / elem_k;
  g1.N = a.I;
  g1.n_rows = 2 * a.I;
  g1.A = (const uint8_t*)a.x;
  g1.a_row_bytes = a.fmt == Fmt::NVF4 ? (uint32_t)a.H / 2 : (uint32_t)a.H * esz;  // NVF4: packed E2M1
  g1.a_bytes = g1.a_row_bytes * (uint32_t)a.T;
  g1.A_sf = a.x_sf;
  g1.a_sf_row = a.fmt == Fmt::NVF4 ? a.H / 16 : a.H / sf_div;  // NVF4: one E4M3 scale per 16
  g1.a_sf_bytes = (uint32_t)a.T * (uint32_t)g1.a_sf_row * (a.fmt == Fmt::FP8 ? 4u : 1u);
  g1.B = (const uint8_t*)a.w13;
  g1.b_tile = (uint32_t)prepared_tile_bytes(wf);
  g1.b_expert_bytes = (uint32_t)(prepared_expert_bytes(wf, 2 * a.I, a.H));
  g1.bsc_expert_bytes = (uint32_t)(prepared_scale_expert_bytes(wf, 2 * a.I, a.H));
  g1.C_gs = a.c_scales;
  g1.B_sf = a.w13_sf;
  g1.b_sf_row = a.H / sf_div;
  g1.B_gs = a.w13_gs;
  g1.C = a.h;
  g1.c_row_bytes = (long long)a.I * esz;
  g1.C_sf = a.h_sf;
  g1.c_sf_row = a.I / sf_div;
  g1.clamp = a.clamp;
  // the routing plan built by the gate_up launch itself (weight-bound tiles only)
  if (a.plan_ids != nullptr) {
    if (!ffn_plan_fusable(a.fmt, a.bm, npairs, a.E, a.I, false)) return hipErrorInvalidValue;
    g1.plan_ids = a.plan_ids;
    g1.ids64 = a.ids64 ? 1 : 0;
    g1.npairs = npairs;
    g1.plan_out = a.plan;
  }
  // down: A = h rows, B = w2 [E, H, I]
  g2 = g1;
  g2.plan_ids = nullptr;
  // (n_tiles of both legs are set at launch from their tile widths)
  g2.K = a.I;
  g2.ksteps = (a.I + elem_k - 1) / elem_k;
  g2.N = a.H;
  g2.n_rows = a.H;
  g2.A = (const uint8_t*)a.h;
  g2.a_row_bytes = (uint32_t)a.I * esz;
  g2.a_bytes = g2.a_row_bytes * (uint32_t)npairs;
  g2.A_sf = a.h_sf;
  g2.a_sf_row = a.I / sf_div;
  g2.a_sf_bytes = (uint32_t)npairs * (uint32_t)g2.a_sf_row * (a.fmt == Fmt::FP8 ? 4u : 1u);
  g2.B = (const uint8_t*)a.w2;
  g2.b_expert_bytes = (uint32_t)(prepared_expert_bytes(wf, a.H, a.I));
  g2.bsc_expert_bytes = (uint32_t)(prepared_scale_expert_bytes(wf, a.H, a.I));
  g2.B_sf = a.w2_sf;
  g2.b_sf_row = a.I / sf_div;
  g2.B_gs = a.w2_gs;
  g2.C = a.y;
  g2.c_row_bytes = (long long)a.H * 2;
  g2.C_sf = nullptr;
  g2.c_sf_row = 0;
  // the split tail's buffers (used where the down tiles can split; ffn_split_bytes)
  if (a.split != nullptr && ffn_split_bytes(a.fmt) > 0) {
    g2.split_cnt = (int*)a.split;
    g2.split_part = (float*)((uint8_t*)a.split + ffn_split_counter_bytes());
  }
  if (a.fuse_combine) {
    g2.fuse = 1;
    g2.T = a.T;
    g2.pair_row = a.pair_row;
    g2.topk_w = a.topk_w;
    g2.counters = a.counters;
    g2.cnt_stride = combine_counter_stride(a.H);
    g2.out = a.out;
    g2.shared = (const uint16_t*)a.shared;
    g2.residual = (const uint16_t*)a.residual;
    g2.out_f32 = a.out_f32 ? 1 : 0;
    g2.y_bytes = (uint32_t)((size_t)npairs * a.H * 2);
  }
  switch (a.fmt) {
    case Fmt::FP8:
      if (a.bm == 128) launch_pair<Fmt::FP8, 128>(g1, g2, a.fast, s, stage, a.ev);
      else launch_pair<Fmt::FP8, 80>(g1, g2, a.fast, s, stage, a.ev);
      break;
    case Fmt::BF16:
      if (bm == 128) launch_pair<Fmt::BF16, 128>(g1, g2, a.fast, s, stage, a.ev);
      else launch_pair<Fmt::BF16, 96>(g1, g2, a.fast, s, stage, a.ev);
      break;
    case Fmt::MX:
      if (a.bm == 128) launch_pair<Fmt::MX, 128>(g1, g2, a.fast, s, stage, a.ev);
      else launch_pair<Fmt::MX, 80>(g1, g2, a.fast, s, stage, a.ev);
      break;
    case Fmt::NV4:
      if (bm == 128) launch_pair<Fmt::NV4, 128>(g1, g2, a.fast, s, stage, a.ev);
      else launch_pair<Fmt::NV4, 96>(g1, g2, a.fast, s, stage, a.ev);
      break;
    case Fmt::NVF4:  // gate_up decodes the NVFP4 activations; down is NV4's on the bf16 intermediate
      if (bm == 128) {
        if (stage != 2) launch_pair<Fmt::NVF4, 128>(g1, g2, a.fast, s, 1, a.ev);
        if (stage != 1) launch_pair<Fmt::NV4, 128>(g1, g2, a.fast, s, 2, a.ev);
      } else {
        if (stage != 2) launch_pair<Fmt::NVF4, 96>(g1, g2, a.fast, s, 1, a.ev);
        if (stage != 1) launch_pair<Fmt::NV4, 96>(g1, g2, a.fast, s, 2, a.ev);
      }
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
