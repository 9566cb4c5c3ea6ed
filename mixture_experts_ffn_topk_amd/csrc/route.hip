// Routing kernels: top-k from router logits, and the routing plan
// (per-expert counts, prefix-sum start offsets, active-expert list and the
// stable (token, slot) -> row permutation).
//
// Plan outputs follow the fused FFN's operands on the Struct_mega_ffn_ep_combine_send
// page: expert_start_indices (per-expert prefix-sum offsets), expert_ids (active
// local experts, -1 = masked), num_active_experts, src_info (per-row origin).
// FromLogits routing follows the routing_input_mode entry of the
// flashinfer.fused_moe MoEActivationPack page.
//
// Everything here is integer work except the softmax weights, so the plan is
// bit-exact and deterministic: rows of one expert are ordered by pair index
// p = t*k + j, built from wavefront ballots (no global sort, no atomics whose
// order could leak into the result).
#include "device.h"
#include "launch.h"

namespace moe {

constexpr int kPlanThreads = 1024;  // 16 waves; also the largest expert count
constexpr int kPlanWaves = kPlanThreads / 64;

// ------------------------------------------------------------------ top-k
// Order-preserving map of a float key to 32 bits (larger key, larger value;
// -0 and +0 equal, as the float comparison has them).
MOE_DEV uint32_t key_bits(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The wave's largest 64-bit (key, ~index) word, uniform: butterflies inside each
// row of 16 lanes by DPP (quad swaps, half-row and row mirrors), then the four
// row results read into scalars.  (Cross-lane shuffles through the LDS crossbar
// made each of the k selection rounds a chain of 18 round trips.)
template <int CTRL>
MOE_DEV uint64_t dpp_max_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t y = ((uint64_t)hi << 32) | lo;
  return y > x ? y : x;
}
MOE_DEV uint64_t wave_max_u64(uint64_t x) {
  x = dpp_max_u64<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_max_u64<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_max_u64<0x141>(x);  // row_half_mirror
  x = dpp_max_u64<0x140>(x);  // row_mirror
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t v = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 16 * r);
    m = v > m ? v : m;
  }
  return m;
}

// The wave's maximum and sum of a float (uniform), by the same DPP butterflies
// and row read-outs; the sum adds the four row sums in row order.
template <int CTRL>
MOE_DEV float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
MOE_DEV float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
#pragma unroll
  for (int r = 1; r < 4; ++r)
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16 * r)));
  return m;
}
MOE_DEV float wave_sum_f32(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
#pragma unroll
  for (int r = 1; r < 4; ++r) m += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16 * r));
  return m;
}

// One wavefront per token.  Each lane holds logits e = lane + 64*i (i < 8),
// k rounds of wave-wide argmax with key (logit + bias desc, index asc), then a
// softmax over the k selected logits.  The optional per-expert bias (the
// routing_bias of bias-aware methods on the MoEActivationPack page) only ranks
// the experts: the weights come from the logits themselves.
template <typename IdxT, bool FAST>
__global__ __launch_bounds__(256) void route_logits_topk_kernel(const float* __restrict__ logits,
                                                                const float* __restrict__ bias, int T, int E, int k,
                                                                IdxT* __restrict__ idx_out,
                                                                float* __restrict__ w_out) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[8], key[8];
  const float* row = logits + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int e = lane + 64 * i;
    float x = e < E ? row[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;  // NaN ranks as -inf
    const float kb = (bias != nullptr && e < E) ? v[i] + bias[e] : v[i];
    key[i] = (kb != kb) ? -INFINITY : kb;
  }
  unsigned taken = 0;
  float my_v = -INFINITY;
  int my_i = 0;
  for (int s = 0; s < k; ++s) {
    float bk = -INFINITY, bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int e = lane + 64 * i;
      bool ok = e < E && !((taken >> i) & 1u);
      if (ok && (key[i] > bk || (key[i] == bk && e < bi))) {
        bk = key[i];
        bv = v[i];
        bi = e;
      }
    }
    // the wave's winner: largest key, then smallest index (a lane without a
    // candidate, ~0x7FFFFFFF, loses to any expert at an equal key)
    const uint64_t w = wave_max_u64(((uint64_t)key_bits(bk) << 32) | (uint32_t)~bi);
    bi = (int)~(uint32_t)w;
    bv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), bi & 63));
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == s) {
      my_v = bv;
      my_i = bi;
    }
  }
  // the largest selected logit (the first one when there is no bias)
  const float vmax = wave_max_f32(lane < k ? my_v : -INFINITY);
  float ex = 0.0f;
  if (lane < k) ex = FAST ? __builtin_amdgcn_exp2f((my_v - vmax) * 1.4426950408889634f) : expf(my_v - vmax);
  const float sum = wave_sum_f32(ex);
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = (IdxT)my_i;
    w_out[(size_t)t * k + lane] = FAST ? ex * __builtin_amdgcn_rcpf(sum) : ex / sum;
  }
}

// ------------------------------------------------------------------ plan pieces
// Expert of pair p: its id if in [0, E), else -1 (a masked slot); ids other
// than -1 outside [0, E) are counted as bad.
template <typename IdxT>
MOE_DEV int load_expert(const IdxT* ids, int p, int E, int* bad) {
  long long e = (long long)ids[p];
  if (e >= 0 && e < E) return (int)e;
  if (e != -1) *bad += 1;
  return -1;
}

// Exclusive scan of cnt[0..E) (LDS) by one block of kPlanThreads threads:
// writes (if write) counts, E+1 start offsets, the active list (ascending, -1
// padded) and num_active; base_lds (if given) receives the start offsets.
// wave_tot is LDS scratch of 2*kPlanWaves ints.
MOE_DEV void plan_scan_and_active(const int* cnt, int E, int* __restrict__ counts_out, int* __restrict__ start_out,
                                  int* __restrict__ ids_out, int* __restrict__ num_active_out, int* base_lds,
                                  int* wave_tot, bool write = true) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int c = tid < E ? cnt[tid] : 0;  // one expert per thread (E <= kPlanThreads)
  const int a = c > 0;
  int cs = c, as = a;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int oc = __shfl_up(cs, d), oa = __shfl_up(as, d);
    if (lane >= d) {
      cs += oc;
      as += oa;
    }
  }
  if (lane == 63) {
    wave_tot[wave] = cs;
    wave_tot[kPlanWaves + wave] = as;
  }
  __syncthreads();
  int cb = 0, ab = 0, ctot = 0, atot = 0;
  for (int w = 0; w < kPlanWaves; ++w) {
    if (w < wave) {
      cb += wave_tot[w];
      ab += wave_tot[kPlanWaves + w];
    }
    ctot += wave_tot[w];
    atot += wave_tot[kPlanWaves + w];
  }
  const int run_c = cb + cs - c, run_a = ab + as - a;  // exclusive
  if (tid < E && base_lds) base_lds[tid] = run_c;
  if (write) {
    if (tid < E) {
      counts_out[tid] = c;
      start_out[tid] = run_c;
      if (a) ids_out[run_a] = tid;
    }
    if (tid == 0) {
      start_out[E] = ctot;
      *num_active_out = atot;
    }
    if (tid >= atot && tid < E) ids_out[tid] = -1;
  }
  __syncthreads();
}

// Stable scatter of the pairs whose experts are in ex_lds[0..n) (pair index
// p0 + i), in chunks of kPlanThreads.  run[e] (LDS) holds the next free row of
// expert e and is advanced.  wcnt is LDS scratch of kPlanWaves * E bytes, zero
// on entry and on exit.
MOE_DEV void plan_scatter(const short* ex_lds, int p0, int n, int E, int* run, uint8_t* wcnt,
                          int* __restrict__ src_info, int* __restrict__ pair_row) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int ebits = 1;
  while ((1 << ebits) < E + 1) ++ebits;
  for (int c0 = 0; c0 < n; c0 += kPlanThreads) {
    const int i = c0 + tid;
    const int e = i < n ? (int)ex_lds[i] : -1;
    // lanes holding the same expert: intersect ballots over the bits of (e + 1)
    const int key = e + 1;  // 0 for a masked slot or past the end
    uint64_t match = ~0ull;
    for (int b = 0; b < ebits; ++b) {
      const uint64_t bal = __ballot((key >> b) & 1);
      match &= ((key >> b) & 1) ? bal : ~bal;
    }
    const int rank = __popcll(match & lt_mask);
    // the lowest lane of each group publishes the group's size for this wave
    if (e >= 0 && rank == 0) wcnt[wave * E + e] = (uint8_t)__popcll(match);
    __syncthreads();
    if (e >= 0) {
      int off = run[e] + rank;
      for (int w = 0; w < wave; ++w) off += wcnt[w * E + e];
      src_info[off] = p0 + i;
      pair_row[p0 + i] = off;
    } else if (i < n) {
      pair_row[p0 + i] = -1;
    }
    __syncthreads();
    if (tid < E) {
      int sum = 0;
      for (int w = 0; w < kPlanWaves; ++w) sum += wcnt[w * E + tid];
      run[tid] += sum;
    }
    __syncthreads();
    if (e >= 0 && rank == 0) wcnt[wave * E + e] = 0;
  }
}

// ------------------------------------------------------------------ fused plan (one block)
template <typename IdxT>
__global__ __launch_bounds__(kPlanThreads) void plan_fused_kernel(const IdxT* __restrict__ ids, int npairs, int E,
                                                                  PlanPtrs out) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  int* cnt = lds;                                      // [E]
  int* run = lds + E;                                  // [E]
  int* misc = lds + 2 * E;                             // [2*kPlanWaves + 1]
  uint8_t* wcnt = (uint8_t*)(misc + 2 * kPlanWaves + 1);  // [kPlanWaves * E]
  short* ex = (short*)(wcnt + ((kPlanWaves * E + 15) & ~15));  // [npairs]
  const int tid = threadIdx.x;
  // the fused combine's arrival counters start every call at zero
  if (out.counters != nullptr)
    for (int i = tid; i < out.n_counters; i += kPlanThreads) out.counters[i] = 0;
  // and so do the down leg's split-tail counters
  if (out.split_counters != nullptr)
    for (int i = tid; i < out.n_split; i += kPlanThreads) out.split_counters[i] = 0;
  for (int e = tid; e < E; e += kPlanThreads) cnt[e] = 0;
  for (int i = tid; i < kPlanWaves * E; i += kPlanThreads) wcnt[i] = 0;
  if (tid == 0) misc[2 * kPlanWaves] = 0;
  __syncthreads();
  int bad = 0;
  for (int p = tid; p < npairs; p += kPlanThreads) {
    const int e = load_expert(ids, p, E, &bad);
    ex[p] = (short)e;
    if (e >= 0) atomicAdd(&cnt[e], 1);
  }
  if (bad) atomicAdd(&misc[2 * kPlanWaves], bad);
  __syncthreads();
  plan_scan_and_active(cnt, E, out.expert_counts, out.expert_start_indices, out.expert_ids, out.num_active, run,
                       misc);
  if (tid == 0) *out.status = misc[2 * kPlanWaves];
  plan_scatter(ex, 0, npairs, E, run, wcnt, out.src_info, out.pair_row);
}

// ------------------------------------------------------------------ multi-block plan
// 1) per-block histograms of contiguous pair ranges
template <typename IdxT>
__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(const IdxT* __restrict__ ids, int npairs, int E,
                                                                  int per_block, int* __restrict__ hist,
                                                                  int* __restrict__ bad_out, int* __restrict__ counters,
                                                                  int n_counters) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  int* cnt = lds;
  const int tid = threadIdx.x, b = blockIdx.x;
  // the fused combine's arrival counters start every call at zero
  if (counters != nullptr)
    for (int i = b * kPlanThreads + tid; i < n_counters; i += gridDim.x * kPlanThreads) counters[i] = 0;
  for (int e = tid; e < E; e += kPlanThreads) cnt[e] = 0;
  if (tid == 0) lds[E] = 0;
  __syncthreads();
  const int begin = b * per_block, end = min(npairs, begin + per_block);
  int bad = 0;
  for (int p = begin + tid; p < end; p += kPlanThreads) {
    const int e = load_expert(ids, p, E, &bad);
    if (e >= 0) atomicAdd(&cnt[e], 1);
  }
  if (bad) atomicAdd(&lds[E], bad);
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) hist[(size_t)b * E + e] = cnt[e];
  if (tid == 0) bad_out[b] = lds[E];
}

// 2) per-block stable scatter.  Every block sums the per-block histograms itself:
// each expert's total (the scan over experts gives its start) and the counts of
// the blocks before it (its base within the expert); block 0 also writes the
// counts, offsets, active list, status, and zeroes the split tail's counters.
// (One launch instead of a scan block between two: at the W4A8 shape, 8 blocks,
// the scan and scatter kernels' 6.3 + 4.7 us became 9.0 us.)
template <typename IdxT>
__global__ __launch_bounds__(kPlanThreads) void plan_scatter_kernel(const IdxT* __restrict__ ids, int npairs, int E,
                                                                    int per_block, int nblocks,
                                                                    const int* __restrict__ hist,
                                                                    const int* __restrict__ bad_in, PlanPtrs out) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  int* cnt = lds;                        // [E]
  int* run = lds + E;                    // [E]
  int* misc = lds + 2 * E;               // [2*kPlanWaves + 1]
  int* pre = misc + 2 * kPlanWaves + 1;  // [E]
  uint8_t* wcnt = (uint8_t*)(pre + E);   // [kPlanWaves * E]
  short* ex = (short*)(wcnt + ((kPlanWaves * E + 15) & ~15));  // [per_block]
  const int tid = threadIdx.x, b = blockIdx.x;
  const bool head = b == 0;
  if (head && out.split_counters != nullptr)
    for (int i = tid; i < out.n_split; i += kPlanThreads) out.split_counters[i] = 0;
  if (tid < E) {
    int tot = 0, before = 0;
    for (int bb = 0; bb < nblocks; ++bb) {
      const int c = hist[(size_t)bb * E + tid];
      before += bb < b ? c : 0;
      tot += c;
    }
    cnt[tid] = tot;
    pre[tid] = before;
  }
  if (head && tid == 0) {
    int sb = 0;
    for (int bb = 0; bb < nblocks; ++bb) sb += bad_in[bb];
    *out.status = sb;
  }
  for (int i = tid; i < kPlanWaves * E; i += kPlanThreads) wcnt[i] = 0;
  const int begin = b * per_block, end = min(npairs, begin + per_block);
  int dummy = 0;
  for (int p = begin + tid; p < end; p += kPlanThreads) ex[p - begin] = (short)load_expert(ids, p, E, &dummy);
  __syncthreads();
  plan_scan_and_active(cnt, E, out.expert_counts, out.expert_start_indices, out.expert_ids, out.num_active, run, misc,
                       head);
  if (tid < E) run[tid] += pre[tid];
  __syncthreads();
  plan_scatter(ex, begin, end - begin, E, run, wcnt, out.src_info, out.pair_row);
}

// ------------------------------------------------------------------ launchers
hipError_t launch_route_logits_topk(const float* logits, const float* bias, int T, int E, int k, void* idx_out,
                                    bool idx64, float* w_out, bool fast, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  if (idx64) {
    if (fast)
      hipLaunchKernelGGL((route_logits_topk_kernel<long long, true>), grid, block, 0, s, logits, bias, T, E, k,
                         (long long*)idx_out, w_out);
    else
      hipLaunchKernelGGL((route_logits_topk_kernel<long long, false>), grid, block, 0, s, logits, bias, T, E, k,
                         (long long*)idx_out, w_out);
  } else {
    if (fast)
      hipLaunchKernelGGL((route_logits_topk_kernel<int, true>), grid, block, 0, s, logits, bias, T, E, k,
                         (int*)idx_out, w_out);
    else
      hipLaunchKernelGGL((route_logits_topk_kernel<int, false>), grid, block, 0, s, logits, bias, T, E, k,
                         (int*)idx_out, w_out);
  }
  return hipGetLastError();
}

size_t plan_workspace_bytes(int npairs, int E) {
  int nb = plan_num_blocks(npairs);
  if (nb <= 1) return 0;
  return ((size_t)nb * E + nb) * sizeof(int);
}

int plan_pairs_per_block(int npairs) {
  const int per = ((npairs + 15) / 16 + 1023) / 1024 * 1024;  // 16 blocks, whole 1024-pair chunks
  return per < 1024 ? 1024 : per > kPlanMaxPairsPerBlock ? kPlanMaxPairsPerBlock : per;
}

int plan_num_blocks(int npairs) {
  if (npairs <= kPlanSingleBlockMaxPairs) return 1;
  const int per = plan_pairs_per_block(npairs);
  return (npairs + per - 1) / per;
}

static size_t wcnt_bytes(int E) { return (size_t)((kPlanWaves * E + 15) & ~15); }

template <typename IdxT>
static hipError_t launch_plan_t(const IdxT* ids, int npairs, int E, const PlanPtrs& out, int* ws, hipStream_t s) {
  const int nb = plan_num_blocks(npairs);
  if (nb <= 1) {
    const size_t lds = (2 * (size_t)E + 2 * kPlanWaves + 1) * sizeof(int) + wcnt_bytes(E) + (size_t)npairs * 2;
    hipLaunchKernelGGL(plan_fused_kernel<IdxT>, dim3(1), dim3(kPlanThreads), lds, s, ids, npairs, E, out);
    return hipGetLastError();
  }
  int* hist = ws;
  int* bad = ws + (size_t)nb * E;
  const int per = plan_pairs_per_block(npairs);
  hipLaunchKernelGGL(plan_count_kernel<IdxT>, dim3(nb), dim3(kPlanThreads), (E + 1) * sizeof(int), s, ids, npairs,
                     E, per, hist, bad, out.counters, out.n_counters);
  hipLaunchKernelGGL(plan_scatter_kernel<IdxT>, dim3(nb), dim3(kPlanThreads),
                     (3 * (size_t)E + 2 * kPlanWaves + 1) * sizeof(int) + wcnt_bytes(E) + (size_t)per * 2, s, ids,
                     npairs, E, per, nb, (const int*)hist, (const int*)bad, out);
  return hipGetLastError();
}

hipError_t launch_plan(const void* ids, bool idx64, int npairs, int E, const PlanPtrs& out, int* ws,
                       hipStream_t s) {
  if (idx64) return launch_plan_t((const long long*)ids, npairs, E, out, ws, s);
  return launch_plan_t((const int*)ids, npairs, E, out, ws, s);
}

}  // namespace moe
