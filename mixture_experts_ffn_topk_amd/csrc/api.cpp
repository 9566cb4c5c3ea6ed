// Host runtime behind the C ABI declared in include/moe_ffn.h: argument
// validation, tile-regime choice, workspace carving and launch sequencing.
// Nothing here allocates device memory, synchronises, or reads device data.
#include "moe_ffn.h"

#include <cmath>
#include <cstring>
#include <new>

#include "launch.h"

struct moe_handle {
  moe_config cfg;
};

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  // moe_forward: [plan buffers, split tail][y][union(plan scratch, h + h_sf)]
  size_t counts, start, ids, nact, status, src, prow, cnt, split, plan_end;
  size_t y, y_end;
  size_t scratch;  // plan scratch or h, h_sf
  size_t h_off, hsf_off, ffn_bytes, plan_scratch_bytes, total;
};

moe::Fmt to_fmt(int f) {
  switch (f) {
    case MOE_FMT_FP8_BLOCK128: return moe::Fmt::FP8;
    case MOE_FMT_BF16: return moe::Fmt::BF16;
    case MOE_FMT_NVFP4_W4A16: return moe::Fmt::NV4;
    case MOE_FMT_NVFP4: return moe::Fmt::NVF4;
    default: return moe::Fmt::MX;
  }
}
// the encoding of the weights (NVFP4 x NVFP4 shares NVFP4 x BF16's)
moe::Fmt weight_fmt(int f) { return f == MOE_FMT_NVFP4 ? moe::Fmt::NV4 : to_fmt(f); }
// bf16 activations, no activation scales
bool bf16_acts(int f) { return f == MOE_FMT_BF16 || f == MOE_FMT_NVFP4_W4A16; }
// bf16 intermediate, no intermediate scales
bool bf16_inter(int f) { return bf16_acts(f) || f == MOE_FMT_NVFP4; }

int choose_bm(const moe_config& c, int T);

Layout layout_for(const moe_config& c, int T) {
  Layout L{};
  const size_t E = (size_t)c.num_experts, np = (size_t)T * c.num_topk;
  size_t o = 0;
  L.counts = o; o = align_up(o + E * 4);
  L.start = o; o = align_up(o + (E + 1) * 4);
  L.ids = o; o = align_up(o + E * 4);
  L.nact = o; o = align_up(o + 4);
  L.status = o; o = align_up(o + 4);
  L.src = o; o = align_up(o + np * 4);
  L.prow = o; o = align_up(o + np * 4);
  L.cnt = o; o = align_up(o + (size_t)T * moe::combine_counter_stride(c.hidden) * 4);
  // the down leg's split tail, where T tokens take the prefill tile regime
  L.split = o; o = align_up(o + (choose_bm(c, T) > 96 ? moe::ffn_split_bytes(to_fmt(c.format)) : 0));
  L.plan_end = o;
  L.y = o; o = align_up(o + np * (size_t)c.hidden * 2);
  L.y_end = o;
  L.scratch = o;
  const moe::Fmt f = to_fmt(c.format);
  L.h_off = 0;
  L.hsf_off = align_up(moe::ffn_h_bytes(f, (int)np, c.intermediate_hidden));
  L.ffn_bytes = align_up(L.hsf_off + moe::ffn_hsf_bytes(f, (int)np, c.intermediate_hidden));
  L.plan_scratch_bytes = align_up(moe::plan_workspace_bytes((int)np, c.num_experts));
  L.total = L.scratch + (L.ffn_bytes > L.plan_scratch_bytes ? L.ffn_bytes : L.plan_scratch_bytes);
  return L;
}

bool valid_T(const moe_handle* h, int32_t T) { return h && T >= 0 && T <= h->cfg.max_num_tokens; }

moe::PlanPtrs plan_ptrs(const moe_plan_buffers* p, int T, int H) {
  return moe::PlanPtrs{p->expert_counts,
                       p->expert_start_indices,
                       p->expert_ids,
                       p->num_active_experts,
                       p->src_info,
                       p->pair_row,
                       p->status,
                       p->combine_counters,
                       p->combine_counters ? T * moe::combine_counter_stride(H) : 0,
                       (int*)p->down_split,
                       p->down_split ? moe::kSplitMaxSlots : 0};
}

// (down_split is optional, 256-byte aligned)
bool plan_complete(const moe_plan_buffers* p) {
  return p && p->expert_counts && p->expert_start_indices && p->expert_ids && p->num_active_experts && p->src_info &&
         p->pair_row && p->status && ((uintptr_t)p->down_split & 255) == 0;
}

int choose_bm(const moe_config& c, int T) {
  if (c.tile_regime == MOE_TILES_DECODE) return 80;
  if (c.tile_regime == MOE_TILES_PREFILL) return 128;
  // Regime gate on the host-known mean rows per expert (the pages' estimated_total_m):
  // up to 64 rows on average, one 80-row tile holds almost every expert under
  // uniform load, and the weight stream dominates.
  const long long mean = ((long long)T * c.num_topk + c.num_experts - 1) / c.num_experts;
  return mean <= 64 ? 80 : 128;
}

// The down leg splits only in the prefill tile regime (some token count up to
// the capacity reaches it).
size_t down_split_bytes(const moe_config& c) {
  if (choose_bm(c, c.max_num_tokens) <= 96) return 0;
  return moe::ffn_split_bytes(to_fmt(c.format));
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Alignment the kernels rely on: 16-byte vector loads and stores of activation,
// intermediate and output rows, 4-byte scale loads, and the 256-byte workspace
// carving.  A null pointer passes (presence is checked separately).
bool al(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// FROM_LOGITS: the top-k launch; returns the ids the plan reads (the caller's
// PRECOMPUTED ids, or idx_out)
moe_status do_route(const moe_handle* h, int32_t T, const void* idx_in, const float* logits, const float* bias,
                    void* idx_out, float* w_out, hipStream_t s, const void** ids) {
  const moe_config& c = h->cfg;
  *ids = idx_in;
  if (c.route_mode != MOE_ROUTE_FROM_LOGITS) return MOE_OK;
  hipError_t e = moe::launch_route_logits_topk(logits, bias, T, c.num_experts, c.num_topk, idx_out,
                                               c.topk_idx_bits == 64, w_out, c.fast_math != 0, s);
  *ids = idx_out;
  return hip_status(e);
}

moe_status do_plan(const moe_handle* h, int32_t T, const void* idx_in, const float* logits, const float* bias,
                   void* idx_out, float* w_out, const moe_plan_buffers* plan, void* scratch, hipStream_t s) {
  const moe_config& c = h->cfg;
  const void* ids = nullptr;
  moe_status st = do_route(h, T, idx_in, logits, bias, idx_out, w_out, s, &ids);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_plan(ids, c.topk_idx_bits == 64, T * c.num_topk, c.num_experts,
                                     plan_ptrs(plan, T, c.hidden), (int*)scratch, s));
}

// Whether the gate_up launch builds the plan itself for T tokens.
// (fuse_plan 2: wherever the sizes allow, without the cost rule)
bool plan_in_gate_up(const moe_config& c, int32_t T) {
  return T > 0 && moe::ffn_plan_fusable(to_fmt(c.format), choose_bm(c, T), T * c.num_topk, c.num_experts,
                                        c.intermediate_hidden, c.fuse_plan != 2);
}

// The combine fused into the down leg: router weights, addends and the output.
struct Fused {
  const float* topk_w;
  const void* shared;
  const void* residual;
  void* out;
};

// plan_ids: the gate_up launch builds the plan from these ids (plan_in_gate_up)
moe_status do_ffn(const moe_handle* h, int32_t T, const void* x, const void* x_sf, const moe_weights* w,
                  const moe_plan_buffers* plan, void* y, void* hbuf, void* hsf, hipStream_t s, int stage,
                  hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr, const Fused* fused = nullptr,
                  const void* plan_ids = nullptr) {
  const moe_config& c = h->cfg;
  moe::FfnArgs a{};
  a.fmt = to_fmt(c.format);
  a.T = T;
  a.E = c.num_experts;
  a.topk = c.num_topk;
  a.H = c.hidden;
  a.I = c.intermediate_hidden;
  a.clamp = c.activation_clamp;
  a.fast = c.fast_math != 0;
  a.bm = choose_bm(c, T);
  a.start = plan->expert_start_indices;
  a.src_info = plan->src_info;
  a.x = x;
  a.x_sf = x_sf;
  a.w13 = w->w13;
  a.w13_sf = w->w13_sf;
  a.w2 = w->w2;
  a.w2_sf = w->w2_sf;
  a.w13_gs = w->w13_gs;
  a.w2_gs = w->w2_gs;
  a.c_scales = w->c_input_scales;
  a.h = hbuf;
  a.h_sf = hsf;
  a.y = y;
  a.split = plan->down_split;
  if (stage == 1) a.ev[0] = e0, a.ev[1] = e1;
  if (stage == 2) a.ev[2] = e0, a.ev[3] = e1;
  if (fused) {
    a.fuse_combine = true;
    a.pair_row = plan->pair_row;
    a.topk_w = fused->topk_w;
    a.counters = plan->combine_counters;
    a.out = fused->out;
    a.shared = fused->shared;
    a.residual = fused->residual;
    a.out_f32 = c.out_fp32 != 0;
  }
  if (plan_ids) {
    a.plan_ids = plan_ids;
    a.ids64 = c.topk_idx_bits == 64;
    a.plan = plan_ptrs(plan, T, c.hidden);
  }
  return hip_status(moe::launch_ffn(a, s, stage));
}

bool weights_ok(const moe_config& c, const moe_weights* w) {
  if (!w || !w->w13 || !w->w2) return false;
  if (c.format != MOE_FMT_BF16 && (!w->w13_sf || !w->w2_sf)) return false;
  if ((c.format == MOE_FMT_NVFP4_W4A16 || c.format == MOE_FMT_NVFP4) && (!w->w13_gs || !w->w2_gs)) return false;
  if (c.format == MOE_FMT_NVFP4 && !w->c_input_scales) return false;
  return true;
}

bool x_ok(const moe_config& c, const void* x, const void* x_sf) {
  return x && (bf16_acts(c.format) || x_sf);
}

// The GEMM kernels address every operand through buffer resources with 32-bit
// lane offsets (an offset of 2^31 or more reads zeros), FP8 stages the weight
// scales of at most 256 K-steps of 128 in LDS, and a weight-bound MX tile stages
// its rows' activation-scale rows (K/32 bytes each, K up to 32768) in LDS.
bool sizes_supported(const moe_config& c) {
  constexpr unsigned long long kMaxBytes = 0x7FFFFFFFull;
  const unsigned long long T = (unsigned long long)c.max_num_tokens, H = (unsigned long long)c.hidden,
                           I = (unsigned long long)c.intermediate_hidden, k = (unsigned long long)c.num_topk;
  const unsigned long long act = bf16_acts(c.format) ? 2 : 1;  // bytes per activation element
  const unsigned long long inter = bf16_inter(c.format) ? 2 : 1;  // bytes per intermediate element
  if (T * H * act > kMaxBytes || T * k * I * inter > kMaxBytes) return false;
  // prepared weight bytes per expert
  const moe::Fmt f = weight_fmt(c.format);
  if (moe::prepared_expert_bytes(f, (int)(2 * I), (int)H) > kMaxBytes ||
      moe::prepared_expert_bytes(f, (int)H, (int)I) > kMaxBytes)
    return false;
  if ((c.format == MOE_FMT_FP8_BLOCK128 || c.format == MOE_FMT_W4A8_MX) && (H > 32768 || I > 32768)) return false;
  // the fused combine addresses y [T*k, H] bf16 through a buffer resource
  if (c.fuse_combine && T * k * H * 2 > kMaxBytes) return false;
  return true;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported combination";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t moe_abi_version(void) { return MOE_FFN_ABI_VERSION; }

moe_status moe_create(const moe_config* cfg, moe_handle** out) {
  if (!cfg || !out) return MOE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const moe_config& c = *cfg;
  if (c.hidden <= 0 || c.intermediate_hidden <= 0 || c.num_experts <= 0 || c.num_experts > 1024) return MOE_ERR_INVALID_ARGUMENT;
  if (c.num_topk <= 0 || c.num_topk > c.num_experts || c.num_topk > 32) return MOE_ERR_INVALID_ARGUMENT;
  if (c.max_num_tokens < 0 || (long long)c.max_num_tokens * c.num_topk > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  if (!(c.activation_clamp > 0.0f)) return MOE_ERR_INVALID_ARGUMENT;  // also rejects NaN
  if (c.topk_idx_bits != 32 && c.topk_idx_bits != 64) return MOE_ERR_INVALID_ARGUMENT;
  if (c.route_mode != MOE_ROUTE_PRECOMPUTED && c.route_mode != MOE_ROUTE_FROM_LOGITS) return MOE_ERR_INVALID_ARGUMENT;
  if (c.tile_regime < MOE_TILES_AUTO || c.tile_regime > MOE_TILES_PREFILL) return MOE_ERR_INVALID_ARGUMENT;
  if (c.out_fp32 != 0 && c.out_fp32 != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c.fuse_combine != 0 && c.fuse_combine != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c.fuse_plan < 0 || c.fuse_plan > 2) return MOE_ERR_INVALID_ARGUMENT;
  switch (c.format) {
    case MOE_FMT_FP8_BLOCK128:
      if (c.hidden % 128 || c.intermediate_hidden % 128) return MOE_ERR_INVALID_ARGUMENT;
      break;
    case MOE_FMT_BF16:
      if (c.hidden % 64 || c.intermediate_hidden % 64) return MOE_ERR_INVALID_ARGUMENT;
      break;
    case MOE_FMT_W4A8_MX:
      if (c.hidden % 32 || c.intermediate_hidden % 32) return MOE_ERR_INVALID_ARGUMENT;
      break;
    case MOE_FMT_NVFP4_W4A16:
    case MOE_FMT_NVFP4:
      if (c.hidden % 64 || c.intermediate_hidden % 64) return MOE_ERR_INVALID_ARGUMENT;
      break;
    default:
      return MOE_ERR_INVALID_ARGUMENT;
  }
  if (c.route_mode == MOE_ROUTE_FROM_LOGITS && c.num_experts > 512) return MOE_ERR_UNSUPPORTED;
  if (!sizes_supported(c)) return MOE_ERR_UNSUPPORTED;
  moe_handle* h = new (std::nothrow) moe_handle;
  if (!h) return MOE_ERR_INVALID_ARGUMENT;
  h->cfg = c;
  *out = h;
  return MOE_OK;
}

void moe_destroy(moe_handle* h) { delete h; }

moe_status moe_prepared_weights_size(const moe_handle* h, moe_prepared_sizes* out) {
  if (!h || !out) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config& c = h->cfg;
  const moe::Fmt f = weight_fmt(c.format);
  const size_t E = (size_t)c.num_experts;
  const int H = c.hidden, I = c.intermediate_hidden;
  out->w13 = E * moe::prepared_expert_bytes(f, 2 * I, H);
  out->w2 = E * moe::prepared_expert_bytes(f, H, I);
  if (f == moe::Fmt::FP8) {
    out->w13_sf = E * (size_t)(2 * I / 128) * (H / 128) * 4;
    out->w2_sf = E * (size_t)(H / 128) * (I / 128) * 4;
  } else {
    out->w13_sf = E * moe::prepared_scale_expert_bytes(f, 2 * I, H);
    out->w2_sf = E * moe::prepared_scale_expert_bytes(f, H, I);
  }
  return MOE_OK;
}

moe_status moe_prepare_weights(const moe_handle* h, const moe_weights* canonical, const moe_weights* prepared,
                               hipStream_t stream) {
  if (!h || !weights_ok(h->cfg, canonical) || !weights_ok(h->cfg, prepared)) return MOE_ERR_INVALID_ARGUMENT;
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  if (!aligned(canonical->w13) || !aligned(canonical->w2) || !aligned(prepared->w13) || !aligned(prepared->w2))
    return MOE_ERR_INVALID_ARGUMENT;
  if (prepared->w13 == canonical->w13 || prepared->w2 == canonical->w2) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config& c = h->cfg;
  const moe::Fmt f = weight_fmt(c.format);
  hipError_t e = moe::launch_prepare(f, c.num_experts, 2 * c.intermediate_hidden, c.hidden, true, canonical->w13,
                                     canonical->w13_sf, (void*)prepared->w13, (void*)prepared->w13_sf, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_prepare(f, c.num_experts, c.hidden, c.intermediate_hidden, false, canonical->w2, canonical->w2_sf,
                          (void*)prepared->w2, (void*)prepared->w2_sf, stream);
  return hip_status(e);
}

size_t moe_workspace_size(const moe_handle* h, int32_t T) {
  if (!valid_T(h, T)) return 0;
  return layout_for(h->cfg, T).total;
}

size_t moe_down_split_size(const moe_handle* h) { return h ? down_split_bytes(h->cfg) : 0; }

int32_t moe_plan_in_gate_up(const moe_handle* h, int32_t T) {
  if (!valid_T(h, T)) return 0;
  return plan_in_gate_up(h->cfg, T) ? 1 : 0;
}

moe_status moe_plan_ex(const moe_handle* h, int32_t T, const void* topk_idx_in, const float* routing_logits,
                       const float* routing_bias, void* topk_idx_out, float* topk_weights_out,
                       const moe_plan_buffers* plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_T(h, T) || !plan_complete(plan)) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config& c = h->cfg;
  if (c.route_mode == MOE_ROUTE_PRECOMPUTED) {
    if ((T > 0 && !topk_idx_in) || routing_bias) return MOE_ERR_INVALID_ARGUMENT;
  } else if (T > 0 && (!routing_logits || !topk_idx_out || !topk_weights_out)) {
    return MOE_ERR_INVALID_ARGUMENT;
  }
  const size_t need = layout_for(c, T).plan_scratch_bytes;
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!al(ws, 256)) return MOE_ERR_INVALID_ARGUMENT;
  return do_plan(h, T, topk_idx_in, routing_logits, routing_bias, topk_idx_out, topk_weights_out, plan, ws, stream);
}

moe_status moe_plan(const moe_handle* h, int32_t T, const void* topk_idx_in, const float* routing_logits,
                    void* topk_idx_out, float* topk_weights_out, const moe_plan_buffers* plan, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  return moe_plan_ex(h, T, topk_idx_in, routing_logits, nullptr, topk_idx_out, topk_weights_out, plan, ws, ws_bytes,
                     stream);
}

moe_status moe_ffn(const moe_handle* h, int32_t T, const void* x, const void* x_sf, const moe_weights* w,
                   const moe_plan_buffers* plan, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_T(h, T) || !plan_complete(plan) || !weights_ok(h->cfg, w)) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!x_ok(h->cfg, x, x_sf) || !y)) return MOE_ERR_INVALID_ARGUMENT;
  if (!al(x, 16) || !al(x_sf, 4) || !al(y, 16) || !al(ws, 256)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = layout_for(h->cfg, T).ffn_bytes;
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (T == 0) return MOE_OK;
  const Layout L = layout_for(h->cfg, T);
  return do_ffn(h, T, x, x_sf, w, plan, y, (char*)ws + L.h_off, (char*)ws + L.hsf_off, stream, 0);
}

moe_status moe_ffn_gate_up_timed(const moe_handle* h, int32_t T, const void* x, const void* x_sf,
                                 const moe_weights* w, const moe_plan_buffers* plan, void* h_out, void* h_sf_out,
                                 hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (!valid_T(h, T) || !plan_complete(plan) || !weights_ok(h->cfg, w)) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!x_ok(h->cfg, x, x_sf) || !h_out || (!bf16_inter(h->cfg.format) && !h_sf_out)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!al(x, 16) || !al(x_sf, 4) || !al(h_out, 16) || !al(h_sf_out, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  return do_ffn(h, T, x, x_sf, w, plan, nullptr, h_out, h_sf_out, stream, 1, start, stop);
}

moe_status moe_ffn_gate_up(const moe_handle* h, int32_t T, const void* x, const void* x_sf, const moe_weights* w,
                           const moe_plan_buffers* plan, void* h_out, void* h_sf_out, hipStream_t stream) {
  return moe_ffn_gate_up_timed(h, T, x, x_sf, w, plan, h_out, h_sf_out, stream, nullptr, nullptr);
}

moe_status moe_plan_ffn_gate_up_timed(const moe_handle* h, int32_t T, const void* topk_idx_in,
                                      const float* routing_logits, void* topk_idx_out, float* topk_weights_out,
                                      const void* x, const void* x_sf, const moe_weights* w,
                                      const moe_plan_buffers* plan, void* h_out, void* h_sf_out, void* ws,
                                      size_t ws_bytes, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  // the union of moe_plan's and moe_ffn_gate_up's checks, all before any launch
  if (!valid_T(h, T) || !plan_complete(plan) || !weights_ok(h->cfg, w)) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config& c = h->cfg;
  if (c.route_mode == MOE_ROUTE_PRECOMPUTED) {
    if (T > 0 && !topk_idx_in) return MOE_ERR_INVALID_ARGUMENT;
  } else if (T > 0 && (!routing_logits || !topk_idx_out || !topk_weights_out)) {
    return MOE_ERR_INVALID_ARGUMENT;
  }
  if (T > 0 && (!x_ok(c, x, x_sf) || !h_out || (!bf16_inter(c.format) && !h_sf_out))) return MOE_ERR_INVALID_ARGUMENT;
  if (!al(x, 16) || !al(x_sf, 4) || !al(h_out, 16) || !al(h_sf_out, 4) || !al(ws, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = layout_for(c, T).plan_scratch_bytes;
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!plan_in_gate_up(c, T)) {
    moe_status st = do_plan(h, T, topk_idx_in, routing_logits, nullptr, topk_idx_out, topk_weights_out, plan, ws,
                            stream);
    if (st != MOE_OK || T == 0) return st;
    return do_ffn(h, T, x, x_sf, w, plan, nullptr, h_out, h_sf_out, stream, 1, start, stop);
  }
  const void* ids = nullptr;
  moe_status st = do_route(h, T, topk_idx_in, routing_logits, nullptr, topk_idx_out, topk_weights_out, stream, &ids);
  if (st != MOE_OK) return st;
  return do_ffn(h, T, x, x_sf, w, plan, nullptr, h_out, h_sf_out, stream, 1, start, stop, nullptr, ids);
}

moe_status moe_plan_ffn_gate_up(const moe_handle* h, int32_t T, const void* topk_idx_in, const float* routing_logits,
                                void* topk_idx_out, float* topk_weights_out, const void* x, const void* x_sf,
                                const moe_weights* w, const moe_plan_buffers* plan, void* h_out, void* h_sf_out,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_plan_ffn_gate_up_timed(h, T, topk_idx_in, routing_logits, topk_idx_out, topk_weights_out, x, x_sf, w,
                                    plan, h_out, h_sf_out, ws, ws_bytes, stream, nullptr, nullptr);
}

moe_status moe_ffn_down_timed(const moe_handle* h, int32_t T, const void* h_in, const void* h_sf_in,
                              const moe_weights* w, const moe_plan_buffers* plan, void* y, hipStream_t stream,
                              hipEvent_t start, hipEvent_t stop) {
  if (!valid_T(h, T) || !plan_complete(plan) || !weights_ok(h->cfg, w)) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!h_in || !y || (!bf16_inter(h->cfg.format) && !h_sf_in))) return MOE_ERR_INVALID_ARGUMENT;
  if (!al(h_in, 16) || !al(h_sf_in, 4) || !al(y, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  return do_ffn(h, T, nullptr, nullptr, w, plan, y, const_cast<void*>(h_in), const_cast<void*>(h_sf_in), stream, 2,
                start, stop);
}

moe_status moe_ffn_down(const moe_handle* h, int32_t T, const void* h_in, const void* h_sf_in, const moe_weights* w,
                        const moe_plan_buffers* plan, void* y, hipStream_t stream) {
  return moe_ffn_down_timed(h, T, h_in, h_sf_in, w, plan, y, stream, nullptr, nullptr);
}

moe_status moe_ffn_down_combine_timed(const moe_handle* h, int32_t T, const void* h_in, const void* h_sf_in,
                                      const moe_weights* w, const moe_plan_buffers* plan, const float* topk_weights,
                                      void* y, const void* shared, const void* residual, void* out,
                                      hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (!valid_T(h, T) || !plan_complete(plan) || !weights_ok(h->cfg, w)) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!h_in || !y || !out || !topk_weights || !plan->combine_counters ||
                (!bf16_inter(h->cfg.format) && !h_sf_in)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!al(h_in, 16) || !al(h_sf_in, 4) || !al(y, 16) || !al(out, 16) || !al(shared, 16) || !al(residual, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  if ((unsigned long long)h->cfg.max_num_tokens * h->cfg.num_topk * h->cfg.hidden * 2 > 0x7FFFFFFFull)
    return MOE_ERR_UNSUPPORTED;  // y is addressed through a 32-bit buffer offset
  if (T == 0) return MOE_OK;
  const Fused f{topk_weights, shared, residual, out};
  return do_ffn(h, T, nullptr, nullptr, w, plan, y, const_cast<void*>(h_in), const_cast<void*>(h_sf_in), stream, 2,
                start, stop, &f);
}

moe_status moe_ffn_down_combine(const moe_handle* h, int32_t T, const void* h_in, const void* h_sf_in,
                                const moe_weights* w, const moe_plan_buffers* plan, const float* topk_weights,
                                void* y, const void* shared, const void* residual, void* out, hipStream_t stream) {
  return moe_ffn_down_combine_timed(h, T, h_in, h_sf_in, w, plan, topk_weights, y, shared, residual, out, stream,
                                    nullptr, nullptr);
}

moe_status moe_combine_ex(const moe_handle* h, int32_t T, const void* y, const float* topk_weights,
                          const moe_plan_buffers* plan, const void* shared, const void* residual, void* out,
                          hipStream_t stream) {
  if (!valid_T(h, T) || !plan || !plan->pair_row) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!y || !topk_weights || !out)) return MOE_ERR_INVALID_ARGUMENT;
  if (!al(y, 16) || !al(out, 16) || !al(shared, 16) || !al(residual, 16)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_combine(y, topk_weights, plan->pair_row, T, h->cfg.num_topk, h->cfg.hidden, shared,
                                        residual, out, h->cfg.out_fp32 != 0, stream));
}

moe_status moe_combine(const moe_handle* h, int32_t T, const void* y, const float* topk_weights,
                       const moe_plan_buffers* plan, void* out, hipStream_t stream) {
  return moe_combine_ex(h, T, y, topk_weights, plan, nullptr, nullptr, out, stream);
}

moe_status moe_forward_ex(const moe_handle* h, int32_t T, const void* x, const void* x_sf, void* topk_idx,
                          float* topk_weights, const float* routing_logits, const float* routing_bias,
                          const moe_weights* w, const void* shared, const void* residual, void* out, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  if (!valid_T(h, T) || !weights_ok(h->cfg, w)) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config& c = h->cfg;
  if (T > 0) {
    if (!x_ok(c, x, x_sf) || !out || !topk_idx || !topk_weights) return MOE_ERR_INVALID_ARGUMENT;
    if (c.route_mode == MOE_ROUTE_FROM_LOGITS && !routing_logits) return MOE_ERR_INVALID_ARGUMENT;
  }
  if (c.route_mode == MOE_ROUTE_PRECOMPUTED && routing_bias) return MOE_ERR_INVALID_ARGUMENT;
  if (!al(x, 16) || !al(x_sf, 4) || !al(out, 16) || !al(shared, 16) || !al(residual, 16) || !al(ws, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = layout_for(c, T);
  if (ws_bytes < L.total || !ws) return MOE_ERR_WORKSPACE_TOO_SMALL;
  char* base = (char*)ws;
  moe_plan_buffers plan{(int32_t*)(base + L.counts), (int32_t*)(base + L.start), (int32_t*)(base + L.ids),
                        (int32_t*)(base + L.nact),   (int32_t*)(base + L.src),   (int32_t*)(base + L.prow),
                        (int32_t*)(base + L.status),
                        c.fuse_combine ? (int32_t*)(base + L.cnt) : nullptr,
                        L.split < L.plan_end ? (void*)(base + L.split) : nullptr};
  // fuse_plan: the gate_up launch builds the plan (the top-k from logits keeps its launch)
  const void* in_launch = nullptr;
  moe_status st;
  if (c.fuse_plan && plan_in_gate_up(c, T)) {
    st = do_route(h, T, topk_idx, routing_logits, routing_bias, topk_idx, topk_weights, stream, &in_launch);
  } else {
    st = do_plan(h, T, topk_idx, routing_logits, routing_bias, topk_idx, topk_weights, &plan, base + L.scratch, stream);
  }
  if (st != MOE_OK || T == 0) return st;
  void* y = base + L.y;
  if (c.fuse_combine) {
    const Fused f{topk_weights, shared, residual, out};
    return do_ffn(h, T, x, x_sf, w, &plan, y, base + L.scratch + L.h_off, base + L.scratch + L.hsf_off, stream, 0,
                  nullptr, nullptr, &f, in_launch);
  }
  st = do_ffn(h, T, x, x_sf, w, &plan, y, base + L.scratch + L.h_off, base + L.scratch + L.hsf_off, stream, 0, nullptr,
              nullptr, nullptr, in_launch);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_combine(y, topk_weights, plan.pair_row, T, c.num_topk, c.hidden, shared, residual, out,
                                        c.out_fp32 != 0, stream));
}

moe_status moe_forward(const moe_handle* h, int32_t T, const void* x, const void* x_sf, void* topk_idx,
                       float* topk_weights, const float* routing_logits, const moe_weights* w, void* out, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  return moe_forward_ex(h, T, x, x_sf, topk_idx, topk_weights, routing_logits, nullptr, w, nullptr, nullptr, out, ws,
                        ws_bytes, stream);
}

}  // extern "C"
