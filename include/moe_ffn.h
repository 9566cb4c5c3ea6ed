/*
 * moe_ffn.h — C ABI of the routed MoE expert-FFN library for MI355X (gfx950).
 *
 * One GPU's share of experts, end to end:
 *   top-k routing -> per-expert permutation (expert_start_indices, src_info)
 *   -> gate/up grouped GEMM with clamped SwiGLU and intermediate requantisation
 *   -> down grouped GEMM -> router-weighted combine back into token order.
 *
 * Sources (API documentation pages; cited by page title and parameter):
 *   [SymmBuffer]  flashinfer.megamoe.MegaMoESymmBuffer — geometry (hidden,
 *                 intermediate_hidden, num_experts, num_topk,
 *                 num_max_tokens_per_rank, activation_clamp, fast_math) and the
 *                 staging views x / x_sf / topk_idx / topk_weights.
 *   [MegaFFN]     Struct_mega_ffn_ep_combine_send (MAX mega_ffn) — the fused FFN's
 *                 operands: gate_up_weight, down_weight and their scale tiles,
 *                 expert_start_indices, expert_ids, num_active_experts, src_info,
 *                 estimated_total_m (tile-regime gate), clamp_activation.
 *   [ActPack]     flashinfer.fused_moe.MoEActivationPack — operand encodings
 *                 (DeepSeek FP8, MXFP8, MXFP4 x MXFP8, BF16, NVFP4) and routing input
 *                 modes (precomputed ids/weights, FromLogits).
 *   [EPCombine]   DistributedEPCombine (MAX ep) — router_weights scale each
 *                 expert's contribution in the combine.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer; the library keeps only its immutable host-side handle.
 *   - Calls are asynchronous on the given hipStream_t, never allocate device
 *     memory, never synchronise and never read device data on the host, so a
 *     sequence of calls can be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed validation launches nothing and returns a status != MOE_OK.
 *   - Alignment: activation, intermediate, y and output buffers (x, h, y, out,
 *     shared, residual) 16 bytes; scale buffers 4 bytes; workspaces 256 bytes.
 *     A misaligned pointer is MOE_ERR_INVALID_ARGUMENT.
 *   - Data errors found on the device (an expert id outside [0, E) that is not
 *     -1) never trap: that slot is treated as masked and counted in
 *     plan->status[0].
 *   - T = 0 tokens is a valid no-op.
 *   - Bytes of every tensor are row-major with the last dimension contiguous.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_ABI_VERSION 11

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* bad geometry, null pointer, T out of range */
  MOE_ERR_UNSUPPORTED = 2,        /* a valid but unsupported combination (raised, never degraded) */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a launch failed; see hipGetLastError() */
} moe_status;

/* Operand encodings ([ActPack] encodings list). */
typedef enum {
  /* "DeepSeek FP8": x E4M3 [T,H] + fp32 scales [T,H/128] (token-major, as the
     [SymmBuffer] x_sf view); w13 E4M3 [E,2I,H] + fp32 [E,2I/128,H/128];
     w2 E4M3 [E,H,I] + fp32 [E,H/128,I/128].  H and I multiples of 128. */
  MOE_FMT_FP8_BLOCK128 = 0,
  /* "BF16": x [T,H], w13 [E,2I,H], w2 [E,H,I] bf16, no scales.  H, I multiples of 64. */
  MOE_FMT_BF16 = 1,
  /* "MXFP4 x MXFP8 (W4A8)": x E4M3 [T,H] + UE8M0 bytes [T,H/32] (token-major);
     w13 packed E2M1 [E,2I,H/2] + UE8M0 [E,2I,H/32]; w2 packed E2M1 [E,H,I/2]
     + UE8M0 [E,H,I/32].  Element 2i is the low nibble of byte i.
     H and I multiples of 32. */
  MOE_FMT_W4A8_MX = 2,
  /* "NVFP4 x BF16 (W4A16)": x bf16 [T,H], no activation scale; w13 packed
     E2M1 [E,2I,H/2] + E4M3 block scales [E,2I,H/16] + one fp32 global scale
     per expert (moe_weights.w13_gs [E]); w2 packed E2M1 [E,H,I/2] + E4M3
     [E,H,I/16] + w2_gs [E].  A weight is e2m1 * block scale * global scale
     ([MegaFFN] gate_up_expert_scales / down_expert_scales carry the per-expert
     scale).  The intermediate is bf16.  H and I multiples of 64. */
  MOE_FMT_NVFP4_W4A16 = 3,
  /* "NVFP4 x NVFP4": x packed E2M1 [T,H/2] + E4M3 block scales [T,H/16] (x_sf);
     weights as MOE_FMT_NVFP4_W4A16.  The per-expert scales are those of [MegaFFN]:
     w13_gs = gate_up_expert_scales (the gate_up leg's output scale: the
     activations' global scale times the weight's), w2_gs = down_expert_scales
     (the down leg's output scale), c_input_scales = the global scale the
     intermediate is requantised against: per (row, 16 columns) block scale
     E4M3_RNE_sat(amax / (6 c)) and codes E2M1_RNE_sat(h / (s c)); the down leg
     consumes codes x block scales (held exactly as bf16 in the caller-visible h
     [T*k, I] of the split legs, h_sf unused).  H and I multiples of 64. */
  MOE_FMT_NVFP4 = 4
} moe_format;

/* Routing input modes ([ActPack] routing_input_mode). */
typedef enum {
  MOE_ROUTE_PRECOMPUTED = 0,   /* caller passes topk_idx + topk_weights */
  MOE_ROUTE_FROM_LOGITS = 1    /* caller passes routing_logits [T,E] fp32; the
                                  library selects top-k (ties -> lower expert id)
                                  and writes ids + softmax-over-k weights */
} moe_route_mode;

/* GEMM tile regime ([MegaFFN] estimated_total_m gates the tile regime).
   AUTO picks from the mean rows per expert T*k/E known on the host. */
typedef enum { MOE_TILES_AUTO = 0, MOE_TILES_DECODE = 1, MOE_TILES_PREFILL = 2 } moe_tile_regime;

/* (host) Problem statement, copied by moe_create ([SymmBuffer] constructor). */
typedef struct moe_config {
  int32_t hidden;               /* H */
  int32_t intermediate_hidden;  /* I */
  int32_t num_experts;          /* E: experts resident on this GPU ([MegaFFN]: local count) */
  int32_t num_topk;             /* k, 1 <= k <= E, k <= 32 */
  int32_t max_num_tokens;       /* capacity, like num_max_tokens_per_rank */
  float activation_clamp;       /* SwiGLU clamp c > 0 (default 10.0); +inf disables */
  int32_t format;               /* moe_format */
  int32_t route_mode;           /* moe_route_mode */
  int32_t topk_idx_bits;        /* 64 (INT64 ids, [SymmBuffer]) or 32 (int32 ids, [ActPack]) */
  int32_t fast_math;            /* 1: hardware exp/reciprocal in SiLU and softmax ([SymmBuffer]) */
  int32_t tile_regime;          /* moe_tile_regime */
  int32_t out_fp32;             /* dtype of the combine output ([EPConfig] combine_dtype and the
                                   mega_ffn combine_dtype parameter leave it open): 0 = bf16
                                   [T,H] (one rounding of the fp32 sum), 1 = fp32 [T,H] */
  int32_t fuse_combine;         /* 1: moe_forward runs the combine inside the down GEMM's
                                   epilogue (moe_ffn_down_combine) instead of as its own
                                   launch ([EPConfig] fuse_ffn_combine_send); same result, bit
                                   for bit */
  int32_t fuse_plan;            /* routing plan inside the gate_up launch (moe_plan_ffn_gate_up;
                                   same plan and result, bit for bit): 0 = moe_forward keeps the
                                   plan's own launch; 1 = moe_forward builds it in the gate_up
                                   launch where that pays; 2 = wherever the sizes allow (also
                                   for moe_plan_ffn_gate_up) */
} moe_config;

/* (host struct of device pointers) Expert weights of this GPU: the canonical
   tensors of moe_format (input of moe_prepare_weights) or their prepared
   layout (input of every FFN entry point). */
typedef struct moe_weights {
  const void* w13;     /* gate_up_weight: rows [0,I) gate, rows [I,2I) up */
  const void* w13_sf;  /* its scales (NULL for BF16) */
  const void* w2;      /* down_weight */
  const void* w2_sf;   /* its scales (NULL for BF16) */
  const float* w13_gs; /* NVFP4: fp32 global scale per expert [E], read as given
                          (no relayout; a prepared struct points at the same
                          buffer); NULL for the other formats */
  const float* w2_gs;  /* NVFP4: likewise for down_weight */
  const float* c_input_scales; /* NVFP4 x NVFP4: per-expert global scale of the requantised
                                  intermediate [E] ([MegaFFN] c_input_scales); NULL otherwise */
} moe_weights;

/* (host struct of device pointers) Routing plan, int32 each ([MegaFFN] Args). */
typedef struct moe_plan_buffers {
  int32_t* expert_counts;         /* [E]   valid pairs per expert */
  int32_t* expert_start_indices;  /* [E+1] exclusive prefix sum of the counts */
  int32_t* expert_ids;            /* [E]   active experts ascending, then -1 */
  int32_t* num_active_experts;    /* [1] */
  int32_t* src_info;              /* [T*k] row -> pair p = t*k + j (rows of an expert keep p order) */
  int32_t* pair_row;              /* [T*k] pair -> row, -1 for a masked slot */
  int32_t* status;                /* [1]   count of ids outside [0,E) other than -1 */
  int32_t* combine_counters;      /* [T * ceil(H/128)] or NULL: arrival counters of the fused
                                     combine ([MegaFFN] arrival_count), zeroed by moe_plan;
                                     needed by moe_ffn_down_combine only */
  void* down_split;               /* moe_down_split_size bytes, 256-byte aligned, or NULL: the
                                     down leg's split tail (below); its arrival counters are
                                     zeroed by moe_plan / moe_plan_ffn_gate_up of the same
                                     plan and left zero by the down leg */
} moe_plan_buffers;

typedef struct moe_handle moe_handle;

/* (host) Byte sizes of the prepared weight tensors (0 where a tensor is absent). */
typedef struct moe_prepared_sizes {
  size_t w13, w13_sf, w2, w2_sf;
} moe_prepared_sizes;

/* Validate *cfg and create a host handle.  Returns MOE_ERR_INVALID_ARGUMENT for
   bad geometry (see moe_format for the divisibility rules), k > E, k > 32,
   E > 1024, clamp <= 0 or NaN, an unknown enum; MOE_ERR_UNSUPPORTED for
   FROM_LOGITS with E > 512, for FP8 and W4A8 with hidden or intermediate_hidden
   above 32768, and where max_num_tokens x hidden (activations), max_num_tokens x k x
   intermediate_hidden (intermediate) or one expert's gate_up weight reaches
   2^31 bytes. */
moe_status moe_create(const moe_config* cfg /* host */, moe_handle** out /* host */);
/* Release the host handle ([SymmBuffer] destroy(): release what the object
   holds).  The handle owns no device memory, so nothing on the device is freed
   and no stream is touched; NULL is a no-op.  The caller must not pass the
   handle to any call afterwards. */
void moe_destroy(moe_handle* h);

/* Prepared weight layout ([MegaFFN] takes its gate_up weight pre-permuted; here
   both weights are).  A weight matrix of R rows and K elements per row (w13: R =
   2I, K = H; w2: R = H, K = I) is cut into tiles of RT rows x one K-step,
   stored expert-major, then by row block rb = row / RT, then by K-step ks, each
   tile contiguous:
     FP8   RT 16, K-step 128, 2048-byte tile: byte 1024*piece + 16*l + b
           (piece < 2, l = 16*g + r, g < 4, r < 16, b < 16) holds byte
           ks*128 + 64*piece + 16*g + b of row 16*rb + r
     MX    RT 16, K-step 128, 1024-byte tile: byte 16*l + b (l = 16*g + r) holds
           byte ks*64 + 16*g + b of packed E2M1 row 16*rb + r, zero past the row's end
     MX scales: 64-byte tile: byte l (l = 16*g + r) holds the UE8M0 byte of
           K-block 4*ks + g of row 16*rb + r, zero past the row's end
     BF16  RT 32, K-step 64, 4096-byte tile: byte 1024*sub + 16*l + b
           (sub < 4, l = 32*h + r, h < 2, r < 32) holds byte ks*128 + 32*sub + 16*h + b
           of tile row 32*rb + r; for w13 tile row 32*j + q is gate row 16*j + q
           (q < 16) or up row 16*j + q - 16 (q >= 16), for w2 it is row 32*j + q
     NVFP4 RT 32, K-step 64, 1024-byte tile: byte 16*l + 4*sub + b (l = 32*h + r,
           sub < 4, b < 4) holds byte ks*32 + 8*sub + 4*h + b of packed E2M1 tile
           row r (rows mapped as for BF16), zero past the row's end
     NVFP4 scales: 128-byte tile: byte 4*r + sub holds the E4M3 scale of
           K-block (16 elements) 4*ks + sub of tile row r, zero past the end
     FP8 scales unchanged; NVFP4 global scales are not part of the layout.
   moe_prepared_weights_size gives the sizes; moe_prepare_weights writes them. */
moe_status moe_prepared_weights_size(const moe_handle* h, moe_prepared_sizes* out /* host */);

/* One-time relayout of canonical weights (moe_format) into the prepared layout,
   asynchronously on `stream`.  `prepared` points to caller-owned buffers of the
   sizes above (16-byte aligned, not overlapping the canonical ones; for FP8 the
   scale buffers may alias the canonical scales).  Canonical buffers must be
   16-byte aligned.  Every FFN entry point below reads the prepared layout. */
moe_status moe_prepare_weights(const moe_handle* h, const moe_weights* canonical /* host struct */,
                               const moe_weights* prepared /* host struct */, hipStream_t stream);

/* Bytes of workspace moe_plan / moe_ffn / moe_forward need for num_tokens tokens
   ([EPConfig] estimate_memory_usage(): the bytes a configuration needs per device,
   known before anything runs), 0 if num_tokens is out of range.  The workspace
   is caller-owned device memory, 256-byte aligned (a misaligned workspace is
   MOE_ERR_INVALID_ARGUMENT); one workspace per concurrently running stream. */
size_t moe_workspace_size(const moe_handle* h, int32_t num_tokens);

/* Bytes of plan->down_split for this handle (0: its down leg never splits, and
   the field may stay NULL).  Split tail of the down leg: when the prefill-regime
   down tiles (see moe_tile_regime) leave a last partial round of at most half
   the workgroups the part runs at once, each of those tiles is cut over K into
   up to 8 pieces that run side by side; each piece stores an fp32 partial tile
   there and the last to arrive ([MegaFFN] arrival_count: cross-workgroup arrival
   counts) sums them in piece order and writes the tile.  The result is
   deterministic; it differs from the unsplit sum only in fp32 summation order.
   With down_split NULL nothing splits.  Calls that share a plan's down_split must
   not overlap. */
size_t moe_down_split_size(const moe_handle* h);

/* Routing plan ([MegaFFN] expert_start_indices, expert_ids, num_active_experts,
   src_info; [ActPack] routing modes).
   PRECOMPUTED: topk_idx_in [T,k] int64/int32 ids (-1 = masked slot).
   FROM_LOGITS: routing_logits [T,E] fp32 in; topk_idx_out [T,k] (dtype per
   topk_idx_bits) and topk_weights_out [T,k] fp32 out.
   Writes every buffer of *plan. */
moe_status moe_plan(const moe_handle* h, int32_t num_tokens, const void* topk_idx_in,
                    const float* routing_logits, void* topk_idx_out, float* topk_weights_out,
                    const moe_plan_buffers* plan /* host struct */, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* moe_plan with bias-aware FROM_LOGITS routing ([ActPack] routing_bias of the
   bias-aware routing methods).  routing_bias [E] fp32 (device; NULL = none)
   ranks the experts by routing_logits[t,e] + routing_bias[e] (fp32 sum; ties ->
   lower expert id); the weights stay a softmax over the k selected experts'
   unbiased logits.  A non-NULL routing_bias in PRECOMPUTED mode is
   MOE_ERR_INVALID_ARGUMENT.  moe_plan(...) is moe_plan_ex(..., NULL, ...). */
moe_status moe_plan_ex(const moe_handle* h, int32_t num_tokens, const void* topk_idx_in,
                       const float* routing_logits, const float* routing_bias, void* topk_idx_out,
                       float* topk_weights_out, const moe_plan_buffers* plan /* host struct */, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* Expert FFN over the plan's rows ([MegaFFN]: gate/up GEMM -> clamped SwiGLU ->
   intermediate requantisation -> down GEMM).  x, x_sf per the format; y [T,k,H]
   bf16 receives each row's result at its pair slot p = src_info[row]; slots of
   masked pairs are left untouched.  w: prepared layout. */
moe_status moe_ffn(const moe_handle* h, int32_t num_tokens, const void* x, const void* x_sf,
                   const moe_weights* w /* host struct */, const moe_plan_buffers* plan /* host struct */,
                   void* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* The two legs of moe_ffn, for callers that schedule or time them separately.
   The requantised intermediate is caller-owned here:
     h    [T*k, I]   E4M3 bytes (FP8, MX) or bf16 (BF16), row = plan row
     h_sf            fp32 [T*k, I/128] (FP8), UE8M0 bytes [T*k, I/32] (MX), NULL (BF16)
   moe_ffn_gate_up: gate/up GEMM of every plan row, clamped SwiGLU, requantisation
   ([MegaFFN]: L1 GEMM, clamp_activation, the re-quant ahead of L2).
   moe_ffn_down: down GEMM of every plan row into y [T,k,H] bf16 at p = src_info[row]
   (with plan->down_split set, the split tail of moe_down_split_size may run).
   w: prepared layout. */
moe_status moe_ffn_gate_up(const moe_handle* h, int32_t num_tokens, const void* x, const void* x_sf,
                           const moe_weights* w /* host struct */, const moe_plan_buffers* plan /* host struct */,
                           void* h_out, void* h_sf_out, hipStream_t stream);
moe_status moe_ffn_down(const moe_handle* h, int32_t num_tokens, const void* h_in, const void* h_sf_in,
                        const moe_weights* w /* host struct */, const moe_plan_buffers* plan /* host struct */,
                        void* y, hipStream_t stream);

/* moe_ffn_gate_up / moe_ffn_down with timing: start and stop are hipEvent_t
   handles owned by the caller (created with timing enabled; either may be NULL).
   They travel with the leg's GEMM kernel launch itself (hipExtLaunchKernel), so
   hipEventElapsedTime(start, stop) is that kernel's own execution time, with no
   separate marker commands between kernels of the stream.  Nothing is recorded
   when no kernel is launched (num_tokens = 0).  Same validation and errors as
   the untimed calls; the events are not checked. */
moe_status moe_ffn_gate_up_timed(const moe_handle* h, int32_t num_tokens, const void* x, const void* x_sf,
                                 const moe_weights* w /* host struct */,
                                 const moe_plan_buffers* plan /* host struct */, void* h_out, void* h_sf_out,
                                 hipStream_t stream, hipEvent_t start, hipEvent_t stop);
moe_status moe_ffn_down_timed(const moe_handle* h, int32_t num_tokens, const void* h_in, const void* h_sf_in,
                              const moe_weights* w /* host struct */, const moe_plan_buffers* plan /* host struct */,
                              void* y, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/* moe_plan followed by moe_ffn_gate_up, as one kernel launch where the sizes
   allow ([EPConfig] fused_moe_ready: dispatch, FFN and combine as few launches;
   here the routing plan moves into the gate_up launch).  Arguments are those of
   the two calls: routing as moe_plan (PRECOMPUTED: topk_idx_in; FROM_LOGITS:
   routing_logits with topk_idx_out / topk_weights_out, whose top-k keeps its own
   launch), the plan buffers (outputs, complete when the call's work is done),
   ws / ws_bytes as for moe_plan, then x, x_sf, w, h_out, h_sf_out as for
   moe_ffn_gate_up.  Where it pays -- the weight-bound tile regime, at most 8192
   pairs, and pairs x rounds of gate_up workgroups per CU (worst-case grid over 512
   workgroup slots) at most 4096, since every workgroup reads all the ids; with the
   handle's fuse_plan = 2, wherever the first two hold -- every workgroup of the
   gate_up launch counts the ids and gathers its own rows itself, and the launch
   writes the whole plan; otherwise the call launches moe_plan's kernels and then
   the gate_up leg.  Plan and h are bit for bit those of the two
   separate calls.  Validation and errors: the union of theirs.  The _timed form's
   events travel with the gate_up kernel's launch (which then includes the plan's
   work where it is built in that launch). */
moe_status moe_plan_ffn_gate_up(const moe_handle* h, int32_t num_tokens, const void* topk_idx_in,
                                const float* routing_logits, void* topk_idx_out, float* topk_weights_out,
                                const void* x, const void* x_sf, const moe_weights* w /* host struct */,
                                const moe_plan_buffers* plan /* host struct */, void* h_out, void* h_sf_out,
                                void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_plan_ffn_gate_up_timed(const moe_handle* h, int32_t num_tokens, const void* topk_idx_in,
                                      const float* routing_logits, void* topk_idx_out, float* topk_weights_out,
                                      const void* x, const void* x_sf, const moe_weights* w /* host struct */,
                                      const moe_plan_buffers* plan /* host struct */, void* h_out, void* h_sf_out,
                                      void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t start,
                                      hipEvent_t stop);

/* (host) 1 if moe_plan_ffn_gate_up (and moe_forward with fuse_plan set) builds the
   routing plan inside the gate_up launch for num_tokens tokens (the rule above:
   [EPConfig] fused_moe_ready), 0 if it launches the plan kernels first or if
   h or num_tokens is invalid.  Launches nothing. */
int32_t moe_plan_in_gate_up(const moe_handle* h, int32_t num_tokens);

/* The down leg with the router-weighted combine fused into its epilogue
   ([EPConfig] fuse_ffn_combine_send: the expert FFN's down epilogue feeds the
   combine; [MegaFFN] arrival_count: per-destination arrival counts).  Each tile
   stores its y rows, then counts them as arrived at their (token, column tile)
   counters in plan->combine_counters (which moe_plan of the same plan zeroed;
   NULL is MOE_ERR_INVALID_ARGUMENT); the tile whose arrival completes a token's
   valid slots reduces that token's columns in slot order, exactly as moe_combine
   (moe_combine_ex's addends shared / residual, NULL = absent; bf16 or fp32 out per
   out_fp32).  y [T,k,H] bf16 is still written (the tiles exchange rows through
   it); out [T,H] receives the result, bit for bit that of moe_ffn_down followed
   by moe_combine_ex.  Tokens with no valid slot get the addends (or zeros). */
moe_status moe_ffn_down_combine(const moe_handle* h, int32_t num_tokens, const void* h_in, const void* h_sf_in,
                                const moe_weights* w /* host struct */,
                                const moe_plan_buffers* plan /* host struct */, const float* topk_weights,
                                void* y, const void* shared, const void* residual, void* out, hipStream_t stream);
/* moe_ffn_down_combine with the launch-carried timing events of moe_ffn_down_timed. */
moe_status moe_ffn_down_combine_timed(const moe_handle* h, int32_t num_tokens, const void* h_in,
                                      const void* h_sf_in, const moe_weights* w /* host struct */,
                                      const moe_plan_buffers* plan /* host struct */, const float* topk_weights,
                                      void* y, const void* shared, const void* residual, void* out,
                                      hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/* Router-weighted combine ([EPCombine] router_weights): out[t] = sum over valid
   slots j in ascending order of topk_weights[t,j] * y[t,j,:], accumulated in
   fp32, written as bf16 [T,H] (fp32 [T,H] when moe_config.out_fp32).  A token with
   no valid slot gets zeros. */
moe_status moe_combine(const moe_handle* h, int32_t num_tokens, const void* y, const float* topk_weights,
                       const moe_plan_buffers* plan /* host struct */, void* out, hipStream_t stream);

/* moe_combine with fused addends (MAX mega_ffn / EP pages: fused_shared_expert,
   "a shared expert is fused into the combine kernel", and has_epilogue_fusion,
   "the combine output is fused with a downstream elementwise epilogue"):
     out[t] = bf16( sum over valid slots j of topk_weights[t,j] * y[t,j,:]
                    + shared[t,:] + residual[t,:] ),
   accumulated in fp32 in that order.  shared and residual are bf16 [T,H]
   (device, 16-byte aligned; NULL = absent).  A shared expert's output comes from
   moe_ffn of a handle with num_experts = 1, num_topk = 1 and every token routed
   to expert 0: its y [T,1,H] is [T,H] in token order.  moe_combine(...) is
   moe_combine_ex(..., NULL, NULL, ...). */
moe_status moe_combine_ex(const moe_handle* h, int32_t num_tokens, const void* y, const float* topk_weights,
                          const moe_plan_buffers* plan /* host struct */, const void* shared, const void* residual,
                          void* out, hipStream_t stream);

/* The whole path in one call: plan (into ws), FFN (y in ws), combine into out
   [T,H] bf16 (fused into the down leg when fuse_combine).  PRECOMPUTED: topk_idx / topk_weights are inputs and are not
   modified.  FROM_LOGITS: routing_logits is the input and topk_idx / topk_weights
   receive the routing result.  w: prepared layout. */
moe_status moe_forward(const moe_handle* h, int32_t num_tokens, const void* x, const void* x_sf,
                       void* topk_idx, float* topk_weights, const float* routing_logits,
                       const moe_weights* w /* host struct */, void* out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* moe_forward with the routing bias of moe_plan_ex and the combine addends of
   moe_combine_ex (each NULL = absent). */
moe_status moe_forward_ex(const moe_handle* h, int32_t num_tokens, const void* x, const void* x_sf,
                          void* topk_idx, float* topk_weights, const float* routing_logits,
                          const float* routing_bias, const moe_weights* w /* host struct */, const void* shared,
                          const void* residual, void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the scratch array moe_forward_static uses as its workspace, one array
   per device. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate device memory: code under HIP
   graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
   arguments and results as moe_forward without ws / ws_bytes: the workspace is a
   scratch array of MOE_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on
   each device it runs on until the process ends; the call itself allocates
   nothing.  Its address on the current device is resolved at the first call on
   that device.  Limit: num_tokens whose moe_workspace_size exceeds 64 MiB gets
   MOE_ERR_WORKSPACE_TOO_SMALL before any launch (at the decode shape H = 7168,
   I = 2048, k = 8, up to 456 tokens).  Every call on one device shares that
   device's array, which keeps the last call's contents (nothing in it needs to
   start at zero); calls that overlap on one device (other streams, other
   threads) race on it and must be serialised by the caller. */
moe_status moe_forward_static(const moe_handle* h, int32_t num_tokens, const void* x, const void* x_sf,
                              void* topk_idx, float* topk_weights, const float* routing_logits,
                              const moe_weights* w /* host struct */, void* out, hipStream_t stream);

const char* moe_status_string(moe_status s);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */
