/*
 * moe.h - C ABI of the MI355X (gfx950) forward pass of a DeepSeek-V3-style
 * Mixture-of-Experts layer.
 *
 * The layer, as the DeepSeek-V3.2-Exp pages define it:
 *   gate    ("Expert scores": formula z = x_ffn W_r, Gate.forward excerpt)
 *           z = x W_r^T in fp32; s = sigmoid(z) or softmax(z); s' = s + bias
 *           (selection only); keep the topk_groups best of n_groups groups
 *           (group score = sum of its two largest s' when a bias is given,
 *           else its largest s'); take the topk largest s'; weights are the
 *           unbiased s of the chosen experts, divided by their sum for
 *           sigmoid, times route_scale.
 *   experts (routed experts and one shared MLP, SwiGLU):
 *           FFN(v) = W2 (silu(W1 v) * (W3 v)), weights stored [out, in].
 *   combine ("Weighted expert sum": formula y_routed = sum_i G_i E_i, the
 *           MoE.forward excerpt and its fp32-accumulate note)
 *           y_t = cast( sum_k w[t,k] FFN_{idx[t,k]}(x_t) + FFN_shared(x_t) ),
 *           summed in fp32 and cast back to x's dtype.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers, row-major, owned by the caller.
 *     The library never allocates or frees device memory; scratch space comes
 *     from the caller's workspace (size from moe_workspace_size()).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; no call copies to the host or
 *     synchronises.  Results are valid once the stream has reached them.
 *   - Inputs are never written.  Outputs are fully overwritten (no need to
 *     zero them).  Outputs must not alias inputs.
 *   - Validation happens on the host before anything is enqueued; on an error
 *     nothing is enqueued, outputs are untouched, and moe_last_error() gives a
 *     readable reason (thread-local).  T == 0 is a successful no-op.
 *   - Results are deterministic: the same inputs give bitwise-equal outputs.
 *   - Calls that share a workspace must be ordered (same stream).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* a shape, pointer or hyper-parameter is invalid          */
  MOE_ERR_UNSUPPORTED = 2,  /* valid, but outside what the kernels implement           */
  MOE_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than moe_workspace_size()     */
  MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed              */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,              /* IEEE binary32                                          */
  MOE_BF16 = 1,             /* bfloat16 (uint16 storage)                              */
  MOE_FP8_E4M3 = 2          /* OCP e4m3fn (uint8 storage), with fp32 block scales     */
} moe_dtype;

typedef enum moe_score {
  MOE_SCORE_SIGMOID = 0,
  MOE_SCORE_SOFTMAX = 1
} moe_score;

/* Accumulator of the combine.
 *   MOE_ACC_F32   ("Weighted expert sum", MoE.forward excerpt and its note:
 *                 y starts as fp32 zeros): y_t = cast( sum_k w O + S ), fp32
 *                 throughout, one cast at the end.
 *   MOE_ACC_LAYER (the original DeepSeek-V3 MoE.forward in the hackaday.io log
 *                 "Time to jump right in and swim with the big fish": the
 *                 running sum lives in x's dtype, the routed experts add their
 *                 weighted outputs in ascending id, the shared output last):
 *                 y_t = 0 in the layer dtype; for each of the token's experts
 *                 in ascending id, y_t = cast(y_t + O*w) with the product and
 *                 the sum in fp32 (torch's promotion of a bf16 tensor times
 *                 fp32 weights); finally y_t = cast(y_t + S_t).  With fp32
 *                 layers every cast is the identity.                         */
typedef enum moe_accumulate {
  MOE_ACC_F32 = 0,
  MOE_ACC_LAYER = 1
} moe_accumulate;

/* Shapes and hyper-parameters ("Expert scores", Gate constructor excerpt:
 * dim, topk = activated experts, n_groups, topk_groups = limited groups,
 * score_func, route_scale; routed and shared widths from the MoE constructor
 * Expert(dim, moe_inter_dim) and MLP(dim, n_shared_experts * moe_inter_dim)).
 *
 * Supported combinations:
 *   act_dtype = router_dtype = weight_dtype = MOE_F32, or
 *   act_dtype = router_dtype = MOE_BF16 with weight_dtype MOE_BF16 or MOE_FP8_E4M3.
 * Limits: 1 <= n_experts <= 512; n_experts % n_groups == 0; n_groups <= 64;
 *   1 <= topk_groups <= n_groups; 1 <= topk <= 32 and topk <= topk_groups *
 *   n_experts / n_groups; with a bias and n_groups > 1 each group needs >= 2
 *   experts; dim, inter and shared_inter multiples of 64 (of 128 for fp8)
 *   and at most 65536; T < 2^24 tokens.  moe_expert_ffn, moe_combine and moe_forward also
 *   return MOE_ERR_UNSUPPORTED, before enqueuing anything, when an expert
 *   launch for T tokens would exceed the 2^32 - 1 work-items a dispatch can
 *   count (only at extreme T x width products).                             */
typedef struct moe_params {
  int32_t dim;           /* model width                                          */
  int32_t n_experts;     /* E, routed experts                                    */
  int32_t n_groups;      /* expert groups (1 = no group limit)                   */
  int32_t topk_groups;   /* groups kept per token                                */
  int32_t topk;          /* experts per token                                    */
  int32_t inter;         /* inner width of every routed expert                   */
  int32_t shared_inter;  /* inner width of the shared expert, 0 = none           */
  int32_t score_func;    /* moe_score                                            */
  float route_scale;     /* multiplies the routing weights                       */
  int32_t act_dtype;     /* dtype of x and y: MOE_F32 or MOE_BF16                */
  int32_t router_dtype;  /* dtype of W_r (applied in fp32)                       */
  int32_t weight_dtype;  /* dtype of routed and shared expert weights            */
  int32_t accumulate;    /* moe_accumulate of the combine (MOE_ACC_F32 default)  */
  int32_t expert_begin;  /* routed experts computed: [expert_begin, expert_end);  */
  int32_t expert_end;    /* expert_end = 0 means n_experts (all experts)          */
} moe_params;

/* Expert range ("DeepSeek MoE.__init__: experts" and the V3 class: a rank
 * builds only experts [experts_start_idx, experts_end_idx) and its forward
 * loops over that range): the gate and the dispatch always cover all
 * n_experts; moe_expert_ffn computes only the routed experts in the range
 * (rows of other experts are left untouched), and the combine of moe_forward
 * adds only their slots, so y is this range's share of the routed sum plus
 * the shared output.  The routed weight stacks (w1, w3, w2 and their scales)
 * then hold only the experts of the range: expert e is entry e - expert_begin.  A slice of the shared expert (rows of W1/W3 and the
 * matching columns of W2, as a [dim, slice] matrix) is passed as a shared
 * expert of width shared_inter = slice.  moe_combine itself needs the full
 * range (it has no offsets to tell the rows apart). */

/* Expert weights, device pointers.  The router weight is [E, dim] row-major.
 * The expert matrices w1, w3, w2, ws1, ws3, ws2 (logically [out, in], stacked
 * over experts for the routed ones) are stored in the tiled layout that
 * moe_pack_weights writes from the row-major matrix; the shapes below are the
 * logical ones and the byte sizes are unchanged.
 * fp8 scales: one fp32 per 128x128 block, [out/128, in/128] per matrix,
 * row-major, stacked over experts for the routed ones; NULL unless
 * weight_dtype is fp8.  Each scale must be finite (the library reads them
 * only on the device and does not check them); a zero scale encodes an
 * all-zero block whatever its codes.  Each 128-wide K block's partial product
 * is multiplied by its own scale product, so tiny and zero scales stay exact. */
typedef struct moe_weights {
  const void* w_router;   /* [E, dim], router_dtype                             */
  const float* bias;      /* [E] fp32 selection bias, or NULL for none          */
  const void* w1;         /* [E, inter, dim]  (gate branch, goes through silu)  */
  const void* w3;         /* [E, inter, dim]  (linear branch)                   */
  const void* w2;         /* [E, dim, inter]  (down projection)                 */
  const float* w1_scale;  /* [E, inter/128, dim/128]                            */
  const float* w3_scale;  /* [E, inter/128, dim/128]                            */
  const float* w2_scale;  /* [E, dim/128, inter/128]                            */
  const void* ws1;        /* [shared_inter, dim]; all ws* NULL if shared_inter=0 */
  const void* ws3;        /* [shared_inter, dim]                                */
  const void* ws2;        /* [dim, shared_inter]                                */
  const float* ws1_scale; /* [shared_inter/128, dim/128]                        */
  const float* ws3_scale; /* [shared_inter/128, dim/128]                        */
  const float* ws2_scale; /* [dim/128, shared_inter/128]                        */
} moe_weights;

/* Bytes of device workspace that moe_forward (and each step below) needs for
 * T tokens.  Host only; enqueues nothing. */
moe_status moe_workspace_size(const moe_params* p, int64_t T, size_t* bytes);

/* Gate ("Expert scores": formula z = x_ffn W_r, Gate.forward excerpt).
 *   x [T, dim] act_dtype; w_router [E, dim] router_dtype; bias [E] or NULL.
 *   out topk_idx [T, topk] int32: chosen experts in descending s' order, equal
 *       s' broken towards the lower expert id (groups likewise);
 *   out topk_w   [T, topk] fp32: routing weights, same order.
 *   Logits and scores are fp32.  Uses the workspace for the logits. */
moe_status moe_gate(const moe_params* p, int64_t T, const void* x, const void* w_router,
                    const float* bias, int32_t* topk_idx, float* topk_w,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Dispatch ("Weighted expert sum", MoE.forward excerpt: bincount of the
 * indices, then per expert the (token, slot) pairs in row-major order).
 *   topk_idx [T, topk] int32, every id in [0, E) and distinct within a row
 *       (ids outside [0, E) are ignored; a repeated id in a row is placed once
 *       and both slots get its row).
 *   out counts [E]: assignments per expert;
 *   out offsets [E+1]: exclusive prefix sum of counts (offsets[E] = T*topk);
 *   out sorted_token [T*topk]: token of each expert-contiguous row; inside an
 *       expert's segment tokens ascend;
 *   out row_of [T, topk]: row of assignment (t, k) in that order.
 *   Bit-exact and deterministic (no order-dependent atomics). */
moe_status moe_permute(const moe_params* p, int64_t T, const int32_t* topk_idx,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                       int32_t* row_of, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Routed experts (SwiGLU; MoE constructor: Expert(dim, moe_inter_dim) per
 * routed expert).
 *   x [T, dim]; sorted_token and offsets as produced by moe_permute (read on
 *   the device: no host synchronisation on the per-expert counts); w: the
 *   routed weights w1, w3, w2 (and scales) are used.
 *   out expert_out [T*topk, dim] act_dtype: row r = FFN_e(x[sorted_token[r]])
 *       for the expert e whose segment holds r (rows of experts outside the
 *       expert range are left untouched).
 *   SwiGLU pre-activations are fp32; h = silu(a1)*a3 is rounded once (bf16,
 *   fp32, or e4m3 per 1x128 block for fp8 weights, where x is quantised the
 *   same way); outputs are rounded to act_dtype. */
moe_status moe_expert_ffn(const moe_params* p, int64_t T, const void* x,
                          const int32_t* sorted_token, const int32_t* offsets,
                          const moe_weights* w, void* expert_out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Shared expert and combine ("Weighted expert sum": the weighted routed
 * outputs summed in fp32, the shared expert's output added, one cast back at
 * the end; the shared expert is the MoE constructor's MLP(dim,
 * n_shared_experts * moe_inter_dim)).
 *   x [T, dim] act_dtype (the shared expert's input; may be NULL when
 *   shared_inter = 0); expert_out [T*topk, dim] act_dtype; row_of [T, topk];
 *   topk_w [T, topk] fp32; w: the shared weights ws1, ws3, ws2 (and scales)
 *   are used when shared_inter > 0.
 *   out y [T, dim] act_dtype = cast(sum_k topk_w[t,k] * expert_out[row_of[t,k]]
 *       + S_t) with S = FFN_shared(x) rounded to act_dtype (h rounded as in
 *       moe_expert_ffn); the k sum visits the token's experts in ascending id
 *       (ascending row, since rows are expert-contiguous; a token's rows must be
 *       distinct) and adds S last; each product and each sum is rounded to
 *       fp32 (no fused multiply-add); MOE_ACC_LAYER also casts the running sum
 *       to act_dtype after every addition.
 *   With a shared expert and topk <= 8 the sum is formed in the epilogue of
 *   the shared expert's down projection (S never leaves the chip); otherwise
 *   S goes through the workspace to a separate combine kernel.  Same result
 *   either way.  Needs the full expert range. */
moe_status moe_combine(const moe_params* p, int64_t T, const void* x, const void* expert_out,
                       const int32_t* row_of, const float* topk_w, const moe_weights* w,
                       void* y, void* workspace, size_t workspace_bytes, void* stream);

/* fp8 activation quantiser (the block scheme of fp8 experts: each row split
 * into 1x128 blocks; scale = amax / 448, or 1 when the block is all zero;
 * code = e4m3fn(v / scale) with IEEE fp32 division, round to nearest even,
 * saturating to +-448; a zero result is code 0).  moe_expert_ffn applies it
 * to x and to h when weight_dtype is MOE_FP8_E4M3; it is exported so the
 * step can be used and checked on its own.
 *   x [rows, cols] bf16, cols a multiple of 128, rows * cols / 128 <= 2^28 - 16
 *   (MOE_ERR_UNSUPPORTED beyond);
 *   out q [rows, cols] e4m3fn codes; out scales [rows, cols/128] fp32. */
moe_status moe_quant_fp8(const void* x, int64_t rows, int32_t cols, uint8_t* q, float* scales,
                         void* stream);

/* Expert weight layout (a storage format of this library; the pages fix no
 * memory layout).  Rewrites a row-major matrix of `rows` rows of `row_bytes`
 * bytes into 16-row x 64-byte tiles: tile (i/16, j/64) of byte (i, j) is
 * stored at ((i/16) * (row_bytes/64) + j/64) * 1024, and inside the tile the
 * 16-byte piece (i%16, (j%64)/16) is piece number (i%16) + 16*((j%64)/16),
 * byte j%16 within it.  Stacked expert matrices are packed in one call (rows =
 * E * out); any element type, since the rule is on bytes.
 *   src [rows, row_bytes] device bytes; out dst, the same size, distinct from
 *   src.  rows must be a multiple of 16 and row_bytes a positive multiple of
 *   64, else MOE_ERR_INVALID_ARG and nothing is enqueued. */
moe_status moe_pack_weights(const void* src, int64_t rows, int64_t row_bytes, void* dst,
                            void* stream);

/* The whole layer: gate, dispatch, experts, combine, in one call.
 *   x [T, dim]; out y [T, dim] act_dtype.
 *   Optional outputs (NULL to skip): topk_idx [T, topk], topk_w [T, topk],
 *   counts [E]. */
moe_status moe_forward(const moe_params* p, int64_t T, const void* x, const moe_weights* w,
                       void* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and result as moe_forward
 * minus the workspace; the scratch is the library's own device array of
 * MOE_NOALLOC_SCRATCH_BYTES on each GPU (held until the process ends; its
 * address is looked up on the first call on a device).  A shape whose
 * moe_workspace_size() exceeds that returns MOE_ERR_UNSUPPORTED before
 * anything is enqueued (64 MiB covers the DeepSeek-V3 layer shape up to
 * about 350 tokens).  Allocates nothing.  Every call on one GPU uses the same
 * array: calls that may overlap on one GPU (several streams or threads) race
 * and must be ordered by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_params* p, int64_t T, const void* x,
                               const moe_weights* w, void* y, int32_t* topk_idx,
                               float* topk_w, int32_t* counts, void* stream);

/* Kernel timing for benchmarks (not needed to use the layer).
 * moe_profile_start(n) creates n sets of HIP events (host-side objects, no
 * device memory).  While started, each moe_expert_ffn / moe_forward call
 * records an event before and after its up-projection and its
 * down-projection grouped-GEMM launches, on the call's stream, into the next
 * set; calls beyond n are not recorded.  moe_profile_stop() waits for the
 * recorded events, returns the number of calls recorded and the summed
 * durations in milliseconds, and destroys the events.  Not for concurrent use
 * from several host threads. */
moe_status moe_profile_start(int32_t max_calls);
moe_status moe_profile_stop(int32_t* calls, float* up_ms, float* down_ms);

/* Measurement helper (not part of the layer): enqueue one kernel that reads
 * every byte of buf once, 16-byte coalesced loads, 8 per lane in flight, 8
 * workgroups of 256 threads per CU.  Timing it gives the HBM read rate this
 * library's kernels can reach on the machine, to set beside the published
 * peak.  buf: device, bytes a positive multiple of 16; sink: one device
 * uint32, written only in a case that does not arise for zero-filled buffers.
 * MOE_ERR_INVALID_ARG on NULL pointers or a bad size, MOE_ERR_HIP if the
 * launch fails. */
moe_status moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Readable name of a status; never NULL. */
const char* moe_status_string(moe_status s);

/* Reason for the last error returned on this thread ("" if none). */
const char* moe_last_error(void);

/* ABI version of this header (bumped on any incompatible change). */
int32_t moe_abi_version(void);

#define MOE_ABI_VERSION 3

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
