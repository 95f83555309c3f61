/*
 * moe_wq.h -- C ABI of the weight-only-quantized fused MoE layer for MI355X (gfx950).
 *
 * What is computed (the pages' statement of the problem):
 *   experts_int8 page (vllm.model_executor.layers.quantization.experts_int8):
 *     - quantize_in_place_and_get_scales: per-row symmetric int8 weights;
 *     - ExpertsInt8MoEMethod.create_weights: w13 int8 [E, 2I, H] (gate rows
 *       0..I-1, up rows I..2I-1), w2 int8 [E, H, I], w13_scale fp32 [E, 2I],
 *       w2_scale fp32 [E, H];
 *     - ExpertsInt8MoEMethod.apply: select_experts (softmax, top_k,
 *       renormalize) then fused_experts (activation "silu",
 *       use_int8_w8a16, apply_router_weight_on_input=False, inplace=True).
 *   moe_wna16 page (vllm.model_executor.layers.quantization.moe_wna16):
 *     - MoeWNA16Method.create_weights: 4-bit codes packed along K, group
 *       scales [E, N, K/g], zeros packed along N; the weight loader stores the
 *       true zero point (GPTQ zeros get +1).
 *     - MoeWNA16Method.apply: the layer takes precomputed topk_weights and
 *       topk_ids (routing is a separate call).
 *
 * Conventions for every call:
 *   - Pointers named "device" are device memory of the current HIP device;
 *     the caller allocates and owns every buffer.  The library allocates no
 *     device memory and keeps no state apart from a thread-local error text
 *     and the static workspace of moe_w8a16_forward_noalloc (one per device).
 *   - Work is enqueued on `stream` (NULL = the default stream) and never
 *     synchronised; results are ready when the stream reaches them.
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is launched.  No C++ exception crosses this boundary.
 *   - Layouts are row-major with the last index contiguous.
 *   - Return value: MOE_OK (0) or an moe_status code; moe_last_error() gives
 *     the detail of the last failure on the calling thread.
 */
#ifndef MOE_WQ_H_
#define MOE_WQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad dimension, k > E, misaligned size  */
  MOE_ERR_UNSUPPORTED = 2,        /* dtype or size outside what the kernels implement     */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP launch or runtime call failed                  */
};

enum moe_act_dtype { MOE_BF16 = 0, MOE_FP16 = 1 };

/* Text of a status code (static storage). */
const char* moe_status_string(int status);
/* Detail of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------------------
 * a1. Per-output-channel symmetric int8 quantization.
 * experts_int8 page, quantize_in_place_and_get_scales: for every row n of
 * every expert e, s[e,n] = max_k |w[e,n,k]| / 127 (fp32 IEEE divide), then
 * q[e,n,k] = clamp(rint(w[e,n,k] / s[e,n]), -127, 127) with the fp32 IEEE
 * divide and round half to even.  An all-zero row gets s = 0 and q = 0.
 *   w     device fp32 [E, N, K]   (read only)
 *   q     device int8 [E, N, K]   (written)
 *   scale device fp32 [E, N]      (written)
 * For w13 pass N = 2I, K = H (gate rows then up rows); for w2 N = H, K = I.
 * Errors: MOE_ERR_INVALID_ARGUMENT for null pointers or E, N, K < 1.
 * ---------------------------------------------------------------------- */
int moe_quantize_weights_int8(const float* w, int64_t E, int64_t N, int64_t K,
                              int8_t* q, float* scale, hipStream_t stream);

/* ------------------------------------------------------------------------
 * a2. Softmax top-k router.
 * experts_int8 page, ExpertsInt8MoEMethod.apply -> select_experts with
 * scoring_func "softmax", top_k, renormalize.  For each token t: the k ids
 * with the largest logits in descending order (equal logits: lower id
 * first); p = softmax over all E in fp32; topk_w[t,j] = p[id_j], divided by
 * the sum of the k chosen p when renormalize != 0.
 *   logits   device fp32  [T, E]
 *   topk_w   device fp32  [T, k]  (written)
 *   topk_ids device int32 [T, k]  (written)
 * Errors: MOE_ERR_INVALID_ARGUMENT (null pointer with T > 0, E < 1, k < 1,
 * k > E, T < 0); MOE_ERR_UNSUPPORTED if E > 1024.  T = 0 launches nothing.
 * ---------------------------------------------------------------------- */
int moe_route_topk(const float* logits, int64_t T, int64_t E, int64_t k, int renormalize,
                   float* topk_w, int32_t* topk_ids, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Routing options of select_experts (experts_int8 page,
 * ExpertsInt8MoEMethod.apply: use_grouped_topk, topk_group,
 * num_expert_group, scoring_func, e_score_correction_bias; moe_wna16 page,
 * MoeWNA16Method.apply_monolithic: routed_scaling_factor).  The pages show
 * the options, not the procedure; this library computes, per token:
 *   1. scores s_e: softmax over the E logits, or sigmoid of each logit
 *      (computed in fp64);
 *   2. choice keys: the fp32 logit when e_score_correction_bias is NULL (the
 *      same order as the scores), else fp32(s_e) + bias_e added in fp32;
 *   3. num_expert_group = G > 1: E splits into G groups of E/G consecutive
 *      experts; a group's key is its largest choice key; the topk_group
 *      groups with the largest keys (equal keys: lower group) keep their
 *      experts, the others' experts cannot be chosen;
 *   4. the k largest choice keys among the experts left, in descending
 *      order, equal keys by lower id;
 *   5. topk_w = the chosen unbiased s, divided by their sum when
 *      renormalize != 0, times routed_scaling_factor (fp64, rounded to fp32).
 * With the defaults (softmax, no groups, no bias, factor 1) this is
 * moe_route_topk.  A NULL moe_routing pointer means those defaults with
 * renormalize = 1.
 * ---------------------------------------------------------------------- */
enum moe_scoring { MOE_SCORING_SOFTMAX = 0, MOE_SCORING_SIGMOID = 1 };
typedef struct moe_routing {
  int scoring;                          /* MOE_SCORING_SOFTMAX or MOE_SCORING_SIGMOID           */
  int renormalize;                      /* divide the chosen scores by their sum                 */
  int64_t num_expert_group;             /* G: 0 or 1 = no groups; else G <= 64, E % G == 0      */
  int64_t topk_group;                   /* groups kept, 1 <= topk_group <= G (ignored if G < 2)  */
  const float* e_score_correction_bias; /* device fp32 [E] or NULL                               */
  float routed_scaling_factor;          /* multiplies the weights (finite)                       */
} moe_routing;

/* moe_route_select: the routing above.
 *   logits   device fp32  [T, E]
 *   topk_w   device fp32  [T, k]  (written)
 *   topk_ids device int32 [T, k]  (written)
 * Errors: MOE_ERR_INVALID_ARGUMENT (null pointer with T > 0, E < 1, k < 1,
 * k > E, T < 0, unknown scoring, G not dividing E, topk_group outside
 * [1, G], k above topk_group * E / G, non-finite factor);
 * MOE_ERR_UNSUPPORTED if E > 1024 or G > 64.  T = 0 launches nothing. */
int moe_route_select(const float* logits, int64_t T, int64_t E, int64_t k, const moe_routing* routing,
                     float* topk_w, int32_t* topk_ids, hipStream_t stream);

/* ------------------------------------------------------------------------
 * a3. Token -> expert align: histogram, prefix scan, padded-block permutation.
 * The pages call the fused kernel that consumes this grouping without
 * printing it (experts_int8 page, ExpertsInt8MoEMethod.apply).  Definition:
 * with f = t*k + j the flat assignment index and c_e the number of f with
 * topk_ids[f] == e (ids outside [0, E) are dropped), each expert owns
 * ceil(c_e / block_m) blocks of block_m rows, experts in ascending order;
 * inside an expert the f ascend, and the rest of its last block holds the
 * sentinel T*k.  block_expert[b] is the expert of block b.  Rows and blocks
 * past the used ones hold T*k and -1.  *num_padded = block_m * (blocks used).
 *   topk_ids     device int32 [T*k]
 *   sorted_ids   device int32 [moe_align_capacity(T,k,E,block_m)]         (written)
 *   block_expert device int32 [moe_align_capacity(T,k,E,block_m)/block_m] (written)
 *   num_padded   device int32 [1]                                         (written)
 * Errors: MOE_ERR_INVALID_ARGUMENT (null pointer with T*k > 0, E < 1,
 * block_m < 1); MOE_ERR_UNSUPPORTED if E > 1024 or block_m > 1024.
 * T*k = 0 writes *num_padded = 0 only.
 * ---------------------------------------------------------------------- */
int64_t moe_align_capacity(int64_t T, int64_t k, int64_t E, int64_t block_m);
int moe_align_block(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int64_t block_m,
                    int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * a4-a6. The W8A16 layer forward.
 * experts_int8 page, ExpertsInt8MoEMethod.apply -> fused_experts with
 * use_int8_w8a16: for every assignment (t, j) to expert e = topk_ids[t,j]:
 *   h = (w13[e] * w13_scale[e]) x_t              (fp32 accumulation, scale on the accumulator)
 *   a = silu(h[0:I]) * h[I:2I]                   (silu(g) = g / (1 + exp(-g)))
 *   y = (w2[e] * w2_scale[e]) a
 *   out_t = sum_j topk_w[t,j] * y                (fp32, j ascending; cast to the activation type)
 *   x          device bf16/fp16 [T, H] (act_dtype)
 *   w13        device int8 [E, 2I, w13_row_stride]  (row stride in elements, 0 means H)
 *   w13_scale  device fp32 [E, 2I]
 *   w2         device int8 [E, H, w2_row_stride]    (0 means I)
 *   w2_scale   device fp32 [E, H]
 *   topk_w     device fp32 [T, k];  topk_ids device int32 [T, k]
 *   block_m    rows per align block: 0 = moe_w8a16_block_m(...), else 16, 32, 64 or 128
 *              (other multiples of 16 up to 256 use the large-tile path)
 *   out        device bf16/fp16 [T, H]; may be the same buffer as x (inplace=True)
 *   workspace  device, at least moe_w8a16_workspace_bytes(...) bytes, 256-byte aligned
 * Requirements: H and I multiples of 128; row strides multiples of 16 and
 * at least the row length; 1 <= k <= E <= 1024.
 * Errors: MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED (act_dtype, block_m),
 * MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP.  T = 0 launches nothing.
 * ---------------------------------------------------------------------- */
int64_t moe_w8a16_block_m(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k);
size_t moe_w8a16_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                                 int64_t block_m);
int moe_w8a16_forward(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I,
                      int64_t E, int64_t k,
                      const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                      const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                      const float* topk_w, const int32_t* topk_ids, int64_t block_m,
                      void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Options of fused_experts / apply beyond the defaults.
 *   apply_router_weight_on_input (experts_int8 page, ExpertsInt8MoEMethod.apply
 *     -> fused_experts): != 0 scales each assignment's input by its routing
 *     weight instead of the output: out_t = sum_j FFN_e(w[t,j] * x_t), with
 *     w * x rounded to the activation type.
 *   num_shared_experts (moe_wna16 page, MoeWNA16Method.apply: shared_experts,
 *     whose output is added to the routed output): S gated MLPs of the routed
 *     experts' shape stored after the E routed ones in every weight tensor
 *     (tensors of E + S experts), taken by every token with weight 1 (a
 *     shared MLP of intermediate S * I is S such experts).  topk_ids still
 *     index the E routed experts; routed ids outside [0, E) are dropped.
 * A NULL pointer means both off.  The _ex calls below take these options;
 * their workspace is moe_*_workspace_bytes_ex(..., opts).
 * ---------------------------------------------------------------------- */
typedef struct moe_fused_opts {
  int apply_router_weight_on_input;
  int64_t num_shared_experts;
} moe_fused_opts;

size_t moe_w8a16_workspace_bytes_ex(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m,
                                    const moe_fused_opts* opts);
/* moe_w8a16_forward with the options (weights [E + S, ...], topk [T, k] of routed experts). */
int moe_w8a16_forward_ex(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                         const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                         const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                         const float* topk_w, const int32_t* topk_ids, const moe_fused_opts* opts,
                         int64_t block_m, void* out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);
/* moe_w8a16_apply with routing options (moe_route_select) and the options above. */
int moe_w8a16_apply_ex(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                       const float* router_logits, const moe_routing* routing,
                       const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                       const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                       const moe_fused_opts* opts, float* topk_w, int32_t* topk_ids, int64_t block_m,
                       void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * moe_w8a16_forward without allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc) nor provide a workspace.
 * Same arguments and result as moe_w8a16_forward (bit for bit: the same
 * kernels), minus workspace / workspace_bytes: the workspace is a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES bytes (256-byte aligned) that
 * each GPU the library runs on holds until the process ends.  The first call
 * on a device looks its address up (hipGetSymbolAddress) with that device
 * current; no call allocates or frees memory.
 * Every call on one GPU uses that GPU's one array: calls that overlap on the
 * same GPU (two streams, two threads) race and must be serialised by the
 * caller.  Nothing is carried from one call to the next (every region a call
 * reads it first writes), so no clearing is needed between calls.
 * Errors: those of moe_w8a16_forward, and MOE_ERR_WORKSPACE_TOO_SMALL when
 * moe_w8a16_workspace_bytes(T, H, I, E, k, block_m) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB covers the decode-sized batches, e.g.
 * E 8, top-2, H 4096, I 14336 up to T = 64, 33 MiB); nothing is launched then.
 * ---------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int moe_w8a16_forward_noalloc(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I,
                              int64_t E, int64_t k,
                              const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                              const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                              const float* topk_w, const int32_t* topk_ids, int64_t block_m,
                              void* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Routing + forward in one call, from router logits (the moe_wna16 page's
 * MoeWNA16Method.apply_monolithic form: the layer takes router_logits and
 * routes itself).  Same result as moe_route_topk followed by
 * moe_w8a16_forward; for T <= 8 one workgroup routes and aligns, which
 * saves a launch.  topk_w / topk_ids (device fp32 / int32 [T, k]) receive
 * the routing.  Arguments and errors as moe_route_topk + moe_w8a16_forward.
 * ---------------------------------------------------------------------- */
int moe_w8a16_apply(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                    const float* router_logits, int renormalize,
                    const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                    const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                    float* topk_w, int32_t* topk_ids, int64_t block_m, void* out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Stages of the forward, exported so that each kernel can be checked and
 * timed alone.  moe_w8a16_forward is exactly moe_align_block followed by
 * these four calls on the workspace regions.
 *
 * moe_w8a16_gemm1: for every padded row r < *num_padded with
 * f = sorted_ids[r] < T*k, t = f / k, e = block_expert[r / block_m]:
 *   v[r, i] = silu(h_i) * h_{I+i},  h_n = w13_scale[e,n] * sum_c x[t,c] w13[e,n,c]
 * `a` is the intermediate, device memory of moe_w8a16_intermediate_bytes
 * bytes (16-byte aligned; passed as float*), cap = moe_align_capacity.  The
 * 16-bit fixed-point form of v is: int8 hi codes [cap, I], then int8 lo codes
 * [cap, I] (each region rounded up to 256 bytes), then fp32 scales
 * [cap, I/g], with v ~= s[r, i/g] * (256 * hi + lo), s = max |v| over the
 * g-column group / 32639 and |error| <= s/2.  What gemm1 writes:
 *   block_m 16 or 32: the fixed-point form with g = 64, at offset 0;
 *   block_m 256 with H a multiple of 256 and (T+1)*H*2 < 2^32 (the prefill
 *     form): the fixed-point form with g = 128, at offset 0;
 *   otherwise: two bf16 planes [2, cap, I] (hi plane first), hi = rne(v) and
 *     lo = rne(v - hi) (16 significant bits).
 * Padding rows of a block that holds rows get v = 0; 16-row groups made only
 * of padding may be left unwritten (GEMM2 never reads them).
 *
 * moe_w8a16_requant: for block_m in (32, 64] or 128 (a no-op otherwise) turns the
 * planes into the fixed-point form with g = 128, stored right after them (at
 * byte offset round_up(4*cap*I, 256)), for the same rows as gemm1.
 *
 * moe_w8a16_gemm2: for every valid padded row r (f = sorted_ids[r] < T*k),
 * split s < splits, h < H:
 *   y[s, f, h] = w2_scale[e,h] * sum_{i in split s} v[r, i] w2[e,h,i]
 * with v as moe_w8a16_gemm1 and moe_w8a16_requant left it in `a` (the
 * fixed-point form for block_m up to 64, 128 and for the prefill form of
 * block_m = 256; the hi + lo planes otherwise).  The K range [0, I) is cut
 * into `splits` parts of whole 128-wide steps (1 <= splits <= I/128; part z
 * covers steps [z*(I/128)/splits, (z+1)*(I/128)/splits) in integer division;
 * block_m > 64 needs equal parts, so splits must divide I/128, except for
 * the prefill form of block_m = 256).  y is device fp32 [splits, T*k, H];
 * rows of dropped ids are not
 * written.  moe_w8a16_splits gives the split count the forward uses.
 *
 * moe_combine_topk: out[t, h] = sum_j topk_w[t,j] * sum_s y[s, t*k+j, h]
 * over the j with topk_ids in [0, E), in fp32 with j and s ascending, cast
 * to act_dtype (round to nearest even).
 * ---------------------------------------------------------------------- */
int64_t moe_w8a16_splits(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m);
/* Bytes of the intermediate buffer `a` of the stage calls (0 for T <= 0). */
size_t moe_w8a16_intermediate_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m);
int moe_w8a16_gemm1(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E,
                    int64_t k, const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                    const int32_t* sorted_ids, const int32_t* block_expert,
                    const int32_t* num_padded, int64_t block_m, float* a, hipStream_t stream);
int moe_w8a16_requant(float* a, int64_t T, int64_t I, int64_t E, int64_t k, const int32_t* sorted_ids,
                      const int32_t* num_padded, int64_t block_m, hipStream_t stream);
int moe_w8a16_gemm2(const float* a, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                    const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                    const int32_t* sorted_ids, const int32_t* block_expert,
                    const int32_t* num_padded, int64_t block_m, int64_t splits, float* y,
                    hipStream_t stream);
int moe_combine_topk(const float* y, int64_t splits, int64_t T, int64_t k, int64_t H, int64_t E,
                     const float* topk_w, const int32_t* topk_ids, int act_dtype, void* out,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * a7. Group-wise asymmetric 4-bit weights with zero points (W4A16).
 * moe_wna16 page, MoeWNA16Method.create_weights: codes packed 8 per int32
 * along K (code k at bits 4*(k mod 8), byte-identical to the page's uint8
 * packing with the even code in the low nibble), scales fp16 [E, N, K/g],
 * zeros packed 8 per int32 along N (row n at bits 4*(n mod 8)), the zero
 * being the true zero: W[n,k] = (q[n,k] - z[n,k/g]) * s[n,k/g].
 *
 * moe_quantize_weights_w4 (the pages print no 4-bit quantizer; this is the
 * min/max reading): per row n and group of g consecutive K,
 * lo = min(w, 0), hi = max(w, 0), s = fp16((hi - lo) / 15) (s = 1 if that
 * rounds to 0), z = clamp(rint(-lo / s), 0, 15),
 * q = clamp(rint(w / s) + z, 0, 15), all in fp32 with the fp16 s.
 *   w        device fp32 [E, N, K]
 *   qweight  device int32  [E, N, K/8]    (written)
 *   scales   device uint16 [E, N, K/g]    (fp16 bits, written)
 *   qzeros   device int32  [E, N/8, K/g]  (written)
 * Requirements: N % 8 == 0, g % 8 == 0, K % g == 0.
 *
 * moe_w4a16_forward: as moe_w8a16_forward with the weights above
 * (w13: N = 2I, K = H; w2: N = H, K = I).  Requirements: H and I multiples
 * of 128 and of g; g a multiple of 128 (MOE_ERR_UNSUPPORTED otherwise).
 * With fp16 activations the intermediate a is carried in fp16 (hi + lo
 * pair), so it must stay inside the fp16 range like the activations.
 * Workspace: moe_w4a16_workspace_bytes (same regions as the int8 path).
 * ---------------------------------------------------------------------- */
int moe_quantize_weights_w4(const float* w, int64_t E, int64_t N, int64_t K, int64_t group_size,
                            int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                            hipStream_t stream);
size_t moe_w4a16_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                                 int64_t block_m);
int moe_w4a16_forward(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I,
                      int64_t E, int64_t k,
                      const int32_t* w13_qweight, const uint16_t* w13_scales,
                      const int32_t* w13_qzeros,
                      const int32_t* w2_qweight, const uint16_t* w2_scales,
                      const int32_t* w2_qzeros, int64_t group_size,
                      const float* topk_w, const int32_t* topk_ids, int64_t block_m,
                      void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_w4a16_forward with routing from logits (see moe_w8a16_apply). */
int moe_w4a16_apply(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                    const float* router_logits, int renormalize,
                    const int32_t* w13_qweight, const uint16_t* w13_scales, const int32_t* w13_qzeros,
                    const int32_t* w2_qweight, const uint16_t* w2_scales, const int32_t* w2_qzeros,
                    int64_t group_size, float* topk_w, int32_t* topk_ids, int64_t block_m, void* out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t moe_w4a16_workspace_bytes_ex(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m,
                                    const moe_fused_opts* opts);
/* moe_w4a16_forward / moe_w4a16_apply with the options (see moe_fused_opts, moe_routing). */
int moe_w4a16_forward_ex(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                         const int32_t* w13_qweight, const uint16_t* w13_scales, const int32_t* w13_qzeros,
                         const int32_t* w2_qweight, const uint16_t* w2_scales, const int32_t* w2_qzeros,
                         int64_t group_size, const float* topk_w, const int32_t* topk_ids,
                         const moe_fused_opts* opts, int64_t block_m, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
int moe_w4a16_apply_ex(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                       const float* router_logits, const moe_routing* routing,
                       const int32_t* w13_qweight, const uint16_t* w13_scales, const int32_t* w13_qzeros,
                       const int32_t* w2_qweight, const uint16_t* w2_scales, const int32_t* w2_qzeros,
                       int64_t group_size, const moe_fused_opts* opts, float* topk_w, int32_t* topk_ids,
                       int64_t block_m, void* out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * GPTQ / AWQ 4-bit checkpoint import (moe_wna16 page,
 * MoeWNA16Method.get_weight_loader: convert_awq_tensor, convert_gptq_int4_qzeros,
 * moe_wna16_weight_loader; MoeWNA16Method.create_weights: group size halving).
 *
 * moe_wna16_group_size: the group size create_weights settles on: halved
 * (and *repeat doubled) until it divides both H and I.  Returns MOE_OK and
 * writes *group / *repeat, or MOE_ERR_INVALID_ARGUMENT if it would fall
 * below 32 (or on non-positive sizes / null pointers).
 *
 * moe_w4_import: one [N, K] matrix of a checkpoint (one expert's gate, up or
 * down projection; gate and up go to rows [0, I) and [I, 2I) of w13):
 *   format MOE_W4_AWQ:  qweight device int32 [K, N/8], packed along N in
 *                       AWQ's nibble order (column c of each group of eight
 *                       in nibble (0,4,1,5,2,6,3,7)[c]); qzeros device int32
 *                       [ceil(K/group_size), N/8] the same way;
 *   format MOE_W4_GPTQ: qweight device int32 [K/8, N], packed along K
 *                       (code k at bits 4(k mod 8)); qzeros device int32
 *                       [ceil(K/group_size), N/8] holding zero - 1 (the
 *                       loader adds 1 per nibble in uint8 arithmetic, so a
 *                       stored 15 carries into its pair's high nibble);
 *   scales device fp16 [ceil(K/group_size), N] (both formats);
 *   repeat: from moe_wna16_group_size (1 = none).
 * Writes this library's layout with groups of group_size / repeat columns:
 *   out_qweight device int32 [N, K/8], out_scales device fp16 [N, K*repeat/group_size],
 *   out_qzeros device int32 [N/8, K*repeat/group_size];
 * output group j takes input group j / repeat.  Integer work: bit exact.
 * Errors: MOE_ERR_INVALID_ARGUMENT (null pointers, unknown format, N or K
 * not multiples of 8, repeat < 1, group_size not a multiple of repeat, the
 * output group not dividing K).
 * ---------------------------------------------------------------------- */
enum moe_w4_format { MOE_W4_AWQ = 0, MOE_W4_GPTQ = 1 };
int moe_wna16_group_size(int64_t H, int64_t I, int64_t group_size, int64_t* group, int64_t* repeat);
int moe_w4_import(int format, const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                  int64_t N, int64_t K, int64_t group_size, int64_t repeat,
                  int32_t* out_qweight, uint16_t* out_scales, int32_t* out_qzeros, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Weight-only fp8 experts (fp8 page: Fp8MoEMethod.__init__ keeps a
 * weight-only path for GPUs without fp8 arithmetic; create_weights: w13
 * [E, 2I, H] and w2 [E, H, I] in float8_e4m3fn (OCP: 1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, largest finite 448, codes 0x7F/0xFF NaN),
 * w13 scales [E, 2] merged into w13_weight_scale [E], w2_weight_scale [E];
 * process_weights_after_loading).  Activations stay bf16 / fp16:
 *   h = w13_scale[e] * sum_c x[t,c] e4m3(w13[e,n,c]),  a = silu(h_gate) h_up,
 *   y = w2_scale[e] * sum_i a[i] e4m3(w2[e,h,i]),     out_t = sum_j w_j y.
 *
 * moe_quantize_weights_fp8: one scale per [N, K] tensor (scaled_fp8_quant of a
 * 16-bit checkpoint): scale[e] = max |w[e]| / 448 (fp32 IEEE divide), code =
 * e4m3fn(clamp(w / scale, -448, 448)), fp32 divide, round to nearest even,
 * the sign bit kept (so -0 codes 0x80); a zero tensor gets scale 0 and codes 0.
 *   w device fp32 [E, N, K]; q device uint8 [E, N, K]; scale device fp32 [E].
 *   (For w13 pass N = 2I: one scale for the merged gate and up rows.)
 * moe_fp8_merge_w13_scales: an fp8 checkpoint's two w13 shard scales
 * (device fp32 [E, 2]) become one (device fp32 [E], their maximum): each
 * shard is dequantized with its own scale (fp32 code value * scale) and
 * quantized again with the maximum as above; w13 (device uint8 [E, 2I, H]) is
 * rewritten in place.
 * moe_wfp8a16_forward / moe_wfp8a16_apply: the layer, as moe_w8a16_forward_ex /
 * moe_w8a16_apply_ex (routing and fused options may be NULL) with the weights
 * above, w13 [E, 2I, w13_row_stride] and w2 [E, H, w2_row_stride] (row strides
 * in elements, 0 meaning unpadded; rows a multiple of 512 bytes long read
 * faster padded by 256 bytes; w13 and w2 16-byte aligned).  Workspace:
 * moe_wfp8a16_workspace_bytes.  Requirements as moe_w8a16_forward.
 * ---------------------------------------------------------------------- */
int moe_quantize_weights_fp8(const float* w, int64_t E, int64_t N, int64_t K, uint8_t* q, float* scale,
                             hipStream_t stream);
int moe_fp8_merge_w13_scales(uint8_t* w13, const float* w13_shard_scales, int64_t E, int64_t I, int64_t H,
                             float* w13_scale, hipStream_t stream);
size_t moe_wfp8a16_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m,
                                   const moe_fused_opts* opts);
int moe_wfp8a16_forward(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                        const uint8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                        const uint8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                        const float* topk_w, const int32_t* topk_ids, const moe_fused_opts* opts,
                        int64_t block_m, void* out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);
int moe_wfp8a16_apply(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                      const float* router_logits, const moe_routing* routing,
                      const uint8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                      const uint8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                      const moe_fused_opts* opts, float* topk_w, int32_t* topk_ids, int64_t block_m,
                      void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * W8A8: the int8 experts above with int8 activations (fused_moe oracle/int8
 * page, select_int8_moe_backend: default keys kInt8StaticChannelSym for the
 * weights, kInt8DynamicTokenSym for the activations).  Both GEMM inputs are
 * quantized per row (token / assignment) with the weights' rule:
 * s = max|row| / 127, code = clamp(rint(v / s), -127, 127) in fp32 (IEEE
 * divide, half to even; a zero row gets s = 0 and codes 0):
 *   x8, sx = quant(x_t);  h = sx * w13_scale[e,n] * sum_c x8[c] w13[e,n,c] (exact int32)
 *   a = silu(h_gate) * h_up (fp32);  a8, sa = quant(a)
 *   y = sa * w2_scale[e,h] * sum_i a8[i] w2[e,h,i];  out_t = sum_j w_j y.
 * moe_quantize_act_int8: the activation quantizer alone (x device bf16/fp16
 * [T, H], 8-byte aligned, H a multiple of 4; q device int8 [T, H], 4-byte
 * aligned; scale device fp32 [T]).
 * moe_w8a8_forward / moe_w8a8_apply: the layer, with arguments, options and
 * requirements as moe_w8a16_forward_ex / moe_w8a16_apply_ex (the same int8
 * weights and scales).  Workspace: moe_w8a8_workspace_bytes.
 * ---------------------------------------------------------------------- */
int moe_quantize_act_int8(const void* x, int act_dtype, int64_t T, int64_t H, int8_t* q, float* scale,
                          hipStream_t stream);
size_t moe_w8a8_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t block_m,
                                const moe_fused_opts* opts);
int moe_w8a8_forward(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                     const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                     const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                     const float* topk_w, const int32_t* topk_ids, const moe_fused_opts* opts,
                     int64_t block_m, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);
int moe_w8a8_apply(const void* x, int act_dtype, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k,
                   const float* router_logits, const moe_routing* routing,
                   const int8_t* w13, const float* w13_scale, int64_t w13_row_stride,
                   const int8_t* w2, const float* w2_scale, int64_t w2_row_stride,
                   const moe_fused_opts* opts, float* topk_w, int32_t* topk_ids, int64_t block_m,
                   void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_WQ_H_ */
