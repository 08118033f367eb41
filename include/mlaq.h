/*
 * mlaq.h -- C ABI of libmlaq, the MI355X (gfx950) fused MLA decode query
 * projection and assembly.
 *
 * The operation (sparkinfer PR #75 "[GG] Add BF16 MLA query projection and
 * assembly", sections "What" and "Contract"; vLLM PR #174 "[GG] Fuse MXFP8 and
 * BF16 MLA query assembly", section "What"): for every decode token m < M and
 * local head h < H,
 *
 *   out[m,h,0:512]   = cvt( bf16_rne( sum_k q_nope[m,h,k] * W[h,k,n] ) )   fp32 accumulation
 *   out[m,h,512:576] = cvt( q_pe[m,h,0:64] )                                same launch, no concat
 *
 * where cvt is the identity for BF16 output and x -> e4m3_satfinite(fp32(x) / q_scale)
 * for E4M3 output, and W is either BF16 or MXFP8 (E4M3 payload times an E8M0
 * scale 2^(S-127) shared by 32 contiguous latent columns of one k row; the
 * weight is N-major with its scales along n, per the review thread on api.py
 * of the sparkinfer page). The summation order over k is unspecified, so the
 * BF16 projection is not a bitwise contract (sparkinfer page, "Contract").
 *
 * Sizes: latent (N) = 512 and rope (R) = 64, so each output row holds 576
 * elements; nope (K) = 128, or 192 (the GLM shape of the sparkinfer page,
 * section "What") through mlaq_run_ex. Supported plans: H in {8, 11, 16}
 * local heads and 1 <= M <= 32 tokens (vLLM page, "What" and "Layout and
 * topology behavior"); anything else is MLAQ_ERR_UNSUPPORTED and the caller
 * keeps its staged path (vLLM page, "Safety scope and PR 173").
 *
 * All entry points are thread-safe. No C++ exception crosses the ABI. Every
 * buffer is caller-owned device memory; the library keeps no pointer after a
 * call returns and allocates nothing in mlaq_run.
 */
#ifndef MLAQ_H_
#define MLAQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats. */
#define MLAQ_WEIGHT_BF16 0  /* W_UK_T bf16 [H,128,512], n fastest */
#define MLAQ_WEIGHT_MXFP8 1 /* E4M3FN payload [H,128,512] + E8M0 scales [H,128,16] */

/* Output element types. */
#define MLAQ_OUT_BF16 0 /* bf16 [M,H,576] */
#define MLAQ_OUT_E4M3 1 /* OCP E4M3FN [M,H,576]: value / q_scale, saturating at +-448 */

/* Cache hints of mlaq_run_ex (timing only; results are identical). */
#define MLAQ_CACHE_DEFAULT 0 /* weights may stay cached between calls */
#define MLAQ_CACHE_STREAM 1  /* weights read once per step, cold in HBM */

/* Status codes. */
#define MLAQ_OK 0
#define MLAQ_ERR_UNSUPPORTED 1 /* plan outside the fused path: keep the staged path */
#define MLAQ_ERR_INVALID_ARG 2 /* bad pointer, alignment, scale presence, overlap or enum */
#define MLAQ_ERR_DEVICE 3      /* a HIP call failed (device query or launch) */

#define MLAQ_NOPE_DIM 128     /* K of mlaq_run */
#define MLAQ_NOPE_DIM_GLM 192 /* the other K mlaq_run_ex accepts */
#define MLAQ_LATENT_DIM 512
#define MLAQ_ROPE_DIM 64
#define MLAQ_MAX_M 32
#define MLAQ_V_DIM 128 /* value width of the UV projection */

/*
 * mlaq_plan_supported -- the pure capability gate (no HIP call).
 * Mirrors can_implement(num_heads, max_m, nope_dim, latent_dim, output_dtype,
 * weight_format, device) of the sparkinfer page (review thread on api.py), with
 * the device replaced by its architecture name (e.g. "gfx950:sramecc+:xnack-")
 * and the rope width made explicit. Each weight format has its own gate, so
 * the BF16 plan does not inherit MXFP8-only requirements (same thread).
 * Returns MLAQ_OK when the fused path covers the plan, MLAQ_ERR_UNSUPPORTED
 * when it does not (arch not gfx950, H not in {8,11,16}, max_m outside
 * 1..32, nope_dim not 128 or 192, latent/rope not 512/64), MLAQ_ERR_INVALID_ARG for an unknown
 * enum or a NULL arch. mlaq_last_error() says which.
 */
int mlaq_plan_supported(int num_heads, int max_m, int nope_dim, int latent_dim, int rope_dim,
                        int weight_format, int out_dtype, const char* arch);

/*
 * mlaq_can_implement -- 1 when the fused path covers the plan on HIP device
 * `device` (an ordinal), else 0. Queries the device's architecture once and
 * caches it; enqueues nothing and never synchronizes.
 */
int mlaq_can_implement(int num_heads, int max_m, int nope_dim, int latent_dim, int rope_dim,
                       int weight_format, int out_dtype, int device);

/*
 * mlaq_prewarm -- load the kernels that serve the given token counts
 * (`m_regimes[0..n_regimes)`, each in 1..32, for both nope widths and both
 * cache hints) for H
 * heads on `device`, and
 * cache the device's architecture, so later mlaq_run calls do no first-use
 * work and can be captured into a hipGraph. Deduplicates regimes that share a
 * kernel, allocates nothing that outlives the call, may block. Idempotent.
 * (sparkinfer page, walkthrough: prewarm of weight and M regimes; vLLM page,
 * "Layout and topology behavior": prewarm only the graph-visible M regimes.)
 * Returns MLAQ_OK, MLAQ_ERR_UNSUPPORTED, MLAQ_ERR_INVALID_ARG (NULL regimes
 * with n_regimes > 0, bad enum) or MLAQ_ERR_DEVICE.
 */
int mlaq_prewarm(int num_heads, const int* m_regimes, int n_regimes, int weight_format,
                 int out_dtype, int device);

/*
 * mlaq_run -- enqueue one fused call on `stream` (a hipStream_t passed as
 * void*; NULL is the null stream) of the current HIP device. Asynchronous:
 * no host synchronization, no allocation, capturable into a hipGraph; the
 * kernel reads *q_scale when it runs, so graph replays see new scale values.
 *
 *   q_nope   bf16 [M,H,128], contiguous, 16-byte aligned
 *   q_pe     bf16 [M,H,64], contiguous, 16-byte aligned
 *   w        bf16 [H,128,512] (MLAQ_WEIGHT_BF16) or E4M3FN bytes [H,128,512]
 *            (MLAQ_WEIGHT_MXFP8), n fastest, 16-byte aligned
 *   w_scales E8M0 bytes [H,128,16]: byte [h,k,j] scales columns 32j..32j+31
 *            of row k; required for MXFP8, must be NULL for BF16 weights
 *   q_scale  device fp32[1], 4-byte aligned; required for E4M3 output, must be
 *            NULL for BF16 output (the BF16 output takes no scale). Every
 *            value is accepted: x / q_scale is the IEEE fp32 quotient (so 0,
 *            inf and NaN scales act as IEEE division says), then rounded to
 *            nearest-even E4M3, finite or infinite results past 448 giving
 *            +-448 and NaN giving 0x7F / 0xFF
 *   out      bf16 or E4M3 [M,H,576], contiguous, 16-byte aligned, must not
 *            overlap any input
 *   M        tokens, 0..32 (M = 0 is a no-op that returns MLAQ_OK)
 *   H        heads, 8, 11 or 16
 *
 * MXFP8 weights decode exactly for scale bytes 10..246, where every nonzero
 * decoded weight is a normal bf16 value (2^-126 <= |w| <= 448 * 2^119);
 * NaN payload codes propagate, and scale byte 255 gives NaN. For bytes 0..9
 * and 247..254 each weight is decoded to bf16 first: a weight in the bf16
 * subnormal range is within one subnormal step (2^-133) of its exact value,
 * one past the bf16 range is an infinity of its sign.
 * Results are deterministic: the same inputs give the same bits.
 * Returns MLAQ_OK, or a non-OK status with `out` untouched and nothing
 * enqueued; mlaq_last_error() describes it.
 */
int mlaq_run(const void* q_nope, const void* q_pe, const void* w, const void* w_scales,
             const float* q_scale, void* out, int M, int H, int weight_format, int out_dtype,
             void* stream);

/*
 * Strided / wider form of mlaq_run (same operation). Every tensor's innermost
 * dimension is contiguous; the two outer strides are given in elements, so a
 * head-major q_nope view ([H,M,K] storage, the batch view of the sparkinfer
 * page's "What") and an output inside a wider, pitched workspace (vLLM page,
 * "Layout and topology behavior": direct writes into the attention backend's
 * query workspace; "pitched outputs" in the sparkinfer page's "Validation")
 * need no copy.
 *
 *   q_nope[m,h,k]  at q_nope + m*q_stride_m + h*q_stride_h + k      (bf16)
 *   q_pe[m,h,r]    at q_pe + m*pe_stride_m + h*pe_stride_h + r       (bf16)
 *   out[m,h,c]     at out + m*out_stride_m + h*out_stride_h + c, c < 576
 *   w, w_scales    contiguous [H, nope_dim, 512] and [H, nope_dim, 16]
 *
 * Requirements (else MLAQ_ERR_INVALID_ARG): strides >= 0, below 2^24 and
 * multiples of 8 elements, the head strides of q_nope and q_pe (q_stride_h,
 * pe_stride_h) below 2^16 (a head-major [H,M,K] view needs M*K <= 6144);
 * base pointers 16-byte aligned (q_scale 4-byte); the M*H output
 * rows pairwise disjoint (one outer stride >= 576 and the other >= the first
 * times its extent); the output's address span disjoint from every input's.
 * nope_dim must be 128 or 192 (else MLAQ_ERR_UNSUPPORTED). Everything else is
 * as for mlaq_run.
 *
 * cache_hint tells the kernel how the weight slab will be used next; it
 * changes timing only, never a result bit (else MLAQ_ERR_INVALID_ARG):
 *   MLAQ_CACHE_DEFAULT (0, what mlaq_run uses): ordinary loads and stores, so
 *       a weight set that fits in the caches stays there across calls (the
 *       same layer called back to back);
 *   MLAQ_CACHE_STREAM (1): the weights are read once per decode step and are
 *       cold in HBM when the call starts (a model's layers in turn, as in
 *       serving). BF16 weight rows are then loaded, and a BF16 output stored,
 *       with the nontemporal hint, which shortens a cold call and lengthens a
 *       warm one (an E4M3 output keeps the default store policy, which
 *       measured faster). MXFP8 weights ignore the hint: their 32-byte row segments
 *       share each 128-byte line among four workgroups, and the hint made
 *       those calls slower.
 * A zero-initialised struct gets MLAQ_CACHE_DEFAULT.
 */
typedef struct mlaq_run_args {
  const void* q_nope;
  int64_t q_stride_m, q_stride_h;
  const void* q_pe;
  int64_t pe_stride_m, pe_stride_h;
  const void* w;
  const void* w_scales;
  const float* q_scale;
  void* out;
  int64_t out_stride_m, out_stride_h;
  int M, H, nope_dim, weight_format, out_dtype;
  int cache_hint; /* MLAQ_CACHE_*; occupies what was tail padding, so the size is unchanged */
} mlaq_run_args;

int mlaq_run_ex(const mlaq_run_args* args, void* stream);

/*
 * V up-projection, the step after MLA decode attention (vLLM page, "Layout and
 * topology behavior" and "Safety scope and PR 173", where the UV projection
 * sits beside the fused query path): for every token m < M and head h < H,
 *
 *   out[m,h,v] = bf16_rne( sum_{c<512} x[m,h,c] * W_UV[h,v,c] )   fp32 accumulation, v < 128
 *
 *   x           bf16 [M,H,512] (attention output in the latent space), contiguous
 *   w_uv        bf16 or E4M3FN bytes [H,128,512]: one latent row per value
 *               column (the checkpoint's layout), latent contiguous
 *   w_uv_scales E8M0 [H,128,16]: byte [h,v,j] scales latent 32j..32j+31 of row v;
 *               required for MXFP8, must be NULL for BF16 weights
 *   out         bf16 [M,H,128], contiguous
 * All 16-byte aligned; out must not overlap an input. Sizes: latent 512,
 * value 128, H in {8, 11, 16}, M in 0..32 (0: no-op). Same status codes,
 * asynchrony, graph-capturability and determinism as mlaq_run.
 * mlaq_uv_prewarm loads the kernels of the listed token counts.
 */
int mlaq_uv_plan_supported(int num_heads, int max_m, int latent_dim, int v_dim, int weight_format,
                           const char* arch);
int mlaq_uv_can_implement(int num_heads, int max_m, int latent_dim, int v_dim, int weight_format,
                          int device);
int mlaq_uv_prewarm(int num_heads, const int* m_regimes, int n_regimes, int weight_format, int device);
int mlaq_uv_run(const void* x, const void* w_uv, const void* w_uv_scales, void* out, int M, int H,
                int weight_format, void* stream);
/*
 * mlaq_uv_run with a cache hint (MLAQ_CACHE_*, as for mlaq_run_ex; anything
 * else is MLAQ_ERR_INVALID_ARG). The hint is accepted so that a caller can
 * pass one policy to every projection of a layer, and the UV kernels ignore
 * it: nontemporal W_UV loads measured slower both warm and with every layer
 * of a decode step cold. mlaq_uv_run is this call with MLAQ_CACHE_DEFAULT.
 */
int mlaq_uv_run_ex(const void* x, const void* w_uv, const void* w_uv_scales, void* out, int M, int H,
                   int weight_format, int cache_hint, void* stream);

/*
 * Dense MLA decode attention with split partials, the consumer of the
 * 576-wide query row (b12x PR #441 "Allow FP32 split partials in prepared
 * dense MLA": commit text, walkthrough, "Behavior"). For each decode token m
 * (one sequence with T_m = seq_lens[m] cached tokens) and head h < H:
 *
 *   s_t  = softmax_scale * q[m,h,0:576] . kv_t[0:576]      t < T_m
 *   out[m,h,:] = bf16_rne( sum_t softmax(s)_t kv_t[0:512] )
 *   lse[m,h]   = log sum_t exp(s_t)                         (natural log)
 *
 * Token t of sequence m is row (t mod page_size) of physical page
 * block_table[m * block_table_stride + t / page_size] of the paged cache;
 * a row is 512 latent values then 64 rotary values (bf16), the key is the
 * whole row and the value its latent part, shared by all heads.
 *
 * The tokens are cut into num_splits ranges of ceil(T/S) rounded up to 64
 * tokens; each range stores its normalized output (MLAQ_PARTIAL_BF16, the
 * default, or MLAQ_PARTIAL_FP32, which avoids the intermediate roundings --
 * the softmax weights enter the value product with 16 significant bits
 * instead of 8 -- and doubles the partial bytes) and its lse in fp32 in the caller's workspace,
 * and a merge kernel forms the BF16 output. With num_splits = 1 the single
 * range is written straight to `out` (identical result, no merge launch).
 * T_m = 0 gives out = 0 and lse = -inf.
 *
 *   q             bf16 [M,H,576] at q + m*q_stride_m + h*q_stride_h (elements,
 *                 multiples of 8 below 2^31), rows contiguous, 16-byte aligned
 *   kv_cache      bf16 [num_pages, page_size, 576], contiguous, 16-byte aligned
 *   block_table   int32 [M, block_table_stride], 4-byte aligned
 *   seq_lens      int32 [M], 4-byte aligned
 *   out           bf16 [M,H,512], contiguous, 16-byte aligned
 *   lse           fp32 [M,H] or NULL
 *   workspace     mlaq_attn_workspace_size(M, H, num_splits, partial_dtype)
 *                 bytes, 256-byte aligned (NULL allowed when that size is 0);
 *                 scratch owned by the caller, overwritten by every call
 *
 * Device-side values are never trusted: seq_lens[m] is clamped into
 * [0, block_table_stride * page_size] and every block-table entry that is
 * read into [0, num_pages); only the entries of blocks below the clamped
 * length are read. Limits (else MLAQ_ERR_UNSUPPORTED): 1 <= H <= 16,
 * 1 <= page_size <= 4096, 1 <= num_splits <= 256, M <= 65536,
 * block_table_stride * page_size <= 2^30 tokens. M = 0 is a
 * no-op. Same status codes, asynchrony, graph-capturability and determinism
 * as mlaq_run; out, lse and workspace must not overlap the inputs or each
 * other. A non-OK status leaves out and lse untouched and enqueues nothing,
 * with one exception: MLAQ_ERR_DEVICE from the merge launch of a call with
 * num_splits > 1, when the split kernel (which writes only the workspace) has
 * already been enqueued.
 */
#define MLAQ_PARTIAL_BF16 0
#define MLAQ_PARTIAL_FP32 1
#define MLAQ_ATTN_ROW 576
#define MLAQ_ATTN_MAX_HEADS 16
#define MLAQ_ATTN_MAX_SPLITS 256
#define MLAQ_ATTN_SPLIT_ALIGN 64

typedef struct mlaq_attn_args {
  const void* q;
  int64_t q_stride_m, q_stride_h;
  const void* kv_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  float softmax_scale;
  int M, H, page_size, num_pages, block_table_stride, num_splits, partial_dtype;
} mlaq_attn_args;

/* Workspace bytes for a plan (0 when num_splits = 1, or for an invalid plan). */
size_t mlaq_attn_workspace_size(int M, int H, int num_splits, int partial_dtype);
/* Split count that fills `device` for M sequences of at most max_seq_len
 * tokens (M * num_splits at most two split workgroups per compute unit,
 * ranges of at least 256 tokens, at most MLAQ_ATTN_MAX_SPLITS, at least 1);
 * written to *num_splits. */
int mlaq_attn_num_splits(int M, int max_seq_len, int device, int* num_splits);
int mlaq_attn_plan_supported(int num_heads, int page_size, int num_splits, int partial_dtype, const char* arch);
int mlaq_attn_can_implement(int num_heads, int page_size, int num_splits, int partial_dtype, int device);
/* Loads the split kernel of a partial dtype, every merge kernel shape it may
 * pair with, and the one-split kernel, and looks up the device address of the
 * scratch array of mlaq_attn_run_noalloc on `device`. */
int mlaq_attn_prewarm(int partial_dtype, int device);
int mlaq_attn_run(const mlaq_attn_args* args, void* stream);

/*
 * Allocation-free form of mlaq_attn_run, for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The same operation, kernels and results as
 * mlaq_attn_run, with the partials and their lse kept in a library-owned
 * device array of MLAQ_ATTN_SCRATCH_BYTES (one per device, created when the
 * library's code object is loaded on it and held until the process ends)
 * instead of a caller workspace:
 *
 *   args->workspace must be NULL and args->workspace_bytes 0
 *   (else MLAQ_ERR_INVALID_ARG); plans whose
 *   mlaq_attn_workspace_size(M, H, num_splits, partial_dtype) exceeds
 *   MLAQ_ATTN_SCRATCH_BYTES are rejected with MLAQ_ERR_UNSUPPORTED (e.g.
 *   32 sequences x 16 heads x 16 splits need 8.4 MB with BF16 partials and
 *   16.8 MB with FP32 ones).
 *
 * No call allocates (no hipMalloc, hipFree or allocating library routine);
 * the array's device address is looked up once per device, in
 * mlaq_attn_prewarm or else in the first call on that device. All calls on
 * one device share its array and it keeps the last call's contents; every
 * call writes each partial before reading it, so nothing needs clearing.
 * Calls that overlap in time on one device (different streams without an
 * ordering between them) race on the array and give undefined results;
 * calls ordered on one stream, or in one graph, are safe. Status codes and
 * the rest of the contract are mlaq_attn_run's.
 */
#define MLAQ_ATTN_SCRATCH_BYTES (32u << 20)
int mlaq_attn_run_noalloc(const mlaq_attn_args* args, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none).
 * The pointer stays valid until the thread's next mlaq_* call. */
const char* mlaq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLAQ_H_ */
