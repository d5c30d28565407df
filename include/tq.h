/*
 * tq.h -- C ABI of the TurboQuant hot path on AMD Instinct MI355X (gfx950).
 *
 * The library quantizes key/value vectors online and estimates attention
 * logits (and vector-search scores) straight from the packed codes.  Every
 * call returns a tq_status (TQ_OK == 0); nothing throws across the ABI.  On
 * failure tq_last_error() returns a thread-local message for the last failed
 * call made by this thread.
 *
 * Method (sources are web pages on TurboQuant; section names are given so a
 * reader can find the passage):
 *  - turboquant.net, "PolarQuant" section: after a random rotation the
 *    coordinates of a unit vector follow
 *      f_d(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - x^2)^((d-3)/2)
 *    on [-1, 1], so a scalar Lloyd-Max quantizer per coordinate needs no
 *    per-block constants.
 *  - turboquant.net, "pseudo-code implementation steps": Lloyd-Max centroids
 *    precomputed once; Pi = Q factor of a Gaussian d x d matrix, generated
 *    once and reused ("potential challenges" section); quant: rotate, nearest
 *    centroid; dequant: centroids[idx] rotated back; attention estimates inner
 *    products with QJL.
 *  - admirer.cn article on Google Research's TurboQuant: (b-1) bits of scalar
 *    codes plus one QJL sign bit of the residual make b bits per coordinate;
 *    the QJL sign sketch gives unbiased inner products.
 *  - turboquant.net, "potential challenges": the residual norm is kept as one
 *    fp16 scalar per vector.
 *
 * Readings of what the pages leave open (the library and its test oracle
 * share them):
 *  - vectors are normalised first; nu = ||x|| is stored as fp16 next to the
 *    residual norm gamma = ||r|| (fp16, round to nearest even);
 *  - S is a d x d matrix of iid N(0,1) (m = d sketch rows); the QJL scale is
 *    alpha = sqrt(pi/2) / d, which makes the estimate unbiased over S;
 *  - sign(0) = +1; nearest-centroid ties go to the lower index;
 *  - a zero vector stores nu = gamma = 0, the codes of y = 0, all signs +1.
 *
 * Estimator (used by tq_attn_logits, tq_search_topk and, with q = e_j, by
 * tq_dequantize):
 *   est(q, rec) = nu * ( <Pi q, c[idx]> + alpha * gamma * <S q, s> )
 *
 * Packed record layout ("canonical layout", caller-owned device memory):
 *  W = ceil(d/32).  planes: uint32 [n_records][W][b]; for word group w the b
 *  words are: words 0..b-2 = bit p of the code index of coordinates
 *  32w..32w+31 (bit j%32 <-> coordinate j), word b-1 = QJL signs (1 <-> +1).
 *  Bits of coordinates >= d are 0.  norms: uint16 [n_records][2] holding the
 *  fp16 bit patterns of (nu, gamma).  A record is b*d bits + 4 bytes.
 *  The b words of a word group are adjacent (rather than each plane being
 *  contiguous over W words) so that one 16-byte load brings every plane of
 *  32 coordinates at b = 4; the two norms share one 4-byte slot so one load
 *  brings both.  Planes and norms are passed as two pointers, not a struct.
 *
 * Device arrays (seq_start, seq_len, slots) are never read on the host: their
 * contents are not validated, and the caller keeps the logit ranges of
 * different sequences disjoint.  Entry points that need scratch memory
 * (prepared queries, chunk partials, search candidates, blocked-quantize
 * residuals) take a caller workspace sized by the matching *_workspace_bytes
 * call; tq_attn_logits also takes max_seq_len (an upper bound of seq_len)
 * to size its grid without reading seq_len.
 *
 * Device pointers must come from the HIP device the context was created on;
 * `stream` is a hipStream_t (NULL = default stream).  Calls are asynchronous:
 * outputs are valid once the stream has been synchronised.  The context is
 * immutable after creation, so concurrent calls on different streams may share
 * it.  No call on the hot path allocates memory.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(_WIN32)
#define TQ_API
#else
#define TQ_API __attribute__((visibility("default")))
#endif

typedef int32_t tq_status;
#define TQ_OK 0
#define TQ_ERR_INVALID_ARG (-1)   /* bad pointer, size, stride or alignment */
#define TQ_ERR_UNSUPPORTED (-2)   /* d or b outside the supported set */
#define TQ_ERR_NOT_CONVERGED (-3) /* tq_lloyd_max hit max_iter */
#define TQ_ERR_HIP (-4)           /* a HIP runtime call or launch failed */
#define TQ_ERR_ALLOC (-5)         /* device allocation failed (context creation) */

/* Input element types of tq_quantize_kv. */
#define TQ_F32 0
#define TQ_BF16 1

/* Supported shapes on the device: d a multiple of 8 in 8..2048, b in {2, 3, 4}
 * (b-1 code bits + 1 sign bit).  The host set-up calls accept 3 <= d <= 2048. */
#define TQ_MAX_D 2048

/* Human-readable name of a status code (static string, never NULL). */
TQ_API const char* tq_status_string(tq_status s);

/* Message of the last failure on the calling thread ("" if none). */
TQ_API const char* tq_last_error(void);

/* W = ceil(d/32): 32-bit words per bit plane; 0 if d < 1. */
TQ_API int32_t tq_words_per_plane(int32_t d);

/* Words of one packed record: W * b (the record also has 2 fp16 norms). */
TQ_API int32_t tq_record_words(int32_t d, int32_t b);

/* ---- offline set-up (host memory, deterministic, no device needed) ------ */

/* Rotation and sketch (turboquant.net pseudo-code, "generate random rotation
 * matrix"; reuse per "potential challenges"; QJL sketch per the admirer.cn
 * QJL paragraph).  Gaussians come from SplitMix64 (key = output `stream` of
 * state `seed`, value i = output i of state key) and Box-Muller (pair j uses
 * uniforms 2j, 2j+1, giving r cos, r sin); G uses stream 0 and S stream 1,
 * both filled row-major.  pi receives the Q factor of G with column signs
 * fixed so that diag(R) > 0 (computed in double, rounded to fp32); y = pi x.
 * s receives S (m = d rows).
 *   pi, s: host float[d*d], row-major, caller-owned.  Either may be NULL.
 * Errors: TQ_ERR_INVALID_ARG if d < 3 or d > TQ_MAX_D. */
TQ_API tq_status tq_make_rotation(int32_t d, uint64_t seed, float* pi, float* s);

/* Lloyd-Max codebook of f_d with 2^lm_bits levels (turboquant.net
 * pseudo-code, "precompute Lloyd-Max centroids"; admirer.cn: Lloyd-Max solves
 * the continuous 1-D k-means problem).  For the two-stage quantizer use
 * lm_bits = b - 1.  Computed in double: thresholds at midpoints, centroids at
 * the conditional means of f_d (incomplete-beta cell masses, closed-form first
 * moments), until max |delta c| < tol; the result is exactly symmetric
 * (c[k] == -c[K-1-k]).
 *   centroids: host float[1 << lm_bits], ascending, caller-owned.
 *   distortion_out (nullable): d * E[(X - c(X))^2], the per-vector MSE of a
 *   unit vector.  iters_out (nullable): iterations run.
 * Errors: TQ_ERR_INVALID_ARG for d < 3, d > TQ_MAX_D, lm_bits outside 1..4,
 * max_iter < 1, tol <= 0 or centroids == NULL; TQ_ERR_NOT_CONVERGED if
 * max_iter was reached (centroids then hold the last iterate). */
TQ_API tq_status tq_lloyd_max(int32_t d, int32_t lm_bits, int32_t max_iter, double tol,
                              float* centroids, double* distortion_out, int32_t* iters_out);

/* ---- context: device copies of the tables --------------------------------
 * Uploads to the current HIP device: Pi and S (fp32 and hi/lo fp16 splits),
 * M = S Pi^T (formed in double), the centroids, their midpoints and the
 * Walsh expansion of the codebook used by the logit kernel.
 *   pi, s: host float[d*d] (as from tq_make_rotation); centroids: host
 *   float[1 << (b-1)], ascending and exactly symmetric.
 * Errors: TQ_ERR_UNSUPPORTED if d is not a multiple of 8 in 8..TQ_MAX_D or b is
 * outside {2,3,4};
 * TQ_ERR_INVALID_ARG for NULL pointers, non-finite values or a codebook that
 * is not strictly ascending and symmetric; TQ_ERR_ALLOC / TQ_ERR_HIP if the
 * device copies fail (nothing is leaked). */
typedef struct tq_ctx tq_ctx;
TQ_API tq_status tq_ctx_create(int32_t d, int32_t b, const float* pi, const float* s,
                               const float* centroids, tq_ctx** out);
/* Frees the device tables (synchronises the device first).  NULL is a no-op. */
TQ_API tq_status tq_ctx_destroy(tq_ctx* ctx);
TQ_API int32_t tq_ctx_dim(const tq_ctx* ctx);
TQ_API int32_t tq_ctx_bits(const tq_ctx* ctx);

/* MSE-only context (turboquant.net pseudo-code "quant" / "dequant" without
 * the QJL stage; admirer.cn: the first stage alone is the MSE-optimal
 * quantizer, whose inner products are biased): every one of the b bits per
 * coordinate is a code bit, records hold b code planes per 32-coordinate
 * group and no sign plane, and the gamma slot of the norms is stored as 0.
 *   pi: host float[d*d]; centroids: host float[1 << b] (tq_lloyd_max with
 *   lm_bits = b), ascending and exactly symmetric.
 * Every hot-path entry point below takes such a context and then computes
 *   quantize: idx_j = nearest centroid of (Pi x / nu)_j, norms (nu, 0)
 *   dequantize: out = nu Pi^T c[idx]
 *   est(q, k) = nu <Pi q, c[idx]>   (logits, search, attention output and
 *   fused decode use this estimate and these dequantized values)
 * with the same record layout rules (W groups of b words).
 * Errors: TQ_ERR_UNSUPPORTED if d is not a multiple of 8 in 8..TQ_MAX_D or b
 * is outside {1,2,3}; otherwise as tq_ctx_create. */
TQ_API tq_status tq_ctx_create_mse(int32_t d, int32_t b, const float* pi,
                                   const float* centroids, tq_ctx** out);
/* 1 for a context from tq_ctx_create_mse, 0 otherwise (and for NULL). */
TQ_API int32_t tq_ctx_is_mse(const tq_ctx* ctx);

/* ---- hot path -------------------------------------------------------------- */

/* Quantize n_heads * n_tokens vectors (turboquant.net pseudo-code "quant",
 * plus the QJL stage of the admirer.cn two-stage description):
 *   nu = ||x||, y = Pi x / nu, idx_j = nearest centroid, r = x/nu - Pi^T c[idx],
 *   gamma = ||r||, s = sign(S r); codes, signs and fp16 (nu, gamma) packed.
 * x: device, element (h, t, j) at x[h*x_stride_head + t*x_stride_token + j]
 *   (strides in elements; rows contiguous), x_dtype TQ_F32 or TQ_BF16.
 * Output record of (h, t) at index h*dst_stride_head + dst_token0 + t of
 *   planes (uint32 [.][W][b], 16-byte aligned base) and norms (uint16 [.][2]).
 * Errors: TQ_ERR_INVALID_ARG for NULL ctx/pointers with n > 0, negative sizes,
 * strides below d, misaligned planes/x, unknown dtype.  n_tokens == 0 or
 * n_heads == 0 is a no-op.  Inputs with ||x|| > 65504 overflow fp16 and are
 * not supported (not checked on the hot path). */
TQ_API tq_status tq_quantize_kv(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                                int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                                int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                                int64_t dst_stride_head, int64_t dst_token0, void* stream);

/* tq_quantize_kv with a caller workspace, for large head dimensions.  For d
 * above 480 (32-coordinate words >= 16) the quantization runs as two blocked
 * matrix products (Y = Pi x, then Z = M r) over tiles of 256 vectors, the
 * residual r kept in `workspace` between them; the tables are then read once
 * per 256 vectors instead of once per 16.  Arguments, record indexing and
 * results as tq_quantize_kv (codes and signs equal up to accumulation-order
 * rounding at decision boundaries, within the parity margins).  Rows are
 * processed in chunks of as many 256-row tiles as the workspace holds.
 * workspace: device memory, 256-byte aligned, at least
 * tq_quantize_workspace_bytes(ctx, 1) bytes (one tile); the bytes for n_rows
 * rows at once (capped at 65536 rows) are tq_quantize_workspace_bytes(ctx,
 * n_rows).  Smaller d: the tq_quantize_kv path, workspace unused (may be
 * NULL).
 * Errors: as tq_quantize_kv; TQ_ERR_INVALID_ARG also for a missing, too small
 * or misaligned workspace when d needs one. */
TQ_API size_t tq_quantize_workspace_bytes(const tq_ctx* ctx, int64_t n_rows);
TQ_API tq_status tq_quantize_kv_ws(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                                   int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                                   int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                                   int64_t dst_stride_head, int64_t dst_token0, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* tq_quantize_kv with a destination per input token (turboquant.net
 * pseudo-code, "integrate into Transformer attention": each step's new keys
 * and values are quantized into the cache), for appends that land at
 * different positions in one call: the new tokens of a batch of sequences
 * (a chunk each, or one token each in decoding), gathered into one input.
 * Record (h, t) goes to index h*dst_stride_head + slots[t] of planes and
 * norms; a token with slots[t] < 0 or slots[t] >= dst_stride_head is skipped
 * (nothing written: padding rows of a batch).  slots: device int64
 * [n_tokens], 8-byte aligned; distinct slots give distinct records (two
 * tokens with one slot race).  Everything else, the results included, as
 * tq_quantize_kv: a token's record is bit-identical to what tq_quantize_kv
 * writes for it.
 * Errors: as tq_quantize_kv; TQ_ERR_INVALID_ARG also for NULL slots with work
 * to do, dst_stride_head < 1 or misaligned slots. */
TQ_API tq_status tq_quantize_kv_slots(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                                      int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                                      int64_t x_stride_head, const int64_t* slots,
                                      uint32_t* planes, uint16_t* norms,
                                      int64_t dst_stride_head, void* stream);

/* Dequantize n records (turboquant.net pseudo-code "dequant", with the QJL
 * term so that <q, out_i> equals est(q, record i) for every q):
 *   out_i = nu * (Pi^T c[idx] + alpha * gamma * S^T s).
 * out: device float, row i at out + i*out_ld (out_ld >= d).
 * Errors: TQ_ERR_INVALID_ARG for NULL pointers with n > 0, n < 0, out_ld < d,
 * misaligned planes.  n == 0 is a no-op. */
TQ_API tq_status tq_dequantize(const tq_ctx* ctx, const uint32_t* planes,
                               const uint16_t* norms, int64_t n, float* out, int64_t out_ld,
                               void* stream);

/* Workspace for tq_attn_logits (prepared queries), in bytes. */
TQ_API size_t tq_attn_logits_workspace_bytes(const tq_ctx* ctx, int32_t batch,
                                             int32_t n_q_heads, int32_t n_kv_heads);

/* Attention logits from packed keys (turboquant.net pseudo-code "integrate
 * into attention": keys stored quantized, inner products estimated with QJL;
 * admirer.cn: 4-bit keys for logits).  Each query is rotated and projected
 * once (Pi q, S q), then every cached key record is streamed:
 *   logits[hq*logits_stride_head + seq_start[bi] + t] =
 *       scale * est(q[bi, hq], key record (hq / G, bi, t)),  G = n_q/n_kv,
 * with the key record of (kv head h, sequence bi, token t) at index
 *   h*keys_stride_head + seq_start[bi] + t.
 * q: device float [batch][n_q_heads][d] with row stride d and batch stride
 *   q_stride_batch (elements).  seq_start (int64) and seq_len (int32): device
 *   arrays [batch]; max_seq_len (host) bounds every seq_len[bi] (the grid is
 *   sized from it; the caller guarantees 0 <= seq_len[bi] <= max_seq_len and
 *   that the addressed records exist).
 * workspace: device memory of at least tq_attn_logits_workspace_bytes(),
 *   16-byte aligned; it may be overwritten.  With d <= 128 and at most 4
 *   query heads per kv head the call is one launch that prepares the query
 *   operands on chip and leaves the workspace untouched (same results as
 *   tq_attn_prepare + tq_attn_logits_prepared, bit for bit); otherwise the
 *   prepared operands go through the workspace.
 * Errors: TQ_ERR_INVALID_ARG for NULL pointers with work to do, batch < 0,
 * n_kv_heads < 1, n_q_heads % n_kv_heads != 0, a too small workspace,
 * misaligned planes/workspace.  batch == 0 or max_seq_len == 0 is a no-op. */
TQ_API tq_status tq_attn_logits(const tq_ctx* ctx, const float* q, int32_t batch,
                                int32_t n_q_heads, int64_t q_stride_batch,
                                const uint32_t* planes, const uint16_t* norms,
                                int32_t n_kv_heads, int64_t keys_stride_head,
                                const int64_t* seq_start, const int32_t* seq_len,
                                int32_t max_seq_len, float scale, float* logits,
                                int64_t logits_stride_head, void* workspace,
                                size_t workspace_bytes, void* stream);

/* tq_attn_logits for callers that cannot allocate or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, launches and results.  Where
 * tq_attn_logits is one launch (d <= 128, at most 4 query heads per kv
 * head) it needs no memory beyond its arguments; otherwise the prepared
 * query operands go to a static device array of TQ_NOALLOC_SCRATCH_BYTES
 * (4 MiB) that the library holds on each GPU until the process ends.
 * Allocates nothing.  On that two-launch path a call whose prepared queries
 * (tq_attn_logits_workspace_bytes of the same sizes) exceed the array
 * returns TQ_ERR_INVALID_ARG; every call on one GPU shares the array, which
 * keeps the last call's contents, so such calls that overlap on one GPU
 * (other streams, other threads) race.  The context must come from
 * tq_ctx_create on the device the call runs on (context creation looks the
 * array up). */
#define TQ_NOALLOC_SCRATCH_BYTES (4u << 20)
TQ_API tq_status tq_attn_logits_noalloc(const tq_ctx* ctx, const float* q, int32_t batch,
                                        int32_t n_q_heads, int64_t q_stride_batch,
                                        const uint32_t* planes, const uint16_t* norms,
                                        int32_t n_kv_heads, int64_t keys_stride_head,
                                        const int64_t* seq_start, const int32_t* seq_len,
                                        int32_t max_seq_len, float scale, float* logits,
                                        int64_t logits_stride_head, void* stream);

/* The two halves of tq_attn_logits, for callers that reuse prepared queries
 * (several caches or chunks scored against the same queries) or time the key
 * stream on its own.  tq_attn_prepare rotates and projects the queries (Pi q,
 * S q) and writes the prepared operands into `workspace` (same size and
 * alignment rules as tq_attn_logits); tq_attn_logits_prepared streams the
 * keys against a workspace prepared with the same ctx, batch, n_q_heads and
 * n_kv_heads.  Arguments and errors as for tq_attn_logits. */
TQ_API tq_status tq_attn_prepare(const tq_ctx* ctx, const float* q, int32_t batch,
                                 int32_t n_q_heads, int64_t q_stride_batch, int32_t n_kv_heads,
                                 void* workspace, size_t workspace_bytes, void* stream);
TQ_API tq_status tq_attn_logits_prepared(const tq_ctx* ctx, const void* workspace,
                                         size_t workspace_bytes, int32_t batch,
                                         int32_t n_q_heads, const uint32_t* planes,
                                         const uint16_t* norms, int32_t n_kv_heads,
                                         int64_t keys_stride_head, const int64_t* seq_start,
                                         const int32_t* seq_len, int32_t max_seq_len,
                                         float scale, float* logits,
                                         int64_t logits_stride_head, void* stream);

/* The start of a decode step (turboquant.net pseudo-code, "integrate into
 * Transformer attention": the new key and value are quantized into the cache
 * and the query is prepared for the logits over packed keys) in one launch:
 * exactly tq_quantize_kv(k_new -> k_planes/k_norms),
 * tq_quantize_kv(v_new -> v_planes/v_norms) and tq_attn_prepare(q ->
 * workspace), with bit-identical results.  K and V share dtype, sizes,
 * strides and the destination indexing (record (h, t) at
 * h*dst_stride_head + dst_token0 + t of each cache, or with dst_slots
 * non-NULL h*dst_stride_head + dst_slots[t] under the rules of
 * tq_quantize_kv_slots, dst_token0 then 0); the preparation
 * arguments are those of tq_attn_prepare.  At d = 128 the three jobs run in
 * one grid (the small per-step jobs then cost one launch instead of three);
 * other d run them as three launches.
 * Errors: as tq_quantize_kv for either K or V, and as tq_attn_prepare;
 * nothing is launched when any check fails.  n_tokens == 0 (or n_heads == 0)
 * skips the quantization, batch == 0 the preparation. */
TQ_API tq_status tq_decode_step_prepare(const tq_ctx* ctx, const void* k_new, const void* v_new,
                                        int32_t x_dtype, int64_t n_tokens, int32_t n_heads,
                                        int64_t x_stride_token, int64_t x_stride_head,
                                        uint32_t* k_planes, uint16_t* k_norms,
                                        uint32_t* v_planes, uint16_t* v_norms,
                                        int64_t dst_stride_head, int64_t dst_token0,
                                        const int64_t* dst_slots,
                                        const float* q, int32_t batch, int32_t n_q_heads,
                                        int64_t q_stride_batch, int32_t n_kv_heads,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for tq_attn_output, in bytes (0 for invalid sizes). */
TQ_API size_t tq_attn_output_workspace_bytes(const tq_ctx* ctx, int32_t batch,
                                             int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t max_seq_len);

/* Attention output from packed values (turboquant.net pseudo-code "integrate
 * into Transformer attention": values are quantized like keys; a query head's
 * output is the weighted sum of the values, here the dequantized values of
 * the pseudo-code "dequant"):
 *   out[bi*out_stride_batch + hq*d + i] =
 *       sum_{t < seq_len[bi]} p[hq*p_stride_head + seq_start[bi] + t]
 *                             * dequant(value record (hq / G, bi, t))_i,
 * computed as Pi^T (sum_t p nu c[idx]) + alpha S^T (sum_t p nu gamma s) (the
 * transforms applied once per head).  The value record of (kv head h,
 * sequence bi, token t) is at h*values_stride_head + seq_start[bi] + t, as for
 * tq_attn_logits; p uses the logits' indexing (e.g. softmax of those logits).
 * p, seq_start, seq_len, out: device memory; max_seq_len bounds every seq_len.
 * workspace: at least tq_attn_output_workspace_bytes(), 16-byte aligned;
 * overwritten.  Errors: TQ_ERR_INVALID_ARG for NULL pointers with work to do,
 * batch < 0, n_kv_heads < 1, n_q_heads % n_kv_heads != 0, a too small
 * workspace, misaligned planes/workspace.  batch == 0 is a no-op; an empty
 * sequence gets a zero output. */
TQ_API tq_status tq_attn_output(const tq_ctx* ctx, const float* p, int64_t p_stride_head,
                                int32_t batch, int32_t n_q_heads, const uint32_t* planes,
                                const uint16_t* norms, int32_t n_kv_heads,
                                int64_t values_stride_head, const int64_t* seq_start,
                                const int32_t* seq_len, int32_t max_seq_len, float* out,
                                int64_t out_stride_batch, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Workspace for tq_attn_decode, in bytes (0 for invalid sizes). */
TQ_API size_t tq_attn_decode_workspace_bytes(const tq_ctx* ctx, int32_t batch,
                                             int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t max_seq_len);

/* Fused decode attention over packed keys and values (turboquant.net
 * pseudo-code "integrate into Transformer attention": keys and values stored
 * quantized, inner products estimated with QJL):
 *   out[bi*out_stride_batch + hq*d + i] =
 *       sum_t softmax_t(scale * est(q[bi, hq], key (hq/G, bi, t)))
 *             * dequant(value (hq/G, bi, t))_i,
 * in one pass over keys and values (chunks of tokens: logits, running
 * softmax statistics and the value sums stay on chip; the chunks are combined
 * with log-sum-exp rescaling).  Key and value records of (kv head h, sequence
 * bi, token t) are both at h*kv_stride_head + seq_start[bi] + t.  Other
 * arguments as for tq_attn_logits and tq_attn_output; an empty sequence gets
 * a zero output.  workspace: at least tq_attn_decode_workspace_bytes(),
 * 16-byte aligned; overwritten.  Errors as for tq_attn_logits. */
TQ_API tq_status tq_attn_decode(const tq_ctx* ctx, const float* q, int32_t batch,
                                int32_t n_q_heads, int64_t q_stride_batch,
                                const uint32_t* k_planes, const uint16_t* k_norms,
                                const uint32_t* v_planes, const uint16_t* v_norms,
                                int32_t n_kv_heads, int64_t kv_stride_head,
                                const int64_t* seq_start, const int32_t* seq_len,
                                int32_t max_seq_len, float scale, float* out,
                                int64_t out_stride_batch, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Workspace for tq_search_topk, in bytes: the prepared query rows (about
 * 8 x d bytes per query) and per-query candidate lists of one chunk of
 * records (8 bytes x 65536 per query, or x 16384 where that would pass 1 GiB). */
TQ_API size_t tq_search_workspace_bytes(const tq_ctx* ctx, int64_t n_queries, int64_t n_db,
                                        int32_t k);

/* Nearest-neighbour search over a quantized database (zingnex.cn digest,
 * nearest-neighbour section; admirer.cn vector-search paragraph: quantize the
 * database with near-zero indexing time, then score from the codes).  For
 * each query a, the k records with the largest est(q_a, record) (scale 1),
 * ordered by (score descending, index ascending); scores of all pairs are
 * never written to memory.
 * queries: device float [n_queries][d]; planes/norms: n_db records.
 * out_idx: device int64 [n_queries][k]; out_score: device float [n_queries][k]
 *   (entries beyond n_db hold index -1 and score -inf).
 * workspace: device memory of at least tq_search_workspace_bytes(),
 *   16-byte aligned; it is overwritten.
 * Errors: TQ_ERR_INVALID_ARG for NULL pointers with work to do, negative
 * sizes, k outside 1..64, a too small workspace, misaligned pointers.
 * n_queries == 0 is a no-op. */
TQ_API tq_status tq_search_topk(const tq_ctx* ctx, const float* queries, int64_t n_queries,
                                const uint32_t* planes, const uint16_t* norms, int64_t n_db,
                                int32_t k, int64_t* out_idx, float* out_score,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---- fractional bit widths: two instances over a channel split ------------
 *
 * The pages quote quality at 2.5 and 3.5 bits per channel (zingnex.cn digest,
 * section on theoretical guarantees and experiments; turboquant.net, KV cache
 * compression benchmark table; admirer.cn article, LongBench paragraph) but do
 * not say how a fractional width is formed.  Reading implemented here: the d
 * channels of a key/value/query are split in two contiguous groups, channels
 * [0, d_hi) quantized by instance `hi` (its own d = d_hi, b = b_hi, rotation,
 * projection and codebook) and channels [d_hi, d_hi + d_lo) by instance `lo`;
 * a record pair costs d_hi b_hi + d_lo b_lo code bits (64 channels at 3 bits
 * + 64 at 2 = 2.5 bits per channel at d = 128; 4 + 3 = 3.5).  Which channels
 * get the wider code is the caller's choice: order them first (a fixed
 * channel permutation can be folded into the projection weights, since inner
 * products are invariant under a common permutation).
 *   estimate(q, k) = est_hi(q[0:d_hi], k_hi) + est_lo(q[d_hi:], k_lo)
 * (each instance's own estimator, so the sum is unbiased when both are
 * two-stage); dequantized vectors are the concatenation of the two parts.
 * Each group's records follow the layout and indexing of its own instance
 * (two record arrays, same (head, token) indexing).  hi and lo must be both
 * two-stage or both MSE-only and on one device; any of b_hi >= b_lo or
 * b_hi < b_lo is allowed.  Errors as the single-instance calls, plus
 * TQ_ERR_INVALID_ARG for a NULL or mismatched instance. */

/* tq_quantize_kv of x[..][0:d_hi] into (hi_planes, hi_norms) and of
 * x[..][d_hi:d_hi+d_lo] into (lo_planes, lo_norms); x rows hold d_hi + d_lo
 * elements (x_stride_token >= d_hi + d_lo; d_hi a multiple of 8 keeps the
 * second group 16-byte aligned). */
TQ_API tq_status tq_split_quantize_kv(const tq_ctx* hi, const tq_ctx* lo, const void* x,
                                      int32_t x_dtype, int64_t n_tokens, int32_t n_heads,
                                      int64_t x_stride_token, int64_t x_stride_head,
                                      uint32_t* hi_planes, uint16_t* hi_norms,
                                      uint32_t* lo_planes, uint16_t* lo_norms,
                                      int64_t dst_stride_head, int64_t dst_token0, void* stream);
/* out[i][0:d_hi] and out[i][d_hi:d_hi+d_lo] = the two groups' reconstructions
 * of record pair i (out_ld >= d_hi + d_lo). */
TQ_API tq_status tq_split_dequantize(const tq_ctx* hi, const tq_ctx* lo,
                                     const uint32_t* hi_planes, const uint16_t* hi_norms,
                                     const uint32_t* lo_planes, const uint16_t* lo_norms,
                                     int64_t n, float* out, int64_t out_ld, void* stream);
/* Workspace for tq_split_attn_logits in bytes (0 for invalid sizes). */
TQ_API size_t tq_split_attn_logits_workspace_bytes(const tq_ctx* hi, const tq_ctx* lo,
                                                   int32_t batch, int32_t n_q_heads,
                                                   int32_t n_kv_heads);
/* tq_attn_logits over split records: logit = scale * (est_hi + est_lo), with
 * q [batch][n_q_heads][d_hi + d_lo] (batch stride q_stride_batch), both record
 * arrays indexed as keys_stride_head / seq_start / seq_len say.  One
 * preparation launch and one key-stream launch that reads both record arrays.
 * Errors: as tq_attn_logits; TQ_ERR_UNSUPPORTED unless d_hi, d_lo <= 128 and
 * n_q_heads / n_kv_heads <= 4. */
TQ_API tq_status tq_split_attn_logits(const tq_ctx* hi, const tq_ctx* lo, const float* q,
                                      int32_t batch, int32_t n_q_heads, int64_t q_stride_batch,
                                      const uint32_t* hi_planes, const uint16_t* hi_norms,
                                      const uint32_t* lo_planes, const uint16_t* lo_norms,
                                      int32_t n_kv_heads, int64_t keys_stride_head,
                                      const int64_t* seq_start, const int32_t* seq_len,
                                      int32_t max_seq_len, float scale, float* logits,
                                      int64_t logits_stride_head, void* workspace,
                                      size_t workspace_bytes, void* stream);
/* The two halves of tq_split_attn_logits (as tq_attn_prepare and
 * tq_attn_logits_prepared): prepare the queries against both instances into
 * `workspace`, then stream both record arrays against it (same hi, lo,
 * batch, n_q_heads and n_kv_heads).  Arguments and errors as for
 * tq_split_attn_logits. */
TQ_API tq_status tq_split_attn_prepare(const tq_ctx* hi, const tq_ctx* lo, const float* q,
                                       int32_t batch, int32_t n_q_heads, int64_t q_stride_batch,
                                       int32_t n_kv_heads, void* workspace,
                                       size_t workspace_bytes, void* stream);
TQ_API tq_status tq_split_attn_logits_prepared(
    const tq_ctx* hi, const tq_ctx* lo, const void* workspace, size_t workspace_bytes,
    int32_t batch, int32_t n_q_heads, const uint32_t* hi_planes, const uint16_t* hi_norms,
    const uint32_t* lo_planes, const uint16_t* lo_norms, int32_t n_kv_heads,
    int64_t keys_stride_head, const int64_t* seq_start, const int32_t* seq_len,
    int32_t max_seq_len, float scale, float* logits, int64_t logits_stride_head, void* stream);
/* Workspace for tq_split_attn_output in bytes (0 for invalid sizes). */
TQ_API size_t tq_split_attn_output_workspace_bytes(const tq_ctx* hi, const tq_ctx* lo,
                                                   int32_t batch, int32_t n_q_heads,
                                                   int32_t n_kv_heads, int32_t max_seq_len);
/* tq_attn_output over split value records: out[bi][h][0:d_hi] from the hi
 * records and out[bi][h][d_hi:] from the lo records, weights p as for
 * tq_attn_output (out row of a head: d_hi + d_lo floats; out_stride_batch >=
 * n_q_heads (d_hi + d_lo) when batch > 1).  Errors: as tq_attn_output. */
TQ_API tq_status tq_split_attn_output(const tq_ctx* hi, const tq_ctx* lo, const float* p,
                                      int64_t p_stride_head, int32_t batch, int32_t n_q_heads,
                                      const uint32_t* hi_planes, const uint16_t* hi_norms,
                                      const uint32_t* lo_planes, const uint16_t* lo_norms,
                                      int32_t n_kv_heads, int64_t values_stride_head,
                                      const int64_t* seq_start, const int32_t* seq_len,
                                      int32_t max_seq_len, float* out, int64_t out_stride_batch,
                                      void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
