// Internal declarations shared by the host code and the HIP kernels of libtq.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstddef>
#include <cstdint>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxK = 8;         // centroids for b <= 4
constexpr int kMaxVec = 5;       // odd Walsh monomials (b = 4) + QJL signs

// Device tables of a context.  All matrices are zero-padded to Dp = 32*W rows
// and columns so that kernels never branch on the ragged edge of d.
struct DevTables {
  const __half* pi_hi;   // [Dp][Dp] row-major, fp16 hi part of Pi
  const __half* pi_lo;   // [Dp][Dp] fp16 of (Pi - pi_hi)
  const __half* m_hi;    // [Dp][Dp] M = S Pi^T (formed in double), hi part
  const __half* m_lo;    // [Dp][Dp] lo part
  const uint16_t* pib_hi;   // [Dp][Dp] bf16 bits of Pi (round to nearest even)
  const uint16_t* pib_mid;  // [Dp][Dp] bf16 bits of Pi - pib_hi
  const __half* pit_hi;  // [Rp][Dp] Pi^T hi/lo (rows padded to a multiple of 64)
  const __half* pit_lo;
  const __half* st_hi;   // [Rp][Dp] S^T hi/lo
  const __half* st_lo;
  const float* pit32;    // [d][d] Pi^T (column r of Pi is contiguous: pit32[j*d + r] = Pi[r][j])
  const float* st32;     // [d][d] S^T
  const float* pi32;     // [d][d] Pi, row-major
  const float* s32;      // [d][d] S, row-major
};

}  // namespace tq

struct tq_ctx {
  int32_t d, b, W, Dp, K;
  int32_t mse;                // 1: MSE-only records (b code planes, no QJL stage)
  int32_t cp;                 // code planes per group: b - 1, or b in MSE mode
  int device;
  float cent[tq::kMaxK];      // centroids (ascending)
  float mid[tq::kMaxK];       // midpoints t_k = (c_k + c_{k+1}) / 2, k < K-1
  // Walsh expansion of the codebook over the code bits: c[idx] = c0 - 2 sum_m w_m u_m,
  // u_m = XOR of the code planes in mask_m (odd masks only for a symmetric codebook).
  int32_t n_mono;
  int32_t mono_mask[tq::kMaxVec];
  double mono_w[tq::kMaxVec];
  double c0;
  int n_cu;                   // compute units of the device (grid sizing)
  void* dev_block;            // one allocation holding every device table
  tq::DevTables t;
};

namespace tq {

// Launchers (defined in the .hip files).  They assume validated arguments and
// return hipGetLastError() of the launch.
hipError_t launch_quantize(const tq_ctx* ctx, const void* x, int32_t x_dtype, int64_t n_tokens,
                           int32_t n_heads, int64_t x_stride_token, int64_t x_stride_head,
                           uint32_t* planes, uint16_t* norms, int64_t dst_stride_head,
                           int64_t dst_token0, const int64_t* slots, hipStream_t stream);

// Large head dimensions (Dp >= 512): blocked products with a workspace.
bool quantize_big_applies(const tq_ctx* ctx);
size_t quantize_big_workspace_bytes(const tq_ctx* ctx, int64_t n_rows);
hipError_t launch_quantize_big(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                               int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                               int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                               int64_t dst_stride_head, int64_t dst_token0, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

hipError_t launch_quantize128(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                              int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                              int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                              int64_t dst_stride_head, int64_t dst_token0,
                              const int64_t* slots, hipStream_t stream);

// d = 64 as token pairs through the d = 128 kernel: when it applies (no
// slots, at least one pair per head; for odd b, even first record index and
// head stride), and the launch of the pairs (an odd last token per head is
// left to the caller).
bool quantize64_pairs_apply(const tq_ctx* ctx, int64_t n_tokens, int32_t n_heads,
                            int64_t x_stride_token, int64_t dst_stride_head, int64_t dst_token0,
                            const int64_t* slots);
hipError_t launch_quantize64_pairs(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                                   int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                                   int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                                   int64_t dst_stride_head, int64_t dst_token0,
                                   hipStream_t stream);

hipError_t launch_decode_step_prepare(const tq_ctx* ctx, const void* k_new, const void* v_new,
                                      int32_t x_dtype, int64_t n_tokens, int32_t n_heads,
                                      int64_t x_stride_token, int64_t x_stride_head,
                                      uint32_t* k_planes, uint16_t* k_norms, uint32_t* v_planes,
                                      uint16_t* v_norms, int64_t dst_stride_head,
                                      int64_t dst_token0, const int64_t* slots,
                                      const float* q, int32_t batch,
                                      int32_t n_q_heads, int64_t q_stride_batch,
                                      int32_t n_kv_heads, void* workspace, hipStream_t stream);

size_t attn_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t n_q_heads,
                            int32_t n_kv_heads);
// Device address of the static scratch of tq_attn_logits_noalloc on `device`
// (looked up on the first call for a device, which must then be current;
// context creation makes that call).
hipError_t noalloc_scratch(int device, void** out);
// fold: prepare the folded operand layout that the logit stream uses when
// logits_fold() holds (the fused decode kernel reads the unfolded one)
hipError_t launch_attn_prepare(const tq_ctx* ctx, const float* q, int32_t batch,
                               int32_t n_q_heads, int64_t q_stride_batch, int32_t n_kv_heads,
                               void* workspace, bool fold, hipStream_t stream);
// whether tq_attn_logits' stream reads a folded preparation (d <= 64 on the
// resident kernel)
bool logits_fold(const tq_ctx* ctx, int32_t n_q_heads, int32_t n_kv_heads);
// The whole logit call in one launch (query preparation inside the stream
// kernel, no workspace), where attn_one_applies: the resident stream with
// d <= 128 and at most 4 query heads per kv head.
bool attn_one_applies(const tq_ctx* ctx, int32_t n_q_heads, int32_t n_kv_heads);
hipError_t launch_attn_one(const tq_ctx* ctx, const float* q, int32_t batch, int32_t n_q_heads,
                           int64_t q_stride_batch, const uint32_t* planes, const uint16_t* norms,
                           int32_t n_kv_heads, int64_t keys_stride_head,
                           const int64_t* seq_start, const int32_t* seq_len,
                           int32_t max_seq_len, float scale, float* logits,
                           int64_t logits_stride_head, hipStream_t stream);
hipError_t launch_attn_stream(const tq_ctx* ctx, const void* workspace, int32_t batch,
                              int32_t n_q_heads, const uint32_t* planes, const uint16_t* norms,
                              int32_t n_kv_heads, int64_t keys_stride_head,
                              const int64_t* seq_start, const int32_t* seq_len,
                              int32_t max_seq_len, float scale, float* logits,
                              int64_t logits_stride_head, hipStream_t stream);

size_t search_workspace_bytes(const tq_ctx* ctx, int64_t n_queries, int64_t n_db, int32_t k);
hipError_t launch_search_topk(const tq_ctx* ctx, const float* queries, int64_t n_queries,
                              const uint32_t* planes, const uint16_t* norms, int64_t n_db,
                              int32_t k, int64_t* out_idx, float* out_score, void* workspace,
                              hipStream_t stream);
size_t vout_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t max_seq_len);
hipError_t launch_attn_output(const tq_ctx* ctx, const float* p, int64_t p_stride_head,
                              int32_t batch, int32_t n_q_heads, const uint32_t* planes,
                              const uint16_t* norms, int32_t n_kv_heads,
                              int64_t values_stride_head, const int64_t* seq_start,
                              const int32_t* seq_len, int32_t max_seq_len, float* out,
                              int64_t out_stride_batch, int64_t out_stride_head, void* workspace,
                              hipStream_t stream);
// Channel-split records (two instances c1, c2 over channels [0, d1) and
// [d1, d1 + d2)): logits as one preparation launch and one stream launch.
size_t split_attn_workspace_bytes(const tq_ctx* c1, const tq_ctx* c2, int32_t batch,
                                  int32_t n_q_heads, int32_t n_kv_heads);
bool split_logits_supported(const tq_ctx* c1, const tq_ctx* c2, int32_t n_q_heads,
                            int32_t n_kv_heads);
hipError_t launch_split_prepare(const tq_ctx* c1, const tq_ctx* c2, const float* q,
                                int32_t batch, int32_t n_q_heads, int64_t q_stride_batch,
                                int32_t n_kv_heads, void* workspace, hipStream_t stream);
hipError_t launch_split_stream(const tq_ctx* c1, const tq_ctx* c2, const void* workspace,
                               int32_t batch, int32_t n_q_heads, const uint32_t* planes1,
                               const uint16_t* norms1, const uint32_t* planes2,
                               const uint16_t* norms2, int32_t n_kv_heads,
                               int64_t keys_stride_head, const int64_t* seq_start,
                               const int32_t* seq_len, int32_t max_seq_len, float scale,
                               float* logits, int64_t logits_stride_head, hipStream_t stream);
size_t decode_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t n_q_heads,
                              int32_t n_kv_heads, int32_t max_seq_len);
hipError_t launch_attn_decode(const tq_ctx* ctx, const float* q, int32_t batch, int32_t n_q_heads,
                              int64_t q_stride_batch, const uint32_t* k_planes,
                              const uint16_t* k_norms, const uint32_t* v_planes,
                              const uint16_t* v_norms, int32_t n_kv_heads,
                              int64_t kv_stride_head, const int64_t* seq_start,
                              const int32_t* seq_len, int32_t max_seq_len, float scale,
                              float* out, int64_t out_stride_batch, void* workspace,
                              hipStream_t stream);
hipError_t launch_dequantize(const tq_ctx* ctx, const uint32_t* planes, const uint16_t* norms,
                             int64_t n, float* out, int64_t out_ld, hipStream_t stream);

}  // namespace tq
