// Decode-step preparation in one launch (turboquant.net pseudo-code,
// "integrate into Transformer attention": the step's new key and value are
// quantized into the cache, and its queries rotated and projected for the
// logits over packed keys).
//
// The three jobs are independent and each is small at decode time (one new
// token per head and layer), so run as separate kernels their cost is mostly
// per-launch latency.  Here disjoint workgroups of one grid do them side by
// side: the first nbk workgroups quantize the new keys, the next nbv the new
// values (the d = 128 quantizer of tq_q128.h), the rest prepare the queries
// (tq_prep.h).  Results are bit-identical to tq_quantize_kv twice and
// tq_attn_prepare.
#include "tq_prep.h"
#include "tq_q128.h"

namespace tq {
namespace {

constexpr int kStepDynLds = 16 * 1024;

struct StepArgs {
  Q128Args k, v;
  PrepArgs p;
  uint32_t nbk, nbv;            // workgroups of the key and value quantizations
  uint32_t prep_x, prep_y;      // preparation grid (x, y); z = batch
};

template <int NB, bool BF16, bool MSE>
__global__ void __launch_bounds__(256, 2) step_prep_kernel(StepArgs a) {
  const uint32_t b = blockIdx.x;
  if (b < a.nbk) {
    q128_tiles<NB, BF16, MSE>(a.k, b, a.nbk);
  } else if (b < a.nbk + a.nbv) {
    q128_tiles<NB, BF16, MSE>(a.v, b - a.nbk, a.nbv);
  } else {
    const uint32_t r = b - a.nbk - a.nbv;
    const uint32_t bx = r % a.prep_x, byz = r / a.prep_x;
    prep_block(a.p, (int)bx, (int)(byz % a.prep_y), (int)(byz / a.prep_y));
  }
}

template <int NB, bool BF16, bool MSE>
hipError_t launch_step(const StepArgs& a, unsigned grid, size_t shm, hipStream_t st) {
  auto fn = step_prep_kernel<NB, BF16, MSE>;
  // The preparation's dynamic LDS at d = 128 is 12 KB; with the quantizer's
  // static LDS (up to 77 KB) a block passes 64 KB, so allow 16 KB of dynamic
  // LDS explicitly, once (static + allowed dynamic must stay within 160 KB).
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, kStepDynLds);
  if (attr != hipSuccess) return attr;
  if (shm > (size_t)kStepDynLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), shm, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step_prepare(const tq_ctx* ctx, const void* k_new, const void* v_new,
                                      int32_t x_dtype, int64_t n_tokens, int32_t n_heads,
                                      int64_t x_stride_token, int64_t x_stride_head,
                                      uint32_t* k_planes, uint16_t* k_norms, uint32_t* v_planes,
                                      uint16_t* v_norms, int64_t dst_stride_head,
                                      int64_t dst_token0, const int64_t* slots,
                                      const float* q, int32_t batch,
                                      int32_t n_q_heads, int64_t q_stride_batch,
                                      int32_t n_kv_heads, void* workspace, hipStream_t stream) {
  const bool quant = n_tokens > 0 && n_heads > 0;
  const bool prep = batch > 0;
  if (!quant && !prep) return hipSuccess;
  // One grid needs the d = 128 quantizer and one launch's worth of rows;
  // otherwise the same three jobs run as separate launches.
  if (ctx->d != 128 || (quant && ((int64_t)n_heads * n_tokens > kMaxRows ||
                                   x_stride_token >= ((int64_t)1 << 25)))) {
    hipError_t e = hipSuccess;
    if (quant) {
      e = launch_quantize(ctx, k_new, x_dtype, n_tokens, n_heads, x_stride_token, x_stride_head,
                          k_planes, k_norms, dst_stride_head, dst_token0, slots, stream);
      if (e == hipSuccess)
        e = launch_quantize(ctx, v_new, x_dtype, n_tokens, n_heads, x_stride_token,
                            x_stride_head, v_planes, v_norms, dst_stride_head, dst_token0,
                            slots, stream);
    }
    if (e == hipSuccess && prep)
      e = launch_attn_prepare(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads, workspace,
                              logits_fold(ctx, n_q_heads, n_kv_heads), stream);
    return e;
  }
  const bool bf = x_dtype == TQ_BF16;
  StepArgs a{};
  if (quant) {
    Q128Args base;
    hipError_t e = q128_args(ctx, k_new, n_tokens, x_stride_token, x_stride_head, k_planes,
                             k_norms, dst_stride_head, dst_token0, slots, base);
    if (e != hipSuccess) return e;
    a.k = q128_group(base, 0, n_heads, bf);
    e = q128_args(ctx, v_new, n_tokens, x_stride_token, x_stride_head, v_planes, v_norms,
                  dst_stride_head, dst_token0, slots, base);
    if (e != hipSuccess) return e;
    a.v = q128_group(base, 0, n_heads, bf);
    // a persistent loop over tiles: at most one workgroup per CU per job
    a.nbk = a.nbv = std::min<uint32_t>(a.k.n_tiles, (uint32_t)ctx->n_cu);
  }
  size_t shm = 0;
  unsigned n_prep = 0;
  if (prep) {
    dim3 pg;
    prep_args(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads, workspace, a.p, shm, pg,
              logits_fold(ctx, n_q_heads, n_kv_heads));
    a.prep_x = pg.x;
    a.prep_y = pg.y;
    n_prep = pg.x * pg.y * pg.z;
  }
  const unsigned grid = a.nbk + a.nbv + n_prep;
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: return bf ? launch_step<1, true, true>(a, grid, shm, stream) : launch_step<1, false, true>(a, grid, shm, stream);
      case 2: return bf ? launch_step<2, true, true>(a, grid, shm, stream) : launch_step<2, false, true>(a, grid, shm, stream);
      default: return bf ? launch_step<3, true, true>(a, grid, shm, stream) : launch_step<3, false, true>(a, grid, shm, stream);
    }
  }
  switch (ctx->b) {
    case 2: return bf ? launch_step<2, true, false>(a, grid, shm, stream) : launch_step<2, false, false>(a, grid, shm, stream);
    case 3: return bf ? launch_step<3, true, false>(a, grid, shm, stream) : launch_step<3, false, false>(a, grid, shm, stream);
    default: return bf ? launch_step<4, true, false>(a, grid, shm, stream) : launch_step<4, false, false>(a, grid, shm, stream);
  }
}

}  // namespace tq
