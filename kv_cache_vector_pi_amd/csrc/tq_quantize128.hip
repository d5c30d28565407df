// Quantization for head_dim 128, and 64 as token pairs: the kernels and their
// launchers (the method and the organisation of each kernel are described
// in tq_q128.h and tq_q128s.h).  bf16 input at d = 128 with a token count
// that is a multiple of 32 (and no slot map) runs the pipelined kernel of
// tq_q128s.h; everything else runs q128_tiles.
#include "tq_q128.h"
#include "tq_q128s.h"

namespace tq {
namespace {

template <int NB, bool BF16, bool MSE, int D>
__global__ void __launch_bounds__(256, MSE ? 3 : 2) quantize128_kernel(Q128Args a) {
  q128_tiles<NB, BF16, MSE, D>(a, blockIdx.x, gridDim.x);
}

template <int NB, bool BF16, bool MSE, int D>
hipError_t launch128(const Q128Args& a, int n_cu, hipStream_t st) {
  static int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, quantize128_kernel<NB, BF16, MSE, D>, 256,
                                                     0) != hipSuccess ||
        nb < 1)
      nb = 1;
    return nb;
  }();
  const int64_t grid = std::min<int64_t>((int64_t)a.n_tiles, (int64_t)n_cu * per_cu);
  hipLaunchKernelGGL((quantize128_kernel<NB, BF16, MSE, D>), dim3((unsigned)grid), dim3(256), 0, st,
                     a);
  return hipGetLastError();
}

template <int NB, bool MSE>
__global__ void __launch_bounds__(512, 4) quantize128s_kernel(Q128SArgs a) {
  q128s_body<NB, MSE>(a);
}

template <int NB, bool MSE>
hipError_t launch128s(const Q128SArgs& a, int n_cu, hipStream_t st) {
  const uint32_t grid = std::min<uint32_t>(a.n_blocks, (uint32_t)n_cu * 2);
  hipLaunchKernelGGL((quantize128s_kernel<NB, MSE>), dim3(grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

// bf16 at d = 128, n_tokens a multiple of 32, no slots: the pipelined kernel
hipError_t launch_stream128(const tq_ctx* ctx, const void* x, int64_t n_tokens, int32_t n_heads,
                            int64_t x_stride_token, int64_t x_stride_head, uint32_t* planes,
                            uint16_t* norms, int64_t dst_stride_head, int64_t dst_token0,
                            hipStream_t stream) {
  Q128SArgs a{};
  a.x = (const uint16_t*)x;
  a.x_stride_token = x_stride_token;
  a.x_stride_head = x_stride_head;
  a.n_tokens = (uint32_t)n_tokens;
  a.blk_per_head = (uint32_t)(n_tokens / kSB);
  make_div(a.blk_per_head, a.div_m, a.div_s1, a.div_s2);
  a.n_blocks = (uint32_t)((int64_t)n_heads * (n_tokens / kSB));
  a.planes = planes;
  a.norms = (uint32_t*)norms;
  a.dst_stride_head = dst_stride_head;
  a.dst_token0 = dst_token0;
  a.pib_hi = ctx->t.pib_hi;
  a.pib_mid = ctx->t.pib_mid;
  a.m_hi = ctx->t.m_hi;
  a.m_lo = ctx->t.m_lo;
  const int KH = ctx->K / 2;
  for (int k = 0; k < 4; ++k) {
    a.thr[k] = (k < KH - 1) ? ctx->mid[KH + k] : 0.f;
    a.cpos[k] = (k < KH) ? ctx->cent[KH + k] : 0.f;
  }
  const int n_cu = ctx->n_cu;
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: return launch128s<1, true>(a, n_cu, stream);
      case 2: return launch128s<2, true>(a, n_cu, stream);
      default: return launch128s<3, true>(a, n_cu, stream);
    }
  }
  switch (ctx->b) {
    case 2: return launch128s<2, false>(a, n_cu, stream);
    case 3: return launch128s<3, false>(a, n_cu, stream);
    default: return launch128s<4, false>(a, n_cu, stream);
  }
}

// rows: tokens (D = 128) or token pairs (D = 64) per head
template <int D>
hipError_t launch_rows(const tq_ctx* ctx, const void* x, int32_t x_dtype, int64_t rows,
                       int32_t n_heads, int64_t x_stride_token, int64_t x_stride_head,
                       uint32_t* planes, uint16_t* norms, int64_t dst_stride_head,
                       int64_t dst_token0, const int64_t* slots, hipStream_t stream) {
  Q128Args a;
  const hipError_t ea = q128_args(ctx, x, rows, x_stride_token, x_stride_head, planes, norms,
                                  dst_stride_head, dst_token0, slots, a);
  if (ea != hipSuccess) return ea;
  const bool bf = x_dtype == TQ_BF16;
  // launch over groups of heads with fewer than kMaxRows rows
  const int64_t heads_per_launch = std::max<int64_t>(1, kMaxRows / rows);
  for (int64_t h0 = 0; h0 < n_heads; h0 += heads_per_launch) {
    const int64_t nh = std::min<int64_t>(heads_per_launch, n_heads - h0);
    const Q128Args ah = q128_group(a, h0, nh, bf);
    hipError_t e;
    const int n_cu = ctx->n_cu;
    if (ctx->mse) {
      switch (ctx->b) {
        case 1: e = bf ? launch128<1, true, true, D>(ah, n_cu, stream) : launch128<1, false, true, D>(ah, n_cu, stream); break;
        case 2: e = bf ? launch128<2, true, true, D>(ah, n_cu, stream) : launch128<2, false, true, D>(ah, n_cu, stream); break;
        default: e = bf ? launch128<3, true, true, D>(ah, n_cu, stream) : launch128<3, false, true, D>(ah, n_cu, stream); break;
      }
    } else {
      switch (ctx->b) {
        case 2: e = bf ? launch128<2, true, false, D>(ah, n_cu, stream) : launch128<2, false, false, D>(ah, n_cu, stream); break;
        case 3: e = bf ? launch128<3, true, false, D>(ah, n_cu, stream) : launch128<3, false, false, D>(ah, n_cu, stream); break;
        default: e = bf ? launch128<4, true, false, D>(ah, n_cu, stream) : launch128<4, false, false, D>(ah, n_cu, stream); break;
      }
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_quantize128(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                              int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                              int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                              int64_t dst_stride_head, int64_t dst_token0,
                              const int64_t* slots, hipStream_t stream) {
  if (x_dtype == TQ_BF16 && !slots && n_tokens % kSB == 0 &&
      (int64_t)n_heads * (n_tokens / kSB) < ((int64_t)1 << 32))
    return launch_stream128(ctx, x, n_tokens, n_heads, x_stride_token, x_stride_head, planes,
                            norms, dst_stride_head, dst_token0, stream);
  return launch_rows<128>(ctx, x, x_dtype, n_tokens, n_heads, x_stride_token, x_stride_head,
                          planes, norms, dst_stride_head, dst_token0, slots, stream);
}

bool quantize64_pairs_apply(const tq_ctx* ctx, int64_t n_tokens, int32_t n_heads,
                            int64_t x_stride_token, int64_t dst_stride_head, int64_t dst_token0,
                            const int64_t* slots) {
  // pairs of consecutive tokens of one head (at least one per head), 32-bit
  // row offsets, and 16-byte aligned pair records: a d = 64 record is 8 b
  // bytes, so any index serves for even b and an even one for odd b
  return ctx->d == 64 && !slots && n_tokens >= 2 && x_stride_token < ((int64_t)1 << 24) &&
         (ctx->b % 2 == 0 || (dst_token0 % 2 == 0 && (n_heads == 1 || dst_stride_head % 2 == 0)));
}

hipError_t launch_quantize64_pairs(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                                   int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                                   int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                                   int64_t dst_stride_head, int64_t dst_token0,
                                   hipStream_t stream) {
  // the first 2 floor(n_tokens / 2) tokens of each head; an odd last token is
  // the caller's
  return launch_rows<64>(ctx, x, x_dtype, n_tokens / 2, n_heads, x_stride_token, x_stride_head,
                         planes, norms, dst_stride_head, dst_token0, nullptr, stream);
}

}  // namespace tq
