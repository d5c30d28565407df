// Attention output from packed values (turboquant.net pseudo-code
// "integrate into Transformer attention": V is quantized like K; the output
// of a query head is the attention-weighted sum of the values, here of the
// dequantized values of the pseudo-code "dequant").
//
// With v~_t = nu_t (Pi^T c[idx_t] + alpha gamma_t S^T s_t) the output
//   o = sum_t p_t v~_t = Pi^T a_rot + alpha S^T a_sk,
//   a_rot = sum_t (p_t nu_t) c[idx_t],   a_sk = sum_t (p_t nu_t gamma_t) s_t,
// so the token stream accumulates in rotated / sketch space and the two
// d x d transforms run once per query head at the end.
//
//  1. vout_accum_kernel: workgroup = (chunk of 1024 tokens, kv head and
//     block of 4 query heads, sequence), in 4 steps of 256 tokens: the
//     step's weights p nu and p nu gamma are staged in LDS, and
//     dev::vacc_mfma sums the packed bits against them on the int8 matrix
//     cores (tokens as the contraction) into the chunk's partial sums in the
//     workspace.
//  2. vout_final_kernel: workgroup = (query head, sequence): sum the chunk
//     partials, then o_i = sum_j Pi[j][i] a_rot[j] + alpha sum_j S[j][i] a_sk[j].
// MSE-only records (no QJL stage) have no sketch part: a_sk = 0, and the S^T
// product is skipped.
#include <algorithm>
#include <cmath>

#include "tq_dev.h"
#include "tq_vacc.h"
#include "tq_internal.h"

namespace tq {
namespace {

struct VAccArgs {
  const float* p;           // weights, p[hq * p_stride_head + seq_start[bi] + t]
  int64_t p_stride_head;
  const uint32_t* planes;
  const uint32_t* norms;
  int64_t values_stride_head;
  const int64_t* seq_start;
  const int32_t* seq_len;
  float* part;              // [batch][n_kv][n_rb][n_chunk][2][4][Dp]
  int d, W, Dp, G, n_kv, n_rb, n_chunk;
  dev::VaccCoef cf;
};

inline int n_rb_of(int G) { return (G + 3) / 4; }

constexpr int kSub = 1;                          // 256-token steps per chunk
constexpr int kChunk = dev::kVChunk * kSub;      // tokens per chunk (one partial)

template <int NB, bool MSE>
__global__ void __launch_bounds__(256) vout_accum_kernel(VAccArgs a) {
  __shared__ __align__(16) char lds[dev::vacc_lds_bytes(NB)];
  __shared__ __align__(16) float wts[dev::kVChunk * 8];   // p nu (4 heads), p nu gamma (4)
  const int tid = threadIdx.x;
  const int chunk_i = blockIdx.x;
  const int h = blockIdx.y / a.n_rb, rb = blockIdx.y % a.n_rb;
  const int bi = blockIdx.z;
  const int len = a.seq_len[bi];
  const int64_t start = a.seq_start[bi];
  const int RW = a.W * NB;                       // words per record
  float* dst = a.part +
      ((((int64_t)bi * a.n_kv + h) * a.n_rb + rb) * a.n_chunk + chunk_i) * 8 * (int64_t)a.Dp;

  for (int step = 0; step < kSub; ++step) {
    const int t0 = chunk_i * kChunk + step * dev::kVChunk;
    const int nt = max(0, min(dev::kVChunk, len - t0));
    if (step > 0 && nt == 0) break;              // uniform; step 0 always writes the partial
    if (step > 0) __syncthreads();               // the previous step is done with wts and lds
    // ---- stage the step's weights (thread t: token t), with the first slice
    //      of the records loaded behind them --------------------------------------
    const int64_t rec0 = (int64_t)h * a.values_stride_head + start + t0;
    static_assert(dev::kVChunk == 256, "one token per thread");
    const int t = tid;
    uint32_t nr = 0u;
    float pw[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < nt) {
      nr = a.norms[rec0 + t];
#pragma unroll
      for (int hh = 0; hh < 4; ++hh)
        if (4 * rb + hh < a.G)
          pw[hh] = a.p[(int64_t)(h * a.G + 4 * rb + hh) * a.p_stride_head + start + t0 + t];
    }
    dev::VaccSlice<NB> first;
    dev::vacc_load_slice<NB>(a.planes + rec0 * RW, nt, a.W, 0, first);
    {
      const float nu = __half2float(__ushort_as_half((unsigned short)(nr & 0xffffu)));
      const float ga = __half2float(__ushort_as_half((unsigned short)(nr >> 16)));
      float4 w1, w2;
      w1.x = pw[0] * nu; w1.y = pw[1] * nu; w1.z = pw[2] * nu; w1.w = pw[3] * nu;
      w2.x = w1.x * ga; w2.y = w1.y * ga; w2.z = w1.z * ga; w2.w = w1.w * ga;
      *(float4*)&wts[8 * t] = w1;
      *(float4*)&wts[8 * t + 4] = w2;
    }
    __syncthreads();
    // ---- accumulate into the chunk's partial sums ----------------------------------
    dev::vacc_mfma<NB, MSE>(a.planes + rec0 * RW, nt, a.W, wts, a.cf, lds, dst, a.Dp, first,
                            step > 0);
  }
}

struct VFinArgs {
  const float* part;
  const float* pi32;        // [d][d] row-major
  const float* s32;
  float* out;               // out[bi * out_stride_batch + hq * out_stride_head + i]
  int64_t out_stride_batch, out_stride_head;
  int d, Dp, G, n_kv, n_rb, n_chunk;
  int qjl;                  // 0: MSE-only records, no sketch part
  float alpha;
};

__global__ void __launch_bounds__(256) vout_final_kernel(VFinArgs a) {
  extern __shared__ float fsm[];
  float* arot = fsm;               // [Dp]
  float* ask = fsm + a.Dp;         // [Dp]
  __shared__ __align__(16) float red[2048];
  const int hq = blockIdx.x, bi = blockIdx.y;
  const int h = hq / a.G, g = hq % a.G, rb = g / 4, hh = g % 4;
  const float* src = a.part + (((int64_t)bi * a.n_kv + h) * a.n_rb + rb) * a.n_chunk * 8 * (int64_t)a.Dp;
  dev::sum_chunk_partials(src, a.n_chunk, hh, 4 + hh, a.Dp, nullptr, 1.f, red, arot, ask);
  dev::apply_transforms(a.pi32, a.s32, a.d, a.qjl != 0, a.alpha, arot, ask, red,
                        a.out + (int64_t)bi * a.out_stride_batch + (int64_t)hq * a.out_stride_head);
}

}  // namespace

size_t vout_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t max_seq_len) {
  const int G = n_q_heads / n_kv_heads;
  const int ch = kChunk;
  const int64_t n_chunk = std::max<int64_t>(1, ((int64_t)max_seq_len + ch - 1) / ch);
  return (size_t)batch * n_kv_heads * n_rb_of(G) * n_chunk * 8 * ctx->Dp * sizeof(float);
}

hipError_t launch_attn_output(const tq_ctx* ctx, const float* p, int64_t p_stride_head,
                              int32_t batch, int32_t n_q_heads, const uint32_t* planes,
                              const uint16_t* norms, int32_t n_kv_heads,
                              int64_t values_stride_head, const int64_t* seq_start,
                              const int32_t* seq_len, int32_t max_seq_len, float* out,
                              int64_t out_stride_batch, int64_t out_stride_head, void* workspace,
                              hipStream_t stream) {
  const int G = n_q_heads / n_kv_heads;
  VAccArgs a{};
  a.p = p;
  a.p_stride_head = p_stride_head;
  a.planes = planes;
  a.norms = (const uint32_t*)norms;
  a.values_stride_head = values_stride_head;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.part = (float*)workspace;
  a.d = ctx->d;
  a.W = ctx->W;
  a.Dp = ctx->Dp;
  a.G = G;
  a.n_kv = n_kv_heads;
  a.n_rb = n_rb_of(G);
  a.n_chunk = std::max(1, (max_seq_len + kChunk - 1) / kChunk);
  if (!dev::make_vacc_coef(ctx->mono_mask, ctx->mono_w, ctx->n_mono, ctx->c0, ctx->cp, a.cf))
    return hipErrorInvalidValue;
  const size_t shm = 0;
  const dim3 grid(a.n_chunk, n_kv_heads * a.n_rb, batch);
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: hipLaunchKernelGGL((vout_accum_kernel<1, true>), grid, dim3(256), shm, stream, a); break;
      case 2: hipLaunchKernelGGL((vout_accum_kernel<2, true>), grid, dim3(256), shm, stream, a); break;
      default: hipLaunchKernelGGL((vout_accum_kernel<3, true>), grid, dim3(256), shm, stream, a); break;
    }
  } else {
    switch (ctx->b) {
      case 2: hipLaunchKernelGGL((vout_accum_kernel<2, false>), grid, dim3(256), shm, stream, a); break;
      case 3: hipLaunchKernelGGL((vout_accum_kernel<3, false>), grid, dim3(256), shm, stream, a); break;
      default: hipLaunchKernelGGL((vout_accum_kernel<4, false>), grid, dim3(256), shm, stream, a); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  VFinArgs f{};
  f.part = a.part;
  f.pi32 = ctx->t.pi32;
  f.s32 = ctx->t.s32;
  f.out = out;
  f.out_stride_batch = out_stride_batch;
  f.out_stride_head = out_stride_head;
  f.d = ctx->d;
  f.Dp = ctx->Dp;
  f.G = G;
  f.n_kv = n_kv_heads;
  f.n_rb = a.n_rb;
  f.n_chunk = a.n_chunk;
  f.qjl = ctx->mse ? 0 : 1;
  f.alpha = (float)(std::sqrt(M_PI / 2.0) / ctx->d);
  hipLaunchKernelGGL(vout_final_kernel, dim3(n_q_heads, batch), dim3(256),
                     2 * ctx->Dp * sizeof(float), stream, f);
  return hipGetLastError();
}

}  // namespace tq
