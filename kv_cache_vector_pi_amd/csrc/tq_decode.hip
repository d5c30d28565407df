// Fused decode attention over a packed KV cache (turboquant.net pseudo-code
// "integrate into Transformer attention": keys and values stored quantized,
// inner products estimated with QJL; showapi.com's single-kernel reading of
// the attention step, used here only for the fusion).
//
//   out[bi, hq] = sum_t softmax_t(scale * est(q[bi, hq], key t)) * dequant(value t)
//
// in one pass over the keys and values, split over chunks of tokens
// (flash-decoding style):
//  1. the queries are prepared once (tq_attn_prepare's int8 operands);
//  2. decode_chunk_kernel, per (chunk, kv head and block of 4 query heads,
//     sequence): the chunk's logits on the int8 MFMAs into LDS, the chunk's
//     softmax statistics (max m, sum l of exp(logit - m)), then the value
//     accumulation of dev::vacc_mfma (int8 MFMAs, tokens as the contraction)
//     with weights exp(logit - m) nu (and times gamma for the sketch part) --
//     partial sums and (m, l) per chunk;
//  3. decode_final_kernel, per (query head, sequence): rescale the chunks by
//     exp(m_c - M), divide by L = sum_c l_c exp(m_c - M), and apply Pi^T and
//     S^T once.
// An empty sequence gets a zero output.  MSE-only records (no QJL stage)
// drop every sketch term: no sign MFMAs, no S^T product.
#include <algorithm>
#include <cmath>

#include "tq_dev.h"
#include "tq_vacc.h"
#include "tq_internal.h"

namespace tq {
namespace {

using dev::v4i;

struct DecArgs {
  const char* ws;               // prepared queries
  const uint32_t* k_planes;
  const uint32_t* k_norms;
  const uint32_t* v_planes;
  const uint32_t* v_norms;
  int64_t kv_stride_head;
  const int64_t* seq_start;
  const int32_t* seq_len;
  float* part;                  // [batch][n_kv][n_rb][n_chunk][8][Dp]
  float* stats;                 // [batch][n_kv][n_rb][n_chunk][4][2]  (m, l)
  int d, W, Dp, G, n_kv, n_rb, n_chunk;
  float scale, alpha;
  int mask[kMaxVec];
  dev::VaccCoef cf;
};

constexpr int kChunk = dev::kVChunk;     // tokens per chunk

__device__ inline float wmax(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wsum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int NB, bool MSE>
__global__ void __launch_bounds__(256) decode_chunk_kernel(DecArgs a) {
  constexpr int CP = MSE ? NB : NB - 1;          // code planes
  constexpr int NV = 1 << (CP - 1);
  constexpr int NC = 2 * NV + (MSE ? 0 : 2);
  constexpr int CH = kChunk;
  __shared__ __align__(16) char lds[dev::vacc_lds_bytes(NB)];
  __shared__ __align__(16) float lg[4 * CH];           // logits, then softmax numerators
  __shared__ __align__(16) float wts[CH * 8];          // p nu (4 heads), p nu gamma (4)
  const int RW = a.W * NB;
  __shared__ float st_m[4], st_l[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int chunk_i = blockIdx.x;
  const int h = blockIdx.y / a.n_rb, rb = blockIdx.y % a.n_rb;
  const int bi = blockIdx.z;
  const int len = a.seq_len[bi];
  const int64_t start = a.seq_start[bi];
  const int t0 = chunk_i * CH;
  const int nt = max(0, min(CH, len - t0));
  const int64_t rec0 = (int64_t)h * a.kv_stride_head + start + t0;

  // the first slice of the value records, loaded while the logits compute
  dev::VaccSlice<NB> first;
  dev::vacc_load_slice<NB>(a.v_planes + rec0 * RW, nt, a.W, 0, first);

  // ---- 1. logits of the chunk (tiles of 16 tokens, one per wave at a time) ----
  const int nws = dev::n_ws(a.W);
  const size_t rbb = dev::rb_bytes(a.W, NC);
  const char* rbase = a.ws + (((size_t)bi * a.n_kv + h) * a.n_rb + rb) * rbb;
  const float4 cst = ((const float4*)(rbase + (size_t)nws * NC * 64 * 16))[g];
  const bool head_ok = 4 * rb + g < a.G;
  // every load of the phase is issued up front: the first word step of the
  // wave's 4 key tiles with their norms, the operands of that word step, and
  // the value norm of token tid (used for the weights)
  constexpr int TPW = CH / dev::kTile / dev::kWaves;   // key tiles per wave
  uint32_t wd0[TPW][NB], nrm0[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tl = dev::kTile * (wave + dev::kWaves * u) + n;
    const bool valid = tl < nt;
#pragma unroll
    for (int p = 0; p < NB; ++p) wd0[u][p] = 0u;
    if (valid && g < a.W) dev::load_group<NB>(a.k_planes + ((rec0 + tl) * a.W + g) * NB, wd0[u]);
    nrm0[u] = valid ? a.k_norms[rec0 + tl] : 0u;
  }
  v4i A0[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) A0[c] = ((const v4i*)rbase)[c * 64 + lane];
  const uint32_t vnr = tid < nt ? a.v_norms[rec0 + tid] : 0u;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tl = dev::kTile * (wave + dev::kWaves * u) + n;   // token within the chunk
    const bool valid = tl < nt;
    const int64_t rec = rec0 + tl;
    const uint32_t nrm = nrm0[u];
    v4i acc_m = {0, 0, 0, 0}, acc_q = {0, 0, 0, 0};
    for (int wsi = 0; wsi < nws; ++wsi) {
      const int w = 4 * wsi + g;
      uint32_t wd[NB];
#pragma unroll
      for (int p = 0; p < NB; ++p) wd[p] = wd0[u][p];
      if (wsi > 0) {
#pragma unroll
        for (int p = 0; p < NB; ++p) wd[p] = 0u;
        if (valid && w < a.W) dev::load_group<NB>(a.k_planes + (rec * a.W + w) * NB, wd);
      }
      const v4i* fr = (const v4i*)(rbase + (size_t)wsi * NC * 64 * 16);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        uint32_t uw = 0u;
#pragma unroll
        for (int p = 0; p < CP; ++p)
          if ((a.mask[v] >> p) & 1) uw ^= wd[p];
#pragma unroll
        for (int half = 0; half < 2; ++half)
          acc_m = __builtin_amdgcn_mfma_i32_16x16x64_i8(wsi == 0 ? A0[2 * v + half]
                                                                 : fr[(2 * v + half) * 64 + lane],
                                                        dev::bit_lanes(uw, half), acc_m, 0, 0, 0);
      }
#pragma unroll
      for (int half = 0; half < (MSE ? 0 : 2); ++half)
        acc_q = __builtin_amdgcn_mfma_i32_16x16x64_i8(wsi == 0 ? A0[2 * NV + half]
                                                               : fr[(2 * NV + half) * 64 + lane],
                                                      dev::bit_lanes(wd[NB - 1], half), acc_q,
                                                      0, 0, 0);
    }
    const float mse = fmaf(dev::limbs_to_float(acc_m), cst.x, cst.z);
    const float qjl = fmaf(dev::limbs_to_float(acc_q), cst.y, cst.w);
    const float nu = __half2float(__ushort_as_half((unsigned short)(nrm & 0xffffu)));
    const float ga = __half2float(__ushort_as_half((unsigned short)(nrm >> 16)));
    const float logit = a.scale * nu * (MSE ? mse : fmaf(a.alpha * ga, qjl, mse));
    lg[g * CH + tl] = (valid && head_ok) ? logit : -INFINITY;
  }
  __syncthreads();

  // ---- 2. softmax statistics of the chunk: wave hh handles query head hh ----
  {
    const int hh = wave;
    float m = -INFINITY;
    for (int t = lane; t < CH; t += 64) m = fmaxf(m, lg[hh * CH + t]);
    m = wmax(m);
    float l = 0.f;
    for (int t = lane; t < CH; t += 64) {
      const float x = lg[hh * CH + t];
      const float p = (m == -INFINITY) ? 0.f : __expf(x - m);
      lg[hh * CH + t] = p;
      l += p;
    }
    l = wsum(l);
    if (lane == 0) {
      st_m[hh] = m;
      st_l[hh] = l;
    }
  }
  __syncthreads();
  // weights of token tid: p nu and p nu gamma of its value record
  static_assert(CH == 256, "one token per thread");
  {
    const float nu = __half2float(__ushort_as_half((unsigned short)(vnr & 0xffffu)));
    const float ga = __half2float(__ushort_as_half((unsigned short)(vnr >> 16)));
    float4 w1, w2;
    w1.x = lg[tid] * nu; w1.y = lg[CH + tid] * nu; w1.z = lg[2 * CH + tid] * nu;
    w1.w = lg[3 * CH + tid] * nu;
    w2.x = w1.x * ga; w2.y = w1.y * ga; w2.z = w1.z * ga; w2.w = w1.w * ga;
    *(float4*)&wts[8 * tid] = w1;
    *(float4*)&wts[8 * tid + 4] = w2;
  }
  __syncthreads();

  // ---- 3. value accumulation and the chunk's partials -------------------------
  const size_t cidx = (((size_t)bi * a.n_kv + h) * a.n_rb + rb) * a.n_chunk + chunk_i;
  float* dst = a.part + cidx * 8 * (size_t)a.Dp;
  if (tid < 4) {
    a.stats[cidx * 8 + 2 * tid] = st_m[tid];
    a.stats[cidx * 8 + 2 * tid + 1] = st_l[tid];
  }
  dev::vacc_mfma<NB, MSE>(a.v_planes + rec0 * RW, nt, a.W, wts, a.cf, lds, dst, a.Dp, first);
}

struct DecFinArgs {
  const float* part;
  const float* stats;
  const float* pi32;
  const float* s32;
  float* out;
  int64_t out_stride_batch;
  int d, Dp, G, n_kv, n_rb, n_chunk;
  int qjl;                      // 0: MSE-only records, no sketch part
  float alpha;
};

__global__ void __launch_bounds__(256) decode_final_kernel(DecFinArgs a) {
  extern __shared__ float fsm[];
  float* arot = fsm;               // [Dp]
  float* ask = fsm + a.Dp;         // [Dp]
  float* fac = fsm + 2 * a.Dp;     // [n_chunk] exp(m_c - M) / L
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hq = blockIdx.x, bi = blockIdx.y;
  const int h = hq / a.G, g = hq % a.G, rb = g / 4, hh = g % 4;
  const size_t c0 = (((size_t)bi * a.n_kv + h) * a.n_rb + rb) * a.n_chunk;
  // M = max over chunks, L = sum l_c exp(m_c - M)
  float m = -INFINITY;
  for (int c = tid; c < a.n_chunk; c += 256) m = fmaxf(m, a.stats[(c0 + c) * 8 + 2 * hh]);
  m = wmax(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float l = 0.f;
  for (int c = tid; c < a.n_chunk; c += 256) {
    const float mc = a.stats[(c0 + c) * 8 + 2 * hh];
    const float f = (mc == -INFINITY) ? 0.f : __expf(mc - M);
    fac[c] = f;
    l += f * a.stats[(c0 + c) * 8 + 2 * hh + 1];
  }
  l = wsum(l);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  const float L = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  __syncthreads();
  __shared__ __align__(16) float red2[2048];
  dev::sum_chunk_partials(a.part + c0 * 8 * (size_t)a.Dp, a.n_chunk, hh, 4 + hh, a.Dp, fac, inv,
                          red2, arot, ask);
  dev::apply_transforms(a.pi32, a.s32, a.d, a.qjl != 0, a.alpha, arot, ask, red2,
                        a.out + (int64_t)bi * a.out_stride_batch + (int64_t)hq * a.d);
}

struct DecLayout {
  size_t prep, part, stats, total;
  int chunk, n_chunk, n_rb;
};

DecLayout dec_layout(const tq_ctx* ctx, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                     int32_t max_seq_len) {
  DecLayout L{};
  const int G = n_q_heads / n_kv_heads;
  L.n_rb = (G + 3) / 4;
  L.chunk = kChunk;
  L.n_chunk = std::max(1, (max_seq_len + L.chunk - 1) / L.chunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nblk = (size_t)batch * n_kv_heads * L.n_rb * L.n_chunk;
  L.prep = 0;
  L.part = al(attn_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads));
  L.stats = L.part + al(nblk * 8 * ctx->Dp * sizeof(float));
  L.total = L.stats + al(nblk * 8 * sizeof(float));
  return L;
}

}  // namespace

size_t decode_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t n_q_heads,
                              int32_t n_kv_heads, int32_t max_seq_len) {
  return dec_layout(ctx, batch, n_q_heads, n_kv_heads, max_seq_len).total;
}

hipError_t launch_attn_decode(const tq_ctx* ctx, const float* q, int32_t batch, int32_t n_q_heads,
                              int64_t q_stride_batch, const uint32_t* k_planes,
                              const uint16_t* k_norms, const uint32_t* v_planes,
                              const uint16_t* v_norms, int32_t n_kv_heads,
                              int64_t kv_stride_head, const int64_t* seq_start,
                              const int32_t* seq_len, int32_t max_seq_len, float scale,
                              float* out, int64_t out_stride_batch, void* workspace,
                              hipStream_t stream) {
  const DecLayout L = dec_layout(ctx, batch, n_q_heads, n_kv_heads, max_seq_len);
  char* ws = (char*)workspace;
  hipError_t e = launch_attn_prepare(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads,
                                     ws + L.prep, false, stream);
  if (e != hipSuccess) return e;
  DecArgs a{};
  a.ws = ws + L.prep;
  a.k_planes = k_planes;
  a.k_norms = (const uint32_t*)k_norms;
  a.v_planes = v_planes;
  a.v_norms = (const uint32_t*)v_norms;
  a.kv_stride_head = kv_stride_head;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.part = (float*)(ws + L.part);
  a.stats = (float*)(ws + L.stats);
  a.d = ctx->d;
  a.W = ctx->W;
  a.Dp = ctx->Dp;
  a.G = n_q_heads / n_kv_heads;
  a.n_kv = n_kv_heads;
  a.n_rb = L.n_rb;
  a.n_chunk = L.n_chunk;
  a.scale = scale;
  a.alpha = (float)(std::sqrt(M_PI / 2.0) / ctx->d);
  for (int v = 0; v < kMaxVec; ++v) a.mask[v] = v < ctx->n_mono ? ctx->mono_mask[v] : 0;
  if (!dev::make_vacc_coef(ctx->mono_mask, ctx->mono_w, ctx->n_mono, ctx->c0, ctx->cp, a.cf))
    return hipErrorInvalidValue;
  const size_t shm = 0;
  const dim3 grid(L.n_chunk, n_kv_heads * L.n_rb, batch);
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: hipLaunchKernelGGL((decode_chunk_kernel<1, true>), grid, dim3(256), shm, stream, a); break;
      case 2: hipLaunchKernelGGL((decode_chunk_kernel<2, true>), grid, dim3(256), shm, stream, a); break;
      default: hipLaunchKernelGGL((decode_chunk_kernel<3, true>), grid, dim3(256), shm, stream, a); break;
    }
  } else {
    switch (ctx->b) {
      case 2: hipLaunchKernelGGL((decode_chunk_kernel<2, false>), grid, dim3(256), shm, stream, a); break;
      case 3: hipLaunchKernelGGL((decode_chunk_kernel<3, false>), grid, dim3(256), shm, stream, a); break;
      default: hipLaunchKernelGGL((decode_chunk_kernel<4, false>), grid, dim3(256), shm, stream, a); break;
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecFinArgs f{};
  f.part = a.part;
  f.stats = a.stats;
  f.pi32 = ctx->t.pi32;
  f.s32 = ctx->t.s32;
  f.out = out;
  f.out_stride_batch = out_stride_batch;
  f.d = ctx->d;
  f.Dp = ctx->Dp;
  f.G = a.G;
  f.n_kv = n_kv_heads;
  f.n_rb = L.n_rb;
  f.n_chunk = L.n_chunk;
  f.qjl = ctx->mse ? 0 : 1;
  f.alpha = a.alpha;
  hipLaunchKernelGGL(decode_final_kernel, dim3(n_q_heads, batch), dim3(256),
                     (2 * (size_t)ctx->Dp + L.n_chunk) * sizeof(float), stream, f);
  return hipGetLastError();
}

}  // namespace tq
