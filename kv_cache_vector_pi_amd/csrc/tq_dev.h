// Device helpers shared by the logit, value-output and fused decode kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace tq {
namespace dev {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;          // key tokens per MFMA tile
constexpr int kWaves = 4;          // waves per workgroup

// MFMA calls per word step: two per Walsh subset of the cp code planes, and
// two for the sign plane when the records carry the QJL stage
__host__ __device__ inline int n_calls(int cp, bool qjl) { return 2 * (1 << (cp - 1)) + (qjl ? 2 : 0); }
__host__ __device__ inline int n_ws(int W) { return (W + 3) / 4; }                  // word steps of 4 words

// Prepared-query workspace for one (batch, kv head, row block of 4 q heads):
//   int4 frag[n_ws][n_calls][64 lanes]   A operands (16 int8 each)
//   float4 consts[4]                      per q head: mse scale, qjl scale,
//                                         mse offset, qjl offset
__host__ __device__ inline size_t rb_bytes(int W, int nc) {
  return (size_t)n_ws(W) * nc * 64 * 16 + 4 * 16;
}

template <int NB>
__device__ inline void load_group(const uint32_t* p, uint32_t (&w)[NB]) {
  // NB words per record group
  if constexpr (NB == 4) {
    uint4 v = *(const uint4*)p;
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (NB == 2) {
    uint2 v = *(const uint2*)p;
    w[0] = v.x; w[1] = v.y;
  } else {
    for (int i = 0; i < NB; ++i) w[i] = p[i];
  }
}

// masked int8 lanes of a plane word for shifts 4*half .. 4*half+3
__device__ inline v4i bit_lanes(uint32_t u, int half) {
  const uint32_t m = 0x01010101u << (4 * half);
  v4i r;
  r[0] = (int)(u & m);
  r[1] = (int)(u & (m << 1));
  r[2] = (int)(u & (m << 2));
  r[3] = (int)(u & (m << 3));
  return r;
}

// Four balanced base-256 limbs accumulated by the int8 MFMAs -> float.
__device__ inline float limbs_to_float(const v4i& c) {
  return fmaf((float)c[3], 16777216.f, fmaf((float)c[2], 65536.f, fmaf((float)c[1], 256.f, (float)c[0])));
}

// Block-wide value accumulation over nt staged tokens (256 threads, every
// thread calls it): for the 4 query heads hh of the block
//   dst[hh][j]     = sum_t wts[t][hh]     * c[idx_tj]
//   dst[4 + hh][j] = sum_t wts[t][4 + hh] * s_tj        (s = +-1)
// for j < Dp (coordinates j >= d hold the contributions of zero bits and are
// ignored by the consumers).  MSE records (NB code planes, no sign plane)
// leave dst[4 + hh] zero.  words: LDS [nt][RW] packed records (RW = W*NB),
// wts: LDS [nt][8], ctab: LDS centroids, red: LDS scratch of
// max(1, 256 / Dp) * 8 * Dp floats that may alias `words` (a barrier separates
// the reads from the reuse).  Threads own coordinates lc + 256k of token group
// tg (tokens tg, tg + TT, ...).
template <int NB, bool MSE>
__device__ void vacc_block(const uint32_t* words, const float* wts, const float* ctab, int nt,
                           int RW, int d, int Dp, float* red, float* dst) {
  const int tid = threadIdx.x;
  const int NL = min(Dp, 256);
  const int TT = 256 / NL;
  const int lc = tid % NL, tg = tid / NL;
  constexpr int kMaxCpt = 8;                     // Dp <= 2048
  const int cpt = (Dp + 255) / 256;
  float ar[kMaxCpt][4], as[kMaxCpt][4];
#pragma unroll
  for (int k = 0; k < kMaxCpt; ++k)
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) ar[k][hh] = as[k][hh] = 0.f;
  if (tg < TT) {
    for (int t = tg; t < nt; t += TT) {
      const uint32_t* rw = words + t * RW;
      const float4 w1 = *(const float4*)(wts + 8 * t);
      const float4 w2 = *(const float4*)(wts + 8 * t + 4);
#pragma unroll
      for (int k = 0; k < kMaxCpt; ++k) {
        if (k >= cpt) break;
        const int j = lc + 256 * k;
        if (j >= d) continue;
        const uint32_t* gw = rw + (j >> 5) * NB;
        const int bit = j & 31;
        uint32_t idx = 0;
#pragma unroll
        for (int q = 0; q < (MSE ? NB : NB - 1); ++q) idx |= __builtin_amdgcn_ubfe(gw[q], bit, 1) << q;
        const float c = ctab[idx];
        ar[k][0] = fmaf(w1.x, c, ar[k][0]);
        ar[k][1] = fmaf(w1.y, c, ar[k][1]);
        ar[k][2] = fmaf(w1.z, c, ar[k][2]);
        ar[k][3] = fmaf(w1.w, c, ar[k][3]);
        if constexpr (MSE) continue;
        // +1.0 for a set sign bit, -1.0 otherwise
        const float sg =
            __uint_as_float(0xbf800000u ^ (__builtin_amdgcn_ubfe(gw[NB - 1], bit, 1) << 31));
        as[k][0] = fmaf(w2.x, sg, as[k][0]);
        as[k][1] = fmaf(w2.y, sg, as[k][1]);
        as[k][2] = fmaf(w2.z, sg, as[k][2]);
        as[k][3] = fmaf(w2.w, sg, as[k][3]);
      }
    }
  }
  __syncthreads();          // staging area may be reused for the token-group sums
  if (TT > 1) {
    if (tg < TT)
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        red[(tg * 8 + hh) * NL + lc] = ar[0][hh];
        red[(tg * 8 + 4 + hh) * NL + lc] = as[0][hh];
      }
    __syncthreads();
    for (int i = tid; i < 8 * NL; i += 256) {
      float s = 0.f;
      for (int g = 0; g < TT; ++g) s += red[g * 8 * NL + i];
      dst[(i / NL) * Dp + i % NL] = s;           // TT > 1 only when Dp <= 128: NL == Dp
    }
  } else if (tg < TT) {
#pragma unroll
    for (int k = 0; k < kMaxCpt; ++k) {
      if (k >= cpt) break;
      const int j = lc + 256 * k;
      if (j >= Dp) continue;
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        dst[hh * Dp + j] = ar[k][hh];
        dst[(4 + hh) * Dp + j] = as[k][hh];
      }
    }
  }
}

}  // namespace dev
}  // namespace tq
