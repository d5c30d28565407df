// Quantization for head_dim 128 (the KV-cache case), specialised for gfx950.
// Same method and results as the generic kernel (turboquant.net pseudo-code
// "quant"; admirer.cn two-stage description; residual norm as fp16 from the
// "potential challenges" section), organised for throughput:
//
//  * 4 waves per workgroup, wave w owns word w of every plane (output
//    coordinates 32w..32w+31 = one 32-row block of v_mfma_f32_32x32x16_f16);
//    its slices of Pi and M (hi and lo fp16 parts) stay in registers.
//  * 64 vectors per tile (two 32-column blocks); x_s and then the residual
//    live in LDS as fp16 hi/lo pairs.
//  * Register budget <= 256 per lane, so two workgroups share a CU and the
//    matrix phase of one overlaps the per-coordinate work of the other.
//  * Per coordinate: |y| is compared against the K/2-1 positive thresholds
//    (the codebook is symmetric); the centroid is a select chain on those
//    compares, negated for the lower half of the codebook; code bits come
//    from lane-mask algebra on the compares, accumulated with one shift-add
//    per bit and spread to the canonical bit positions once per word.
//  * A vector with ||x|| = 0 gets its signs forced to +1 and gamma to 0 once
//    per vector (its codes, of y = 0, need no fix).
//  * Pure 128-dimensional layout: no padded coordinates (d == 128 only).
#include <algorithm>
#include <cmath>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kT = 64;        // vectors per tile
constexpr int kLdx = 136;     // LDS row stride in halves (128 + 8)

struct Q128Args {
  const void* x;
  int64_t x_stride_token, x_stride_head;
  int64_t n_tokens;
  uint32_t* planes;
  uint32_t* norms;
  int64_t dst_stride_head, dst_token0;
  const __half* pi_hi;
  const __half* pi_lo;
  const __half* m_hi;
  const __half* m_lo;
  int64_t n_tiles, tiles_per_head;
  float thr[4];     // positive thresholds t_{K/2} .. t_{K-2}
  float cpos[4];    // positive centroids c_{K/2} .. c_{K-1}
};

// rows held by lane half h (0/1) of a 32x32 C block: 8*(i/4) + 4*h + i%4.
// Spread a 16-bit value (bit i <-> row of element i) to those word positions.
__device__ inline uint32_t spread16(uint32_t v, int h) {
  uint32_t x = (v & 0xffu) | ((v & 0xff00u) << 8);    // bytes 0 and 2
  x = (x | (x << 4)) & 0x0f0f0f0fu;                     // one nibble per byte
  return x << (4 * h);
}

template <int NB, bool BF16>
__global__ void __launch_bounds__(256, 2) quantize128_kernel(Q128Args a) {
  constexpr int K = 1 << (NB - 1);
  constexpr int KH = K / 2;           // positive centroids
  constexpr int NT = KH - 1;          // positive thresholds
  __shared__ __align__(16) _Float16 bufA[kT * kLdx];   // x_hi, then r_hi
  __shared__ __align__(16) _Float16 bufB[kT * kLdx];   // x_lo, then r_lo
  __shared__ float ysc[kT];
  __shared__ uint32_t nu16[kT];
  __shared__ float gpart[4][kT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;

  // Pi / M rows 32*wave + col, K slots 16*ks + 8*hh .. +8
  v8h Ph[8], Pl[8], Mh[8], Ml[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int off = (32 * wave + col) * 128 + 16 * ks + 8 * hh;
    Ph[ks] = *(const v8h*)(a.pi_hi + off);
    Pl[ks] = *(const v8h*)(a.pi_lo + off);
    Mh[ks] = *(const v8h*)(a.m_hi + off);
    Ml[ks] = *(const v8h*)(a.m_lo + off);
  }

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const int h = (int)(tile / a.tiles_per_head);
    const int64_t t0 = (tile % a.tiles_per_head) * kT;
    const int cnt = (int)std::min<int64_t>(kT, a.n_tokens - t0);

    // ---- 1. x -> norm, power-of-two scale, fp16 (hi/lo) into LDS ----------
    // pass p: vector 4*wave + 16*p + lane/16, 8-element chunk lane%16
    {
      uint4 raw[BF16 ? 4 : 8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int v = 4 * wave + 16 * p + (lane >> 4);
        const int64_t off =
            (int64_t)h * a.x_stride_head + (t0 + v) * a.x_stride_token + 8 * (lane & 15);
        const bool ok = v < cnt;
        if constexpr (BF16) {
          raw[p] = ok ? *(const uint4*)((const uint16_t*)a.x + off) : make_uint4(0u, 0u, 0u, 0u);
        } else {
          raw[2 * p] = ok ? *(const uint4*)((const float*)a.x + off) : make_uint4(0u, 0u, 0u, 0u);
          raw[2 * p + 1] =
              ok ? *(const uint4*)((const float*)a.x + off + 4) : make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int v = 4 * wave + 16 * p + (lane >> 4);
        const int c = lane & 15;
        float xv[8];
        if constexpr (BF16) {
          const uint32_t wv[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[2 * e] = __uint_as_float(wv[e] << 16);
            xv[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
          }
        } else {
          const uint4 u0 = raw[2 * p], u1 = raw[2 * p + 1];
          xv[0] = __uint_as_float(u0.x); xv[1] = __uint_as_float(u0.y);
          xv[2] = __uint_as_float(u0.z); xv[3] = __uint_as_float(u0.w);
          xv[4] = __uint_as_float(u1.x); xv[5] = __uint_as_float(u1.y);
          xv[6] = __uint_as_float(u1.z); xv[7] = __uint_as_float(u1.w);
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(xv[e], xv[e], ss);
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        const float nu = sqrtf(ss);
        int ex = 0;
        if (nu > 0.f) frexpf(nu, &ex);
        const float sc = ldexpf(1.f, -ex);
        v8h hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xs = xv[e] * sc;
          const _Float16 hv = (_Float16)xs;
          hi[e] = hv;
          if constexpr (!BF16) lo[e] = (_Float16)(xs - (float)hv);
        }
        *(v8h*)(bufA + v * kLdx + 8 * c) = hi;
        if constexpr (!BF16) *(v8h*)(bufB + v * kLdx + 8 * c) = lo;
        if (c == 0) {
          ysc[v] = (nu > 0.f) ? ldexpf(1.f / nu, ex) : 0.f;
          nu16[v] = (uint32_t)__half_as_ushort(__float2half_rn(nu));
        }
      }
    }
    __syncthreads();

    // ---- 2. Y = Pi x_s (rows 32*wave.., columns = 2 blocks of 32 vectors) --
    v16f acc[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      v16f c = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = (32 * cb + col) * kLdx + 16 * ks + 8 * hh;
        const v8h xh = *(const v8h*)(bufA + off);
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ph[ks], xh, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(Pl[ks], xh, c, 0, 0, 0);
        if constexpr (!BF16) {
          const v8h xl = *(const v8h*)(bufB + off);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ph[ks], xl, c, 0, 0, 0);
        }
      }
      acc[cb] = c;
    }
    __syncthreads();    // all of x has been read; r may overwrite it

    // ---- 3. codes and residual ----------------------------------------------
    uint32_t codew[2][3];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int v = 32 * cb + col;
      const float s = ysc[v];
      uint32_t bacc[3] = {0u, 0u, 0u};    // code planes, bit i <-> element i
      float g2 = 0.f;
      float rr[16];
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        const float y = acc[cb][i] * s;
        const float ay = fabsf(y);
        const bool pos = y > 0.f;
        bool gt[NT > 0 ? NT : 1];
        float cm = a.cpos[0];
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          gt[k] = ay > a.thr[k];
          cm = gt[k] ? a.cpos[k + 1] : cm;
        }
        const float c = pos ? cm : -cm;      // sign of the code (y = +0 -> lower half)
        const float r = y - c;
        rr[i] = r;
        g2 = fmaf(r, r, g2);
        // idx = pos ? KH + m : KH - 1 - m, m = number of thresholds below |y|;
        // top bit = pos; lower bits = m for pos, ~m otherwise.  With the
        // thermometer code gt[], bit 0 of m is the XOR of all gt, bit 1 (K=8)
        // is gt[1].
        if constexpr (NB == 2) {
          bacc[0] = (bacc[0] << 1) | (pos ? 1u : 0u);
        } else if constexpr (NB == 3) {
          bacc[1] = (bacc[1] << 1) | (pos ? 1u : 0u);
          bacc[0] = (bacc[0] << 1) | ((gt[0] == pos) ? 1u : 0u);
        } else {
          bacc[2] = (bacc[2] << 1) | (pos ? 1u : 0u);
          bacc[1] = (bacc[1] << 1) | ((gt[1] == pos) ? 1u : 0u);
          const bool m0 = gt[0] ^ gt[1] ^ gt[2];
          bacc[0] = (bacc[0] << 1) | ((m0 == pos) ? 1u : 0u);
        }
      }
      // residual -> LDS as hi/lo fp16 (rows 8j + 4hh .. +3 hold 4 consecutive i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v4h rh, rl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float r = rr[4 * j + e];
          const _Float16 hv = (_Float16)r;
          rh[e] = hv;
          rl[e] = (_Float16)(r - (float)hv);
        }
        const int off = v * kLdx + 32 * wave + 8 * j + 4 * hh;
        *(v4h*)(bufA + off) = rh;
        *(v4h*)(bufB + off) = rl;
      }
#pragma unroll
      for (int p = 0; p < NB - 1; ++p) {
        uint32_t w = spread16(bacc[p], hh);
        w |= __shfl_xor(w, 32);
        codew[cb][p] = w;
      }
      g2 += __shfl_xor(g2, 32);
      if (hh == 0) gpart[wave][v] = g2;
    }
    __syncthreads();

    // ---- 4. Z = M r (3 passes), signs, store ----------------------------------
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      v16f z = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = (32 * cb + col) * kLdx + 16 * ks + 8 * hh;
        const v8h rh = *(const v8h*)(bufA + off);
        const v8h rl = *(const v8h*)(bufB + off);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Mh[ks], rh, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ml[ks], rh, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Mh[ks], rl, z, 0, 0, 0);
      }
      uint32_t sb = 0u;
#pragma unroll
      for (int i = 15; i >= 0; --i) sb = (sb << 1) | (z[i] >= 0.f ? 1u : 0u);
      uint32_t sw = spread16(sb, hh);
      sw |= __shfl_xor(sw, 32);
      const int v = 32 * cb + col;
      if (ysc[v] == 0.f) sw = 0xffffffffu;       // ||x|| = 0: r = 0, all signs +1
      if (v < cnt) {
        const int64_t rec = (int64_t)h * a.dst_stride_head + a.dst_token0 + t0 + v;
        uint32_t* dst = a.planes + (rec * 4 + wave) * NB;
        // lane half 0 stores the lower planes, half 1 the upper ones
        if constexpr (NB == 4) {
          if (hh == 0) *(uint2*)dst = make_uint2(codew[cb][0], codew[cb][1]);
          else *(uint2*)(dst + 2) = make_uint2(codew[cb][2], sw);
        } else if constexpr (NB == 3) {       // 12-byte groups: 4-byte stores
          if (hh == 0) {
            dst[0] = codew[cb][0];
            dst[1] = codew[cb][1];
          } else {
            dst[2] = sw;
          }
        } else {
          if (hh == 0) dst[0] = codew[cb][0];
          else dst[1] = sw;
        }
      }
    }
    if (tid < cnt) {
      const float s = (gpart[0][tid] + gpart[1][tid]) + (gpart[2][tid] + gpart[3][tid]);
      const float gam = ysc[tid] == 0.f ? 0.f : sqrtf(s);
      const uint32_t gb = (uint32_t)__half_as_ushort(__float2half_rn(gam));
      const int64_t rec = (int64_t)h * a.dst_stride_head + a.dst_token0 + t0 + tid;
      a.norms[rec] = nu16[tid] | (gb << 16);
    }
    __syncthreads();
  }
}

template <int NB, bool BF16>
hipError_t launch128(const Q128Args& a, int n_cu, hipStream_t st) {
  static int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, quantize128_kernel<NB, BF16>, 256, 0) !=
            hipSuccess ||
        nb < 1)
      nb = 1;
    return nb;
  }();
  const int64_t grid = std::min<int64_t>(a.n_tiles, (int64_t)n_cu * per_cu);
  hipLaunchKernelGGL((quantize128_kernel<NB, BF16>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize128(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                              int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                              int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                              int64_t dst_stride_head, int64_t dst_token0, hipStream_t stream) {
  Q128Args a{};
  a.x = x;
  a.x_stride_token = x_stride_token;
  a.x_stride_head = x_stride_head;
  a.n_tokens = n_tokens;
  a.planes = planes;
  a.norms = (uint32_t*)norms;
  a.dst_stride_head = dst_stride_head;
  a.dst_token0 = dst_token0;
  a.pi_hi = ctx->t.pi_hi;
  a.pi_lo = ctx->t.pi_lo;
  a.m_hi = ctx->t.m_hi;
  a.m_lo = ctx->t.m_lo;
  a.tiles_per_head = (n_tokens + kT - 1) / kT;
  a.n_tiles = a.tiles_per_head * n_heads;
  const int KH = ctx->K / 2;
  for (int k = 0; k < 4; ++k) {
    a.thr[k] = (k < KH - 1) ? ctx->mid[KH + k] : 0.f;
    a.cpos[k] = (k < KH) ? ctx->cent[KH + k] : 0.f;
  }
  const bool bf = x_dtype == TQ_BF16;
  switch (ctx->b) {
    case 2: return bf ? launch128<2, true>(a, ctx->n_cu, stream) : launch128<2, false>(a, ctx->n_cu, stream);
    case 3: return bf ? launch128<3, true>(a, ctx->n_cu, stream) : launch128<3, false>(a, ctx->n_cu, stream);
    default: return bf ? launch128<4, true>(a, ctx->n_cu, stream) : launch128<4, false>(a, ctx->n_cu, stream);
  }
}

}  // namespace tq
