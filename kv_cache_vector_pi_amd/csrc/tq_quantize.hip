// Online quantization of KV vectors (turboquant.net pseudo-code "quant":
// rotate by Pi, nearest Lloyd-Max centroid per coordinate; admirer.cn article:
// (b-1)-bit scalar codes then a 1-bit QJL sign sketch of the residual;
// turboquant.net "potential challenges": the residual norm is one fp16 scalar).
//
//   nu = ||x||, y = Pi x / nu, idx_j = #{k : y_j > t_k}, r = y - c[idx] (rotated
//   residual), gamma = ||r||, z = M r with M = S Pi^T, s_i = [z_i >= 0]
//
// One fused kernel per tile of T vectors of one head:
//  1. load x, nu per vector (wave-shuffle reduction), x_s = x * 2^-e (e from
//     nu, exact) as fp16 into LDS (fp32 input: hi and lo fp16 parts);
//  2. Y = Pi x_s on fp16 MFMA (v_mfma_f32_16x16x32_f16) with Pi split into
//     hi + lo fp16 (2 passes for bf16 input, 3 for fp32), fp32 accumulate;
//  3. per coordinate: threshold count, centroid, residual, code bits; the
//     residual goes back to LDS as hi + lo fp16;
//  4. Z = M r with M and r split hi/lo (3 passes), sign bits;
//  5. packed words, fp16 nu and gamma to HBM.
// Each wave owns whole 32-coordinate words of the output (two 16-row MFMA
// blocks), so every plane word of a vector is assembled inside one wave.
// Errors against exact arithmetic stay near 1e-7 of a unit coordinate, far
// below the 1e-5 decision margins the codes are checked against.
#include <algorithm>
#include <cmath>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct QuantArgs {
  const void* x;
  int64_t x_stride_token, x_stride_head;
  int64_t n_tokens;
  int32_t n_heads;
  uint32_t* planes;
  uint32_t* norms;
  int64_t dst_stride_head, dst_token0;
  const int64_t* slots;   // per-token destination, or null (dst_token0 + t)
  const __half* pi_hi;
  const __half* pi_lo;
  const __half* m_hi;
  const __half* m_lo;
  int d, W, Dp, NW, T, ldx;   // ldx: LDS row stride in halves
  int64_t n_tiles, tiles_per_head;
  float cent[kMaxK];
  float mid[kMaxK];
};

__device__ inline float lane_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// record of (head h, token t), or -1 for a token whose slot lies outside
// [0, dst_stride_head)
__device__ inline int64_t dst_record(const QuantArgs& a, int64_t h, int64_t t) {
  int64_t s = t;
  if (a.slots) {
    s = a.slots[t];
    if (s < 0 || s >= a.dst_stride_head) return -1;
  }
  return h * a.dst_stride_head + a.dst_token0 + s;
}

__device__ inline v8h lds_v8h(const _Float16* p) { return *(const v8h*)p; }
__device__ inline v8h gbl_v8h(const __half* p) { return *(const v8h*)p; }

// NB: words per record group (bits per coordinate); MSE: all NB are code
// planes and the QJL stage (residual, Z = M r, signs, gamma) is left out;
// BF16: input type; NCB: 16-vector column blocks per tile; WPW: words per
// wave (word w = wave + NW * i); RES: one word per wave and Dp == 128 -> Pi
// and M fragments stay in registers for the whole kernel.
template <int NB, bool MSE, bool BF16, int NCB, int WPW, bool RES>
__global__ void __launch_bounds__(RES ? 256 : 512) quantize_kernel(QuantArgs a) {
  constexpr int CP = MSE ? NB : NB - 1;     // code planes
  constexpr int K = 1 << CP;
  constexpr int T = 16 * NCB;
  extern __shared__ __align__(16) char smem[];
  _Float16* bufA = (_Float16*)smem;                       // x_hi, then r_hi  [T][ldx]
  _Float16* bufB = bufA + T * a.ldx;                      // x_lo, then r_lo  [T][ldx]
  float* ysc = (float*)(bufB + T * a.ldx);                // [T] 2^e / nu (0 if nu == 0)
  uint32_t* nu16 = (uint32_t*)(ysc + T);                  // [T] fp16 bits of nu
  float* gpart = (float*)(nu16 + T);                      // [NW][T] partial gamma^2

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int d = a.d, Dp = a.Dp, W = a.W, NW = a.NW, ldx = a.ldx;
  const int KS = RES ? 4 : Dp / 32;   // compile-time 4 when fragments are resident

  // resident Pi / M fragments (Dp == 128, one word per wave)
  v8h rPh[RES ? 8 : 1], rPl[RES ? 8 : 1], rMh[RES ? 8 : 1], rMl[RES ? 8 : 1];
  if constexpr (RES) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int64_t off = (int64_t)(32 * wave + 16 * rb + n) * Dp + 32 * ks + 8 * g;
        rPh[ks * 2 + rb] = gbl_v8h(a.pi_hi + off);
        rPl[ks * 2 + rb] = gbl_v8h(a.pi_lo + off);
        rMh[ks * 2 + rb] = gbl_v8h(a.m_hi + off);
        rMl[ks * 2 + rb] = gbl_v8h(a.m_lo + off);
      }
  }

  // lanes per vector in the load phase (power of two), chunks of 8 elements
  const int nchunk = Dp / 8;
  int LPV = 1;
  while (LPV < nchunk && LPV < 64) LPV <<= 1;
  const int VPP = 64 / LPV;                     // vectors per wave pass
  const int CPL = (nchunk + LPV - 1) / LPV;     // chunks per lane

  // RES (d = 128, 4 waves, 64 vectors per tile): each lane owns one 8-element
  // chunk of 4 vectors per tile -- pass p covers vector 4*wave + 16p + lane/16,
  // chunk lane%16.  The next tile's chunks are fetched into registers while the
  // current tile is in its MFMA phases.
  constexpr int NPRE = RES ? (BF16 ? 4 : 8) : 1;
  uint4 pre[NPRE];
  auto fetch = [&](int64_t tl) {
    if constexpr (RES) {
      const int hf = (int)(tl / a.tiles_per_head);
      const int64_t tf = (tl % a.tiles_per_head) * T;
      const int cf = (int)std::min<int64_t>(T, a.n_tokens - tf);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int v = 4 * wave + 16 * p + (lane >> 4);
        const int64_t off = (int64_t)hf * a.x_stride_head + (tf + v) * a.x_stride_token +
                            8 * (lane & 15);
        if constexpr (BF16) {
          pre[p] = (tl < a.n_tiles && v < cf) ? *(const uint4*)((const uint16_t*)a.x + off)
                                              : make_uint4(0u, 0u, 0u, 0u);
        } else {
          const bool ok = tl < a.n_tiles && v < cf;
          pre[2 * p] = ok ? *(const uint4*)((const float*)a.x + off) : make_uint4(0u, 0u, 0u, 0u);
          pre[2 * p + 1] =
              ok ? *(const uint4*)((const float*)a.x + off + 4) : make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  };
  if constexpr (RES) fetch(blockIdx.x);

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    const int h = (int)(tile / a.tiles_per_head);
    const int64_t t0 = (tile % a.tiles_per_head) * T;
    const int cnt = (int)std::min<int64_t>(T, a.n_tokens - t0);

    // ---- 1. load, norm, scale, fp16 split --------------------------------
    if constexpr (RES) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int v = 4 * wave + 16 * p + (lane >> 4);
        const int c = lane & 15;
        float xv[8];
        if constexpr (BF16) {
          const uint32_t wv[4] = {pre[p].x, pre[p].y, pre[p].z, pre[p].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[2 * e] = __uint_as_float(wv[e] << 16);
            xv[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
          }
        } else {
          const uint4 u0 = pre[2 * p], u1 = pre[2 * p + 1];
          xv[0] = __uint_as_float(u0.x); xv[1] = __uint_as_float(u0.y);
          xv[2] = __uint_as_float(u0.z); xv[3] = __uint_as_float(u0.w);
          xv[4] = __uint_as_float(u1.x); xv[5] = __uint_as_float(u1.y);
          xv[6] = __uint_as_float(u1.z); xv[7] = __uint_as_float(u1.w);
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(xv[e], xv[e], ss);
        ss = lane_sum(ss, 16);
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
          lo[e] = (_Float16)(xs - (float)hv);
        }
        *(v8h*)(bufA + v * ldx + 8 * c) = hi;
        if constexpr (!BF16) *(v8h*)(bufB + v * ldx + 8 * c) = lo;
        if (c == 0) {
          ysc[v] = (nu > 0.f) ? ldexpf(1.f / nu, ex) : 0.f;
          nu16[v] = (uint32_t)__half_as_ushort(__float2half_rn(nu));
        }
      }
    } else
    for (int vb = wave * VPP; vb < T; vb += NW * VPP) {
      const int v = vb + lane / LPV;
      const int sub = lane % LPV;
      const bool vok = v < T && v < cnt;
      float xv[4][8];      // at most 4 chunks per lane (Dp <= 2048)
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = sub + LPV * k;
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[k][e] = 0.f;
        if (k < CPL && vok && 8 * c < d) {
          const int64_t off = (int64_t)h * a.x_stride_head + (t0 + v) * a.x_stride_token + 8 * c;
          if constexpr (BF16) {
            const uint4 raw = *(const uint4*)((const uint16_t*)a.x + off);
            const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              xv[k][2 * e] = __uint_as_float(wv[e] << 16);
              xv[k][2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
            }
          } else {
            const float4 f0 = *(const float4*)((const float*)a.x + off);
            const float4 f1 = *(const float4*)((const float*)a.x + off + 4);
            xv[k][0] = f0.x; xv[k][1] = f0.y; xv[k][2] = f0.z; xv[k][3] = f0.w;
            xv[k][4] = f1.x; xv[k][5] = f1.y; xv[k][6] = f1.z; xv[k][7] = f1.w;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(xv[k][e], xv[k][e], ss);
        }
      }
      ss = lane_sum(ss, LPV);
      const float nu = sqrtf(ss);
      int ex = 0;
      if (nu > 0.f) frexpf(nu, &ex);
      const float sc = ldexpf(1.f, -ex);
      if (v < T) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int c = sub + LPV * k;
          if (k < CPL && c < nchunk) {
            v8h hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float xs = xv[k][e] * sc;
              const _Float16 hv = (_Float16)xs;
              hi[e] = hv;
              lo[e] = (_Float16)(xs - (float)hv);
            }
            *(v8h*)(bufA + v * ldx + 8 * c) = hi;
            if constexpr (!BF16) *(v8h*)(bufB + v * ldx + 8 * c) = lo;
          }
        }
        if (sub == 0) {
          ysc[v] = (nu > 0.f) ? ldexpf(1.f / nu, ex) : 0.f;
          nu16[v] = (uint32_t)__half_as_ushort(__float2half_rn(nu));
        }
      }
    }
    __syncthreads();
    if constexpr (RES) fetch(tile + gridDim.x);   // next tile, in flight during MFMA

    // ---- 2. Y = Pi x_s ------------------------------------------------------
    // words of this wave: w = wave + NW * wi.  The K step is the outer loop,
    // so all waves (and the workgroups in step with them) read one narrow
    // column slice of Pi at a time, which stays in L2.
    v4f acc[WPW][2][NCB];
#pragma unroll
    for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[wi][rb][cb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int ks = 0; ks < KS; ++ks) {
      v8h xh[NCB], xl[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        xh[cb] = lds_v8h(bufA + (16 * cb + n) * ldx + 32 * ks + 8 * g);
        if constexpr (!BF16) xl[cb] = lds_v8h(bufB + (16 * cb + n) * ldx + 32 * ks + 8 * g);
      }
#pragma unroll
      for (int wi = 0; wi < WPW; ++wi) {
        const int w = wave + NW * wi;
        if (w >= W) continue;
        v8h ph[2], pl[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          if constexpr (RES) {
            ph[rb] = rPh[ks * 2 + rb];
            pl[rb] = rPl[ks * 2 + rb];
          } else {
            const int64_t off = (int64_t)(32 * w + 16 * rb + n) * Dp + 32 * ks + 8 * g;
            ph[rb] = gbl_v8h(a.pi_hi + off);
            pl[rb] = gbl_v8h(a.pi_lo + off);
          }
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            v4f c = acc[wi][rb][cb];
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[rb], xh[cb], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl[rb], xh[cb], c, 0, 0, 0);
            if constexpr (!BF16) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[rb], xl[cb], c, 0, 0, 0);
            acc[wi][rb][cb] = c;
          }
      }
    }
    __syncthreads();   // every wave is done reading x before r overwrites it

    // ---- 3. codes, residual -------------------------------------------------
    uint32_t codew[WPW][NCB][3];
    float g2[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) g2[cb] = 0.f;
    {
#pragma unroll
      for (int wi = 0; wi < WPW; ++wi) {
        const int w = wave + NW * wi;
        if (w >= W) continue;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int v = 16 * cb + n;
          const float s = ysc[v];
          uint32_t cw[3] = {0u, 0u, 0u};
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            float rr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int pos = 16 * rb + 4 * g + i;
              const int j = 32 * w + pos;
              const float y = acc[wi][rb][cb][i] * s;
              int idx = 0;
              float c = a.cent[0];
#pragma unroll
              for (int k = 0; k < K - 1; ++k) {
                const bool gt = y > a.mid[k];
                idx += gt ? 1 : 0;
                c = gt ? a.cent[k + 1] : c;
              }
              const bool live = (j < d) && (s > 0.f);
              const float r = live ? y - c : 0.f;
              rr[i] = r;
              g2[cb] = fmaf(r, r, g2[cb]);
              if (j < d) {
#pragma unroll
                for (int p = 0; p < CP; ++p) cw[p] |= (uint32_t)((idx >> p) & 1) << pos;
              }
            }
            if constexpr (MSE) continue;
            // residual to LDS as hi + lo fp16
            const int j0 = 32 * w + 16 * rb + 4 * g;
            typedef _Float16 v4h __attribute__((ext_vector_type(4)));
            v4h rh, rl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const _Float16 hv = (_Float16)rr[i];
              rh[i] = hv;
              rl[i] = (_Float16)(rr[i] - (float)hv);
            }
            *(v4h*)(bufA + v * ldx + j0) = rh;
            *(v4h*)(bufB + v * ldx + j0) = rl;
          }
#pragma unroll
          for (int p = 0; p < CP; ++p) {
            uint32_t x = cw[p];
            x |= __shfl_xor(x, 16);
            x |= __shfl_xor(x, 32);
            codew[wi][cb][p] = x;
          }
        }
      }
    }
    // partial gamma^2 of this wave's coordinates, per vector
#pragma unroll
    for (int cb = 0; cb < (MSE ? 0 : NCB); ++cb) {
      float x = g2[cb];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      if (g == 0) gpart[wave * T + 16 * cb + n] = x;
    }
    __syncthreads();

    // ---- 4. Z = M r (K step outer, as for Y), signs, 5. store ---------------
    if constexpr (MSE) {
#pragma unroll
      for (int wi = 0; wi < WPW; ++wi) {
        const int w = wave + NW * wi;
        if (w >= W) continue;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int v = 16 * cb + n;
          if (g < NB && v < cnt) {
            uint32_t val = 0u;
#pragma unroll
            for (int p = 0; p < NB; ++p)
              if (g == p) val = codew[wi][cb][p];
            const int64_t rec = dst_record(a, h, t0 + v);
            if (rec >= 0) a.planes[(rec * W + w) * NB + g] = val;
          }
        }
      }
    } else {
      v4f zacc[WPW][2][NCB];
#pragma unroll
      for (int wi = 0; wi < WPW; ++wi)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) zacc[wi][rb][cb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int ks = 0; ks < KS; ++ks) {
        v8h rh[NCB], rl[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          rh[cb] = lds_v8h(bufA + (16 * cb + n) * ldx + 32 * ks + 8 * g);
          rl[cb] = lds_v8h(bufB + (16 * cb + n) * ldx + 32 * ks + 8 * g);
        }
#pragma unroll
        for (int wi = 0; wi < WPW; ++wi) {
          const int w = wave + NW * wi;
          if (w >= W) continue;
          v8h mh[2], ml[2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            if constexpr (RES) {
              mh[rb] = rMh[ks * 2 + rb];
              ml[rb] = rMl[ks * 2 + rb];
            } else {
              const int64_t off = (int64_t)(32 * w + 16 * rb + n) * Dp + 32 * ks + 8 * g;
              mh[rb] = gbl_v8h(a.m_hi + off);
              ml[rb] = gbl_v8h(a.m_lo + off);
            }
          }
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              v4f c = zacc[wi][rb][cb];
              c = __builtin_amdgcn_mfma_f32_16x16x32_f16(mh[rb], rh[cb], c, 0, 0, 0);
              c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ml[rb], rh[cb], c, 0, 0, 0);
              c = __builtin_amdgcn_mfma_f32_16x16x32_f16(mh[rb], rl[cb], c, 0, 0, 0);
              zacc[wi][rb][cb] = c;
            }
        }
      }
#pragma unroll
      for (int wi = 0; wi < WPW; ++wi) {
        const int w = wave + NW * wi;
        if (w >= W) continue;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          uint32_t sw = 0u;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int pos = 16 * rb + 4 * g + i;
              if (32 * w + pos < d && zacc[wi][rb][cb][i] >= 0.f) sw |= 1u << pos;
            }
          sw |= __shfl_xor(sw, 16);
          sw |= __shfl_xor(sw, 32);
          const int v = 16 * cb + n;
          if (g < NB && v < cnt) {
            uint32_t val = sw;
#pragma unroll
            for (int p = 0; p < NB - 1; ++p)
              if (g == p) val = codew[wi][cb][p];
            const int64_t rec = dst_record(a, h, t0 + v);
            if (rec >= 0) a.planes[(rec * W + w) * NB + g] = val;
          }
        }
      }
    }
    if (tid < T && tid < cnt) {
      float s = 0.f;
      if (!MSE)
        for (int ww = 0; ww < NW; ++ww) s += gpart[ww * T + tid];
      const float gam = sqrtf(s);
      const uint32_t gb = (uint32_t)__half_as_ushort(__float2half_rn(gam));
      const int64_t rec = dst_record(a, h, t0 + tid);
      if (rec >= 0) a.norms[rec] = nu16[tid] | (gb << 16);
    }
    __syncthreads();   // LDS is reused by the next tile
  }
}

template <int NB, bool MSE, bool BF16, int NCB, int WPW, bool RES>
hipError_t launch_one(const QuantArgs& a, size_t shm, dim3 grid, dim3 block, hipStream_t st) {
  auto fn = quantize_kernel<NB, MSE, BF16, NCB, WPW, RES>;
  // raise the dynamic-LDS limit once per instantiation (the largest tile
  // shape needs ~134 KB); never inside a launch sequence a caller may capture
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(fn, grid, block, shm, st, a);
  return hipGetLastError();
}

// tile shapes by padded dimension: (column blocks, words per wave)
//   Dp <= 256: (4, 1)   Dp <= 512: (4, 2)   Dp <= 1024: (2, 4)   else (1, 8)
template <int NB, bool MSE, bool BF16>
hipError_t launch_nb(const QuantArgs& a, size_t shm, dim3 grid, dim3 block, hipStream_t st) {
  if (a.Dp == 128) return launch_one<NB, MSE, BF16, 4, 1, true>(a, shm, grid, block, st);
  if (a.Dp <= 256) return launch_one<NB, MSE, BF16, 4, 1, false>(a, shm, grid, block, st);
  if (a.Dp <= 512) return launch_one<NB, MSE, BF16, 4, 2, false>(a, shm, grid, block, st);
  if (a.Dp <= 1024) return launch_one<NB, MSE, BF16, 2, 4, false>(a, shm, grid, block, st);
  return launch_one<NB, MSE, BF16, 1, 8, false>(a, shm, grid, block, st);
}

}  // namespace

hipError_t launch_quantize(const tq_ctx* ctx, const void* x, int32_t x_dtype, int64_t n_tokens,
                           int32_t n_heads, int64_t x_stride_token, int64_t x_stride_head,
                           uint32_t* planes, uint16_t* norms, int64_t dst_stride_head,
                           int64_t dst_token0, const int64_t* slots, hipStream_t stream) {
  // the d = 128 kernel computes row offsets within a tile in 32 bits
  if (ctx->d == 128 && x_stride_token < ((int64_t)1 << 25))
    return launch_quantize128(ctx, x, x_dtype, n_tokens, n_heads, x_stride_token, x_stride_head,
                              planes, norms, dst_stride_head, dst_token0, slots, stream);
  // d = 64: the same kernel on token pairs, where they line up; an odd last
  // token of each head goes through the generic kernel below
  if (quantize64_pairs_apply(ctx, n_tokens, n_heads, x_stride_token, dst_stride_head, dst_token0,
                             slots)) {
    const hipError_t e = launch_quantize64_pairs(ctx, x, x_dtype, n_tokens, n_heads,
                                                 x_stride_token, x_stride_head, planes, norms,
                                                 dst_stride_head, dst_token0, stream);
    if (e != hipSuccess || n_tokens % 2 == 0) return e;
    const size_t esz = x_dtype == TQ_BF16 ? 2 : 4;
    x = (const char*)x + (size_t)(n_tokens - 1) * x_stride_token * esz;
    dst_token0 += n_tokens - 1;
    n_tokens = 1;
  }
  QuantArgs a{};
  a.x = x;
  a.x_stride_token = x_stride_token;
  a.x_stride_head = x_stride_head;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.planes = planes;
  a.norms = (uint32_t*)norms;
  a.dst_stride_head = dst_stride_head;
  a.dst_token0 = dst_token0;
  a.slots = slots;
  a.pi_hi = ctx->t.pi_hi;
  a.pi_lo = ctx->t.pi_lo;
  a.m_hi = ctx->t.m_hi;
  a.m_lo = ctx->t.m_lo;
  a.d = ctx->d;
  a.W = ctx->W;
  a.Dp = ctx->Dp;
  a.NW = std::min(ctx->W, 8);
  const int ncb = ctx->Dp <= 512 ? 4 : (ctx->Dp <= 1024 ? 2 : 1);   // as in launch_nb
  a.T = 16 * ncb;
  a.ldx = ctx->Dp + 8;
  for (int k = 0; k < tq::kMaxK; ++k) {
    a.cent[k] = ctx->cent[k];
    a.mid[k] = ctx->mid[k];
  }
  a.tiles_per_head = (n_tokens + a.T - 1) / a.T;
  a.n_tiles = a.tiles_per_head * n_heads;
  const size_t shm = (size_t)2 * a.T * a.ldx * sizeof(_Float16) + (size_t)a.T * (2 + a.NW) * 4;
  // persistent grid: a few workgroups per CU
  const int cus = ctx->n_cu;
  const int per_cu = shm > 80 * 1024 ? 1 : (shm > 50 * 1024 ? 2 : 4);
  const int64_t grid = std::min<int64_t>(a.n_tiles, (int64_t)cus * per_cu);
  const dim3 block(64 * a.NW);
  const bool bf = x_dtype == TQ_BF16;
#define TQ_QNB(NB, MSE)                                                   \
  return bf ? launch_nb<NB, MSE, true>(a, shm, dim3(grid), block, stream) \
            : launch_nb<NB, MSE, false>(a, shm, dim3(grid), block, stream)
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: TQ_QNB(1, true);
      case 2: TQ_QNB(2, true);
      default: TQ_QNB(3, true);
    }
  }
  switch (ctx->b) {
    case 2: TQ_QNB(2, false);
    case 3: TQ_QNB(3, false);
    default: TQ_QNB(4, false);
  }
#undef TQ_QNB
}

}  // namespace tq
