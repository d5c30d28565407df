// Value-side device code: the int8-MFMA value accumulation over packed
// records (bit-plane transposes, weight operands) and the finishing of a query
// head (chunk partials, Pi^T / S^T), shared by the attention-output and fused
// decode kernels.
#pragma once
#include "tq_dev.h"

namespace tq {
namespace dev {

// ---- 32 x 32 bit transpose in registers ------------------------------------
// Within each half of the wave (lanes 0-31 and 32-63): on entry lane l holds
// the word of row l; on exit lane l holds column l, i.e. bit b of its word is
// bit l of the entry word of lane b.  Five exchange stages (partner lane
// l ^ j, j = 16, 8, 4, 2, 1): the lower lane of a pair keeps the bits b with
// b & j == 0 and takes the partner's bits shifted up by j, the upper lane the
// reverse; a rotate and a bitfield insert per stage, with the per-lane mask
// and rotate amount precomputed (TransposeLanes).
struct TransposeLanes {
  uint32_t mk[5], sh[5];
  __device__ explicit TransposeLanes(int lane) {
    const uint32_t m0[5] = {0x0000FFFFu, 0x00FF00FFu, 0x0F0F0F0Fu, 0x33333333u, 0x55555555u};
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      const int j = 16 >> s;
      const bool lower = (lane & j) == 0;
      mk[s] = lower ? m0[s] : ~m0[s];
      sh[s] = lower ? 32 - j : j;        // rotate right: left by j for the lower lane
    }
  }
};
__device__ inline uint32_t xpose_step(uint32_t x, uint32_t p, uint32_t mk, uint32_t sh) {
  const uint32_t r = __builtin_amdgcn_alignbit(p, p, sh);
  return (x & mk) | (r & ~mk);
}
__device__ inline uint32_t transpose32(uint32_t x, const TransposeLanes& t) {
  x = xpose_step(x, (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (16 << 10) | 0x1F), t.mk[0], t.sh[0]);
  x = xpose_step(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false), t.mk[1], t.sh[1]);
  x = xpose_step(x, (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (4 << 10) | 0x1F), t.mk[2], t.sh[2]);
  x = xpose_step(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false), t.mk[3], t.sh[3]);
  x = xpose_step(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false), t.mk[4], t.sh[4]);
  return x;
}

// ---- value accumulation on the int8 matrix cores -----------------------------
// For the 4 query heads hh of the block and a chunk of nt <= kVChunk tokens:
//   dst[hh][j]     = sum_t wts[t][hh]     * c[idx_tj]
//   dst[4 + hh][j] = sum_t wts[t][4 + hh] * s_tj        (s = +-1)
// for j < Dp (coordinates j >= d have zero bits).  MSE records (NB code
// planes, no sign plane) leave dst[4 + hh] zero.
//
// Same algebra as the logit kernel with tokens as the contraction: c[idx] =
// c_0 + sum_m wm2[m] u_m (u_m the XOR of the code planes in Walsh subset m)
// and s = 2 beta - 1 (beta the sign bit), so both sums reduce to
// sum_t w_t * bit_tj, an int8 MFMA (v_mfma_i32_16x16x64_i8) with
//   A (16 x 64 tokens): 4 heads x 4 balanced int8 limbs of the fixed-point
//     weights w_t 2^e, one scale e per head and part for the whole chunk;
//   B (64 tokens x 16 coordinates): bits, as int8 lanes of a word whose bit b
//     is token b's bit (plane words transposed in registers, 32 x 32 at a
//     time), masked in place as 0 or 2^k with the 2^k folded into A.
// Per 128-token block and 32-coordinate word: 2 NB transposes, one
// v_permlane16_swap per plane to gather 4 token groups x 16 coordinates per
// operand, then (NV + 1) x 2 MFMAs per 16 coordinates.  Lane (g, n) of an
// accumulator holds head g's 4 limbs at coordinate n.
//
// The chunk's records are staged from global memory in slices of 4 words
// (wave w takes word w of a slice), plane-major in LDS; the A operands are
// built once per chunk.  All 256 threads call it.
constexpr int kVChunk = 256;                       // tokens per chunk
constexpr int kVAopsBytes = kVChunk / 128 * 4 * 64 * 16;   // A operands: 8 KB
__host__ __device__ constexpr int vacc_words_bytes(int NB) { return 4 * NB * kVChunk * 4; }
__host__ __device__ constexpr int vacc_lds_bytes(int NB) { return kVAopsBytes + vacc_words_bytes(NB); }

template <int NB>
__device__ inline void load_words(const uint32_t* p, uint32_t (&w)[NB]) {
  if constexpr (NB == 4) {
    const uint4 v = *(const uint4*)p;
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (NB == 2) {
    const uint2 v = *(const uint2*)p;
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NB; ++i) w[i] = p[i];
  }
}

// Codebook in Walsh form: c[idx] = c0 + sum_m wm2[m] u_m (wm2 = -2 w_m).
struct VaccCoef {
  float wm2[4];
  float c0;
};

// From the context's Walsh expansion (monomials in the order 1 / 1, 2 /
// 1, 2, 4, 7); false if the masks differ from the ones walsh_mask encodes.
inline bool make_vacc_coef(const int32_t* mono_mask, const double* mono_w, int n_mono, double c0,
                           int cp, VaccCoef& cf) {
  static const int kMasks[3][4] = {{1, 0, 0, 0}, {1, 2, 0, 0}, {1, 2, 4, 7}};
  if (cp < 1 || cp > 3 || n_mono != (1 << (cp - 1))) return false;
  for (int v = 0; v < 4; ++v) {
    if (v < n_mono && mono_mask[v] != kMasks[cp - 1][v]) return false;
    cf.wm2[v] = v < n_mono ? (float)(-2.0 * mono_w[v]) : 0.f;
  }
  cf.c0 = (float)c0;
  return true;
}

// One slice (4 words) of the chunk's records in registers: thread tid holds
// items tid + 256 q (q < 4) = (word it / kVChunk of the slice, token
// it % kVChunk); zero beyond nt and W.  Loaded ahead of use, so that the
// loads are in flight while other work runs.
template <int NB>
struct VaccSlice {
  uint32_t v[4][NB];
};
template <int NB>
__device__ inline void vacc_load_slice(const uint32_t* planes, int nt, int W, int w0,
                                       VaccSlice<NB>& sl) {
  const int RW = W * NB;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int it = (int)threadIdx.x + 256 * q;
    const int wl = it / kVChunk, t = it % kVChunk, w = w0 + wl;
#pragma unroll
    for (int p = 0; p < NB; ++p) sl.v[q][p] = 0u;
    if (w < W && t < nt) load_words<NB>(planes + (int64_t)t * RW + w * NB, sl.v[q]);
  }
}

// planes: global records of the chunk (token t at planes + t * W * NB), of
// which the caller has loaded slice 0 into `first` (vacc_load_slice with
// w0 = 0); wts: LDS [kVChunk][8] (read for t < nt only); lds:
// vacc_lds_bytes(NB) bytes, 16-aligned.  Callers synchronise before reusing
// wts or lds.
template <int NB, bool MSE>
__device__ void vacc_mfma(const uint32_t* planes, int nt, int W, const float* wts,
                          const VaccCoef cf, char* lds, float* dst, int Dp,
                          const VaccSlice<NB>& first, bool accumulate = false) {
  constexpr int CP = MSE ? NB : NB - 1;       // code planes
  constexpr int NV = 1 << (CP - 1);           // Walsh subsets
  constexpr int NP = MSE ? 1 : 2;             // weight parts: code, sign
  __shared__ int s_e[8];                      // fixed-point exponent per (part, head)
  __shared__ float s_sum[8];                  // sum of the weights per (part, head)
  v4i* aops = (v4i*)lds;                      // [block][part][half][64 lanes]
  uint32_t* wordsT = (uint32_t*)(lds + kVAopsBytes);   // [4 words][NB planes][kVChunk]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // 1. scale and sum per (part, head): wave w takes combos 2w, 2w + 1
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int combo = 2 * wave + q, part = combo >> 2, hh = combo & 3;
    float mx = 0.f, sm = 0.f;
    if (part < NP)
      for (int t = lane; t < nt; t += 64) {
        const float w = wts[8 * t + 4 * part + hh];
        mx = fmaxf(mx, fabsf(w));
        sm += w;
      }
    for (int o = 32; o > 0; o >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, o));
      sm += __shfl_xor(sm, o);
    }
    if (lane == 0) {
      int e = 0;
      if (mx > 0.f) { int ex; frexpf(mx, &ex); e = min(30 - ex, 120); }
      s_e[combo] = e;
      s_sum[combo] = sm;
    }
  }
  __syncthreads();
  // 2. A operands: weight of token t (block b, position tb): token group
  //    tb / 32 sits in lane group [0, 2, 1, 3][tb / 32] (the order the
  //    permlane16 swap leaves), bit tb % 32 = 8 e + 4 h + i is byte e of
  //    register i of half h, shift k = 4 h + i.  An item is the 4 tokens
  //    e = 0..3 of one (block, part, head, group, h, i): their limb words
  //    (A' + 0x80808080) ^ 0x80808080 are byte-transposed so that each
  //    register dword (one limb of the 4 tokens) is one LDS write.
  for (int it = tid; it < (kVChunk / 32) * 4 * 8 * NP; it += 256) {
    const int hi = it & 7, h = hi >> 2, i = hi & 3;       // (h, i) fastest: distinct dwords
    const int rest = it >> 3;
    const int hh = rest & 3, r2 = rest >> 2;
    const int tg = r2 % (kVChunk / 32), part = r2 / (kVChunk / 32);   // 32-token group
    const int combo = 4 * part + hh, e2 = s_e[combo], k = 4 * h + i;
    uint32_t D[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 32 * tg + 8 * e + 4 * h + i;
      const int Q = t < nt ? (int)rintf(ldexpf(wts[8 * t + combo], e2)) : 0;
      const int Ap = (k < 7) ? shift_round(Q, k) : -shift_round(Q, 7);
      D[e] = ((uint32_t)Ap + 0x80808080u) ^ 0x80808080u;
    }
    // 4 x 4 byte transpose: O[L] byte e = D[e] byte L
    const uint32_t t0 = __builtin_amdgcn_perm(D[1], D[0], 0x05010400u);
    const uint32_t t1 = __builtin_amdgcn_perm(D[1], D[0], 0x07030602u);
    const uint32_t t2 = __builtin_amdgcn_perm(D[3], D[2], 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(D[3], D[2], 0x07030602u);
    const uint32_t O[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u),
                           __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                           __builtin_amdgcn_perm(t3, t1, 0x05040100u),
                           __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
    const int b = tg >> 2, grp = tg & 3;
    const int g = (grp == 1) ? 2 : (grp == 2 ? 1 : grp);
    uint32_t* base = (uint32_t*)(aops + ((b * 2 + part) * 2 + h) * 64) + i;
#pragma unroll
    for (int L = 0; L < 4; ++L) base[(16 * g + 4 * hh + L) * 4] = O[L];
  }
  const TransposeLanes tl(lane);
  const int gq = lane >> 4, n = lane & 15;
  // 3. slices of 4 words; the next slice is loaded while this one computes
  VaccSlice<NB> sl = first;
  const int nsplit = W <= 2 ? 2 : 1;          // waves per word (token halves)
  __shared__ float xch[2][2][2][64];          // [word][cb][code, sign][lane]
  for (int w0 = 0; w0 < W; w0 += 4) {
    __syncthreads();            // A operands written / previous slice consumed
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int it = tid + 256 * q;
      const int wl = it / kVChunk, t = it % kVChunk;
#pragma unroll
      for (int p = 0; p < NB; ++p) wordsT[(wl * NB + p) * kVChunk + t] = sl.v[q][p];
    }
    __syncthreads();
    if (w0 + 4 < W) vacc_load_slice<NB>(planes, nt, W, w0 + 4, sl);
    // word of this wave; with at most two words per record the other waves
    // are not idle: a second wave per word takes tokens 128..255 and the two
    // partial sums meet in LDS (nsplit = 2)
    const int wl = nsplit == 2 ? wave % W : wave;       // word within the slice
    const int bh = nsplit == 2 ? wave / W : 0;          // first 128-token block
    const int w = w0 + wl;
    const bool active = w < W && bh < nsplit;
    float pc[2] = {0.f, 0.f}, ps[2] = {0.f, 0.f};       // scaled code / sign sums
    if (active) {
      v4i G[2][NV], S[2];
      // one 128-token block; the first starts the accumulators from an inline
      // zero operand instead of zeroed registers (a block with no tokens has
      // zero bits and weights, so running it is harmless)
      auto block = [&](int b, auto first_c) {
        constexpr bool FIRST = decltype(first_c)::value;
        const v4i zero = {0, 0, 0, 0};
        uint32_t X0[NB], X1[NB];
#pragma unroll
        for (int p = 0; p < NB; ++p) {
          const uint32_t* row = wordsT + (wl * NB + p) * kVChunk + 128 * b;
          const uint32_t t1 = transpose32(row[lane], tl);
          const uint32_t t2 = transpose32(row[64 + lane], tl);
          const auto r = __builtin_amdgcn_permlane16_swap(t1, t2, false, false);
          X0[p] = r[0];           // coordinates 32w + n, token groups 0, 2, 1, 3
          X1[p] = r[1];           // coordinates 32w + 16 + n
        }
        const v4i* ab = aops + b * 4 * 64;
        v4i Ac[2], As[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          Ac[h] = ab[h * 64 + lane];
          if constexpr (!MSE) As[h] = ab[(2 + h) * 64 + lane];
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const uint32_t* X = cb ? X1 : X0;
#pragma unroll
          for (int m = 0; m < NV; ++m) {
            uint32_t u = 0u;
#pragma unroll
            for (int p = 0; p < CP; ++p)
              if ((walsh_mask<CP>(m) >> p) & 1) u ^= X[p];
            G[cb][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ac[0], bit_lanes(u, 0),
                                                             FIRST ? zero : G[cb][m], 0, 0, 0);
            G[cb][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ac[1], bit_lanes(u, 1), G[cb][m], 0, 0, 0);
          }
          if constexpr (!MSE) {
            S[cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(As[0], bit_lanes(X[NB - 1], 0),
                                                          FIRST ? zero : S[cb], 0, 0, 0);
            S[cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(As[1], bit_lanes(X[NB - 1], 1), S[cb], 0, 0, 0);
          }
        }
      };
      block(bh, std::true_type{});
      for (int b = bh + nsplit; b * 128 < nt; b += nsplit) block(b, std::false_type{});
      // lane (g, n): head g at coordinate 32w + 16cb + n
      const float sc0 = ldexpf(1.f, -s_e[gq]);
      const float sc1 = MSE ? 0.f : ldexpf(2.f, -s_e[4 + gq]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float code = 0.f;
#pragma unroll
        for (int m = 0; m < NV; ++m) code = fmaf(cf.wm2[m], limbs_to_float(G[cb][m]), code);
        pc[cb] = code * sc0;
        if constexpr (!MSE) ps[cb] = limbs_to_float(S[cb]) * sc1;
      }
    }
    if (nsplit == 2) {                    // uniform: W is the same for the block
      if (active && bh == 1)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          xch[wl][cb][0][lane] = pc[cb];
          xch[wl][cb][1][lane] = ps[cb];
        }
      __syncthreads();
      if (active && bh == 0)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          pc[cb] += xch[wl][cb][0][lane];
          ps[cb] += xch[wl][cb][1][lane];
        }
    }
    if (active && bh == 0) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int j = 32 * w + 16 * cb + n;
        float v0 = pc[cb] + cf.c0 * s_sum[gq];
        float v1 = MSE ? 0.f : ps[cb] - s_sum[4 + gq];
        if (accumulate) {         // this block's own partial from an earlier call
          v0 += dst[gq * Dp + j];
          v1 += dst[(4 + gq) * Dp + j];
        }
        dst[gq * Dp + j] = v0;
        dst[(4 + gq) * Dp + j] = v1;
      }
    }
  }
}

// ---- finishing a query head: chunk partials -> output -----------------------
// Block-wide (256 threads).  Threads split as NL = min(Dp / 4, 256) lanes over
// float4 groups of the outputs x 256 / NL groups over the chunks; the chunk
// groups' partial sums meet in LDS `red` (>= 2048 floats).  Each thread keeps
// 4 chunk steps x 2 rows of float4 loads in flight: the reduction reads the
// whole partial array once and is bound by how many loads are outstanding.

// arot[j] = sc * sum_c f_c part_c[r0][j],  ask[j] = sc * sum_c f_c part_c[r1][j]
// for j < Dp, chunk c's rows at part + c * 8 * Dp (16-byte aligned, Dp a
// multiple of 4); f_c = fac[c] (LDS) or 1.
__device__ inline void sum_chunk_partials(const float* part, int n_chunk, int r0, int r1, int Dp,
                                          const float* fac, float sc, float* red, float* arot,
                                          float* ask) {
  const int tid = threadIdx.x;
  const int D4 = Dp / 4;
  const int NL = min(D4, 256), TT = 256 / NL;
  const int lj = tid % NL, tg = tid / NL;
  float4* red4 = (float4*)red;                  // [2][TT][NL]
  auto fma4 = [](float f, float4 v, float4 acc) {
    return make_float4(fmaf(f, v.x, acc.x), fmaf(f, v.y, acc.y), fmaf(f, v.z, acc.z),
                       fmaf(f, v.w, acc.w));
  };
  auto add4 = [](float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
  };
  for (int j0 = 0; j0 < D4; j0 += NL) {
    const int j4 = j0 + lj;
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 a1[4] = {z4, z4, z4, z4}, a2[4] = {z4, z4, z4, z4};
    if (tg < TT && j4 < D4) {
      const float4* p1 = (const float4*)(part + r0 * Dp) + j4;
      const float4* p2 = (const float4*)(part + r1 * Dp) + j4;
      const int64_t cs = 2 * Dp;                 // float4s per chunk (8 rows)
      int c = tg;
      for (; c + 3 * TT < n_chunk; c += 4 * TT) {
        float4 v1[4], v2[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v1[u] = p1[(int64_t)(c + u * TT) * cs];
          v2[u] = p2[(int64_t)(c + u * TT) * cs];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float f = fac ? fac[c + u * TT] : 1.f;
          a1[u] = fma4(f, v1[u], a1[u]);
          a2[u] = fma4(f, v2[u], a2[u]);
        }
      }
      for (; c < n_chunk; c += TT) {
        const float f = fac ? fac[c] : 1.f;
        a1[0] = fma4(f, p1[(int64_t)c * cs], a1[0]);
        a2[0] = fma4(f, p2[(int64_t)c * cs], a2[0]);
      }
    }
    if (tg < TT) {          // threads past TT * NL (256 % NL != 0) only idle
      red4[tg * NL + lj] = add4(add4(a1[0], a1[1]), add4(a1[2], a1[3]));
      red4[(TT + tg) * NL + lj] = add4(add4(a2[0], a2[1]), add4(a2[2], a2[3]));
    }
    __syncthreads();
    if (tid < NL && j0 + tid < D4) {
      float4 t1 = z4, t2 = z4;
      for (int q = 0; q < TT; ++q) {
        t1 = add4(t1, red4[q * NL + tid]);
        t2 = add4(t2, red4[(TT + q) * NL + tid]);
      }
      const int j = 4 * (j0 + tid);
      arot[j] = t1.x * sc; arot[j + 1] = t1.y * sc; arot[j + 2] = t1.z * sc; arot[j + 3] = t1.w * sc;
      ask[j] = t2.x * sc; ask[j + 1] = t2.y * sc; ask[j + 2] = t2.z * sc; ask[j + 3] = t2.w * sc;
    }
    __syncthreads();
  }
}

// out[i] = sum_j Pi[j][i] arot[j] + alpha sum_j S[j][i] ask[j]  (i < d; the
// second sum only when qjl), with Pi and S row-major fp32 [d][d].  Threads
// split as NI = min(d / 4, 256) lanes over float4 groups of outputs x 256 / NI
// groups over j (4 independent float4 row loads per matrix in flight), met in
// LDS `red` (>= 2048 floats); d is a multiple of 8, so 4 | d, rows are 16-byte
// aligned.
__device__ inline void apply_transforms(const float* pi32, const float* s32, int d, bool qjl,
                                        float alpha, const float* arot, const float* ask,
                                        float* red, float* out) {
  const int tid = threadIdx.x;
  const int D4 = d / 4;
  const int NI = min(D4, 256), TT = 256 / NI;
  const int li = tid % NI, tg = tid / NI;
  float4* red4 = (float4*)red;                  // [TT][NI]
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fma4 = [](float f, float4 v, float4 acc) {
    return make_float4(fmaf(f, v.x, acc.x), fmaf(f, v.y, acc.y), fmaf(f, v.z, acc.z),
                       fmaf(f, v.w, acc.w));
  };
  auto add4 = [](float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
  };
  for (int i0 = 0; i0 < D4; i0 += NI) {
    const int i4 = i0 + li;
    float4 o1[4] = {z4, z4, z4, z4}, o2[4] = {z4, z4, z4, z4};
    if (tg < TT && i4 < D4) {
      const float4* P = (const float4*)pi32 + i4;
      const float4* S = (const float4*)s32 + i4;
      int j = tg;
      for (; j + 3 * TT < d; j += 4 * TT) {
        float4 vp[4], vs[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          vp[u] = P[(int64_t)(j + u * TT) * D4];
          if (qjl) vs[u] = S[(int64_t)(j + u * TT) * D4];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          o1[u] = fma4(arot[j + u * TT], vp[u], o1[u]);
          if (qjl) o2[u] = fma4(ask[j + u * TT], vs[u], o2[u]);
        }
      }
      for (; j < d; j += TT) {
        o1[0] = fma4(arot[j], P[(int64_t)j * D4], o1[0]);
        if (qjl) o2[0] = fma4(ask[j], S[(int64_t)j * D4], o2[0]);
      }
    }
    const float4 s1 = add4(add4(o1[0], o1[1]), add4(o1[2], o1[3]));
    const float4 s2 = add4(add4(o2[0], o2[1]), add4(o2[2], o2[3]));
    const float4 v = make_float4(fmaf(alpha, s2.x, s1.x), fmaf(alpha, s2.y, s1.y),
                                 fmaf(alpha, s2.z, s1.z), fmaf(alpha, s2.w, s1.w));
    if (tg < TT) red4[tg * NI + li] = v;   // threads past TT * NI only idle
    __syncthreads();
    if (tid < NI && i0 + tid < D4) {
      float4 t = z4;
      for (int q = 0; q < TT; ++q) t = add4(t, red4[q * NI + tid]);
      const int i = 4 * (i0 + tid);
      out[i] = t.x;
      out[i + 1] = t.y;
      out[i + 2] = t.z;
      out[i + 3] = t.w;
    }
    __syncthreads();
  }
}

}  // namespace dev
}  // namespace tq
