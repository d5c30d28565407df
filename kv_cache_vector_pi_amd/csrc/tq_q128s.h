// Quantization for head_dim 128 with bf16 input, organised for long calls
// (cache fills): the same method and results as q128_tiles (turboquant.net
// pseudo-code "quant"; admirer.cn two-stage description; residual norm as
// fp16 from the "potential challenges" section), with a different schedule.
//
//  * Blocks of 32 vectors (all in one head: the caller's token count is a
//    multiple of 32) flow through a software pipeline run by two roles of
//    four waves each, which meet at one barrier per step.  In step j
//      - the code waves decide the codes of block j from Y(j) (computed at
//        the end of step j-1), write its residual to LDS, then run the MFMAs
//        of Y(j+1) = Pi x(j+1);
//      - the sketch waves run the MFMAs of Z(j-1) = M r(j-1) (while the code
//        waves' vector units decide codes), take the signs and store block
//        j-1's records and norms, issue the copy of block j+5 from HBM
//        straight into LDS (global_load_lds_dwordx4: no registers held while
//        in flight), compute the norms of block j+2 from LDS, and wait for
//        block j+3's copy.
//  * Y = Pi x runs on v_mfma_f32_32x32x16_bf16 straight on the raw bf16
//    input, with Pi split into two bf16 parts (hi + mid, |Pi - hi - mid| <=
//    2^-18 |Pi| elementwise), so no conversion of x is needed: the rotated
//    coordinate errs by at most 2^-18 ||Pi_j|| ||x|| = 3.8e-6 ||x|| (Cauchy-
//    Schwarz), inside the 1e-5 decision margin.  The codes compare y = acc/nu
//    with the thresholds as acc against t * nu.
//  * The residual r = (acc - nu c) 2^-e (a power-of-two scale keeps it near
//    unit size) is written as fp16 hi/lo and Z = M r takes three fp16
//    passes, as in q128_tiles; sign(z) does not depend on the positive scale,
//    and gamma = ||r|| / (nu 2^-e).
//  * Norms come from the input itself (sum of squares of the bf16 values),
//    so nu is exact to fp32 rounding.  A vector whose squared norm falls
//    outside [2^-120, 2^120] is rescaled in LDS by a power of two before its
//    Y, so the products (and the norm) stay inside fp32's normal range.
//  * x rows land in LDS 256 bytes apart with their 16-byte chunks permuted
//    (chunk c of row r at slot c ^ (r & 15)), so the MFMA operand reads of 16
//    rows at one chunk hit distinct banks.
//  * Code wave w and sketch wave 4 + w own output coordinates 32w..32w+31;
//    their slices of Pi (bf16 hi, mid) and of M (fp16 hi, lo) stay in
//    registers for the whole call.  Every sketch wave stores its record
//    words and (redundantly, identical values) the block's norms with all 64
//    lanes active, so each step issues a fixed number of memory
//    instructions and the wait for a copy in flight can name its exact
//    count.
#pragma once
#include "tq_dma.h"
#include "tq_q128.h"

namespace tq {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kSB = 32;       // vectors per block
constexpr int kSD = 5;        // x blocks resident in LDS: the copy lead in steps
constexpr int kSR = 136;      // LDS row stride of the residual, in halves

struct Q128SArgs {
  const uint16_t* x;                 // bf16 bits
  int64_t x_stride_token, x_stride_head;
  uint32_t n_tokens;                 // per head, a multiple of 32
  uint32_t n_blocks;                 // n_heads * n_tokens / 32
  uint32_t blk_per_head;             // n_tokens / 32
  uint32_t div_m, div_s1, div_s2;    // block / blk_per_head by multiply-shift
  uint32_t* planes;
  uint32_t* norms;
  int64_t dst_stride_head, dst_token0;
  const uint16_t* pib_hi;            // bf16 bits of Pi, [128][128]
  const uint16_t* pib_mid;           // bf16 bits of Pi - hi
  const __half* m_hi;
  const __half* m_lo;
  float thr[4];                      // positive thresholds t_{K/2} .. t_{K-2}
  float cpos[4];                     // positive centroids c_{K/2} .. c_{K-1}
};

// n / blk_per_head (multiply-shift, as fast_div)
__device__ inline uint32_t head_of(uint32_t n, const Q128SArgs& a) {
  const uint32_t t = __umulhi(n, a.div_m);
  return (t + ((n - t) >> a.div_s1)) >> a.div_s2;
}

template <int NB, bool MSE>
__device__ __forceinline__ void q128s_body(const Q128SArgs& a) {
  constexpr int CP = MSE ? NB : NB - 1;   // code planes
  constexpr int K = 1 << CP;
  constexpr int KH = K / 2;               // positive centroids
  constexpr int NT = KH - 1;              // positive thresholds
  constexpr int NR = MSE ? 1 : 2;         // residual buffers
  __shared__ __align__(16) uint16_t xb[kSD][kSB * 128];          // raw bf16 blocks
  __shared__ __align__(16) _Float16 rh_s[NR][MSE ? 8 : kSB * kSR];
  __shared__ __align__(16) _Float16 rl_s[NR][MSE ? 8 : kSB * kSR];
  __shared__ float4 prm[4][kSB];         // per vector: nu', 2^-e', nu' 2^-e', nu16 bits
  __shared__ float gp[2][4][kSB];        // per coordinate group: partial sums of r^2
  __shared__ uint32_t cwb[2][4][kSB][CP];  // code words per (group, vector)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool yrole = wave < 4;            // uniform per wave
  const int grp = wave & 3;               // coordinates 32 grp .. 32 grp + 31
  const int col = lane & 31, hh = lane >> 5;
  const uint32_t G = gridDim.x, g = blockIdx.x;
  if (g >= a.n_blocks) return;
  const int nb = (int)((a.n_blocks - 1 - g) / G) + 1;     // blocks of this workgroup

  // ---- copy of local block j into LDS buffer j % kSD (sketch waves) -------
  // sketch wave grp copies rows 8 grp .. 8 grp + 7 as two 1 KB pieces (4 rows
  // each); lane l of piece i fills slot l % 16 of row 8 grp + 4i + l / 16
  // with the row's chunk (slot ^ (row & 15))
  auto copy_block = [&](int j) {
    const uint32_t blk = g + (uint32_t)j * G;
    const uint32_t h = head_of(blk, a);
    const uint32_t t0 = (blk - h * a.blk_per_head) * kSB;
    const uint16_t* base = a.x + (int64_t)h * a.x_stride_head + (int64_t)t0 * a.x_stride_token;
    const int buf = j % kSD;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 8 * grp + 4 * i + (lane >> 4);
      const int chunk = (lane & 15) ^ (row & 15);
      const uint16_t* src = base + (int64_t)row * a.x_stride_token + 8 * chunk;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(
          lds_addr(&xb[buf][(8 * grp + 4 * i) * 128]));
      copy16_to_lds(src, m0);
    }
  };

  // ---- norms of local block j (sketch waves): vectors 8 grp .. 8 grp + 7 --
  // lane: vector 8 grp + lane / 8, chunks 2 (lane % 8) and +1
  auto norms_block = [&](int j) {
    const int buf = j % kSD;
    const int v = 8 * grp + (lane >> 3);
    const int q = lane & 7;
    uint16_t* rowp = &xb[buf][v * 128];
    uint4* p0 = (uint4*)(rowp + 8 * ((2 * q) ^ (v & 15)));
    uint4* p1 = (uint4*)(rowp + 8 * ((2 * q + 1) ^ (v & 15)));
    uint4 u0 = *p0, u1 = *p1;
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const v2bf pr = __builtin_bit_cast(v2bf, w[e]);
      ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
    }
    ss = row8_sum(ss);
    // the common case: ||x||^2 inside [2^-120, 2^120]
    float nu = __builtin_amdgcn_sqrtf(ss), nup = nu;
    // otherwise (zero, tiny, huge or not finite): scale the vector's bf16
    // values in LDS by 2^k (exact) so that its largest magnitude is in
    // [0.5, 1), recompute the norm, and keep nu = nu' 2^-k; the products of
    // Y then stay inside fp32's normal range.  All 8 lanes of a vector take
    // the same branch.
    const bool odd = !(ss >= 0x1p-120f && ss <= 0x1p120f);
    if (__builtin_amdgcn_ballot_w64(odd)) {
      if (odd) {
        uint32_t mx = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          mx = max(mx, max(w[e] & 0x7fffu, (w[e] >> 16) & 0x7fffu));
        mx = row8_max(mx);
        if (mx == 0u || mx >= 0x7f80u) {       // zero, or inf / NaN present: no scaling
          nu = nup = (mx == 0u) ? 0.f : __builtin_amdgcn_sqrtf(ss);
        } else {
          int ex;
          frexpf(__uint_as_float(mx << 16), &ex);
          const int k = -ex;
          uint32_t o[8];
          float s2 = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float lo = ldexpf(__uint_as_float(w[e] << 16), k);
            const float hi = ldexpf(__uint_as_float(w[e] & 0xffff0000u), k);
            o[e] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
            const v2bf pr = __builtin_bit_cast(v2bf, o[e]);
            s2 = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, s2, false);
          }
          *p0 = make_uint4(o[0], o[1], o[2], o[3]);
          *p1 = make_uint4(o[4], o[5], o[6], o[7]);
          nup = __builtin_amdgcn_sqrtf(row8_sum(s2));
          nu = ldexpf(nup, -k);
        }
      }
    }
    int ex = 0;
    if (nup > 0.f) frexpf(nup, &ex);
    const float s = ldexpf(1.f, -ex);
    if (q == 0)
      prm[j & 3][v] = make_float4(nup, s, nup * s,
                                  __uint_as_float((uint32_t)__half_as_ushort(__float2half_rn(nu))));
  };

  if (yrole) {
    // ======== code waves: Y = Pi x on the raw bf16 input, codes, residual ===
    v8bf Ph[8], Pm[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int off = (32 * grp + col) * 128 + 16 * ks + 8 * hh;
      Ph[ks] = *(const v8bf*)(a.pib_hi + off);
      Pm[ks] = *(const v8bf*)(a.pib_mid + off);
    }
    // Y(j): 16 MFMAs on block j's raw rows (chunk c of row r at slot c ^ (r & 15)),
    // hi and mid products in one accumulator (back-to-back MFMAs on the same
    // accumulator issue without a stall), the operand read of step ks + 1
    // issued before the MFMAs of step ks
    auto y_block = [&](v16f& acc, int j) {
      const uint16_t* xr = &xb[j % kSD][col * 128];
      acc = v16f{};
      v8bf xf = *(const v8bf*)(xr + 8 * (hh ^ (col & 15)));
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        v8bf xn = xf;
        if (ks < 7) xn = *(const v8bf*)(xr + 8 * ((2 * ks + 2 + hh) ^ (col & 15)));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ph[ks], xf, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Pm[ks], xf, acc, 0, 0, 0);
        xf = xn;
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    // Codes of block j from acc = Y(j).  Element i of a lane is coordinate
    // 32 grp + 8 (i/4) + 4 hh + i%4 of vector col.  acc = Pi x' with x' = x 2^k
    // (k = 0 but for rescaled vectors) and nu' = ||x'||: y = acc / nu'.
    // idx = pos ? KH + m : KH-1-m with m the number of positive thresholds
    // below |y| (|acc| > t nu'); the top code bit is pos, the lower bits m
    // (pos) or ~m, from lane-mask algebra on the compares, shifted in from
    // i = 15 down.  Residual in acc units scaled by s = 2^-e':
    // r = (acc - nu' c) s = +-(|acc| s - c nu' s), written as fp16 hi/lo in
    // groups of four consecutive coordinates as soon as each group is done.
    auto codes = [&](const v16f& acc, int j) {
      const float4 pv = prm[j & 3][col];
      const float nup = pv.x, s = pv.y, nus = pv.z;
      float thr_v[NT > 0 ? NT : 1], cs[KH];
#pragma unroll
      for (int k = 0; k < NT; ++k) thr_v[k] = a.thr[k] * nup;
#pragma unroll
      for (int k = 0; k < KH; ++k) cs[k] = a.cpos[k] * nus;
      uint32_t bacc[3] = {0u, 0u, 0u};
      float g2 = 0.f;
      float rr[4];
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        const float y = acc[i];
        const float ay = fabsf(y);
        const bool pos = y > 0.f;
        const uint64_t P = __builtin_amdgcn_ballot_w64(pos);
        uint64_t Gm[NT > 0 ? NT : 1];
        float cm = cs[0];
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          const bool gt = ay > thr_v[k];
          Gm[k] = __builtin_amdgcn_ballot_w64(gt);
          cm = gt ? cs[k + 1] : cm;
        }
        const float ra = fmaf(ay, s, -cm);
        const float r = pos ? ra : -ra;
        rr[i & 3] = r;
        g2 = fmaf(r, r, g2);
        bacc[CP - 1] = shift_in(bacc[CP - 1], P);
        if constexpr (CP == 2) {
          bacc[0] = shift_in(bacc[0], ~(Gm[0] ^ P));
        } else if constexpr (CP == 3) {
          bacc[1] = shift_in(bacc[1], ~(Gm[1] ^ P));
          bacc[0] = shift_in(bacc[0], ~(Gm[0] ^ Gm[1] ^ Gm[2] ^ P));
        }
        if constexpr (!MSE) {
          if ((i & 3) == 0) {         // coordinates 8 (i/4) + 4 hh .. +3 complete
            typedef uint32_t u2v __attribute__((ext_vector_type(2)));
            v4h rh;
#pragma unroll
            for (int e = 0; e < 4; ++e) rh[e] = (_Float16)rr[e];
            const u2v hb = __builtin_bit_cast(u2v, rh);
            u2v lb;
            lb[0] = lo_pair(rr[0], rr[1], hb[0]);
            lb[1] = lo_pair(rr[2], rr[3], hb[1]);
            const int off = col * kSR + 32 * grp + 8 * (i >> 2) + 4 * hh;
            *(v4h*)(rh_s[j & 1] + off) = rh;
            *(u2v*)(rl_s[j & 1] + off) = lb;
          }
        }
      }
      if constexpr (!MSE) gp[j & 1][grp][col] = halves_sum(g2);   // both halves: same value
#pragma unroll
      for (int p = 0; p < CP; ++p) cwb[j & 1][grp][col][p] = halves_or(spread16(bacc[p], hh));
    };

    __syncthreads();            // copies of blocks 0-2 landed
    __syncthreads();            // norms (and rescales) of blocks 0, 1 written
    v16f ya;
    y_block(ya, 0);
    __syncthreads();            // Y(0) has read buffer 0, which step 0 refills
    for (int j = 0; j <= nb; ++j) {
      codes(ya, j);             // block nb: stale buffers, results unused
      __builtin_amdgcn_sched_barrier(0);
      y_block(ya, j + 1);
      __syncthreads();
    }
  } else {
    // ======== sketch waves: copies, norms, Z = M r, signs, stores ==========
    v8h Mh[8], Ml[8];
    if constexpr (!MSE) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = (32 * grp + col) * 128 + 16 * ks + 8 * hh;
        Mh[ks] = *(const v8h*)(a.m_hi + off);
        Ml[ks] = *(const v8h*)(a.m_lo + off);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): tables in before the copies start
    // Z(j) = M r(j): 24 MFMAs on the residual's fp16 hi and lo parts, in one
    // accumulator (a second would not fit the register budget; the other
    // waves' work fills the chain's gaps), with the operand reads of step
    // ks + 1 issued before the MFMAs of step ks
    auto z_block = [&](v16f& z, int j) {
      z = v16f{};
      if constexpr (!MSE) {
        const _Float16* rh = rh_s[j & 1] + col * kSR + 8 * hh;
        const _Float16* rl = rl_s[j & 1] + col * kSR + 8 * hh;
        v8h h0 = *(const v8h*)rh, l0 = *(const v8h*)rl;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          v8h h1 = h0, l1 = l0;
          if (ks < 7) {
            h1 = *(const v8h*)(rh + 16 * (ks + 1));
            l1 = *(const v8h*)(rl + 16 * (ks + 1));
          }
          z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Mh[ks], h0, z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ml[ks], h0, z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Mh[ks], l0, z, 0, 0, 0);
          h0 = h1;
          l0 = l1;
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks < 6; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
      }
    };
    // signs of Z(j) and the stores of block j's record group grp and norms;
    // every lane stores (identical values where two lanes or waves write the
    // same word)
    auto finish = [&](const v16f& z, int j) {
      uint32_t sw = 0u;
      if constexpr (!MSE) {
        // sign bits of z shifted in from i = 15 down (v_alignbit: one vector op
        // per coordinate), then inverted: bit set <=> z >= 0 (z is never -0:
        // the accumulators start at +0)
        uint32_t sn = 0u;
#pragma unroll
        for (int i = 15; i >= 0; --i) sn = __builtin_amdgcn_alignbit(sn, __float_as_uint(z[i]), 31);
        sw = halves_or(spread16(~sn, hh));
      }
      const uint32_t blk = g + (uint32_t)j * G;
      const uint32_t h = head_of(blk, a);
      const uint32_t t0 = (blk - h * a.blk_per_head) * kSB;
      const int64_t rec = (int64_t)h * a.dst_stride_head + a.dst_token0 + t0 + col;
      uint32_t* gw = a.planes + (rec * 4 + grp) * NB;     // group grp of record col
      uint32_t wd[NB];
#pragma unroll
      for (int p = 0; p < CP; ++p) wd[p] = cwb[j & 1][grp][col][p];
      if constexpr (!MSE) wd[NB - 1] = sw;
      if constexpr (NB == 4) {
        *(uint2*)(gw + 2 * hh) = hh ? make_uint2(wd[2], wd[3]) : make_uint2(wd[0], wd[1]);
      } else if constexpr (NB == 3) {
        *(uint2*)(gw + hh) = hh ? make_uint2(wd[1], wd[2]) : make_uint2(wd[0], wd[1]);
      } else if constexpr (NB == 2) {
        gw[hh] = hh ? wd[1] : wd[0];
      } else {
        gw[0] = wd[0];
      }
      // norms: (nu16, gamma16); gamma = ||r|| / (nu' 2^-e')
      const float4 pv = prm[j & 3][col];
      float gam = 0.f;
      if constexpr (!MSE) {
        const float sq = (gp[j & 1][0][col] + gp[j & 1][1][col]) +
                         (gp[j & 1][2][col] + gp[j & 1][3][col]);
        gam = pv.z > 0.f ? __builtin_amdgcn_sqrtf(sq) * __builtin_amdgcn_rcpf(pv.z) : 0.f;
      }
      const uint32_t gb = (uint32_t)__half_as_ushort(__float2half_rn(gam));
      a.norms[rec] = __float_as_uint(pv.w) | (gb << 16);
    };

    // prologue: copies of blocks 0 .. kSD-1, norms of 0 and 1
    const int pre = nb < kSD ? nb : kSD;
    for (int j = 0; j < pre; ++j) copy_block(j);
    wait_vmcnt(2 * (pre - (nb < 3 ? nb : 3)));     // blocks 0, 1, 2 landed
    __syncthreads();
    norms_block(0);
    if (nb > 1) norms_block(1);
    __syncthreads();
    __syncthreads();            // the code waves' Y(0) is done with buffer 0
    for (int j = 0; j <= nb; ++j) {
      // Z first: its MFMAs run while the code waves decide codes
      if (j >= 1) {
        v16f z;
        z_block(z, j - 1);
        finish(z, j - 1);
      }
      if (j + kSD < nb) copy_block(j + kSD);
      if (j + 2 < nb) norms_block(j + 2);
      // block j + 3 must have landed before its norms in the next step.
      // Issued after it: copies of blocks j+4 .. min(j+kSD, nb-1) (2 each),
      // and the stores of steps max(1, s+1) .. j (2 each), s the step that
      // issued it (its own stores precede the copy; s < 0: the prologue)
      if (j + 3 < nb) {
        const int issued_at = j + 3 - kSD;
        const int last_copy = (j + kSD < nb ? j + kSD : nb - 1);
        int after = 2 * (last_copy - (j + 3));
        const int from = issued_at < 0 ? 1 : issued_at + 1;
        for (int s = (from < 1 ? 1 : from); s <= j; ++s) after += 2;
        wait_vmcnt(after);
      }
      __syncthreads();
    }
  }
}

}  // namespace
}  // namespace tq
