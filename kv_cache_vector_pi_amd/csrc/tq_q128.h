// Quantization for head_dim 128 (the KV-cache case), specialised for gfx950.
// Same method and results as the generic kernel (turboquant.net pseudo-code
// "quant"; admirer.cn two-stage description; residual norm as fp16 from the
// "potential challenges" section), organised for throughput:
//
//  * 4 waves per workgroup, wave w owns word w of every plane (output
//    coordinates 32w..32w+31 = one 32-row block of v_mfma_f32_32x32x16_f16);
//    its slices of Pi and M (hi and lo fp16 parts) stay in registers.
//  * 64 vectors per tile (two 32-column blocks); x_s and the residual live
//    in separate LDS buffers as fp16 hi/lo pairs (two barriers per tile), and
//    the next tile's x is loaded into registers while this one computes.
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
//  * Tiles run over the flattened (head, token) rows of a launch, so many
//    short heads (one new token per head and layer in decoding) share a
//    tile; a tile inside one head reads and writes contiguous rows.
//  * Head dimension 64 (template D = 64) runs the same code on token pairs: a
//    tile row is two consecutive tokens of one head (coordinates 0..63 the
//    first, 64..127 the second), waves 0-1 take the first token's two words
//    and waves 2-3 the second's, each against the 64 x 64 tables over its
//    token's 64 coordinates (half the MFMAs and table registers).  The pair's
//    four record groups are exactly the two tokens' records back to back, so
//    the staging and stores are unchanged; norms and scales are per token.
#pragma once
#include <algorithm>
#include <cmath>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kT = 64;        // vectors per tile
constexpr int kLdx = 136;     // LDS row stride in halves (128 + 8)

struct Q128Args {
  const void* x;
  int64_t x_stride_token, x_stride_head;
  int64_t n_tokens;
  uint32_t* planes;
  uint32_t* norms;
  int64_t dst_stride_head, dst_token0;
  const int64_t* slots;              // per-token destination, or null (dst_token0 + t)
  const __half* pi_hi;
  const __half* pi_lo;
  const __half* m_hi;
  const __half* m_lo;
  uint32_t n_tiles, n_rows;          // rows: n_heads * n_tokens of this launch
  uint32_t div_m, div_s1, div_s2;   // row / n_tokens by multiply-shift
  float thr[4];     // positive thresholds t_{K/2} .. t_{K-2}
  float cpos[4];    // positive centroids c_{K/2} .. c_{K-1}
};

// n / d for 32-bit n by the round-up multiply-shift method (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1.
inline void make_div(uint32_t d, uint32_t& m, uint32_t& s1, uint32_t& s2) {
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
  s1 = l < 1 ? l : 1;
  s2 = l > 0 ? l - 1 : 0;
}
__device__ inline uint32_t fast_div(uint32_t n, const Q128Args& a) {
  const uint32_t t = __umulhi(n, a.div_m);
  return (t + ((n - t) >> a.div_s1)) >> a.div_s2;
}

// rows held by lane half h (0/1) of a 32x32 C block: 8*(i/4) + 4*h + i%4.
// Spread a 16-bit value (bit i <-> row of element i) to those word positions.
__device__ inline uint32_t spread16(uint32_t v, int h) {
  uint32_t x = (v & 0xffu) | ((v & 0xff00u) << 8);    // bytes 0 and 2
  x = (x | (x << 4)) & 0x0f0f0f0fu;                     // one nibble per byte
  return x << (4 * h);
}

// acc * 2 + (bit of this lane in `mask`): one v_addc with the lane mask of a
// compare as carry-in, so a code or sign bit costs one vector op.
__device__ inline uint32_t shift_in(uint32_t acc, uint64_t mask) {
  uint32_t out;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(out), "=s"(carry_out) : "v"(acc), "s"(mask));
  return out;
}

// Low fp16 parts of a residual pair: fp16(r - hi) for (r0, hi0) and (r1, hi1),
// hi0 / hi1 the low / high half of h01.  v_fma_mix forms r * 1 - hi in fp32
// and rounds once to fp16; r - hi is exact in fp32 (hi is r rounded to
// fp16), so this is the plain conversion of (r - (float)hi) in one
// instruction per element instead of three.
__device__ inline uint32_t lo_pair(float r0, float r1, uint32_t h01) {
  uint32_t out;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(out) : "v"(r0), "v"(h01));
  asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "+v"(out) : "v"(r1), "v"(h01));
  return out;
}

// Combine a value with the one in lane l ^ 32 (v_permlane32_swap: with both
// operands v it returns v[l mod 32] and v[32 + l mod 32] in every lane l).
__device__ inline uint32_t halves_or(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] | r[1];
}
__device__ inline float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over each row of 16 lanes (DPP: swap neighbours, swap pairs, mirror
// within 8, mirror within 16); every lane of the row gets the total.
__device__ inline float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
  return x;
}

// Sum over each group of 8 lanes (the first three steps of row16_sum).
__device__ inline float row8_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  return x;
}

// Maximum over each group of 8 lanes (the row8_sum pattern with max).
__device__ inline uint32_t row8_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, true));
  return x;
}

template <bool BF16>
struct RawX {
  uint4 v[BF16 ? 4 : 8];
};

// Rows f0 .. f0 + cnt - 1 of a tile: (head, token) of row f is
// (f / n_tokens, f % n_tokens).  `one` (uniform): all in head h0 from t0.
struct TileRows {
  uint32_t f0, h0, t0;
  int cnt;
  bool one;
};
__device__ inline TileRows tile_rows(uint32_t tile, const Q128Args& a) {
  TileRows r;
  r.f0 = tile * kT;
  r.h0 = fast_div(r.f0, a);
  r.t0 = r.f0 - r.h0 * (uint32_t)a.n_tokens;
  r.cnt = (int)min((uint32_t)kT, a.n_rows - r.f0);
  r.one = (int64_t)r.t0 + r.cnt <= a.n_tokens;
  return r;
}
// (head, token) of row f0 + v
__device__ inline void row_ht(const TileRows& r, int v, const Q128Args& a, uint32_t& h,
                              uint32_t& t) {
  if (r.one) {
    h = r.h0;
    t = r.t0 + v;
  } else {
    const uint32_t f = r.f0 + v;
    h = fast_div(f, a);
    t = f - h * (uint32_t)a.n_tokens;
  }
}

// Loads of one 64-row tile: pass p covers row 4*wave + 16*p + lane/16,
// 8-element chunk lane%16 (D = 64: token (lane%16)/8 of the row's pair, chunk
// lane%8).  Rows past the end of the launch read as zero.
template <bool BF16, int D>
__device__ inline void load_tile(RawX<BF16>& raw, const Q128Args& a, uint32_t tile, int wave,
                                 int lane) {
  constexpr int TPV = 128 / D;                       // tokens per row
  const int tp = D == 64 ? (lane & 15) >> 3 : 0;     // token of the pair
  const int cc = D == 64 ? (lane & 7) : (lane & 15); // 8-element chunk of the token
  const TileRows r = tile_rows(tile, a);
  // vectors past the end re-read the tile's first row (always valid); the
  // consumer zeroes them, so no lane branches around a load and nothing
  // waits for it
  auto load = [&](int p, int64_t off) {
    if constexpr (BF16) {
      raw.v[p] = *(const uint4*)((const uint16_t*)a.x + off);
    } else {
      raw.v[2 * p] = *(const uint4*)((const float*)a.x + off);
      raw.v[2 * p + 1] = *(const uint4*)((const float*)a.x + off + 4);
    }
  };
  if (r.one) {        // uniform branch: rows t0 .. t0 + cnt - 1 of head h0
    // row offsets within the tile in 32 bits (the launcher keeps
    // x_stride_token below 2^25 elements, 2^24 for D = 64)
    const int64_t base =
        (int64_t)r.h0 * a.x_stride_head + (int64_t)TPV * r.t0 * a.x_stride_token;
    const int32_t xst = (int32_t)a.x_stride_token;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int v = 4 * wave + 16 * p + (lane >> 4);
      load(p, base + (int64_t)((TPV * (v < r.cnt ? v : 0) + tp) * xst + 8 * cc));
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int v = 4 * wave + 16 * p + (lane >> 4);
      const uint32_t f = r.f0 + (v < r.cnt ? v : 0);
      const uint32_t h = fast_div(f, a), t = f - h * (uint32_t)a.n_tokens;
      load(p, (int64_t)h * a.x_stride_head + ((int64_t)TPV * t + tp) * a.x_stride_token + 8 * cc);
    }
  }
}

// NB: words per record group; MSE: all NB planes are code planes (no QJL
// stage, gamma stored as 0), else NB-1 code planes and the sign plane.
// The tiles tile0, tile0 + stride, ... of a launch, by one 256-thread
// workgroup (the kernel body; launch bounds: 256 threads, 2 workgroups per CU,
// 3 for MSE-only records).
template <int NB, bool BF16, bool MSE, int D = 128>
__device__ __forceinline__ void q128_tiles(const Q128Args& a, uint32_t tile0, uint32_t stride) {
  static_assert(D == 128 || D == 64, "head dimension 128, or 64 as token pairs");
  constexpr int TPV = 128 / D;            // tokens per tile row
  constexpr int KS = D / 16;              // K steps of one product
  constexpr int CP = MSE ? NB : NB - 1;   // code planes
  constexpr int K = 1 << CP;
  constexpr int KH = K / 2;           // positive centroids
  constexpr int NT = KH - 1;          // positive thresholds
  constexpr int YP = BF16 ? 2 : 3;    // MFMA passes per K step of Y
  constexpr int ZN = KS * 3;          // MFMAs of Z = M r per 32-vector block
  // x (scaled, fp16 hi/lo) and the residual (hi/lo) in separate buffers, so
  // a tile needs two barriers: x of the next tile is written while the
  // residual of this one is still being read.
  __shared__ __align__(16) _Float16 xh_s[kT * kLdx];
  __shared__ __align__(16) _Float16 xl_s[BF16 ? 8 : kT * kLdx];
  __shared__ __align__(16) _Float16 rh_s[kT * kLdx];
  __shared__ __align__(16) _Float16 rl_s[kT * kLdx];
  // per token (row v, token k of the row at TPV * v + k), by tile parity
  __shared__ float ysc[2][TPV * kT];  // 2^e / nu (0 for x = 0)
  __shared__ float sinv[2][TPV * kT]; // nu 2^-e (1 for x = 0): thresholds to acc units
  __shared__ uint32_t nu16[2][TPV * kT];
  __shared__ float gpart[4][kT];
  // packed records and norms of the tile (the global layout), written out
  // one tile later with contiguous stores
  __shared__ __align__(16) uint32_t outw[2][kT * 4 * NB];
  __shared__ __align__(16) uint32_t outn[2][TPV * kT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  // D = 64: this wave's token of the pair, and where its coordinates start
  const int half = D == 64 ? wave >> 1 : 0;
  const int kofs = 64 * half;

  // Pi / M rows 32*wave + col (D = 64: 32*(wave&1) + col of the 64 x 64
  // tables), K slots 16*ks + 8*hh .. +8
  v8h Ph[KS], Pl[KS], Mh[KS], Ml[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int off = (32 * (D == 64 ? (wave & 1) : wave) + col) * D + 16 * ks + 8 * hh;
    Ph[ks] = *(const v8h*)(a.pi_hi + off);
    Pl[ks] = *(const v8h*)(a.pi_lo + off);
    Mh[ks] = *(const v8h*)(a.m_hi + off);
    Ml[ks] = *(const v8h*)(a.m_lo + off);
  }
  // wait for the table loads here, once: otherwise the first iteration's
  // pending loads leave waits inside the loop that stall every tile
  __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0) expcnt(7) lgkmcnt(15)

  auto tile_cnt = [&](uint32_t tile) -> int { return (int)min((uint32_t)kT, a.n_rows - tile * kT); };

  // ---- x -> norm, power-of-two scale, fp16 (hi/lo) into LDS, pass p --------
  // pass p: vector 4*wave + 16*p + lane/16, 8-element chunk lane%16; the 16
  // lanes of a row hold one vector and all get its norm
  RawX<BF16> raw;
  auto x_pass = [&](int p, int cnt, int pb) {
    const int v = 4 * wave + 16 * p + (lane >> 4);
    const int c = lane & 15;
    const bool live = v < cnt;              // past the end: zero vector
    uint4 u0 = raw.v[BF16 ? p : 2 * p];
    uint4 u1 = BF16 ? u0 : raw.v[2 * p + 1];
    if (!live) u0 = u1 = make_uint4(0u, 0u, 0u, 0u);
    float xv[8];
    float ss = 0.f;
    if constexpr (BF16) {
      const uint32_t wv[4] = {u0.x, u0.y, u0.z, u0.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[2 * e] = __uint_as_float(wv[e] << 16);
        xv[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
        const v2bf pr = __builtin_bit_cast(v2bf, wv[e]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
      }
    } else {
      xv[0] = __uint_as_float(u0.x); xv[1] = __uint_as_float(u0.y);
      xv[2] = __uint_as_float(u0.z); xv[3] = __uint_as_float(u0.w);
      xv[4] = __uint_as_float(u1.x); xv[5] = __uint_as_float(u1.y);
      xv[6] = __uint_as_float(u1.z); xv[7] = __uint_as_float(u1.w);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(xv[e], xv[e], ss);
    }
    ss = D == 64 ? row8_sum(ss) : row16_sum(ss);
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
    *(v8h*)(xh_s + v * kLdx + 8 * c) = hi;
    if constexpr (!BF16) *(v8h*)(xl_s + v * kLdx + 8 * c) = lo;
    // the 16 lanes of the row (8 of each token for D = 64) write the same values
    const int vk = TPV * v + (D == 64 ? c >> 3 : 0);
    ysc[pb][vk] = (nu > 0.f) ? ldexpf(__builtin_amdgcn_rcpf(nu), ex) : 0.f;
    sinv[pb][vk] = (nu > 0.f) ? ldexpf(nu, -ex) : 1.f;
    nu16[pb][vk] = (uint32_t)__half_as_ushort(__float2half_rn(nu));
  };

  // ---- MFMA m (0 .. 8*YP-1) of Y = Pi x_s for the 32 vectors of block cb ---
  v8h xf_h, xf_l;
  auto y_mfma = [&](v16f& acc, int cb, int m) {
    const int ks = m / YP, ps = m % YP;
    if (ps == 0) {
      const int off = (32 * cb + col) * kLdx + kofs + 16 * ks + 8 * hh;
      xf_h = *(const v8h*)(xh_s + off);
      if constexpr (!BF16) xf_l = *(const v8h*)(xl_s + off);
    }
    if (ps == 0) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ph[ks], xf_h, acc, 0, 0, 0);
    else if (ps == 1) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(Pl[ks], xf_h, acc, 0, 0, 0);
    else acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ph[ks], xf_l, acc, 0, 0, 0);
  };

  // ---- codes and residual of block cb; after element i, `hook(i)` ---------
  // Element i of a lane is coordinate 32*wave + 8(i/4) + 4hh + i%4 of vector
  // 32cb + col.  y = s * acc with s > 0 the vector's scale: thresholds and
  // centroids are taken to acc's units (t / s, c / s) once per vector and the
  // residual stays in those units (z changes by the factor 1/s, which keeps
  // its sign; gamma^2 = s^2 * sum r^2); s = 0 (x = 0) uses 1.
  // idx = pos ? KH + m : KH - 1 - m with m the number of positive thresholds
  // below |y|: the top code bit is pos, the lower bits are m (pos) or ~m; for
  // the thermometer gt[], bit 0 of m is the XOR of all gt and bit 1 (K = 8) is
  // gt[1].  Bits enter by shift-in from i = 15 down, so bit i of each
  // accumulator belongs to element i.
  uint32_t codew[2][3];
  auto codes = [&](const v16f& acc, int cb, int pb, auto&& hook) {
    const int v = 32 * cb + col;
    const float sv = ysc[pb][TPV * v + half];
    const float inv = sinv[pb][TPV * v + half];
    float thr_v[NT > 0 ? NT : 1], cpos_v[KH];
#pragma unroll
    for (int k = 0; k < NT; ++k) thr_v[k] = a.thr[k] * inv;
#pragma unroll
    for (int k = 0; k < KH; ++k) cpos_v[k] = a.cpos[k] * inv;
    uint32_t bacc[3] = {0u, 0u, 0u};
    float g2 = 0.f;
    float rr[16];
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      const float y = acc[i];
      const float ay = fabsf(y);
      const bool pos = y > 0.f;
      const uint64_t P = __builtin_amdgcn_ballot_w64(pos);
      bool gt[NT > 0 ? NT : 1];
      uint64_t G[NT > 0 ? NT : 1];
      float cm = cpos_v[0];
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        gt[k] = ay > thr_v[k];
        G[k] = __builtin_amdgcn_ballot_w64(gt[k]);
        cm = gt[k] ? cpos_v[k + 1] : cm;
      }
      const float c = pos ? cm : -cm;      // y = +0 -> lower half
      const float r = y - c;
      rr[i] = r;
      g2 = fmaf(r, r, g2);
      bacc[CP - 1] = shift_in(bacc[CP - 1], P);
      if constexpr (CP == 2) {
        bacc[0] = shift_in(bacc[0], ~(G[0] ^ P));
      } else if constexpr (CP == 3) {
        bacc[1] = shift_in(bacc[1], ~(G[1] ^ P));
        bacc[0] = shift_in(bacc[0], ~(G[0] ^ G[1] ^ G[2] ^ P));
      }
      hook(15 - i);
    }
    // residual -> LDS as hi/lo fp16 (rows 8j + 4hh .. +3 hold 4 consecutive i)
#pragma unroll
    for (int j = 0; j < (MSE ? 0 : 4); ++j) {
      typedef uint32_t u2v __attribute__((ext_vector_type(2)));
      v4h rh;
#pragma unroll
      for (int e = 0; e < 4; ++e) rh[e] = (_Float16)rr[4 * j + e];
      const u2v hb = __builtin_bit_cast(u2v, rh);
      u2v lb;
      lb[0] = lo_pair(rr[4 * j], rr[4 * j + 1], hb[0]);
      lb[1] = lo_pair(rr[4 * j + 2], rr[4 * j + 3], hb[1]);
      const int off = v * kLdx + 32 * wave + 8 * j + 4 * hh;
      *(v4h*)(rh_s + off) = rh;
      *(u2v*)(rl_s + off) = lb;
    }
#pragma unroll
    for (int p = 0; p < CP; ++p) codew[cb][p] = halves_or(spread16(bacc[p], hh));
    if constexpr (!MSE)
      gpart[wave][v] = halves_sum(g2) * (sv * sv);  // both halves write the same value
  };

  // ---- MFMA m (0..23) of Z = M r for block cb ------------------------------
  v8h rf_h, rf_l;
  auto z_mfma = [&](v16f& z, int cb, int m) {
    const int ks = m / 3, ps = m % 3;
    if (ps == 0) {
      const int off = (32 * cb + col) * kLdx + kofs + 16 * ks + 8 * hh;
      rf_h = *(const v8h*)(rh_s + off);
      rf_l = *(const v8h*)(rl_s + off);
    }
    if (ps == 0) z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Mh[ks], rf_h, z, 0, 0, 0);
    else if (ps == 1) z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ml[ks], rf_h, z, 0, 0, 0);
    else z = __builtin_amdgcn_mfma_f32_32x32x16_f16(Mh[ks], rf_l, z, 0, 0, 0);
  };

  // ---- signs of block cb and its record words into the staging buffer ------
  auto signs = [&](const v16f& z, int cb, int pb, auto&& hook) {
    if constexpr (MSE) {      // code words only
      const int v = 32 * cb + col;
      uint32_t* dst = outw[pb] + (v * 4 + wave) * NB;
      if (hh == 0)
#pragma unroll
        for (int p = 0; p < NB; ++p) dst[p] = codew[cb][p];
#pragma unroll
      for (int e = 0; e < 16; ++e) hook(e);
      return;
    }
    uint32_t sb = 0u;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      sb = shift_in(sb, __builtin_amdgcn_ballot_w64(z[i] >= 0.f));
      hook(15 - i);
    }
    uint32_t sw = halves_or(spread16(sb, hh));
    const int v = 32 * cb + col;
    if (ysc[pb][TPV * v + half] == 0.f) sw = 0xffffffffu;   // ||x|| = 0: r = 0, all signs +1
    // group `wave` of record v; each lane half writes the words it owns
    // (a word both halves write gets the same value from both)
    uint32_t* dst = outw[pb] + (v * 4 + wave) * NB;
    if constexpr (NB == 4) {
      *(uint2*)(dst + 2 * hh) = hh ? make_uint2(codew[cb][2], sw) : make_uint2(codew[cb][0], codew[cb][1]);
    } else if constexpr (NB == 3) {
      dst[hh] = hh ? codew[cb][1] : codew[cb][0];
      dst[hh + 1] = hh ? sw : codew[cb][1];
    } else {
      dst[hh] = hh ? sw : codew[cb][0];
    }
  };

  auto none = [](int) {};
  uint32_t tile = tile0;
  if (tile >= a.n_tiles) return;
  // prologue: x of the first tile
  load_tile<BF16, D>(raw, a, tile, wave, lane);
  {
    const int cnt0 = tile_cnt(tile);
#pragma unroll
    for (int p = 0; p < 4; ++p) x_pass(p, cnt0, 0);
  }
  int par = 0;
  bool have_prev = false;
  TileRows prev{};
  // record of row v, or -1 for a token whose slot lies outside [0, dst_stride_head)
  auto rec_of = [&](const TileRows& r, int v) -> int64_t {
    uint32_t h, t;
    row_ht(r, v, a, h, t);
    int64_t s = t;
    if (a.slots) {
      s = a.slots[t];
      if (s < 0 || s >= a.dst_stride_head) return -1;
    }
    return (int64_t)h * a.dst_stride_head + a.dst_token0 + TPV * s;   // first token of the row
  };
  // Copy the staged records and norms of the previous tile (buffer pb) to
  // memory: prev.cnt * NB <= 256 chunks of 16 bytes, one per thread, and the
  // norms.  Stores are issued before the next tile's loads, so that waiting
  // for those loads (the memory counter covers loads and stores alike) never
  // waits for fresh stores.
  auto flush = [&](int pb) {
    if (!have_prev) return;
    if (prev.one && !a.slots) {
      // a row's 4 record groups are its TPV records, back to back
      const int64_t rec0 = rec_of(prev, 0);
      if (tid < prev.cnt * NB)
        ((uint4*)(a.planes + rec0 * (D / 32) * NB))[tid] = ((const uint4*)outw[pb])[tid];
      if (tid < TPV * prev.cnt) a.norms[rec0 + tid] = outn[pb][tid];
    } else {
      if (tid < prev.cnt * NB) {
        const int v = tid / NB;
        const int64_t rec = rec_of(prev, v);
        if (rec >= 0)
          ((uint4*)(a.planes + rec * (D / 32) * NB))[tid - v * NB] = ((const uint4*)outw[pb])[tid];
      }
      if (tid < TPV * prev.cnt) {
        const int64_t rec = rec_of(prev, tid / TPV);
        if (rec >= 0) a.norms[rec + tid % TPV] = outn[pb][tid];
      }
    }
  };
  for (; tile < a.n_tiles; tile += stride, par ^= 1) {
    const TileRows cur = tile_rows(tile, a);
    const int cnt = cur.cnt;
    const uint32_t next = tile + stride;
    const bool has_next = next < a.n_tiles;
    __syncthreads();
    // every wave has finished the previous tile and x of this one is in LDS:
    // write the previous records, then prefetch the next tile
    flush(par ^ 1);
    if (BF16 && has_next) load_tile<BF16, D>(raw, a, next, wave, lane);

    // Y of block 0, then the codes of block 0 with Y of block 1 interleaved
    v16f acc0 = {}, acc1 = {};
#pragma unroll
    for (int m = 0; m < KS * YP; ++m) y_mfma(acc0, 0, m);
    codes(acc0, 0, par, [&](int e) {
#pragma unroll
      for (int m = e * KS * YP / 16; m < (e + 1) * KS * YP / 16; ++m) y_mfma(acc1, 1, m);
    });
    codes(acc1, 1, par, none);
    __syncthreads();

    // Z of block 0 with x of the next tile converted in between (its LDS
    // buffer is free: every wave has finished Y), then Z of block 1 with the
    // signs of block 0
    v16f z0 = {}, z1 = {};
    const int cnt_n = has_next ? tile_cnt(next) : 0;
    if (!BF16 && has_next) load_tile<BF16, D>(raw, a, next, wave, lane);    // fp32: no prefetch
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if constexpr (!MSE)
#pragma unroll
        for (int m = p * ZN / 4; m < p * ZN / 4 + ZN / 8; ++m) z_mfma(z0, 0, m);
      x_pass(p, cnt_n, par ^ 1);
      if constexpr (!MSE)
#pragma unroll
        for (int m = p * ZN / 4 + ZN / 8; m < (p + 1) * ZN / 4; ++m) z_mfma(z0, 0, m);
    }
    signs(z0, 0, par, [&](int e) {
      if (!MSE && e < ZN / 2) {
#pragma unroll
        for (int m = 2 * e; m < 2 * e + 2; ++m) z_mfma(z1, 1, m);
      }
    });
    signs(z1, 1, par, none);

    if (tid < TPV * cnt) {            // token tid % TPV of row tid / TPV
      const int v = tid / TPV, k = tid % TPV;
      const float sq = MSE ? 0.f
                     : D == 64 ? gpart[2 * k][v] + gpart[2 * k + 1][v]
                               : (gpart[0][v] + gpart[1][v]) + (gpart[2][v] + gpart[3][v]);
      const float gam = (MSE || ysc[par][tid] == 0.f) ? 0.f : sqrtf(sq);
      const uint32_t gb = (uint32_t)__half_as_ushort(__float2half_rn(gam));
      outn[par][tid] = nu16[par][tid] | (gb << 16);
    }
    prev = cur;
    have_prev = true;
  }
  __syncthreads();
  flush(par ^ 1);
}

// ---- host side -------------------------------------------------------------
constexpr int64_t kMaxRows = ((int64_t)1 << 32) - 2 * kT;   // 32-bit row indices per launch

// Arguments shared by every launch of one quantize call (hipErrorInvalidValue
// for n_tokens beyond 32-bit row indices).  slots: null, or the destination
// token of each input token (device int64 [n_tokens]; record (h, t) at
// h * dst_stride_head + dst_token0 + slots[t], skipped for a slot outside
// [0, dst_stride_head)).
inline hipError_t q128_args(const tq_ctx* ctx, const void* x, int64_t n_tokens,
                            int64_t x_stride_token, int64_t x_stride_head, uint32_t* planes,
                            uint16_t* norms, int64_t dst_stride_head, int64_t dst_token0,
                            const int64_t* slots, Q128Args& a) {
  a = Q128Args{};
  a.x = x;
  a.x_stride_token = x_stride_token;
  a.x_stride_head = x_stride_head;
  a.n_tokens = n_tokens;
  a.planes = planes;
  a.norms = (uint32_t*)norms;
  a.dst_stride_head = dst_stride_head;
  a.dst_token0 = dst_token0;
  a.slots = slots;
  a.pi_hi = ctx->t.pi_hi;
  a.pi_lo = ctx->t.pi_lo;
  a.m_hi = ctx->t.m_hi;
  a.m_lo = ctx->t.m_lo;
  if (n_tokens > kMaxRows) return hipErrorInvalidValue;
  make_div((uint32_t)n_tokens, a.div_m, a.div_s1, a.div_s2);
  const int KH = ctx->K / 2;
  for (int k = 0; k < 4; ++k) {
    a.thr[k] = (k < KH - 1) ? ctx->mid[KH + k] : 0.f;
    a.cpos[k] = (k < KH) ? ctx->cent[KH + k] : 0.f;
  }
  return hipSuccess;
}

// The launch over heads h0 .. h0 + nh - 1 (nh * n_tokens <= kMaxRows).
inline Q128Args q128_group(const Q128Args& a, int64_t h0, int64_t nh, bool bf16) {
  Q128Args ah = a;
  ah.x = (const char*)a.x + h0 * a.x_stride_head * (bf16 ? 2 : 4);
  ah.dst_token0 = a.dst_token0 + h0 * a.dst_stride_head;
  ah.n_rows = (uint32_t)(nh * a.n_tokens);
  ah.n_tiles = (ah.n_rows + kT - 1) / kT;
  return ah;
}

}  // namespace
}  // namespace tq
