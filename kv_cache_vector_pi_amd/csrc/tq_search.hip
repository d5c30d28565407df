// Vector search over a quantized database and dequantization
// (zingnex.cn digest, nearest-neighbour section; admirer.cn vector-search
// paragraph; turboquant.net pseudo-code "dequant").
//
// Both are "decoded GEMMs" over the packed records:
//   score[q][n] = nu_n * ( sum_j QR[q][j] c[idx_nj] + alpha * gamma_n * sum_j QP[q][j] s_nj )
// For search QR = Pi q and QP = S q (one row per query).  For dequantization
// the rows are the unit vectors e_j, i.e. QR = Pi^T and QP = S^T, so the
// "score" of row j is coordinate j of nu (Pi^T c[idx] + alpha gamma S^T s).
//
// Search: the query rows (Pi q, S q; row_prep_kernel on the fp32 matrix
// cores) are split into fp16 hi parts plus fp8 copies for the correction
// products, with alpha folded into the sketch half, and stored in K-slot
// order.  search_gemm_kernel copies a 256-query tile's rows and a 256-record
// tile's plane words into LDS two words ahead, and each MFMA wave decodes its
// own records' words into its B operands in registers (v_perm_b32 lookups in
// byte tables of the codebook and of each record's gamma).  Per 32-coordinate
// word and 32 x 32 block one accumulator takes
//   acc += QR_hi c_hi + (alpha QP)_hi gamma s        (v_mfma_f32_32x32x16_f16)
//        + QR_lo c_hi + QR_hi c_lo                   (v_mfma_scale_f32_32x32x64_f8f6f4)
// (gamma s is exact in fp16: gamma is an fp16 value and s = +-1), and score
// = nu * acc.  Instead of writing every score, the epilogue keeps only those
// above the query's running k-th best score (candidates appended with one
// atomic per wave and query row), and a one-wave-per-query merge after each
// chunk of records folds them into the running top-k (score descending,
// index ascending) and raises the threshold.
//
// Dequantization has two kernels, picked by tq_dequantize: at d = 128 with
// at least 64 records per compute unit, dequant128_kernel keeps each wave's
// 32 rows of Pi^T and S^T in registers for a persistent loop over 64-record
// tiles (32x32x16 MFMAs, output straight from the accumulators); every other
// d, and smaller calls, run decoded_gemm_kernel in its two-accumulator form
// on 16x16x32 tiles (the rows of Pi^T and S^T as the "queries").
#include <algorithm>
#include <cmath>

#include "tq_dma.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kRowsTile = 64;    // dequantize: rows per workgroup
constexpr int kRecTile = 64;     // dequantize: records per workgroup
constexpr int kLdsRow = 40;      // halves per staged row of one word (32 + pad)
constexpr int kQT = 256;         // search: queries per workgroup
constexpr int kRT = 256;         // search: records per workgroup
constexpr int kFirst = 2048;     // search: records of the first chunk (sets the thresholds)
constexpr int kChunk = 65536;    // search: records per later chunk = candidate capacity ...
constexpr int kChunkSmall = 16384;   // ... unless n_q x kChunk candidates exceed kCandCap bytes
constexpr int64_t kCandCap = (int64_t)1 << 30;

// records per chunk after the first: the candidate lists hold a chunk's worth
inline int search_chunk(int64_t n_queries) {
  return n_queries * (int64_t)kChunk * 8 <= kCandCap ? kChunk : kChunkSmall;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Position, within its 32-coordinate word, of coordinate c in the staged query
// rows: K-slot 4g + t holds coordinate g + 8t.  Slots 4g .. 4g + 3 are then the
// bits at positions g, g + 8, g + 16, g + 24 of a plane word, which one AND with
// 0x01010101 << g spreads over four bytes.
__host__ __device__ inline int kslot_of(int c) { return 4 * (c & 7) + (c >> 3); }

// float -> fp8 e4m3 (OCP: exponent bias 7, largest finite 448, no infinity),
// round to nearest even; saturates at 448.  Host and device share it (the
// codebook's tables are built on the host, the query rows on the device).
__host__ __device__ inline uint8_t to_e4m3(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sg = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
  if (a >= 0x43E80000u) return (uint8_t)(sg | 0x7Eu);          // >= 464, inf, nan: 448
  if (a < 0x3C800000u) {                                        // below 2^-6: steps of 2^-9
    const float y = __builtin_bit_cast(float, a) * 512.0f;      // exact, < 8
    uint32_t q = (uint32_t)y;
    const float r = y - (float)q;
    if (r > 0.5f || (r == 0.5f && (q & 1u))) ++q;
    return (uint8_t)(sg | q);                                   // q == 8: 2^-6
  }
  uint32_t q = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);    // exponent field 1 .. 15
  const uint32_t rem = a & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;    // carries into the exponent
  return (uint8_t)(sg | (q > 0x7Eu ? 0x7Eu : q));
}

// Byte of K-slot kappa (0 .. 31) in a lane half's fp8 operand: lane half hh
// holds the byte groups g (kappa = 4 g + t) with (g >> 1) & 1 == hh, in the
// order g = 2 hh, 2 hh + 1, 4 + 2 hh, 5 + 2 hh, i.e. the groups its decode of
// the two 16-slot halves of a word produces.  Returns 16 hh + 4 gi + t.
__host__ __device__ inline int fp8_byte_of(int kappa) {
  const int g = kappa >> 2, t = kappa & 3;
  return 16 * ((g >> 1) & 1) + 4 * ((g & 1) + 2 * (g >> 2)) + t;
}

// ---- row preparation: Pi q and S q, split into hi/lo fp16 -----------------
// On the fp32 matrix cores: a workgroup computes 32 query rows x 128 outputs
// of [Pi rows | S rows] (4 waves, 32 outputs each) with
// v_mfma_f32_32x32x2_f32 over the d coordinates, two per instruction.  Lane
// l supplies q[row0 + l % 32][j + l / 32] (A) and coordinate j + l / 32 of
// output row o = o0 + l % 32 of Pi or S, read as Pi^T[j + l / 32][o] (B,
// coalesced across the wave).  The sum of squares of the A values gives
// ||q|| per row for the fp8 scales.
constexpr int kPrepRows = 32;
constexpr int kPrepOut = 128;

struct RowPrepArgs {
  const float* q;        // [n][d]
  const float* pit;      // [d][d] Pi^T
  const float* st;       // [d][d] S^T
  __half* qr_hi;         // [n_pad][Dp]
  uint8_t* q8;           // [n_pad][Dp / 32][64]: per word, fp8 (QR lo) 2^e_lo then (QR hi) 2^e_hi
  __half* qp_hi;
  uint32_t* q8scale;     // [n_pad]: E8M0 codes of 2^-e_lo (byte 0) and 2^-e_hi (byte 1)
  float pscale;          // factor on S q (alpha for search)
  int d, Dp;
  int64_t n, n_pad;      // n_pad: a multiple of kPrepRows
};

__global__ void __launch_bounds__(256) row_prep_kernel(RowPrepArgs a) {
  __shared__ float qn2[kPrepRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int64_t row0 = (int64_t)blockIdx.x * kPrepRows;
  const int o = blockIdx.y * kPrepOut + 32 * wave + col;   // output column of this lane
  const bool sk = o >= a.Dp;
  const int r = sk ? o - a.Dp : o;
  const bool live = o < 2 * a.Dp && r < a.d;
  const float* tc = (sk ? a.st : a.pit) + (live ? r : 0);  // Pi^T / S^T column r
  const bool qlive = row0 + col < a.n;
  const float* qp = a.q + (qlive ? row0 + col : 0) * (int64_t)a.d;
  v16f acc = {};
  float ssq = 0.f;
  int j = 0;
  // batches of 8 coordinates as 4 MFMAs: lane half hh takes coordinates
  // j + 4 hh .. + 3, one per MFMA, so its query values are one 16-byte load
  // (the contraction order within a batch is free: A and B agree on it)
  if (a.d % 4 == 0 && ((uintptr_t)a.q & 15) == 0) {
    constexpr int U = 8;                         // batches in flight
    for (; j + 8 * U <= a.d; j += 8 * U) {
      float4 av[U];
      float bv[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jb = j + 8 * u + 4 * hh;
        av[u] = qlive ? *(const float4*)(qp + jb) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int c = 0; c < 4; ++c) bv[u][c] = live ? tc[(int64_t)(jb + c) * a.d] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float aq[4] = {av[u].x, av[u].y, av[u].z, av[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          ssq = fmaf(aq[c], aq[c], ssq);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(aq[c], bv[u][c], acc, 0, 0, 0);
        }
      }
    }
  }
  for (; j < a.d; j += 2) {
    const int jj = j + hh;
    const float av = (qlive && jj < a.d) ? qp[jj] : 0.f;
    const float bv = (live && jj < a.d) ? tc[(int64_t)jj * a.d] : 0.f;
    ssq = fmaf(av, av, ssq);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
  }
  // ||q||^2 of row col: the two lane halves hold the two halves of its coordinates
  ssq += __shfl_xor(ssq, 32);
  if (wave == 0 && hh == 0) qn2[col] = ssq;
  __syncthreads();
  if (o >= 2 * a.Dp) return;
  const int kappa = kslot_of(r & 31);
  const int pos = (r & ~31) + kappa;                // K-slot order within the word
  const int64_t b8 = (int64_t)(r >> 5) * 64 + fp8_byte_of(kappa);
  // element i: query row 8 (i / 4) + 4 hh + i % 4 of the tile, output o
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rl = 8 * (i >> 2) + 4 * hh + (i & 3);
    const int64_t row = row0 + rl;
    if (row < a.n_pad) {
      const float v = live ? (sk ? a.pscale * acc[i] : acc[i]) : 0.f;
      const __half vh = __float2half(v);
      if (sk) {
        a.qp_hi[row * a.Dp + pos] = vh;
      } else {
        a.qr_hi[row * a.Dp + pos] = vh;
        // fp8 copies of the hi and lo parts for the correction products,
        // scaled by powers of two: |Pi q|_j <= ||q|| < 2^e puts (QR hi) 2^(8-e)
        // below 256, and |QR lo| <= 2^-11 |QR| (fp16 rounding) the lo part too
        int e = 0;
        frexpf(sqrtf(qn2[rl]), &e);
        const int ehi = min(100, max(-100, 8 - e)), elo = ehi + 11;
        const float vl = v - __half2float(vh);
        uint8_t* q8 = a.q8 + row * (int64_t)(2 * a.Dp) + b8;
        q8[0] = to_e4m3(ldexpf(vl, elo));
        q8[32] = to_e4m3(ldexpf(__half2float(vh), ehi));
        if (o == 0) a.q8scale[row] = (uint32_t)(127 - elo) | ((uint32_t)(127 - ehi) << 8);
      }
    }
  }
}

// ---- decoded GEMM ------------------------------------------------------------
struct GemmArgs {
  const __half* qr_hi;
  const __half* qr_lo;
  const __half* qp_hi;
  const __half* qp_lo;   // [rows_pad][Dp]
  int64_t n_rows;        // valid rows (queries or coordinates)
  const uint32_t* planes;
  const uint32_t* norms;
  int64_t rec0, n_rec;   // records rec0 .. rec0 + n_rec - 1
  int W, Dp;
  float alpha;
  _Float16 c_hi[kMaxK];
  _Float16 c_lo[kMaxK];
  // output: out[rec * out_ld + row]
  float* out;
  int64_t out_ld;
  int out_vec4;          // out 16-byte aligned and out_ld % 4 == 0 (dequant128_kernel)
};

// MSE: records of NB code planes without the QJL stage (no sketch term).
template <int NB, bool MSE, int MODE>
__global__ void __launch_bounds__(256) decoded_gemm_kernel(GemmArgs a) {
  constexpr int CP = MSE ? NB : NB - 1;
  __shared__ __align__(16) _Float16 dh[kRecTile * kLdsRow];
  __shared__ __align__(16) _Float16 dl[kRecTile * kLdsRow];
  __shared__ __align__(16) _Float16 ds[kRecTile * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int64_t rt = blockIdx.x, qt = blockIdx.y;
  const int64_t row = qt * kRowsTile + 16 * wave + n;       // A-operand row of this lane
  // decode role: record dr = tid / 4, coordinates 8 * (tid % 4) .. +8 of the word
  const int dr = tid >> 2, dq = tid & 3;
  const int64_t drec = rt * kRecTile + dr;
  const bool dlive = drec < a.n_rec;

  v4f am[4], aq[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    am[cb] = (v4f){0.f, 0.f, 0.f, 0.f};
    aq[cb] = (v4f){0.f, 0.f, 0.f, 0.f};
  }
  // The next word's record words and A fragments load into registers while
  // this word's MFMAs run.
  uint32_t wn[NB];
  v8h rhn, rln, phn = {}, pln = {};
  auto load_word = [&](int ks) {
#pragma unroll
    for (int p = 0; p < NB; ++p) wn[p] = 0u;
    if (dlive) {
      const uint32_t* src = a.planes + ((a.rec0 + drec) * a.W + ks) * NB;
#pragma unroll
      for (int p = 0; p < NB; ++p) wn[p] = src[p];
    }
    const int64_t aoff = row * a.Dp + 32 * ks + 8 * g;
    rhn = *(const v8h*)(a.qr_hi + aoff);
    rln = *(const v8h*)(a.qr_lo + aoff);
    if constexpr (!MSE) {
      phn = *(const v8h*)(a.qp_hi + aoff);
      pln = *(const v8h*)(a.qp_lo + aoff);
    }
  };
  load_word(0);
  for (int ks = 0; ks < a.W; ++ks) {
    uint32_t wd[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) wd[p] = wn[p];
    const v8h rh = rhn, rl = rln;
    const v8h ph = phn, pl = pln;
    // decode word ks of record dr, coordinates 8dq .. 8dq+7
    {
      v8h vh, vl, vs;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int bit = 8 * dq + e;
        int idx = 0;
#pragma unroll
        for (int p = 0; p < CP; ++p) idx |= (int)((wd[p] >> bit) & 1u) << p;
        vh[e] = a.c_hi[idx];
        vl[e] = a.c_lo[idx];
        if constexpr (!MSE) vs[e] = ((wd[NB - 1] >> bit) & 1u) ? (_Float16)1.0f : (_Float16)-1.0f;
      }
      *(v8h*)(dh + dr * kLdsRow + 8 * dq) = vh;
      *(v8h*)(dl + dr * kLdsRow + 8 * dq) = vl;
      if constexpr (!MSE) *(v8h*)(ds + dr * kLdsRow + 8 * dq) = vs;
    }
    __syncthreads();
    if (ks + 1 < a.W) load_word(ks + 1);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int off = (16 * cb + n) * kLdsRow + 8 * g;
      const v8h bh = *(const v8h*)(dh + off);
      const v8h bl = *(const v8h*)(dl + off);
      am[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rh, bh, am[cb], 0, 0, 0);
      am[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rl, bh, am[cb], 0, 0, 0);
      am[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rh, bl, am[cb], 0, 0, 0);
    }
    if constexpr (!MSE) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const v8h bs = *(const v8h*)(ds + (16 * cb + n) * kLdsRow + 8 * g);
        aq[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bs, aq[cb], 0, 0, 0);
        aq[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bs, aq[cb], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // epilogue: lane holds rows 4g+i of the wave's 16-row block, record 16cb+n.
  // The tile is staged in LDS as [record][row] and written one record row at
  // a time, consecutive threads on consecutive outputs (a lane's own values
  // sit 16 records apart, one float each).
  __shared__ float ot[kRecTile * (kRowsTile + 1)];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int rl = 16 * cb + n;
    const int64_t rec = rt * kRecTile + rl;
    float nu = 0.f, ag = 0.f;
    if (rec < a.n_rec) {
      const uint32_t nr = a.norms[a.rec0 + rec];
      nu = __half2float(__ushort_as_half((unsigned short)(nr & 0xffffu)));
      ag = a.alpha * __half2float(__ushort_as_half((unsigned short)(nr >> 16)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ot[rl * (kRowsTile + 1) + 16 * wave + 4 * g + i] = nu * fmaf(ag, aq[cb][i], am[cb][i]);
  }
  __syncthreads();
  for (int k = tid; k < kRecTile * kRowsTile; k += 256) {
    const int rl = k / kRowsTile, rr = k - rl * kRowsTile;
    const int64_t rec = rt * kRecTile + rl;
    const int64_t r = qt * kRowsTile + rr;
    if (rec < a.n_rec && r < a.n_rows) a.out[(a.rec0 + rec) * a.out_ld + r] = ot[rl * (kRowsTile + 1) + rr];
  }
}

// ---- dequantization at d = 128 ------------------------------------------------
// Wave w computes output rows 32w .. 32w + 31 (v_mfma_f32_32x32x16_f16): its
// rows of Pi^T and S^T, hi and lo fp16, stay in registers for the whole
// persistent loop.  A tile of 64 records is decoded once into LDS -- centroid
// hi and lo parts and the signs as +-1 -- the codebook looked up in LDS; then
// am = Pi^T c (3 passes) and aq = S^T s (2 passes), and the output
// nu (am + alpha gamma aq) is stored from the accumulators as float4 runs of
// four rows (or, for an unaligned output stride, staged in LDS over the
// decoded tile and written one record row at a time).  The next tile's
// record words load during the MFMAs.
constexpr int kDqT = 64;      // records per tile
constexpr int kDqLd = 136;    // LDS row stride of a decoded record, in halves
constexpr int kDqOut = 132;   // LDS row stride of a staged output record, in floats

template <int NB, bool MSE>
__global__ void __launch_bounds__(256, 2) dequant128_kernel(GemmArgs a) {
  constexpr int CP = MSE ? NB : NB - 1;
  __shared__ __align__(16) _Float16 bufs[3 * kDqT * kDqLd];
  __shared__ uint32_t ctab_s[kMaxK];
  __shared__ float nu_s[kDqT], ag_s[kDqT];
  _Float16* bch = bufs;
  _Float16* bcl = bufs + kDqT * kDqLd;
  _Float16* bsg = bufs + 2 * kDqT * kDqLd;
  float* ot = (float*)bufs;          // [kDqT][kDqOut] floats, over bch and bcl
  static_assert(kDqT * kDqOut * 4 <= 2 * kDqT * kDqLd * 2, "output staging fits");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  if (tid < kMaxK)
    ctab_s[tid] = (uint32_t)__builtin_bit_cast(uint16_t, a.c_hi[tid]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, a.c_lo[tid]) << 16);
  // Pi^T / S^T rows 32 wave + col, K slots 16 ks + 8 hh .. +8
  v8h Th[8], Tl[8], Sh[8], Sl[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int off = (32 * wave + col) * 128 + 16 * ks + 8 * hh;
    Th[ks] = *(const v8h*)(a.qr_hi + off);
    Tl[ks] = *(const v8h*)(a.qr_lo + off);
    if constexpr (!MSE) {
      Sh[ks] = *(const v8h*)(a.qp_hi + off);
      Sl[ks] = *(const v8h*)(a.qp_lo + off);
    }
  }
  // decode role: record tid / 4 of the tile, word tid % 4 (coordinates 32 w ..)
  const int dr = tid >> 2, dw = tid & 3;
  const int64_t n_tiles = (a.n_rec + kDqT - 1) / kDqT;
  uint32_t wn[NB];
  auto load_words = [&](int64_t tile) {
    const int64_t rec = tile * kDqT + dr;
#pragma unroll
    for (int p = 0; p < NB; ++p) wn[p] = 0u;
    if (tile < n_tiles && rec < a.n_rec) {
      const uint32_t* src = a.planes + ((a.rec0 + rec) * 4 + dw) * NB;
#pragma unroll
      for (int p = 0; p < NB; ++p) wn[p] = src[p];
    }
  };
  int64_t tile = blockIdx.x;
  load_words(tile);
  __syncthreads();                          // ctab_s written
  for (; tile < n_tiles; tile += gridDim.x) {
    const int64_t r0 = tile * kDqT;
    // ---- decode: 32 coordinates of one record word per thread ----------------
    {
      uint32_t wd[NB];
#pragma unroll
      for (int p = 0; p < NB; ++p) wd[p] = wn[p];
#pragma unroll
      for (int c8 = 0; c8 < 4; ++c8) {
        v8h vh, vl, vs;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int bit = 8 * c8 + e;
          uint32_t idx = 0;
#pragma unroll
          for (int p = 0; p < CP; ++p) idx |= ((wd[p] >> bit) & 1u) << p;
          const uint32_t hl = ctab_s[idx];
          vh[e] = __builtin_bit_cast(_Float16, (uint16_t)(hl & 0xffffu));
          vl[e] = __builtin_bit_cast(_Float16, (uint16_t)(hl >> 16));
          if constexpr (!MSE) vs[e] = ((wd[NB - 1] >> bit) & 1u) ? (_Float16)1.0f : (_Float16)-1.0f;
        }
        const int off = dr * kDqLd + 32 * dw + 8 * c8;
        *(v8h*)(bch + off) = vh;
        *(v8h*)(bcl + off) = vl;
        if constexpr (!MSE) *(v8h*)(bsg + off) = vs;
      }
      if (tid < kDqT) {
        const int64_t rec = r0 + tid;
        float nu = 0.f, ag = 0.f;
        if (rec < a.n_rec) {
          const uint32_t nr = a.norms[a.rec0 + rec];
          nu = __half2float(__ushort_as_half((unsigned short)(nr & 0xffffu)));
          ag = a.alpha * __half2float(__ushort_as_half((unsigned short)(nr >> 16)));
        }
        nu_s[tid] = nu;
        ag_s[tid] = ag;
      }
    }
    __syncthreads();
    load_words(tile + gridDim.x);          // the next tile's words, in flight during the MFMAs
    // ---- products: two 32-record blocks --------------------------------------
    v16f am[2], aq[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      am[cb] = (v16f){};
      aq[cb] = (v16f){};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = (32 * cb + col) * kDqLd + 16 * ks + 8 * hh;
        const v8h bh = *(const v8h*)(bch + off);
        const v8h bl = *(const v8h*)(bcl + off);
        am[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Th[ks], bh, am[cb], 0, 0, 0);
        am[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Tl[ks], bh, am[cb], 0, 0, 0);
        am[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Th[ks], bl, am[cb], 0, 0, 0);
        if constexpr (!MSE) {
          const v8h bs = *(const v8h*)(bsg + off);
          aq[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Sh[ks], bs, aq[cb], 0, 0, 0);
          aq[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Sl[ks], bs, aq[cb], 0, 0, 0);
        }
      }
    }
    // element i of block cb: row 32 wave + 8 (i / 4) + 4 hh + i % 4, record 32 cb + col
    if (a.out_vec4) {
      // four consecutive rows per (lane, i / 4): float4 stores straight from
      // the accumulators, 32 contiguous bytes per record and instruction
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int rl = 32 * cb + col;
        const int64_t rec = r0 + rl;
        const float nu = nu_s[rl], ag = ag_s[rl];
        if (rec < a.n_rec) {
          float* dst = a.out + (a.rec0 + rec) * a.out_ld + 32 * wave + 4 * hh;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(float4*)(dst + 8 * j) = make_float4(nu * fmaf(ag, aq[cb][4 * j], am[cb][4 * j]),
                                                  nu * fmaf(ag, aq[cb][4 * j + 1], am[cb][4 * j + 1]),
                                                  nu * fmaf(ag, aq[cb][4 * j + 2], am[cb][4 * j + 2]),
                                                  nu * fmaf(ag, aq[cb][4 * j + 3], am[cb][4 * j + 3]));
        }
      }
    } else {
      __syncthreads();                      // every wave is done with the decoded tile
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int rl = 32 * cb + col;
        const float nu = nu_s[rl], ag = ag_s[rl];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 32 * wave + 8 * (i >> 2) + 4 * hh + (i & 3);
          ot[rl * kDqOut + row] = nu * fmaf(ag, aq[cb][i], am[cb][i]);
        }
      }
      __syncthreads();
      for (int k = tid; k < kDqT * 128; k += 256) {
        const int rl = k >> 7, row = k & 127;
        const int64_t rec = r0 + rl;
        if (rec < a.n_rec) a.out[(a.rec0 + rec) * a.out_ld + row] = ot[rl * kDqOut + row];
      }
    }
    __syncthreads();                        // the decode buffers (and staging) are free again
  }
}

// ---- search GEMM with threshold-filter epilogue -------------------------------
struct SearchArgs {
  const __half* qa[4];   // [rows_pad][Dp] halves each, coordinates of each 32-word in K-slot
                         // order (below): QR hi; the fp8 correction rows (64 bytes per
                         // word, row preparation); (alpha QP) hi; qa[3] holds q8scale
  int64_t qa_step;       // qa[i] = qa[0] + i * qa_step (halves)
  int64_t n_q;
  const uint32_t* planes;
  const uint32_t* norms;
  int64_t rec0, n_rec;   // records rec0 .. rec0 + n_rec - 1 of this chunk
  int W, Dp;
  uint32_t tb[8];        // byte tables of the codebook for v_perm: bytes of centroid k's
                         // fp16 hi part (low byte: tb[0] k < 4, tb[1] k >= 4; high byte:
                         // tb[2], tb[3]); fp8 (c hi) 2^e_chi (tb[4], tb[5]) and fp8
                         // (c lo) 2^e_clo (tb[6], tb[7])
  uint32_t bscale;       // E8M0 codes of 2^-e_chi (byte 0) and 2^-e_clo (byte 1)
  const uint32_t* q8scale;   // [rows_pad]: the query rows' fp8 scale codes (row preparation)
  const float* thr;      // [n_q] running k-th best score (-inf: fewer than k yet)
  int* cnt;              // [n_q] candidates of this chunk
  float* cand_s;         // [n_q][chunk]
  int* cand_i;           // [n_q][chunk] record index within the chunk
  int64_t chunk;         // candidate capacity per query (records per chunk)
};

// One workgroup per (256-record tile, 256-query tile), 8 waves, each owning
// 128 queries x 64 records (4 x 2 blocks of 32 x 32).  Per 32-coordinate word:
//  * the word's query rows (NA arrays x 256 rows x 64 bytes) and the tile's
//    plane words go from memory straight into LDS (global_load_lds, two words
//    ahead, three buffers); 16-byte chunk c of query row r lands at position
//    c ^ ((r >> 2) & 3), so an operand read of 16 consecutive rows covers all
//    64 banks;
//  * every wave reads the plane words of its own 64 records and turns them into
//    the fp16 B operands in registers: the code index of four coordinates as
//    four bytes (an AND-OR of the shifted planes), then v_perm_b32 lookups in
//    the codebook's byte tables (centroid hi and lo parts) and in a per-record
//    table of gamma's bytes (gamma * s, exact in fp16), with no per-coordinate
//    table reads;
//  * one barrier per word.
// The MFMAs per word and 32 x 32 block are those of the decoded product:
//   acc += QR_hi c_hi + (alpha QP)_hi gamma s       (fp16, two per K-slice)
//        + QR_lo c_hi + QR_hi c_lo                  (one scaled fp8 MFMA per word).
// The two correction terms are each about 2^-11 of the code term, so fp8
// (3 mantissa bits, about 2^-4 relative per factor) leaves them an error near
// 2^-14 of the code term, while the per-block power-of-two scales of
// v_mfma_scale_f32_32x32x64_f8f6f4 keep both products inside fp8's range.  The
// fp8 MFMA covers 64 K-slots (both terms of a word) in the time of two fp16 ones,
// so the matrix cores do three quarters of the work of four fp16 passes.
template <int NB, bool MSE>
__global__ void __launch_bounds__(512, 2) search_gemm_kernel(SearchArgs a) {
  constexpr int CP = MSE ? NB : NB - 1;         // code planes
  // staged query arrays: QR hi, the fp8 correction rows and (alpha QP) hi.
  // The sketch term alpha gamma <QP, s> is a small part of a score, so its
  // fp16 rounding of QP (2^-12 relative) stays ~1e-4 of the scores' rms;
  // (alpha QP) lo is not used.
  constexpr int NA = MSE ? 2 : 3;
  constexpr int NRC = 4 * NB;                    // record copies (256 lanes x 4 B) per word
  __shared__ __align__(16) _Float16 As[3][NA][kQT * 32];
  __shared__ __align__(16) uint32_t Rs[4][kRT * NB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int wq = wave & 1, wr = wave >> 1;       // queries 128 wq .., records 64 wr ..
  const int64_t r0 = (int64_t)blockIdx.x * kRT, q0 = (int64_t)blockIdx.y * kQT;

  // Copies of one word, in items a wave issues one at a time (spread over the
  // products, so that the address units work beside the matrix cores instead
  // of stalling every wave at the start of a step).  A lane's byte offsets are
  // fixed for the whole loop; only the scalar bases move with the word.
  // Query rows of word s into buffer s % 3, items 0 .. 2 NA - 1: wave w copies
  // rows 32w .. 32w + 31 of every array, 16 rows (1 KB) per copy; lane l
  // fills slot l % 4 of row 16 i + l / 4 with chunk slot ^ ((row >> 2) & 3).
  uint32_t qoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * wave + 16 * i + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    qoff[i] = (uint32_t)((row * a.Dp + 8 * chunk) * 2);
  }
  const char* qbase = (const char*)(a.qa[0] + q0 * a.Dp);
  auto stage_q = [&](int s, int item) {
    const int buf = s % 3, ar = item >> 1;
    const int rbase = 32 * wave + 16 * (item & 1);
    const int sw_ = s < a.W ? s : a.W - 1;          // past the last word: a harmless copy
    copy16_to_lds_s(qoff[item & 1], qbase + ((int64_t)ar * a.qa_step + 32 * sw_) * 2,
                    __builtin_amdgcn_readfirstlane(lds_addr(&As[buf][ar][rbase * 32])));
  };
  // Plane words of word s into buffer s % 4, items 0 .. NRI - 1: copy j = w +
  // 8 item (if j < NRC) moves dwords 64 j .. 64 j + 63 of the tile's
  // [record][plane] block (a record past the chunk's end reads the last one;
  // its scores are dropped).
  constexpr int NRI = (NRC + 7) / 8;
  const int n_rc = wave < NRC ? (NRC - 1 - wave) / 8 + 1 : 0;   // copies per wave
  uint32_t roff[NRI];
#pragma unroll
  for (int i = 0; i < NRI; ++i) {
    const int e = 64 * (wave + 8 * i) + lane, r = e / NB, p = e - r * NB;
    const int64_t rl = r0 + r;
    roff[i] = (uint32_t)(((rl < a.n_rec ? rl : a.n_rec - 1) * (int64_t)(a.W * NB) + p) * 4);
  }
  const char* rbase_p = (const char*)(a.planes + a.rec0 * (int64_t)(a.W * NB));
  auto stage_r = [&](int s, int item) {
    const int j = wave + 8 * item;
    if (NRC % 8 == 0 || j < NRC) {
      const int buf = s & 3;
      const int sw_ = s < a.W ? s : a.W - 1;
      copy4_to_lds_s(roff[item], rbase_p + (int64_t)sw_ * NB * 4,
                     __builtin_amdgcn_readfirstlane(lds_addr(&Rs[buf][64 * j])));
    }
  };
  // item i of step st: rows of word st + 2, then planes of word st + 3.  Every
  // step issues all of them (no branch splits the step's schedule): past the
  // last word they refill a buffer that no later step reads with a valid word.
  auto stage_item = [&](int st, int i) {
    if (i < 2 * NA)
      stage_q(st + 2, i);
    else if (i < 2 * NA + NRI)
      stage_r(st + 3, i - 2 * NA);
  };

  // this lane's records 64 wr + 32 rb + col
  uint32_t tg[2];            // bytes: gamma_hi ^ 0x80, gamma_hi, gamma_lo
  float nu_r[2];
  bool rlive[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int64_t rl = r0 + 64 * wr + 32 * rb + col;
    rlive[rb] = rl < a.n_rec;
    const int64_t rc = a.rec0 + (rlive[rb] ? rl : a.n_rec - 1);
    const uint32_t nn = a.norms[rc];
    nu_r[rb] = __half2float(__ushort_as_half((unsigned short)(nn & 0xffffu)));
    const uint32_t g = nn >> 16, glo = g & 0xffu, ghi = (g >> 8) & 0xffu;
    tg[rb] = (ghi ^ 0x80u) | (ghi << 8) | (glo << 16);
  }
  uint32_t tb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) tb[i] = a.tb[i];

  // B operands of one 32 x 32 block for K-slots 16 kk + 8 hh .. + 7, i.e. byte
  // groups g = 4 kk + 2 hh and g + 1; w holds the plane words shifted right by
  // 2 hh, so group g + j's bits are at 4 kk + j for every lane.  Dwords of an
  // fp16 operand: (slots 0,1), (2,3) of group g, then of group g + 1.  One call
  // fills the two dwords of group g + j in B[0] (centroid hi) and B[1]
  // (gamma s), and dword 2 kk + j (fp8 centroid hi) and 4 + 2 kk + j (fp8
  // centroid lo) of the lane's fp8 operand B8 for the word's correction product.
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  auto decode_group = [&](const uint32_t (&w)[NB], uint32_t tgr, int kk, int j, u4v (&B)[2],
                          v8i& B8) {
    const int k = 4 * kk + j;
    uint32_t v = w[0] & (0x01010101u << k);
    if constexpr (CP >= 2) v |= (w[1] << 1) & (0x02020202u << k);
    if constexpr (CP >= 3) v |= (w[2] << 2) & (0x04040404u << k);
    const uint32_t sel = v >> k;                     // code index per byte
    const uint32_t hl = __builtin_amdgcn_perm(tb[1], tb[0], sel);
    const uint32_t hh8 = __builtin_amdgcn_perm(tb[3], tb[2], sel);
    B[0][2 * j] = __builtin_amdgcn_perm(hh8, hl, 0x05010400u);
    B[0][2 * j + 1] = __builtin_amdgcn_perm(hh8, hl, 0x07030602u);
    B8[2 * kk + j] = (int)__builtin_amdgcn_perm(tb[5], tb[4], sel);
    B8[4 + 2 * kk + j] = (int)__builtin_amdgcn_perm(tb[7], tb[6], sel);
    if constexpr (!MSE) {
      const uint32_t sb = (w[NB - 1] >> k) & 0x01010101u;     // sign bits per byte
      // selectors (2, b0, 2, b1) and (2, b2, 2, b3) into tgr
      const uint32_t sa = __builtin_amdgcn_perm(0x02020202u, sb, 0x01040004u);
      const uint32_t sc = __builtin_amdgcn_perm(0x02020202u, sb, 0x03040204u);
      B[1][2 * j] = __builtin_amdgcn_perm(0u, tgr, sa);
      B[1][2 * j + 1] = __builtin_amdgcn_perm(0u, tgr, sc);
    }
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (v16f){};
  v8i B8[2];                 // per record block: the word's fp8 correction operand
  // this lane's plane words of word s (records 64 wr + 32 rb + col), shifted
  // right by 2 hh
  auto rec_words = [&](int s, uint32_t (&w)[2][NB]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const uint32_t* rw = &Rs[s & 3][(64 * wr + 32 * rb + col) * NB];
      if constexpr (NB == 4) {
        const uint4 v = *(const uint4*)rw;
        w[rb][0] = v.x; w[rb][1] = v.y; w[rb][2] = v.z; w[rb][3] = v.w;
      } else {
#pragma unroll
        for (int p = 0; p < NB; ++p) w[rb][p] = rw[p];
      }
#pragma unroll
      for (int p = 0; p < NB; ++p) w[rb][p] >>= 2 * hh;
    }
  };
  // scales of the fp8 correction product: lane (row, hh) gives the code of its
  // row's block hh (A: 2^-e_lo for the lo part, 2^-e_hi for the hi part),
  // lane (record, hh) that of its column's block hh (B: 2^-e_chi, 2^-e_clo)
  int sa8[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
    sa8[qb] = (int)((a.q8scale[q0 + 128 * wq + 32 * qb + col] >> (8 * hh)) & 0xffu);
  const int sb8 = (int)((a.bscale >> (8 * hh)) & 0xffu);

  // fp16 MFMAs of K-slice kk of word s (query rows from buffer s % 3) on the
  // operands Bc: QR hi x centroid hi and (alpha QP) hi x gamma s.  The decode
  // of the next K-slice's operands Bd / B8 (group j of record block rb per
  // 32-query block) is interleaved: per query block, its operand reads, then
  // each MFMA followed by vector instructions.
  constexpr int NF = MSE ? 1 : 2;                // fp16 MFMAs per block and K-slice
  // Operand reads: row 128 wq + 32 qb + col, chunk c sits at halves
  // (row * 32) + ((c ^ ((row >> 2) & 3)) << 3), and (row >> 2) & 3 is the same
  // for every qb, so a lane reads chunk c of all its rows, arrays and buffers
  // at fixed distances from one address per chunk (immediate offsets).
  typedef const __attribute__((address_space(3))) char* lds_cp;
  const uint32_t rsw = (uint32_t)(col >> 2) & 3u;
  const uint32_t as0 = lds_addr(&As[0][0][0]);
  auto a_addr = [&](int buf, int c) -> lds_cp {
    const uint32_t off = (((uint32_t)(128 * wq + col) * 32u + ((((uint32_t)c) ^ rsw) << 3)) * 2u) & 0xffffu;
    return (lds_cp)(uintptr_t)(as0 + (uint32_t)buf * (uint32_t)(NA * kQT * 64) + off);
  };
  constexpr int kArr = kQT * 32 * 2;             // bytes per staged array
  auto products = [&](int s, int kk, const u4v (&Bc)[2][2], const uint32_t (&wd)[2][NB],
                      int kkd, u4v (&Bd)[2][2]) {
    const lds_cp ab = a_addr(s % 3, 2 * kk + hh);
    static_assert(2 * NA + NRI <= 8, "one copy per query block and K-slice");
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const v8h A0 = *(const __attribute__((address_space(3))) v8h*)(ab + qb * 2048);
      v8h A2 = A0;
      if constexpr (!MSE)
        A2 = *(const __attribute__((address_space(3))) v8h*)(ab + 2 * kArr + qb * 2048);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        v16f c = acc[qb][rb];
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, __builtin_bit_cast(v8h, Bc[rb][0]), c, 0,
                                                   0, 0);
        if constexpr (!MSE)
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(A2, __builtin_bit_cast(v8h, Bc[rb][1]), c,
                                                     0, 0, 0);
        acc[qb][rb] = c;
      }
      decode_group(wd[qb >> 1], tg[qb >> 1], kkd, qb & 1, Bd[qb >> 1], B8[qb >> 1]);
      __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);
#pragma unroll
      for (int m = 0; m < 2 * NF; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      stage_item(s, 4 * kk + qb);
    }
  };
  // the word's correction products, one scaled fp8 MFMA per 32 x 32 block:
  // K block 0 = (QR lo) 2^e_lo x (c hi) 2^e_chi, block 1 = (QR hi) 2^e_hi x
  // (c lo) 2^e_clo, over the lane's 16 K-slots of each (query rows from
  // buffer s % 3, array 1: the lo part in chunks 0-1, the hi part in 2-3)
  auto corrections = [&](int s) {
    const lds_cp al = a_addr(s % 3, hh) + kArr;
    const lds_cp ah = a_addr(s % 3, 2 + hh) + kArr;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const u4v lo = *(const __attribute__((address_space(3))) u4v*)(al + qb * 2048);
      const u4v hi = *(const __attribute__((address_space(3))) u4v*)(ah + qb * 2048);
      const v8i A8 = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[qb][rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A8, B8[rb], acc[qb][rb], 0,
                                                                      0, 0, sa8[qb], 0, sb8);
    }
  };

  // Copies run ahead of the products: query rows two words, plane words
  // three.  Step s - 2 issues the rows of word s and the planes of word
  // s + 1, so a step can decode the first K-slice of the next word during its
  // second half and start on products right after the barrier.
  auto stage_r_all = [&](int s) {
#pragma unroll
    for (int i = 0; i < NRI; ++i) stage_r(s, i);
  };
  auto stage_q_all = [&](int s) {
#pragma unroll
    for (int i = 0; i < 2 * NA; ++i) stage_q(s, i);
  };
  stage_r_all(0);
  stage_q_all(0);
  if (a.W > 1) stage_r_all(1);
  if (a.W > 1) stage_q_all(1);
  if (a.W > 2) stage_r_all(2);
  wait_vmcnt((a.W > 1 ? 2 * NA : 0) + (a.W > 2 ? n_rc : 0));   // rows of word 0, planes of 0 and 1
  __syncthreads();
  u4v Bn[2][2], Bk[2][2];    // K-slice 0 of the current word (decoded one step early), slice 1
  uint32_t w[2][NB];         // the current word's plane words (read one step early)
  rec_words(0, w);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    decode_group(w[rb], tg[rb], 0, 0, Bn[rb], B8[rb]);
    decode_group(w[rb], tg[rb], 0, 1, Bn[rb], B8[rb]);
  }
  for (int st = 0; st < a.W; ++st) {
    if (st > 0) {
        // rows of word st and planes of word st + 1 landed (the copies of
      // step st - 1 may still be in flight), then for every wave
      wait_vmcnt(2 * NA + n_rc);
      __syncthreads();
    }
    // the products issue the copies of rows st + 2 and planes st + 3:
    // buffers (st + 2) % 3 and (st + 3) % 4 were last read in step st - 1
    // (after the last word, the "next" plane words are a stale buffer:
    // decoded, never used)
    products(st, 0, Bn, w, 1, Bk);
    corrections(st);           // B8 complete: slice 0 (a step early) and slice 1
    uint32_t wn[2][NB];        // planes of word st + 1 landed before this step's barrier
    rec_words(st + 1, wn);
    products(st, 1, Bk, wn, 0, Bn);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int p = 0; p < NB; ++p) w[rb][p] = wn[rb][p];
  }

  // thresholds of the tile's queries, in the (now free) query-row buffers;
  // no copy may still be writing LDS
  wait_vmcnt(0);
  float* thr_s = (float*)&As[0][0][0];
  __syncthreads();
  if (tid < kQT) {
    const int64_t q = q0 + tid;
    thr_s[tid] = q < a.n_q ? a.thr[q] : INFINITY;   // padded rows never pass
  }
  __syncthreads();

  // epilogue: element i of block (qb, rb) is query 128 wq + 32 qb + 8 (i / 4) +
  // 4 hh + i % 4 and record 64 wr + 32 rb + col; keep scores above the
  // query's threshold
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int64_t rl = r0 + 64 * wr + 32 * rb + col;
    const float nu = nu_r[rb];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ql = 128 * wq + 32 * qb + 8 * (i >> 2) + 4 * hh + (i & 3);
        const float sc = nu * acc[qb][rb][i];
        const bool pass = rlive[rb] && sc > thr_s[ql];
        const uint64_t m = __ballot(pass);
        if (m) {
          // lanes 0..31 share one query row, lanes 32..63 another
          const uint32_t mh = hh ? (uint32_t)(m >> 32) : (uint32_t)m;
          int base = 0;
          if (col == 0 && mh) base = atomicAdd(&a.cnt[q0 + ql], __popc(mh));
          base = __shfl(base, 32 * hh);
          if (pass) {
            const int64_t slot = (q0 + ql) * a.chunk + base + __popc(mh & ((1u << col) - 1u));
            a.cand_s[slot] = sc;
            a.cand_i[slot] = (int)rl;
          }
        }
      }
  }
}

// ---- candidate merge: one wave per query ---------------------------------------
struct MergeArgs {
  int64_t n_q, base;     // candidate indices are relative to record `base`
  int k;
  float* thr;
  int* cnt;
  const float* cand_s;
  const int* cand_i;
  int64_t chunk;         // candidate capacity per query
  float* run_score;      // [n_q][k]
  int64_t* run_idx;
  int first, last;
  float* out_score;
  int64_t* out_idx;
};

__device__ inline bool beats(float as, int64_t ai, float bs, int64_t bi) {
  return as > bs || (as == bs && ai < bi);
}

__global__ void __launch_bounds__(256) cand_merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t q = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= a.n_q) return;
  const int k = a.k;
  float sv = -INFINITY;
  int64_t iv = -1;
  if (!a.first && lane < k) {
    sv = a.run_score[q * k + lane];
    iv = a.run_idx[q * k + lane];
  }
  float ts = __shfl(sv, k - 1);
  int64_t ti = __shfl(iv, k - 1);
  const int n = a.cnt[q];
  const float* cs = a.cand_s + q * a.chunk;
  const int* ci = a.cand_i + q * a.chunk;
  for (int b0 = 0; b0 < n; b0 += 64) {
    const bool in = b0 + lane < n;
    const float v = in ? cs[b0 + lane] : -INFINITY;
    const int64_t id = in ? a.base + ci[b0 + lane] : -1;
    uint64_t mask = __ballot(in && beats(v, id, ts, ti));
    while (mask) {
      const int src = __ffsll((unsigned long long)mask) - 1;
      const float cv = __shfl(v, src);
      const int64_t cid = __shfl(id, src);
      // entries that beat the candidate form a prefix of the sorted list
      const uint64_t bm = __ballot(lane < k && beats(sv, iv, cv, cid));
      const int p = __popcll(bm);
      const float us = __shfl_up(sv, 1);
      const int64_t ui = __shfl_up(iv, 1);
      if (p < k) {
        if (lane > p && lane < k) {
          sv = us;
          iv = ui;
        }
        if (lane == p) {
          sv = cv;
          iv = cid;
        }
      }
      ts = __shfl(sv, k - 1);
      ti = __shfl(iv, k - 1);
      mask &= ~(1ull << src);
      mask &= __ballot(in && beats(v, id, ts, ti));
    }
  }
  if (lane < k) {
    if (a.last) {
      a.out_score[q * k + lane] = sv;
      a.out_idx[q * k + lane] = iv;
    } else {
      a.run_score[q * k + lane] = sv;
      a.run_idx[q * k + lane] = iv;
    }
  }
  if (lane == 0) {
    a.thr[q] = ts;     // k-th best so far (-inf while fewer than k)
    a.cnt[q] = 0;
  }
}

__global__ void search_init_kernel(float* thr, int* cnt, int64_t n_q) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q < n_q) {
    thr[q] = -INFINITY;
    cnt[q] = 0;
  }
}

void fill_centroid_split(const tq_ctx* ctx, GemmArgs& g) {
  for (int k = 0; k < kMaxK; ++k) {
    const float c = k < ctx->K ? ctx->cent[k] : 0.f;
    const _Float16 h = (_Float16)c;
    g.c_hi[k] = h;
    g.c_lo[k] = (_Float16)(c - (float)h);
  }
}

template <int MODE>
hipError_t launch_gemm(const tq_ctx* ctx, const GemmArgs& g, dim3 grid, hipStream_t st) {
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: hipLaunchKernelGGL((decoded_gemm_kernel<1, true, MODE>), grid, dim3(256), 0, st, g); break;
      case 2: hipLaunchKernelGGL((decoded_gemm_kernel<2, true, MODE>), grid, dim3(256), 0, st, g); break;
      default: hipLaunchKernelGGL((decoded_gemm_kernel<3, true, MODE>), grid, dim3(256), 0, st, g); break;
    }
  } else {
    switch (ctx->b) {
      case 2: hipLaunchKernelGGL((decoded_gemm_kernel<2, false, MODE>), grid, dim3(256), 0, st, g); break;
      case 3: hipLaunchKernelGGL((decoded_gemm_kernel<3, false, MODE>), grid, dim3(256), 0, st, g); break;
      default: hipLaunchKernelGGL((decoded_gemm_kernel<4, false, MODE>), grid, dim3(256), 0, st, g); break;
    }
  }
  return hipGetLastError();
}

struct SearchLayout {
  size_t qa[4], thr, cnt, cand_s, cand_i, run_s, run_i, total;
  int64_t rows_pad;
};

SearchLayout search_layout(const tq_ctx* ctx, int64_t n_queries, int32_t k) {
  SearchLayout L{};
  L.rows_pad = (n_queries + kQT - 1) / kQT * kQT;
  const size_t mat = align256((size_t)L.rows_pad * ctx->Dp * sizeof(__half));
  size_t off = 0;
  for (int i = 0; i < 4; ++i) {
    L.qa[i] = off;
    off += mat;
  }
  L.thr = off; off += align256((size_t)n_queries * sizeof(float));
  L.cnt = off; off += align256((size_t)n_queries * sizeof(int));
  const size_t chunk = (size_t)search_chunk(n_queries);
  L.cand_s = off; off += align256((size_t)n_queries * chunk * sizeof(float));
  L.cand_i = off; off += align256((size_t)n_queries * chunk * sizeof(int));
  L.run_s = off; off += align256((size_t)n_queries * k * sizeof(float));
  L.run_i = off; off += align256((size_t)n_queries * k * sizeof(int64_t));
  L.total = off;
  return L;
}

}  // namespace

size_t search_workspace_bytes(const tq_ctx* ctx, int64_t n_queries, int64_t n_db, int32_t k) {
  (void)n_db;
  return search_layout(ctx, n_queries, k).total;
}

hipError_t launch_search_topk(const tq_ctx* ctx, const float* queries, int64_t n_queries,
                              const uint32_t* planes, const uint16_t* norms, int64_t n_db,
                              int32_t k, int64_t* out_idx, float* out_score, void* workspace,
                              hipStream_t stream) {
  const SearchLayout L = search_layout(ctx, n_queries, k);
  char* ws = (char*)workspace;
  const float alpha = (float)(std::sqrt(M_PI / 2.0) / ctx->d);
  RowPrepArgs p{};
  p.q = queries;
  p.pit = ctx->t.pit32;
  p.st = ctx->t.st32;
  p.qr_hi = (__half*)(ws + L.qa[0]);
  p.q8 = (uint8_t*)(ws + L.qa[1]);               // 64 bytes per row and word: as large as QR lo
  p.qp_hi = (__half*)(ws + L.qa[2]);
  p.q8scale = (uint32_t*)(ws + L.qa[3]);
  p.pscale = alpha;
  p.d = ctx->d;
  p.Dp = ctx->Dp;
  p.n = n_queries;
  p.n_pad = L.rows_pad;
  // MSE-only records need the Pi q rows alone (the S q half is never read)
  const int prep_out = ctx->mse ? ctx->Dp : 2 * ctx->Dp;
  hipLaunchKernelGGL(row_prep_kernel,
                     dim3((unsigned)((L.rows_pad + kPrepRows - 1) / kPrepRows),
                          (unsigned)((prep_out + kPrepOut - 1) / kPrepOut)),
                     dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  SearchArgs g{};
  for (int i = 0; i < 4; ++i) g.qa[i] = (const __half*)(ws + L.qa[i]);
  g.qa_step = (int64_t)(L.qa[1] - L.qa[0]) / (int64_t)sizeof(__half);
  g.n_q = n_queries;
  g.planes = planes;
  g.norms = (const uint32_t*)norms;
  g.W = ctx->W;
  g.Dp = ctx->Dp;
  // codebook byte tables: byte k % 4 of tb[half * 2 + (k >= 4)] is byte
  // `half` of centroid k's fp16 hi part; of tb[4 + (k >= 4)] its fp8 hi part
  // (c_hi 2^e_chi), of tb[6 + (k >= 4)] its fp8 lo part (c_lo 2^e_clo).
  // |c| < 2^e puts c_hi 2^(8-e) below 256, and |c_lo| <= 2^-11 |c| the lo part.
  float cmax = 0.f;
  for (int j = 0; j < ctx->K; ++j) cmax = std::max(cmax, std::fabs(ctx->cent[j]));
  int ce = 0;
  std::frexp(cmax, &ce);
  const int echi = std::min(100, std::max(-100, 8 - ce)), eclo = echi + 11;
  g.bscale = (uint32_t)(127 - echi) | ((uint32_t)(127 - eclo) << 8);
  for (int i = 0; i < 8; ++i) g.tb[i] = 0u;
  for (int j = 0; j < kMaxK; ++j) {
    const float c = j < ctx->K ? ctx->cent[j] : 0.f;
    const _Float16 h = (_Float16)c;
    const float l = c - (float)h;
    const uint32_t hb = __builtin_bit_cast(uint16_t, h);
    const int sh = 8 * (j & 3), up = j >> 2;
    g.tb[0 + up] |= (hb & 0xffu) << sh;
    g.tb[2 + up] |= (hb >> 8) << sh;
    g.tb[4 + up] |= (uint32_t)to_e4m3(std::ldexp((float)h, echi)) << sh;
    g.tb[6 + up] |= (uint32_t)to_e4m3(std::ldexp(l, eclo)) << sh;
  }
  g.q8scale = (const uint32_t*)(ws + L.qa[3]);
  g.thr = (float*)(ws + L.thr);
  g.cnt = (int*)(ws + L.cnt);
  g.cand_s = (float*)(ws + L.cand_s);
  g.cand_i = (int*)(ws + L.cand_i);
  g.chunk = search_chunk(n_queries);

  MergeArgs m{};
  m.n_q = n_queries;
  m.k = k;
  m.thr = (float*)(ws + L.thr);
  m.cnt = g.cnt;
  m.cand_s = g.cand_s;
  m.cand_i = g.cand_i;
  m.chunk = g.chunk;
  m.run_score = (float*)(ws + L.run_s);
  m.run_idx = (int64_t*)(ws + L.run_i);
  m.out_score = out_score;
  m.out_idx = out_idx;

  hipLaunchKernelGGL(search_init_kernel, dim3((unsigned)((n_queries + 255) / 256)), dim3(256), 0,
                     stream, m.thr, m.cnt, n_queries);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // chunks: a small first one sets the thresholds, then g.chunk records each
  int64_t base = 0;
  bool first = true;
  do {
    const int64_t len = std::min<int64_t>(n_db - base, first ? kFirst : g.chunk);
    if (len > 0) {
      g.rec0 = base;
      g.n_rec = len;
      const dim3 grid((unsigned)((len + kRT - 1) / kRT), (unsigned)(L.rows_pad / kQT));
      if (ctx->mse) {
        switch (ctx->b) {
          case 1: hipLaunchKernelGGL((search_gemm_kernel<1, true>), grid, dim3(512), 0, stream, g); break;
          case 2: hipLaunchKernelGGL((search_gemm_kernel<2, true>), grid, dim3(512), 0, stream, g); break;
          default: hipLaunchKernelGGL((search_gemm_kernel<3, true>), grid, dim3(512), 0, stream, g); break;
        }
      } else {
        switch (ctx->b) {
          case 2: hipLaunchKernelGGL((search_gemm_kernel<2, false>), grid, dim3(512), 0, stream, g); break;
          case 3: hipLaunchKernelGGL((search_gemm_kernel<3, false>), grid, dim3(512), 0, stream, g); break;
          default: hipLaunchKernelGGL((search_gemm_kernel<4, false>), grid, dim3(512), 0, stream, g); break;
        }
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    m.base = base;
    m.first = first;
    m.last = base + len >= n_db;
    hipLaunchKernelGGL(cand_merge_kernel, dim3((unsigned)((n_queries + 3) / 4)), dim3(256), 0,
                       stream, m);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    base += len;
    first = false;
  } while (base < n_db);
  return hipSuccess;
}

namespace {
template <int NB, bool MSE>
hipError_t launch_dq128(const GemmArgs& g, int n_cu, hipStream_t st) {
  static int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, dequant128_kernel<NB, MSE>, 256, 0) !=
            hipSuccess ||
        nb < 1)
      nb = 1;
    return nb;
  }();
  const int64_t n_tiles = (g.n_rec + kDqT - 1) / kDqT;
  const int64_t grid = std::min<int64_t>(n_tiles, (int64_t)n_cu * per_cu);
  hipLaunchKernelGGL((dequant128_kernel<NB, MSE>), dim3((unsigned)grid), dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_dequant128(const tq_ctx* ctx, const GemmArgs& g, hipStream_t st) {
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: return launch_dq128<1, true>(g, ctx->n_cu, st);
      case 2: return launch_dq128<2, true>(g, ctx->n_cu, st);
      default: return launch_dq128<3, true>(g, ctx->n_cu, st);
    }
  }
  switch (ctx->b) {
    case 2: return launch_dq128<2, false>(g, ctx->n_cu, st);
    case 3: return launch_dq128<3, false>(g, ctx->n_cu, st);
    default: return launch_dq128<4, false>(g, ctx->n_cu, st);
  }
}
}  // namespace

hipError_t launch_dequantize(const tq_ctx* ctx, const uint32_t* planes, const uint16_t* norms,
                             int64_t n, float* out, int64_t out_ld, hipStream_t stream) {
  GemmArgs g{};
  g.qr_hi = ctx->t.pit_hi;
  g.qr_lo = ctx->t.pit_lo;
  g.qp_hi = ctx->t.st_hi;
  g.qp_lo = ctx->t.st_lo;
  g.n_rows = ctx->d;
  g.planes = planes;
  g.norms = (const uint32_t*)norms;
  g.rec0 = 0;
  g.n_rec = n;
  g.W = ctx->W;
  g.Dp = ctx->Dp;
  g.alpha = (float)(std::sqrt(M_PI / 2.0) / ctx->d);
  fill_centroid_split(ctx, g);
  g.out = out;
  g.out_ld = out_ld;
  // d = 128 with enough records to fill the chip: the register-resident form
  // (each workgroup loads 128 KB of tables, which a few tiles do not repay)
  if (ctx->d == 128 && n >= (int64_t)kDqT * ctx->n_cu) {
    g.out_vec4 = (out_ld % 4 == 0 && ((uintptr_t)out & 15) == 0) ? 1 : 0;
    return launch_dequant128(ctx, g, stream);
  }
  const dim3 grid((unsigned)((n + kRecTile - 1) / kRecTile),
                  (unsigned)((ctx->Dp + kRowsTile - 1) / kRowsTile));
  return launch_gemm<1>(ctx, g, grid, stream);
}

}  // namespace tq
