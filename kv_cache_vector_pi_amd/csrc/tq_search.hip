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
// Search: records are decoded once per 128-record tile and 32-coordinate word
// into fp16 LDS operands -- centroid hi and lo parts and gamma * s (gamma is
// an fp16 value and s = +-1, so the product is exact) -- and the query rows,
// split hi + lo with alpha folded into the sketch half, are staged next to
// them.  One accumulator then takes all five passes on
// v_mfma_f32_32x32x16_f16:
//   acc += QR_hi c_hi + QR_lo c_hi + QR_hi c_lo + (alpha QP)_hi gs + (alpha QP)_lo gs,
// and score = nu * acc.  Instead of writing every score, the epilogue keeps
// only those above the query's running k-th best score (candidates appended
// with one atomic per wave and query row), and a one-wave-per-query merge
// after each chunk of records folds them into the running top-k (score
// descending, index ascending) and raises the threshold.
//
// Dequantization keeps the two-accumulator form on 16x16x32 tiles.
#include <algorithm>
#include <cmath>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kRowsTile = 64;    // dequantize: rows per workgroup
constexpr int kRecTile = 64;     // dequantize: records per workgroup
constexpr int kLdsRow = 40;      // halves per staged row of one word (32 + pad)
constexpr int kQT = 128;         // search: queries per workgroup
constexpr int kRT = 128;         // search: records per workgroup
constexpr int kFirst = 2048;     // search: records of the first chunk (sets the thresholds)
constexpr int kChunk = 16384;    // search: records per later chunk = candidate capacity

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- row preparation: Pi q and S q, split into hi/lo fp16 -----------------
// Block (row group of kPrepRows queries, chunk of 256 outputs): each thread
// owns one output row of Pi or S, reads that row as a contiguous column of
// Pi^T / S^T (coalesced across the wave) and accumulates it against the
// group's queries, which are staged through LDS 256 coordinates at a time.
constexpr int kPrepRows = 16;
constexpr int kPrepJ = 256;

struct RowPrepArgs {
  const float* q;        // [n][d]
  const float* pit;      // [d][d] Pi^T
  const float* st;       // [d][d] S^T
  __half* qr_hi;         // [n_pad][Dp]
  __half* qr_lo;
  __half* qp_hi;
  __half* qp_lo;
  float pscale;          // factor on S q (alpha for search)
  int d, Dp;
  int64_t n, n_pad;
};

__global__ void __launch_bounds__(256) row_prep_kernel(RowPrepArgs a) {
  __shared__ __align__(16) float qv[kPrepJ][kPrepRows];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * kPrepRows;
  const int o = blockIdx.y * 256 + tid;          // output index over [Pi rows | S rows]
  const bool sk = o >= a.Dp;
  const int r = sk ? o - a.Dp : o;
  const bool live = o < 2 * a.Dp && r < a.d;
  const float* col = (sk ? a.st : a.pit) + (live ? r : 0);
  float acc[kPrepRows];
#pragma unroll
  for (int i = 0; i < kPrepRows; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < a.d; j0 += kPrepJ) {
    const int nj = min(kPrepJ, a.d - j0);
    __syncthreads();
    for (int it = tid; it < kPrepJ * kPrepRows; it += 256) {
      const int i = it / kPrepJ, j = it % kPrepJ;
      const int64_t row = row0 + i;
      qv[j][i] = (row < a.n && j < nj) ? a.q[row * a.d + j0 + j] : 0.f;
    }
    __syncthreads();
    if (live) {
      auto step = [&](const float t, const int j) {
        const float4* qq = (const float4*)&qv[j][0];
#pragma unroll
        for (int i4 = 0; i4 < kPrepRows / 4; ++i4) {
          const float4 v = qq[i4];
          acc[4 * i4 + 0] = fmaf(t, v.x, acc[4 * i4 + 0]);
          acc[4 * i4 + 1] = fmaf(t, v.y, acc[4 * i4 + 1]);
          acc[4 * i4 + 2] = fmaf(t, v.z, acc[4 * i4 + 2]);
          acc[4 * i4 + 3] = fmaf(t, v.w, acc[4 * i4 + 3]);
        }
      };
      int j = 0;
      // batches of 16 independent column loads in flight
      for (; j + 16 <= nj; j += 16) {
        float t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) t[u] = col[(int64_t)(j0 + j + u) * a.d];
#pragma unroll
        for (int u = 0; u < 16; ++u) step(t[u], j + u);
      }
      for (; j < nj; ++j) step(col[(int64_t)(j0 + j) * a.d], j);
    }
  }
  if (o >= 2 * a.Dp) return;
  __half* hi = sk ? a.qp_hi : a.qr_hi;
  __half* lo = sk ? a.qp_lo : a.qr_lo;
#pragma unroll
  for (int i = 0; i < kPrepRows; ++i) {
    const int64_t row = row0 + i;
    if (row < a.n_pad) {
      const float v = live ? (sk ? a.pscale * acc[i] : acc[i]) : 0.f;
      const __half vh = __float2half(v);
      hi[row * a.Dp + r] = vh;
      lo[row * a.Dp + r] = __float2half(v - __half2float(vh));
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
  const __half* qa[4];   // QR hi, QR lo, (alpha QP) hi, (alpha QP) lo: [rows_pad][Dp]
  int64_t n_q;
  const uint32_t* planes;
  const uint32_t* norms;
  int64_t rec0, n_rec;   // records rec0 .. rec0 + n_rec - 1 of this chunk
  int W, Dp;
  uint32_t ctab[kMaxK];  // centroid k: fp16 hi | fp16 lo << 16
  const float* thr;      // [n_q] running k-th best score (-inf: fewer than k yet)
  int* cnt;              // [n_q] candidates of this chunk
  float* cand_s;         // [n_q][kChunk]
  int* cand_i;           // [n_q][kChunk] record index within the chunk
};

template <int NB, bool MSE>
__global__ void __launch_bounds__(256, 2) search_gemm_kernel(SearchArgs a) {
  constexpr int CP = MSE ? NB : NB - 1;         // code planes
  // staged query arrays: QR hi, QR lo and (alpha QP) hi.  The sketch term
  // alpha gamma <QP, s> is a small part of a score, so its fp16 rounding of
  // QP (2^-12 relative) stays ~1e-4 of the scores' rms; (alpha QP) lo is not
  // used.  The code term keeps hi/lo products (2^-22).
  constexpr int NA = MSE ? 2 : 3;
  __shared__ __align__(16) _Float16 As[NA][kQT * kLdsRow];
  __shared__ __align__(16) _Float16 Bs[3][kRT * kLdsRow];
  __shared__ float thr_s[kQT];
  __shared__ uint32_t ctab_s[kMaxK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int wq = wave & 1, wr = wave >> 1;       // wave tile: 64 queries x 64 records
  const int64_t r0 = (int64_t)blockIdx.x * kRT, q0 = (int64_t)blockIdx.y * kQT;

  if (tid < kQT) {
    const int64_t q = q0 + tid;
    thr_s[tid] = q < a.n_q ? a.thr[q] : INFINITY;   // padded rows never pass
  }
  if (tid < kMaxK) ctab_s[tid] = a.ctab[tid];
  // decode role: record dr, coordinates 16 dh .. 16 dh + 15 of each word
  const int dr = tid >> 1, dh = tid & 1;
  const bool dlive = r0 + dr < a.n_rec;
  const uint32_t* drec = a.planes + (a.rec0 + r0 + dr) * (int64_t)a.W * NB;
  const uint16_t gbits =
      dlive ? (uint16_t)(a.norms[a.rec0 + r0 + dr] >> 16) : (uint16_t)0;   // fp16 gamma

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (v16f){};

  // Word w's query rows (NA arrays x 128 rows x 32 halves, 16 bytes a thread
  // x 2 NA) and record words are loaded into registers one word ahead, so the
  // loads are in flight while the previous word's MFMAs run.
  v8h ra[2 * NA];
  uint32_t wd[NB];
  auto load_word = [&](int w) {
#pragma unroll
    for (int j = 0; j < 2 * NA; ++j) {
      const int c = tid + 256 * j;
      const int ar = c >> 9, row = (c >> 2) & 127, part = c & 3;
      ra[j] = *(const v8h*)(a.qa[ar] + (q0 + row) * a.Dp + 32 * w + 8 * part);
    }
#pragma unroll
    for (int p = 0; p < NB; ++p) wd[p] = dlive ? drec[w * NB + p] : 0u;
  };
  load_word(0);
  for (int w = 0; w < a.W; ++w) {
    __syncthreads();              // previous word's operands fully read
#pragma unroll
    for (int j = 0; j < 2 * NA; ++j) {
      const int c = tid + 256 * j;
      const int ar = c >> 9, row = (c >> 2) & 127, part = c & 3;
      *(v8h*)(&As[ar][row * kLdsRow + 8 * part]) = ra[j];
    }
    // decode word w of record dr
    {
      v8h vh[2], vl[2], vg[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int bit = 16 * dh + e;
        uint32_t idx = 0;
#pragma unroll
        for (int p = 0; p < CP; ++p) idx |= ((wd[p] >> bit) & 1u) << p;
        const uint32_t hl = ctab_s[idx];
        const uint16_t sgn = (MSE || ((wd[NB - 1] >> bit) & 1u)) ? (uint16_t)0 : (uint16_t)0x8000;
        vh[e >> 3][e & 7] = __builtin_bit_cast(_Float16, (uint16_t)(hl & 0xffffu));
        vl[e >> 3][e & 7] = __builtin_bit_cast(_Float16, (uint16_t)(hl >> 16));
        vg[e >> 3][e & 7] = __builtin_bit_cast(_Float16, (uint16_t)(gbits ^ sgn));
      }
      const int off = dr * kLdsRow + 16 * dh;
      *(v8h*)(&Bs[0][off]) = vh[0];
      *(v8h*)(&Bs[0][off + 8]) = vh[1];
      *(v8h*)(&Bs[1][off]) = vl[0];
      *(v8h*)(&Bs[1][off + 8]) = vl[1];
      if constexpr (!MSE) {
        *(v8h*)(&Bs[2][off]) = vg[0];
        *(v8h*)(&Bs[2][off + 8]) = vg[1];
      }
    }
    __syncthreads();
    if (w + 1 < a.W) load_word(w + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v8h A[2][NA], B[2][3];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int off = (64 * wq + 32 * qb + col) * kLdsRow + 16 * kk + 8 * hh;
#pragma unroll
        for (int ar = 0; ar < NA; ++ar) A[qb][ar] = *(const v8h*)(&As[ar][off]);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int off = (64 * wr + 32 * rb + col) * kLdsRow + 16 * kk + 8 * hh;
#pragma unroll
        for (int ar = 0; ar < (MSE ? 2 : 3); ++ar) B[rb][ar] = *(const v8h*)(&Bs[ar][off]);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          v16f c = acc[qb][rb];
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[qb][0], B[rb][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[qb][1], B[rb][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[qb][0], B[rb][1], c, 0, 0, 0);
          if constexpr (!MSE)
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[qb][2], B[rb][2], c, 0, 0, 0);
          acc[qb][rb] = c;
        }
    }
  }

  // epilogue: element i of tile (qb, rb) is query 64wq + 32qb + 8(i/4) + 4hh + i%4
  // and record 64wr + 32rb + col; keep scores above the query's threshold
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int64_t rl = r0 + 64 * wr + 32 * rb + col;
    const bool rlive = rl < a.n_rec;
    const float nu =
        rlive ? __half2float(__ushort_as_half((unsigned short)(a.norms[a.rec0 + rl] & 0xffffu)))
              : 0.f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ql = 64 * wq + 32 * qb + 8 * (i >> 2) + 4 * hh + (i & 3);
        const float sc = nu * acc[qb][rb][i];
        const bool pass = rlive && sc > thr_s[ql];
        const uint64_t m = __ballot(pass);
        if (m) {
          // lanes 0..31 share one query row, lanes 32..63 another
          const uint32_t mh = hh ? (uint32_t)(m >> 32) : (uint32_t)m;
          int base = 0;
          if (col == 0 && mh) base = atomicAdd(&a.cnt[q0 + ql], __popc(mh));
          base = __shfl(base, 32 * hh);
          if (pass) {
            const int64_t slot = (q0 + ql) * (int64_t)kChunk + base + __popc(mh & ((1u << col) - 1u));
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
  const float* cs = a.cand_s + q * (int64_t)kChunk;
  const int* ci = a.cand_i + q * (int64_t)kChunk;
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
  L.cand_s = off; off += align256((size_t)n_queries * kChunk * sizeof(float));
  L.cand_i = off; off += align256((size_t)n_queries * kChunk * sizeof(int));
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
  p.qr_lo = (__half*)(ws + L.qa[1]);
  p.qp_hi = (__half*)(ws + L.qa[2]);
  p.qp_lo = (__half*)(ws + L.qa[3]);
  p.pscale = alpha;
  p.d = ctx->d;
  p.Dp = ctx->Dp;
  p.n = n_queries;
  p.n_pad = L.rows_pad;
  // MSE-only records need the Pi q rows alone (the S q half is never read)
  const int prep_out = ctx->mse ? ctx->Dp : 2 * ctx->Dp;
  hipLaunchKernelGGL(row_prep_kernel,
                     dim3((unsigned)((L.rows_pad + kPrepRows - 1) / kPrepRows),
                          (unsigned)((prep_out + 255) / 256)),
                     dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  SearchArgs g{};
  for (int i = 0; i < 4; ++i) g.qa[i] = (const __half*)(ws + L.qa[i]);
  g.n_q = n_queries;
  g.planes = planes;
  g.norms = (const uint32_t*)norms;
  g.W = ctx->W;
  g.Dp = ctx->Dp;
  for (int j = 0; j < kMaxK; ++j) {
    const float c = j < ctx->K ? ctx->cent[j] : 0.f;
    const _Float16 h = (_Float16)c;
    const _Float16 l = (_Float16)(c - (float)h);
    g.ctab[j] = (uint32_t)__builtin_bit_cast(uint16_t, h) |
                ((uint32_t)__builtin_bit_cast(uint16_t, l) << 16);
  }
  g.thr = (float*)(ws + L.thr);
  g.cnt = (int*)(ws + L.cnt);
  g.cand_s = (float*)(ws + L.cand_s);
  g.cand_i = (int*)(ws + L.cand_i);

  MergeArgs m{};
  m.n_q = n_queries;
  m.k = k;
  m.thr = (float*)(ws + L.thr);
  m.cnt = g.cnt;
  m.cand_s = g.cand_s;
  m.cand_i = g.cand_i;
  m.run_score = (float*)(ws + L.run_s);
  m.run_idx = (int64_t*)(ws + L.run_i);
  m.out_score = out_score;
  m.out_idx = out_idx;

  hipLaunchKernelGGL(search_init_kernel, dim3((unsigned)((n_queries + 255) / 256)), dim3(256), 0,
                     stream, m.thr, m.cnt, n_queries);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // chunks: a small first one sets the thresholds, then kChunk records each
  int64_t base = 0;
  bool first = true;
  do {
    const int64_t len = std::min<int64_t>(n_db - base, first ? kFirst : kChunk);
    if (len > 0) {
      g.rec0 = base;
      g.n_rec = len;
      const dim3 grid((unsigned)((len + kRT - 1) / kRT), (unsigned)(L.rows_pad / kQT));
      if (ctx->mse) {
        switch (ctx->b) {
          case 1: hipLaunchKernelGGL((search_gemm_kernel<1, true>), grid, dim3(256), 0, stream, g); break;
          case 2: hipLaunchKernelGGL((search_gemm_kernel<2, true>), grid, dim3(256), 0, stream, g); break;
          default: hipLaunchKernelGGL((search_gemm_kernel<3, true>), grid, dim3(256), 0, stream, g); break;
        }
      } else {
        switch (ctx->b) {
          case 2: hipLaunchKernelGGL((search_gemm_kernel<2, false>), grid, dim3(256), 0, stream, g); break;
          case 3: hipLaunchKernelGGL((search_gemm_kernel<3, false>), grid, dim3(256), 0, stream, g); break;
          default: hipLaunchKernelGGL((search_gemm_kernel<4, false>), grid, dim3(256), 0, stream, g); break;
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
