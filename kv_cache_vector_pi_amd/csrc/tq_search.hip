// Vector search over a quantized database and dequantization
// (zingnex.cn digest, nearest-neighbour section; admirer.cn vector-search
// paragraph; turboquant.net pseudo-code "dequant").
//
// Both are one "decoded GEMM":
//   score[q][n] = nu_n * ( sum_j QR[q][j] c[idx_nj] + alpha * gamma_n * sum_j QP[q][j] s_nj )
// For search QR = Pi q and QP = S q (one row per query).  For dequantization
// the rows are the unit vectors e_j, i.e. QR = Pi^T and QP = S^T, so the
// "score" of row j is coordinate j of nu (Pi^T c[idx] + alpha gamma S^T s).
//
// Records are decoded once per 64-row tile into fp16 operands in LDS
// (centroid hi and lo parts, signs +-1), the rows are split hi + lo fp16, and
// the contraction runs on v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//   mse += QR_hi c_hi + QR_lo c_hi + QR_hi c_lo,   qjl += QP_hi s + QP_lo s.
// Search then keeps the top-k of each query with a one-wave-per-query merge
// over chunks of scores (ordered by score descending, index ascending).
#include <algorithm>
#include <cmath>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kRowsTile = 64;    // query rows per workgroup
constexpr int kRecTile = 64;     // records per workgroup
constexpr int kChunk = 32768;    // records scored per search pass
constexpr int kLdsRow = 40;      // halves per decoded record row (32 + pad)

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
      const float v = live ? acc[i] : 0.f;
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
  // output: mode 0 -> scores[row * out_ld + (rec - rec0)], mode 1 -> out[rec * out_ld + row]
  float* out;
  int64_t out_ld;
};

template <int NB, int MODE>
__global__ void __launch_bounds__(256) decoded_gemm_kernel(GemmArgs a) {
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
  for (int ks = 0; ks < a.W; ++ks) {
    // decode word ks of record dr, coordinates 8dq .. 8dq+7
    {
      uint32_t wd[NB];
#pragma unroll
      for (int p = 0; p < NB; ++p) wd[p] = 0u;
      if (dlive) {
        const uint32_t* src = a.planes + ((a.rec0 + drec) * a.W + ks) * NB;
#pragma unroll
        for (int p = 0; p < NB; ++p) wd[p] = src[p];
      }
      v8h vh, vl, vs;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int bit = 8 * dq + e;
        int idx = 0;
#pragma unroll
        for (int p = 0; p < NB - 1; ++p) idx |= (int)((wd[p] >> bit) & 1u) << p;
        vh[e] = a.c_hi[idx];
        vl[e] = a.c_lo[idx];
        vs[e] = ((wd[NB - 1] >> bit) & 1u) ? (_Float16)1.0f : (_Float16)-1.0f;
      }
      *(v8h*)(dh + dr * kLdsRow + 8 * dq) = vh;
      *(v8h*)(dl + dr * kLdsRow + 8 * dq) = vl;
      *(v8h*)(ds + dr * kLdsRow + 8 * dq) = vs;
    }
    __syncthreads();
    const int64_t aoff = row * a.Dp + 32 * ks + 8 * g;
    const v8h rh = *(const v8h*)(a.qr_hi + aoff);
    const v8h rl = *(const v8h*)(a.qr_lo + aoff);
    const v8h ph = *(const v8h*)(a.qp_hi + aoff);
    const v8h pl = *(const v8h*)(a.qp_lo + aoff);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int off = (16 * cb + n) * kLdsRow + 8 * g;
      const v8h bh = *(const v8h*)(dh + off);
      const v8h bl = *(const v8h*)(dl + off);
      const v8h bs = *(const v8h*)(ds + off);
      am[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rh, bh, am[cb], 0, 0, 0);
      am[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rl, bh, am[cb], 0, 0, 0);
      am[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rh, bl, am[cb], 0, 0, 0);
      aq[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bs, aq[cb], 0, 0, 0);
      aq[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bs, aq[cb], 0, 0, 0);
    }
    __syncthreads();
  }
  // epilogue: lane holds rows 4g+i of the wave's 16-row block, record 16cb+n
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int64_t rec = rt * kRecTile + 16 * cb + n;
    if (rec >= a.n_rec) continue;
    const uint32_t nr = a.norms[a.rec0 + rec];
    const float nu = __half2float(__ushort_as_half((unsigned short)(nr & 0xffffu)));
    const float ga = __half2float(__ushort_as_half((unsigned short)(nr >> 16)));
    const float ag = a.alpha * ga;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = qt * kRowsTile + 16 * wave + 4 * g + i;
      if (r >= a.n_rows) continue;
      const float v = nu * fmaf(ag, aq[cb][i], am[cb][i]);
      if constexpr (MODE == 0) a.out[r * a.out_ld + rec] = v;
      else a.out[(a.rec0 + rec) * a.out_ld + r] = v;
    }
  }
}

// ---- top-k merge: one wave per query ----------------------------------------
struct TopkArgs {
  const float* scores;   // [n_q][kChunk] for this chunk
  int64_t n_q, chunk_len, base;  // records base .. base + chunk_len - 1
  int k;
  float* run_score;      // [n_q][k]
  int64_t* run_idx;
  int first, last;
  float* out_score;
  int64_t* out_idx;
};

__device__ inline bool beats(float as, int64_t ai, float bs, int64_t bi) {
  return as > bs || (as == bs && ai < bi);
}

__global__ void __launch_bounds__(256) topk_merge_kernel(TopkArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t q = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= a.n_q) return;
  float sv = -INFINITY;
  int64_t iv = -1;
  if (!a.first && lane < a.k) {
    sv = a.run_score[q * a.k + lane];
    iv = a.run_idx[q * a.k + lane];
  }
  const int k = a.k;
  float ts = __shfl(sv, k - 1);
  int64_t ti = __shfl(iv, k - 1);
  const float* row = a.scores + q * (int64_t)kChunk;
  for (int64_t b0 = 0; b0 < a.chunk_len; b0 += 64) {
    const bool in = b0 + lane < a.chunk_len;
    const float v = in ? row[b0 + lane] : -INFINITY;
    const int64_t id = a.base + b0 + lane;
    uint64_t mask = __ballot(in && beats(v, id, ts, ti));
    while (mask) {
      const int src = __ffsll((unsigned long long)mask) - 1;
      const float cv = __shfl(v, src);
      const int64_t ci = __shfl(id, src);
      // entries that beat the candidate form a prefix of the sorted list
      const uint64_t bm = __ballot(lane < k && beats(sv, iv, cv, ci));
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
          iv = ci;
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
hipError_t launch_gemm(int b, const GemmArgs& g, dim3 grid, hipStream_t st) {
  switch (b) {
    case 2: hipLaunchKernelGGL((decoded_gemm_kernel<2, MODE>), grid, dim3(256), 0, st, g); break;
    case 3: hipLaunchKernelGGL((decoded_gemm_kernel<3, MODE>), grid, dim3(256), 0, st, g); break;
    default: hipLaunchKernelGGL((decoded_gemm_kernel<4, MODE>), grid, dim3(256), 0, st, g); break;
  }
  return hipGetLastError();
}

struct SearchLayout {
  size_t qr_hi, qr_lo, qp_hi, qp_lo, scores, run_s, run_i, total;
  int64_t rows_pad;
};

SearchLayout search_layout(const tq_ctx* ctx, int64_t n_queries, int32_t k) {
  SearchLayout L{};
  L.rows_pad = (n_queries + kRowsTile - 1) / kRowsTile * kRowsTile;
  const size_t mat = align256((size_t)L.rows_pad * ctx->Dp * sizeof(__half));
  size_t off = 0;
  L.qr_hi = off; off += mat;
  L.qr_lo = off; off += mat;
  L.qp_hi = off; off += mat;
  L.qp_lo = off; off += mat;
  L.scores = off; off += align256((size_t)L.rows_pad * kChunk * sizeof(float));
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
  RowPrepArgs p{};
  p.q = queries;
  p.pit = ctx->t.pit32;
  p.st = ctx->t.st32;
  p.qr_hi = (__half*)(ws + L.qr_hi);
  p.qr_lo = (__half*)(ws + L.qr_lo);
  p.qp_hi = (__half*)(ws + L.qp_hi);
  p.qp_lo = (__half*)(ws + L.qp_lo);
  p.d = ctx->d;
  p.Dp = ctx->Dp;
  p.n = n_queries;
  p.n_pad = L.rows_pad;
  hipLaunchKernelGGL(row_prep_kernel,
                     dim3((unsigned)((L.rows_pad + kPrepRows - 1) / kPrepRows),
                          (unsigned)((2 * ctx->Dp + 255) / 256)),
                     dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  GemmArgs g{};
  g.qr_hi = p.qr_hi;
  g.qr_lo = p.qr_lo;
  g.qp_hi = p.qp_hi;
  g.qp_lo = p.qp_lo;
  g.n_rows = n_queries;
  g.planes = planes;
  g.norms = (const uint32_t*)norms;
  g.W = ctx->W;
  g.Dp = ctx->Dp;
  g.alpha = (float)(std::sqrt(M_PI / 2.0) / ctx->d);
  fill_centroid_split(ctx, g);
  g.out = (float*)(ws + L.scores);
  g.out_ld = kChunk;

  TopkArgs t{};
  t.scores = g.out;
  t.n_q = n_queries;
  t.k = k;
  t.run_score = (float*)(ws + L.run_s);
  t.run_idx = (int64_t*)(ws + L.run_i);
  t.out_score = out_score;
  t.out_idx = out_idx;
  const int64_t n_chunks = std::max<int64_t>(1, (n_db + kChunk - 1) / kChunk);
  for (int64_t c = 0; c < n_chunks; ++c) {
    const int64_t base = c * kChunk;
    const int64_t len = std::max<int64_t>(0, std::min<int64_t>(kChunk, n_db - base));
    if (len > 0) {
      g.rec0 = base;
      g.n_rec = len;
      const dim3 grid((unsigned)((len + kRecTile - 1) / kRecTile),
                      (unsigned)(L.rows_pad / kRowsTile));
      e = launch_gemm<0>(ctx->b, g, grid, stream);
      if (e != hipSuccess) return e;
    }
    t.chunk_len = len;
    t.base = base;
    t.first = c == 0;
    t.last = c == n_chunks - 1;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)((n_queries + 3) / 4)), dim3(256), 0,
                       stream, t);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

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
  const dim3 grid((unsigned)((n + kRecTile - 1) / kRecTile),
                  (unsigned)((ctx->Dp + kRowsTile - 1) / kRowsTile));
  return launch_gemm<1>(ctx->b, g, grid, stream);
}

}  // namespace tq
