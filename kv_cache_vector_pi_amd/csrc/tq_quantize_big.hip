// Quantization at large head dimensions (Dp >= 512) with a caller workspace
// (turboquant.net pseudo-code "quant", plus the QJL stage of the admirer.cn
// two-stage description): the same results as tq_quantize_kv, organised as
// two blocked matrix products.
//
// At large d the one-kernel quantizer keeps a 16-vector tile of x and of the
// residual in LDS (a 16 x 1536 fp32 tile as fp16 hi/lo is 98 KB), so every 16
// vectors re-read all of Pi and M (19 MB at d = 1536) from L2 / MALL.  Here:
//
//  1. norm kernel: nu = ||x||, the power-of-two scale 2^-e of each row.
//  2. Y kernel: a workgroup owns 256 vectors x 4 words (128 coordinates, one
//     word per wave) and loops over K in blocks of 32 coordinates: the x block
//     (scaled, fp16 hi/lo) is staged in LDS and shared by the 4 waves, each
//     wave streams its 32 rows of Pi.  Pi is read once per 256 vectors instead
//     of once per 16.  Epilogue: codes (written into the records), the
//     residual r = y - c[idx] as fp16 hi/lo into the workspace, and the
//     per-word partial sums of r^2.
//  3. Z kernel (two-stage records): the same blocking for z = M r, reading
//     the residual back from the workspace; epilogue: sign bits (written into
//     the records) and the norms (nu, gamma).
// Codes compare y = acc * 2^e / nu against the midpoints like the other
// quantizers (ties to the lower index); coordinates >= d carry zero bits and
// zero residual; a zero vector stores nu = gamma = 0, the codes of y = 0 and
// all signs +1.
#include <algorithm>
#include <cmath>

#include "tq_q128.h"   // halves_or / halves_sum

namespace tq {
namespace {

constexpr int kBM = 256;     // vectors per tile: 8 column blocks of 32
constexpr int kCB = kBM / 32;
constexpr int kLdk = 40;     // LDS row stride of a 32-coordinate block, in halves

struct BigArgs {
  const void* x;
  int64_t x_stride_token, x_stride_head, n_tokens;
  int64_t f0;                // first row (head-major flattened) of this chunk
  int n_rows;                // rows of this chunk
  uint32_t* planes;
  uint32_t* norms;
  int64_t dst_stride_head, dst_token0;
  const __half* ta_hi;       // Pi (Y kernel) or M (Z kernel), fp16 hi / lo, [Dp][Dp]
  const __half* ta_lo;
  int d, W, Dp;
  float cent[kMaxK];
  float mid[kMaxK];
  // workspace (chunk-local rows)
  float4* sc;                // {2^-e, 2^e / nu (0: x = 0), unused, fp16 bits of nu}
  _Float16* r_hi;            // [n_rows][Dp]
  _Float16* r_lo;
  float* g2;                 // [n_rows][W] partial sums of r^2 (unit space)
  int nvb, nwb;              // vector blocks (kBM rows) and word blocks (4 words)
};

// The Y and Z grids are 1-D: workgroup L runs on XCD L mod 8 (round-robin
// dispatch), and XCD x takes the vector blocks vb = 8 tx + x in order, each
// with all of its word blocks in turn.  The workgroups that share a block of
// x then run together on one XCD and read it from that XCD's L2; the table
// comes from the MALL.  In x-fastest 2-D order every x tile was fetched from
// memory once per word block (12 times at d = 1536), which cost 25% more
// time.  False for the padding workgroups (vb >= nvb), which exit at once.
__device__ inline bool big_tile(const BigArgs& a, int& vb, int& wb) {
  const int L = (int)blockIdx.x, s = L >> 3;
  const int tx = s / a.nwb;
  wb = s - tx * a.nwb;
  vb = 8 * tx + (L & 7);
  return vb < a.nvb;
}

__device__ inline void row_of(const BigArgs& a, int64_t f, int64_t& xoff, int64_t& rec) {
  const int64_t h = f / a.n_tokens, t = f - h * a.n_tokens;
  xoff = h * a.x_stride_head + t * a.x_stride_token;
  rec = h * a.dst_stride_head + a.dst_token0 + t;
}

// 8 consecutive elements of x at element offset off (bf16 or fp32)
template <bool BF16>
__device__ inline void load8(const void* x, int64_t off, float (&v)[8]) {
  if constexpr (BF16) {
    const uint4 raw = *(const uint4*)((const uint16_t*)x + off);
    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(wv[e] << 16);
      v[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
    }
  } else {
    const float4 f0 = *(const float4*)((const float*)x + off);
    const float4 f1 = *(const float4*)((const float*)x + off + 4);
    v[0] = f0.x; v[1] = f0.y; v[2] = f0.z; v[3] = f0.w;
    v[4] = f1.x; v[5] = f1.y; v[6] = f1.z; v[7] = f1.w;
  }
}

// ---- 1. norms and scales: one wave per row --------------------------------
template <bool BF16, bool MSE>
__global__ void __launch_bounds__(256) bigq_norm_kernel(BigArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * 4 + wave;
  if (r >= a.n_rows) return;
  int64_t xoff, rec;
  row_of(a, a.f0 + r, xoff, rec);
  float ss = 0.f;
  for (int j = 8 * lane; j < a.d; j += 512) {     // d is a multiple of 8
    float v[8];
    load8<BF16>(a.x, xoff + j, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) {
    const float nu = sqrtf(ss);
    int ex = 0;
    if (nu > 0.f) frexpf(nu, &ex);
    const uint32_t nb = (uint32_t)__half_as_ushort(__float2half_rn(nu));
    a.sc[r] = make_float4(ldexpf(1.f, -ex), nu > 0.f ? ldexpf(1.f / nu, ex) : 0.f, 0.f,
                          __uint_as_float(nb));
    if (MSE) a.norms[rec] = nb;                    // gamma slot 0
  }
}

// ---- 2. / 3. blocked product over K, shared by the Y and Z kernels ----------
// acc[cb] (32 x 32 block cb of the tile): rows 32 w .. 32 w + 31 of the table
// (this wave's word), columns = vectors 32 cb .. 32 cb + 31 of the tile.
// Lane (col, hh) holds rows 8 (i / 4) + 4 hh + i % 4 of column col.
// ZSRC: B operand from the workspace residual (fp16 hi/lo) instead of x.
// One LDS buffer per block of 32 coordinates: two barriers per block, the
// next block's x (or r) and table fragments load into registers meanwhile.
template <bool BF16, bool ZSRC>
__device__ __forceinline__ void big_product(const BigArgs& a, int vb0, int w, bool wok,
                                            const float4* scs, _Float16* bh, _Float16* bl,
                                            v16f (&acc)[kCB]) {
  constexpr bool LO = ZSRC || !BF16;       // B has a lo part: 3 passes
  constexpr int NP = kBM / 128;            // staged vectors per thread
  const int tid = threadIdx.x, lane = tid & 63;
  const int col = lane & 31, hh = lane >> 5;
  // staging role: vectors tid / 2 + 128 p of the tile, coordinates
  // 16 sh .. 16 sh + 15 of a block
  const int sh = tid & 1;
  bool svok[NP];
  int64_t sxoff[NP], rbase[NP];
  float ssc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sv = (tid >> 1) + 128 * p;
    svok[p] = vb0 + sv < a.n_rows;
    sxoff[p] = 0;
    int64_t srec;
    if (!ZSRC && svok[p]) row_of(a, a.f0 + vb0 + sv, sxoff[p], srec);
    ssc[p] = scs[sv].x;
    rbase[p] = (int64_t)(vb0 + sv) * a.Dp;
  }
  // x (or r) of one block in registers: 16 elements per staged vector
  float xr[NP][16];
  v8h rh2[NP][2], rl2[NP][2];
  auto fetch = [&](int kb) {
    const int k0 = 32 * kb + 16 * sh;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if constexpr (ZSRC) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          rh2[p][c] = svok[p] ? *(const v8h*)(a.r_hi + rbase[p] + k0 + 8 * c) : (v8h){};
          rl2[p][c] = svok[p] ? *(const v8h*)(a.r_lo + rbase[p] + k0 + 8 * c) : (v8h){};
        }
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (svok[p] && k0 + 8 * c < a.d) load8<BF16>(a.x, sxoff[p] + k0 + 8 * c, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) xr[p][8 * c + e] = v[e];
        }
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int sv = (tid >> 1) + 128 * p;
      _Float16* dh = bh + sv * kLdk + 16 * sh;
      _Float16* dl = bl + sv * kLdk + 16 * sh;
      if constexpr (ZSRC) {
        *(v8h*)dh = rh2[p][0];
        *(v8h*)(dh + 8) = rh2[p][1];
        *(v8h*)dl = rl2[p][0];
        *(v8h*)(dl + 8) = rl2[p][1];
      } else {
        v8h hi[2], lo[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float xs = xr[p][e] * ssc[p];
          const _Float16 hv = (_Float16)xs;
          hi[e >> 3][e & 7] = hv;
          lo[e >> 3][e & 7] = (_Float16)(xs - (float)hv);
        }
        *(v8h*)dh = hi[0];
        *(v8h*)(dh + 8) = hi[1];
        if constexpr (LO) {
          *(v8h*)dl = lo[0];
          *(v8h*)(dl + 8) = lo[1];
        }
      }
    }
  };
  // table fragments of a block: row 32 w + col, K 32 kb + 16 ks + 8 hh
  v8h th[2], tl[2];
  auto load_t = [&](int kb) {
    if (!wok) return;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int64_t off = (int64_t)(32 * w + col) * a.Dp + 32 * kb + 16 * ks + 8 * hh;
      th[ks] = *(const v8h*)(a.ta_hi + off);
      tl[ks] = *(const v8h*)(a.ta_lo + off);
    }
  };
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) acc[cb] = (v16f){};
  const int nkb = a.W;                       // Dp = 32 W: blocks of 32 coordinates
  fetch(0);
  load_t(0);
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb > 0) __syncthreads();      // every wave has read block kb - 1
    stage();
    __syncthreads();                  // block kb staged
    const v8h ch[2] = {th[0], th[1]}, cl[2] = {tl[0], tl[1]};
    if (kb + 1 < nkb) {
      fetch(kb + 1);      // next block in flight during the MFMAs
      load_t(kb + 1);
    }
    if (wok) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          const int off = (32 * cb + col) * kLdk + 16 * ks + 8 * hh;
          const v8h xh = *(const v8h*)(bh + off);
          v16f c = acc[cb];
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(ch[ks], xh, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(cl[ks], xh, c, 0, 0, 0);
          if constexpr (LO) {
            const v8h xl = *(const v8h*)(bl + off);
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(ch[ks], xl, c, 0, 0, 0);
          }
          acc[cb] = c;
        }
    }
  }
}

// ---- 2. Y = Pi x, codes, residual ------------------------------------------
template <int NB, bool BF16, bool MSE>
__global__ void __launch_bounds__(256, 2) bigq_y_kernel(BigArgs a) {
  constexpr int CP = MSE ? NB : NB - 1;
  constexpr int K = 1 << CP;
  __shared__ __align__(16) _Float16 bh[kBM * kLdk];
  __shared__ __align__(16) _Float16 bl[kBM * kLdk];
  __shared__ float4 scs[kBM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  int vb, wb;
  if (!big_tile(a, vb, wb)) return;               // uniform over the workgroup
  const int vb0 = vb * kBM;
  const int w = wb * 4 + wave;
  const bool wok = w < a.W;
  for (int t = tid; t < kBM; t += 256)
    scs[t] = vb0 + t < a.n_rows ? a.sc[vb0 + t] : make_float4(1.f, 0.f, 0.f, 0.f);
  __syncthreads();
  v16f acc[kCB];
  big_product<BF16, false>(a, vb0, w, wok, scs, bh, bl, acc);
  if (!wok) return;
  const int jb = 32 * w;                           // first coordinate of the word
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int v = vb0 + 32 * cb + col;             // chunk-local row
    const bool vok = v < a.n_rows;
    const float s = scs[32 * cb + col].y;          // 2^e / nu (0: x = 0)
    uint32_t cw[3] = {0u, 0u, 0u};
    float g2 = 0.f;
    float rr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int pos = 8 * (i >> 2) + 4 * hh + (i & 3);
      const int j = jb + pos;
      const float y = acc[cb][i] * s;
      int idx = 0;
      float c = a.cent[0];
#pragma unroll
      for (int k = 0; k < K - 1; ++k) {
        const bool gt = y > a.mid[k];
        idx += gt ? 1 : 0;
        c = gt ? a.cent[k + 1] : c;
      }
      const bool live = j < a.d && s > 0.f;
      const float r = live ? y - c : 0.f;
      rr[i] = r;
      g2 = fmaf(r, r, g2);
      if (j < a.d) {
#pragma unroll
        for (int p = 0; p < CP; ++p) cw[p] |= (uint32_t)((idx >> p) & 1) << pos;
      }
    }
    uint32_t word[3];
#pragma unroll
    for (int p = 0; p < CP; ++p) word[p] = halves_or(cw[p]);
    const float g2s = halves_sum(g2);
    if (!vok) continue;
    int64_t xoff, rec;
    row_of(a, a.f0 + v, xoff, rec);
    if (hh == 0) {
      uint32_t* dst = a.planes + (rec * a.W + w) * NB;
#pragma unroll
      for (int p = 0; p < CP; ++p) dst[p] = word[p];
      if (!MSE) a.g2[(int64_t)v * a.W + w] = g2s;
    }
    if constexpr (!MSE) {
      typedef _Float16 v4h __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < 4; ++q) {              // rows 8 q + 4 hh .. + 3
        v4h h4, l4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float r = rr[4 * q + e];
          const _Float16 hv = (_Float16)r;
          h4[e] = hv;
          l4[e] = (_Float16)(r - (float)hv);
        }
        const int64_t off = (int64_t)v * a.Dp + jb + 8 * q + 4 * hh;
        *(v4h*)(a.r_hi + off) = h4;
        *(v4h*)(a.r_lo + off) = l4;
      }
    }
  }
}

// ---- 3. Z = M r, signs, norms ---------------------------------------------
template <int NB>
__global__ void __launch_bounds__(256, 2) bigq_z_kernel(BigArgs a) {
  __shared__ __align__(16) _Float16 bh[kBM * kLdk];
  __shared__ __align__(16) _Float16 bl[kBM * kLdk];
  __shared__ float4 scs[kBM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  int vb, wb;
  if (!big_tile(a, vb, wb)) return;               // uniform over the workgroup
  const int vb0 = vb * kBM;
  const int w = wb * 4 + wave;
  const bool wok = w < a.W;
  for (int t = tid; t < kBM; t += 256)
    scs[t] = vb0 + t < a.n_rows ? a.sc[vb0 + t] : make_float4(1.f, 0.f, 0.f, 0.f);
  __syncthreads();
  // norms of the tile's vectors: gamma = ||r|| from the per-word partial sums
  for (int t = tid; wb == 0 && t < kBM && vb0 + t < a.n_rows; t += 256) {
    const int v = vb0 + t;
    float s2 = 0.f;
    for (int ww = 0; ww < a.W; ++ww) s2 += a.g2[(int64_t)v * a.W + ww];
    const float4 sc = scs[t];
    const float gam = sc.y == 0.f ? 0.f : sqrtf(s2);
    int64_t xoff, rec;
    row_of(a, a.f0 + v, xoff, rec);
    a.norms[rec] = __float_as_uint(sc.w) | ((uint32_t)__half_as_ushort(__float2half_rn(gam)) << 16);
  }
  v16f acc[kCB];
  big_product<false, true>(a, vb0, w, wok, scs, bh, bl, acc);
  if (!wok) return;
  const int jb = 32 * w;
  const uint32_t dmask = a.d - jb >= 32 ? 0xffffffffu : ((1u << (a.d - jb)) - 1u);
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int v = vb0 + 32 * cb + col;
    uint32_t sb = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int pos = 8 * (i >> 2) + 4 * hh + (i & 3);
      sb |= (uint32_t)(acc[cb][i] >= 0.f) << pos;
    }
    uint32_t sw = halves_or(sb) & dmask;
    if (scs[32 * cb + col].y == 0.f) sw = dmask;     // x = 0: r = 0, all signs +1
    if (v >= a.n_rows || hh != 0) continue;
    int64_t xoff, rec;
    row_of(a, a.f0 + v, xoff, rec);
    a.planes[(rec * a.W + w) * NB + NB - 1] = sw;
  }
}

struct BigLayout {
  size_t sc, r_hi, r_lo, g2, per_row;
};
inline size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }
// workspace offsets for a chunk of `rows` rows
BigLayout big_layout(const tq_ctx* ctx, int64_t rows) {
  BigLayout L{};
  L.sc = 0;
  L.r_hi = al256(L.sc + (size_t)rows * 16);
  L.r_lo = al256(L.r_hi + (size_t)rows * ctx->Dp * 2);
  L.g2 = al256(L.r_lo + (size_t)rows * ctx->Dp * 2);
  L.per_row = 16 + (size_t)ctx->Dp * 4 + (size_t)ctx->W * 4;
  return L;
}
size_t big_bytes(const tq_ctx* ctx, int64_t rows) {
  const BigLayout L = big_layout(ctx, rows);
  return al256(L.g2 + (size_t)rows * ctx->W * 4);
}

template <int NB, bool BF16, bool MSE>
hipError_t launch_big_chunk(BigArgs a, const tq_ctx* ctx, hipStream_t st) {
  a.nvb = (a.n_rows + kBM - 1) / kBM;
  a.nwb = (a.W + 3) / 4;
  const dim3 grid((unsigned)(8 * ((a.nvb + 7) / 8) * a.nwb));
  hipLaunchKernelGGL((bigq_norm_kernel<BF16, MSE>), dim3((unsigned)((a.n_rows + 3) / 4)),
                     dim3(256), 0, st, a);
  a.ta_hi = ctx->t.pi_hi;
  a.ta_lo = ctx->t.pi_lo;
  hipLaunchKernelGGL((bigq_y_kernel<NB, BF16, MSE>), grid, dim3(256), 0, st, a);
  if constexpr (!MSE) {
    a.ta_hi = ctx->t.m_hi;
    a.ta_lo = ctx->t.m_lo;
    hipLaunchKernelGGL((bigq_z_kernel<NB>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

bool quantize_big_applies(const tq_ctx* ctx) { return ctx->Dp >= 512; }

size_t quantize_big_workspace_bytes(const tq_ctx* ctx, int64_t n_rows) {
  if (!quantize_big_applies(ctx) || n_rows <= 0) return 0;
  const int64_t rows = std::min<int64_t>(((n_rows + kBM - 1) / kBM) * kBM, 65536);
  return big_bytes(ctx, rows);
}

hipError_t launch_quantize_big(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                               int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                               int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                               int64_t dst_stride_head, int64_t dst_token0, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  // rows per chunk: the most whole kBM-row tiles whose workspace fits
  const BigLayout L1 = big_layout(ctx, 1);
  int64_t chunk = std::min<int64_t>((int64_t)(workspace_bytes / L1.per_row) / kBM * kBM, 65536);
  while (chunk >= kBM && big_bytes(ctx, chunk) > workspace_bytes) chunk -= kBM;
  if (chunk < kBM) return hipErrorInvalidValue;
  const bool bf = x_dtype == TQ_BF16;
  const int64_t n_rows = (int64_t)n_heads * n_tokens;
  for (int64_t f0 = 0; f0 < n_rows; f0 += chunk) {
    const int64_t rows = std::min(chunk, n_rows - f0);
    const BigLayout L = big_layout(ctx, rows);
    char* ws = (char*)workspace;
    BigArgs a{};
    a.x = x;
    a.x_stride_token = x_stride_token;
    a.x_stride_head = x_stride_head;
    a.n_tokens = n_tokens;
    a.f0 = f0;
    a.n_rows = (int)rows;
    a.planes = planes;
    a.norms = (uint32_t*)norms;
    a.dst_stride_head = dst_stride_head;
    a.dst_token0 = dst_token0;
    a.d = ctx->d;
    a.W = ctx->W;
    a.Dp = ctx->Dp;
    for (int k = 0; k < kMaxK; ++k) {
      a.cent[k] = ctx->cent[k];
      a.mid[k] = ctx->mid[k];
    }
    a.sc = (float4*)(ws + L.sc);
    a.r_hi = (_Float16*)(ws + L.r_hi);
    a.r_lo = (_Float16*)(ws + L.r_lo);
    a.g2 = (float*)(ws + L.g2);
    hipError_t e;
    if (ctx->mse) {
      switch (ctx->b) {
        case 1: e = bf ? launch_big_chunk<1, true, true>(a, ctx, stream) : launch_big_chunk<1, false, true>(a, ctx, stream); break;
        case 2: e = bf ? launch_big_chunk<2, true, true>(a, ctx, stream) : launch_big_chunk<2, false, true>(a, ctx, stream); break;
        default: e = bf ? launch_big_chunk<3, true, true>(a, ctx, stream) : launch_big_chunk<3, false, true>(a, ctx, stream); break;
      }
    } else {
      switch (ctx->b) {
        case 2: e = bf ? launch_big_chunk<2, true, false>(a, ctx, stream) : launch_big_chunk<2, false, false>(a, ctx, stream); break;
        case 3: e = bf ? launch_big_chunk<3, true, false>(a, ctx, stream) : launch_big_chunk<3, false, false>(a, ctx, stream); break;
        default: e = bf ? launch_big_chunk<4, true, false>(a, ctx, stream) : launch_big_chunk<4, false, false>(a, ctx, stream); break;
      }
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
