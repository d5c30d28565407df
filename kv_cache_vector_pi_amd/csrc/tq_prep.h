// Query preparation for the logit kernels (turboquant.net pseudo-code,
// "integrate into attention": the query is rotated and projected once, the
// keys stay packed): Pi q and S q per query head, turned into the int8-limb
// A operands of v_mfma_i32_16x16x64_i8 in the lane order the logit, fused
// decode and step kernels consume.
#pragma once
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "tq_dev.h"
#include "tq_internal.h"

namespace tq {
namespace {

struct PrepArgs {
  const float* q;          // q[bi * q_stride_batch + head * q_stride_head + j]
  int64_t q_stride_batch, q_stride_head;
  const float* pit;        // [d][d] Pi^T
  const float* st;         // [d][d] S^T
  char* ws;
  int d, W, nc, G, n_kv, n_rb, n_q;     // nc: MFMA calls per word step
  int fold;                // W <= 2 folded layout: lane group g holds word g & 1,
                           // bits 16 (g >> 1) .. +15, so one call per subset
  int n_parts;                          // 2: code and sign parts, 1: MSE-only records
  int nq;                               // output quads per chunk (power of two <= 64)
  float wm2[kMaxVec];      // -2 * w_m of the odd Walsh subsets
  int mask[kMaxVec];       // code-plane subsets
  int nv;                  // number of subsets
  float c0;                // c[0]
};

__device__ inline float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}


// The A operands of one (slot hh, word step wsi, call c, lane group g): 16
// bytes for each of the four lanes 16 g + 4 hh + L, L the limb.  For shift
// k = kbase + sidx (sidx < 4) and byte el of the word, the weight of a bit is
// A' = round(Q / 2^k) (negated for k = 7, where the byte reads -128), Q the
// fixed-point weight round(2^e wv src[j]) of coordinate j = 32 w + 8 el + k
// (0 beyond d); limb L is the balanced base-256 digit
// ((A' + 0x80808080) >> 8L) & 255, minus 128 -- stored as that byte ^ 0x80.
// Each A' is formed once; the four values of a shift (el = 0..3) carry
// their limbs in bytes 0..3 (x_el = biased A' ^ 0x80808080), and a 4 x 4 byte
// transpose (8 v_perm_b32) gives limb L's word: byte el = byte L of x_el.
__device__ inline void limb_operands(const float* src, int e, float wv, int w, int W, int d,
                                     int kbase, uint4 (&o)[4]) {
  uint32_t word[4][4];
#pragma unroll
  for (int sidx = 0; sidx < 4; ++sidx) {
    const int k = kbase + sidx;
    uint32_t x[4];
#pragma unroll
    for (int el = 0; el < 4; ++el) {
      const int j = 32 * w + 8 * el + k;
      const int Q = (w < W && j < d) ? (int)rintf(ldexpf(wv * src[j], e)) : 0;
      const int Ap = (k < 7) ? dev::shift_round(Q, k) : -dev::shift_round(Q, 7);
      x[el] = ((uint32_t)Ap + 0x80808080u) ^ 0x80808080u;
    }
    // v_perm_b32 (s0, s1, sel): result byte i = byte sel_i of {s0 (bytes
    // 4..7), s1 (bytes 0..3)}
    const uint32_t t0 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);   // x0.0 x1.0 x0.1 x1.1
    const uint32_t t1 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);   // x0.2 x1.2 x0.3 x1.3
    const uint32_t t2 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);   // x2.0 x3.0 x2.1 x3.1
    const uint32_t t3 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);   // x2.2 x3.2 x2.3 x3.3
    word[0][sidx] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);           // x0.0 x1.0 x2.0 x3.0
    word[1][sidx] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);           // x0.1 x1.1 x2.1 x3.1
    word[2][sidx] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);           // x0.2 x1.2 x2.2 x3.2
    word[3][sidx] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);           // x0.3 x1.3 x2.3 x3.3
  }
#pragma unroll
  for (int L = 0; L < 4; ++L) o[L] = make_uint4(word[L][0], word[L][1], word[L][2], word[L][3]);
}

// Query preparation: one block per (row block of 4 q heads and part, kv
// head, batch).  Part 0 computes Pi q and the A operands of the code calls,
// part 1 (two-stage records only) S q and those of the sign calls.  Outputs
// come in chunks of 4 nq: thread (quad, jg) accumulates 4 consecutive
// outputs x 4 query slots over the jg-th of nj coordinate ranges (one float4
// row of Pi^T / S^T per coordinate, all of a thread's row loads in flight),
// and the nj partial sums are added in a fixed order (deterministic).  Then
// a power-of-two fixed-point scale per head, and the int8-limb A operands in
// the exact lane order the logit kernels consume.  Slots beyond the GQA
// group size get zero weights.
// The work of block (bx, by, bz) of that grid (the kernel body: 256 threads).
// PREFETCH: load the first batch of table rows before staging the queries
// (the standalone preparation kernels, where the table reads are cold; the
// fused decode-step kernel measured no gain and keeps its registers).
template <bool PREFETCH = false>
__device__ __forceinline__ void prep_block(const PrepArgs& a, int bx, int by, int bz) {
  extern __shared__ float sm[];
  const int Dp = 32 * a.W;
  const int nq = a.nq, nj = 256 / nq;
  float* qv = sm;                 // [d][4]: coordinate j of slot hh at 4j + hh
  float* out = qv + 4 * a.d;      // [4][Dp] this part's outputs (zero padded)
  float* red = out + 4 * Dp;      // [4 waves][16][nq] partial sums
  __shared__ int qfix_e[4];

  const int rb = bx / a.n_parts, part = bx - rb * a.n_parts;
  const int h = by, bi = bz;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* tab = part ? a.st : a.pit;
  const int quad = tid & (nq - 1), jg = tid / nq;    // nq: a power of two <= 64
  const int jl = (a.d + nj - 1) / nj;
  const int ja = min(a.d, jg * jl), jb = min(a.d, ja + jl);
  // PREFETCH: the first batch of this thread's table rows (output chunk 0) is
  // loaded before the queries are staged, so the two memory round trips
  // overlap; the accumulation order below is the same either way.
  float4 t0[PREFETCH ? 16 : 1];
  const bool pre = PREFETCH && 4 * quad < a.d && ja + 16 <= jb;
  if constexpr (PREFETCH) if (pre) {
#pragma unroll
    for (int u = 0; u < 16; ++u) t0[u] = *(const float4*)(tab + 4 * quad + (int64_t)(ja + u) * a.d);
  }

  for (int it = tid; it < 4 * a.d; it += 256) {
    const int hh = it / a.d, j = it - hh * a.d;
    const int slot = 4 * rb + hh;
    qv[4 * j + hh] = slot < a.G
        ? a.q[(int64_t)bi * a.q_stride_batch + (int64_t)(h * a.G + slot) * a.q_stride_head + j]
        : 0.f;
  }
  __syncthreads();
  {
    // one chunk of 4 nq outputs; PRE: the first chunk, which starts from the
    // prefetched rows (a separate instance, so they are dead afterwards)
    auto chunk = [&](int o0, auto pre_tag) {
      constexpr bool PRE = decltype(pre_tag)::value;
      const int r = o0 + 4 * quad;                     // multiple of 4; r < d => r + 3 < d
      float acc[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;
      if (r < a.d) {
        auto fma16 = [&](const float4 t, const float4 qq) {
          const float tv[4] = {t.x, t.y, t.z, t.w}, qs[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(tv[e], qs[i], acc[i][e]);
        };
        const float* tr = tab + r;
        int j = ja;
        if constexpr (PRE && PREFETCH) {
          if (pre) {                                   // the prefetched first batch
#pragma unroll
            for (int u = 0; u < 16; ++u) fma16(t0[u], *(const float4*)&qv[4 * (ja + u)]);
            j = ja + 16;
          }
        }
        for (; j + 16 <= jb; j += 16) {                // 16 independent row loads in flight
          float4 t[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) t[u] = *(const float4*)(tr + (int64_t)(j + u) * a.d);
#pragma unroll
          for (int u = 0; u < 16; ++u) fma16(t[u], *(const float4*)&qv[4 * (j + u)]);
        }
        for (; j < jb; ++j) fma16(*(const float4*)(tr + (int64_t)j * a.d), *(const float4*)&qv[4 * j]);
      }
      // partial sums of the 64 / nq coordinate groups of a wave (lanes nq apart)
      for (int off = nq; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] += __shfl_xor(acc[i][e], off);
      if (lane < nq)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[(wave * 16 + 4 * i + e) * nq + quad] = acc[i][e];
      __syncthreads();
      for (int it = tid; it < 16 * nq; it += 256) {
        const int k = it / nq, qd = it - k * nq;       // k = 4 slot + element
        const float v = (red[k * nq + qd] + red[(16 + k) * nq + qd]) +
                        (red[(32 + k) * nq + qd] + red[(48 + k) * nq + qd]);
        const int o = o0 + 4 * qd + (k & 3);
        if (o < Dp) out[(k >> 2) * Dp + o] = v;
      }
      __syncthreads();
    };
    int o0 = 0;
    if constexpr (PREFETCH) {
      chunk(0, std::true_type{});
      o0 = 4 * nq;
    }
    for (; o0 < Dp; o0 += 4 * nq) chunk(o0, std::false_type{});
  }
  // wave hh: max |out| and sum of out for slot hh -> scale and offsets
  char* rbase = a.ws + (((size_t)bi * a.n_kv + h) * a.n_rb + rb) * dev::rb_bytes(a.W, a.nc);
  {
    const float* r1 = out + wave * Dp;
    float m1 = 0.f, t1 = 0.f;
    for (int j = lane; j < Dp; j += 64) {
      m1 = fmaxf(m1, fabsf(r1[j]));
      t1 += r1[j];
    }
    m1 = wave_max(m1);
    t1 = wave_sum(t1);
    if (lane == 0) {
      float wmax = 2.f;                                 // sign calls: weight 2 S q
      if (part == 0) {
        wmax = 0.f;
        for (int v = 0; v < a.nv; ++v) wmax = fmaxf(wmax, fabsf(a.wm2[v]));
      }
      const float vmax = wmax * m1;
      int e = 0;
      if (vmax > 0.f) { int ex; frexpf(vmax, &ex); e = min(30 - ex, 120); }
      qfix_e[wave] = e;
      // per slot: x mse scale, y qjl scale, z mse offset, w qjl offset
      float* cdst = (float*)(rbase + (size_t)dev::n_ws(a.W) * a.nc * 64 * 16) + 4 * wave;
      if (part == 0) {
        cdst[0] = ldexpf(1.f, -e);
        cdst[2] = a.c0 * t1;
        if (a.n_parts == 1) {        // no sign calls: the QJL terms are zero
          cdst[1] = 0.f;
          cdst[3] = 0.f;
        }
      } else {
        cdst[1] = ldexpf(1.f, -e);
        cdst[3] = -t1;
      }
    }
  }
  __syncthreads();
  const int nws = dev::n_ws(a.W);
  // calls of this part: a code call per Walsh subset and half (one per subset
  // when folded), then the sign calls
  const int code_calls = a.fold ? a.nv : 2 * a.nv;
  const int c_begin = part ? code_calls : 0, n_c = part ? a.nc - code_calls : code_calls;
  // items: (slot hh, ws, call, lane group g) -> the 16 bytes of each lane
  // (16g + 4hh + L), L < 4 (limb_operands); Q is -2 w_vec Pi q, or 2 S q for
  // the sign plane
  const int items = 4 * nws * n_c * 4;
  for (int it = tid; it < items; it += 256) {
    const int g = it & 3;
    const int rest = it >> 2;
    const int cl = rest % n_c, wsi = (rest / n_c) % nws, hh = rest / (n_c * nws);
    const int c = c_begin + cl;
    // word and shift base of lane group g: unfolded, word 4 wsi + g and the
    // call's half; folded, word g & 1 and half g >> 1
    const int w = a.fold ? (g & 1) : 4 * wsi + g;
    const int kbase = a.fold ? 4 * (g >> 1) : (part ? 4 * cl : 4 * (c % 2));
    const float wv = part ? 2.f : a.wm2[a.fold ? c : c / 2];
    uint4 o[4];
    limb_operands(out + hh * Dp, qfix_e[hh], wv, w, a.W, a.d, kbase, o);
    uint4* dst = (uint4*)(rbase + (((size_t)wsi * a.nc + c) * 64 + 16 * g + 4 * hh) * 16);
#pragma unroll
    for (int L = 0; L < 4; ++L) dst[L] = o[L];
  }
}

// ---- host side -------------------------------------------------------------
// Arguments, dynamic LDS bytes and grid of the preparation of `batch` query
// sets of n_q_heads heads against n_kv_heads key heads into `workspace`.
inline void prep_args(const tq_ctx* ctx, const float* q, int32_t batch, int32_t n_q_heads,
                      int64_t q_stride_batch, int32_t n_kv_heads, void* workspace, PrepArgs& p,
                      size_t& shm, dim3& grid, bool fold = false) {
  const int G = n_q_heads / n_kv_heads;
  const int n_rb = (G + 3) / 4;
  p = PrepArgs{};
  p.q = q;
  p.q_stride_batch = q_stride_batch;
  p.q_stride_head = ctx->d;
  p.pit = ctx->t.pit32;
  p.st = ctx->t.st32;
  p.ws = (char*)workspace;
  p.d = ctx->d;
  p.W = ctx->W;
  p.fold = fold ? 1 : 0;
  p.nc = fold ? (1 << (ctx->cp - 1)) + (ctx->mse ? 0 : 1) : dev::n_calls(ctx->cp, !ctx->mse);
  p.G = G;
  p.n_kv = n_kv_heads;
  p.n_rb = n_rb;
  p.n_q = n_q_heads;
  p.nv = ctx->n_mono;
  for (int v = 0; v < ctx->n_mono; ++v) {
    p.wm2[v] = (float)(-2.0 * ctx->mono_w[v]);
    p.mask[v] = ctx->mono_mask[v];
  }
  p.c0 = (float)ctx->c0;
  p.n_parts = ctx->mse ? 1 : 2;
  int nq = 64;
  while (nq > ctx->Dp / 4) nq >>= 1;
  p.nq = nq;
  // q [d][4], outputs [4][Dp], partial sums [4][16][nq]: <= 80 KB at d = 2048
  shm = sizeof(float) * (4 * ctx->d + 4 * ctx->Dp + 64 * nq);
  grid = dim3(n_rb * p.n_parts, n_kv_heads, batch);
}

}  // namespace
}  // namespace tq
