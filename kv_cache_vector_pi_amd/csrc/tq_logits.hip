// Attention logits straight from packed keys (turboquant.net pseudo-code,
// "integrate into attention": keys are stored quantized and inner products
// are estimated with QJL; admirer.cn article: logits computed from 4-bit keys).
//
//   logit = scale * nu * ( <Pi q, c[idx]> + alpha * gamma * <S q, s> )
//
// Design (gfx950): the estimate is rewritten as integer dot products of 0/1
// bit vectors with fixed-point query weights, and those run on the int8
// matrix cores (v_mfma_i32_16x16x64_i8), so a key record is decoded with one
// VALU AND per four coordinates.
//
//  * Codebook: with a symmetric Lloyd-Max codebook, c[idx] expands over the
//    code bits as c[idx] = c_0 - 2 sum_m w_m u_m, where u_m is the XOR of the
//    code planes in an odd-sized subset m (Walsh expansion; 1, 2, 4 subsets for
//    b = 2, 3, 4).  So <Pi q, c[idx]> = c_0 sum(Pi q) - 2 sum_m w_m <Pi q, u_m>.
//  * Signs: <S q, s> = 2 <S q, beta_s> - sum(S q), beta_s the sign plane.
//    MSE-only records (no QJL stage) have b code planes and no sign plane:
//    the estimate is the first term alone and the sign MFMAs are left out.
//  * Bits -> int8 lanes: a 32-bit plane word ANDed with 0x01010101 << k gives
//    four int8 lanes holding bit (8e+k) of the word times 2^k (times -128 for
//    k = 7).  The 2^k is folded into the query weights: the weight for a bit
//    at shift k is round(Q / 2^k), written as four balanced int8 limbs, so no
//    shift is ever applied to the key bits.
//  * MFMA: A = 16 rows = 4 query heads x 4 limbs of the fixed-point weights
//    (prepared once per query), B = 16 key tokens x 64 K-slots of masked bits,
//    C = int32 partial dot products; a lane then holds the 4 limbs of one
//    (head, token) pair and finishes the logit on its own.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "tq_dev.h"
#include "tq_internal.h"
#include "tq_prep.h"

namespace tq {
namespace {

using dev::v4i;
using dev::kTile;
using dev::kWaves;
using dev::n_calls;
using dev::n_ws;
using dev::rb_bytes;
using dev::load_group;
using dev::bit_lanes;
using dev::walsh_mask;

__global__ void __launch_bounds__(256) attn_prep_kernel(PrepArgs a) {
  prep_block<true>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

struct AttnArgs {
  const char* ws;
  const uint32_t* planes;
  const uint32_t* norms;      // (nu, gamma) fp16 pairs as one word per record
  const int64_t* seq_start;
  const int32_t* seq_len;
  float* logits;
  int64_t keys_stride_head, logits_stride_head;
  int W, G, n_kv, n_rb, tiles_per_wave;
  float scale, alpha;
  int mask[kMaxVec];
  struct {                    // second record set of channel-split records
    const char* ws;
    const uint32_t* planes;
    const uint32_t* norms;
    int W;
    float alpha;
  } set2;
};

// Logit stream.  grid = (token chunks, kv heads, batch); each wave owns
// tiles_per_wave tiles of 16 tokens of one (batch, kv head) sequence.
// Lane (g = lane/16, n = lane%16): loads word group g of token n's record
// (per word step), and after the MFMAs holds the 4 limbs of q head 4rb+g
// for token n.  RES: all A operands fit one word step and one row block,
// so they stay in registers for the whole chunk.
template <int NB, bool MSE, bool RES>
__global__ void __launch_bounds__(256) attn_logits_kernel(AttnArgs a) {
  constexpr int CP = MSE ? NB : NB - 1;    // code planes
  constexpr int NV = 1 << (CP - 1);        // Walsh subsets
  constexpr int NC = 2 * NV + (MSE ? 0 : 2);   // MFMA calls per word step
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int len = a.seq_len[bi];
  const int64_t start = a.seq_start[bi];
  const int chunk = a.tiles_per_wave * kTile;
  const int t_begin = (blockIdx.x * kWaves + wave) * chunk;
  if (t_begin >= len) return;
  const int t_end = min(len, t_begin + chunk);
  const int nws = (a.W + 3) >> 2;
  const size_t rbb = (size_t)nws * NC * 64 * 16 + 64;
  const char* wsb = a.ws + ((size_t)bi * a.n_kv + h) * a.n_rb * rbb;
  const int64_t rec0 = (int64_t)h * a.keys_stride_head + start;

  v4i A[RES ? NC : 1];
  float4 cst = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (RES) {
    const v4i* fr = (const v4i*)wsb;
#pragma unroll
    for (int c = 0; c < NC; ++c) A[c] = fr[c * 64 + lane];
    cst = ((const float4*)(wsb + (size_t)NC * 64 * 16))[g];
  }

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    const int tok = t0 + n;
    const bool valid = tok < t_end;
    const int64_t rec = rec0 + tok;
    const uint32_t nrm = valid ? a.norms[rec] : 0u;
    for (int rb = 0; rb < a.n_rb; ++rb) {
      const char* rbase = wsb + rb * rbb;
      v4i acc_m = {0, 0, 0, 0}, acc_q = {0, 0, 0, 0};
      for (int wsi = 0; wsi < nws; ++wsi) {
        const int w = 4 * wsi + g;
        uint32_t wd[NB];
#pragma unroll
        for (int p = 0; p < NB; ++p) wd[p] = 0u;
        if (valid && w < a.W) load_group<NB>(a.planes + (rec * a.W + w) * NB, wd);
        const v4i* fr = (const v4i*)(rbase + (size_t)wsi * NC * 64 * 16);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          uint32_t u = 0u;
#pragma unroll
          for (int p = 0; p < CP; ++p)
            if ((a.mask[v] >> p) & 1) u ^= wd[p];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const v4i Aop = RES ? A[2 * v + half] : fr[(2 * v + half) * 64 + lane];
            acc_m = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aop, bit_lanes(u, half), acc_m, 0, 0, 0);
          }
        }
#pragma unroll
        for (int half = 0; half < (MSE ? 0 : 2); ++half) {
          const v4i Aop = RES ? A[2 * NV + half] : fr[(2 * NV + half) * 64 + lane];
          acc_q = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aop, bit_lanes(wd[NB - 1], half), acc_q,
                                                        0, 0, 0);
        }
      }
      const int hh = 4 * rb + g;
      if (valid && hh < a.G) {
        if constexpr (!RES) cst = ((const float4*)(rbase + (size_t)nws * NC * 64 * 16))[g];
        const float vm = fmaf((float)acc_m[3], 16777216.f,
                              fmaf((float)acc_m[2], 65536.f,
                                   fmaf((float)acc_m[1], 256.f, (float)acc_m[0])));
        const float vq = fmaf((float)acc_q[3], 16777216.f,
                              fmaf((float)acc_q[2], 65536.f,
                                   fmaf((float)acc_q[1], 256.f, (float)acc_q[0])));
        const float mse = fmaf(vm, cst.x, cst.z);
        const float qjl = fmaf(vq, cst.y, cst.w);
        const float nu = __half2float(__ushort_as_half((unsigned short)(nrm & 0xffffu)));
        const float ga = __half2float(__ushort_as_half((unsigned short)(nrm >> 16)));
        const float est = nu * fmaf(a.alpha * ga, qjl, mse);
        a.logits[(int64_t)(h * a.G + hh) * a.logits_stride_head + start + tok] = a.scale * est;
      }
    }
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Cache policy of the record loads: nontemporal.  Each record is read once per
// launch; on the 32-layer stream (570 MB of records) this measured 2-4% faster
// than the default policy.
constexpr int kNT = 2;

template <int NB>
__device__ inline void buf_group(rsrc_t r, uint32_t off, uint32_t (&w)[NB]) {
  if constexpr (NB == 4) {
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (NB == 3) {
    typedef int v3i __attribute__((ext_vector_type(3)));
    const v3i v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, kNT);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else if constexpr (NB == 2) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNT);
    w[0] = v[0]; w[1] = v[1];
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNT);
  }
}

// Resident variant (d <= 128, at most 4 query heads per KV head): the A
// operands and constants stay in registers, and key records are streamed in
// groups of U tiles with double buffering, so every wave keeps 2U tiles of
// loads in flight while its MFMAs run.  Records and norms are read through
// buffer resources bounded to the wave's tokens, so loads past them (and of
// word groups beyond d) return zeros without branches or traffic.
//
// NB2 > 0: channel-split records (fractional bit widths, two instances over
// the first and the remaining channels).  A second record set (a.set2, NB2
// words per group, its own prepared operands) is streamed alongside the
// first; each token's logit is the sum of the two instances' estimates.
//
// FOLD (every set with W <= 2): the lane groups that would hold words 2 and 3
// hold the upper 16 bits of words 0 and 1 instead (lane group g: word g & 1,
// shifts 4 (g >> 1) .. +3), so one MFMA covers all 64 coordinates and each
// Walsh subset (and the sign plane) takes one call instead of two; the query
// operands are prepared in the same folded layout.
// The stream of one wave, wave wi of the wn on sequence bi against kv head h,
// with the prepared operands of the first record set in Asm (LDS, NC x 64
// lanes, then those of set2) and the per-head constants of lane group g at
// cstp[g] / cstp2[g].  The tokens come in groups of U tiles:
//  * IL false: the wave's own contiguous chunk [wi chunk, wi chunk + chunk);
//  * IL true: the sequence's groups in turn (wave wi: groups wi, wi + wn,
//    ...), so the waves of a sequence read one compact window together.
// pre() runs once on every wave (the kernels fill Asm there).  PRIME = 0:
// the first loads follow it; PRIME = 1: the first group's loads are issued
// before it, so they are in flight while the operands are prepared.  On the
// one-call kernel at b >= 3 the interleaved order with one primed group
// measured 2-5% faster than the contiguous order; on the prepared-operand
// stream, and at b = 2, the contiguous order without priming was faster
// (2-3% on the 32-layer stream).
template <int NB, bool MSE, int U, int NB2, bool FOLD, bool IL, int PRIME, typename Pre>
__device__ __forceinline__ void res_stream(const AttnArgs& a, const v4i* Asm, const float4* cstp,
                                           const float4* cstp2, int h, int bi, int wi, int wn,
                                           int chunk, Pre&& pre) {
  static_assert(U % 2 == 0, "tiles are processed in pairs");
  constexpr bool SPLIT = NB2 > 0;
  constexpr int HALVES = FOLD ? 1 : 2;                 // MFMA calls per bit set
  constexpr int CP = MSE ? NB : NB - 1;
  constexpr int NV = 1 << (CP - 1);
  constexpr int NC = HALVES * (NV + (MSE ? 0 : 1));
  constexpr int NBs = SPLIT ? NB2 : NB;                // second set (unused if none)
  constexpr int CP2 = MSE ? NBs : NBs - 1;
  constexpr int NV2 = 1 << (CP2 - 1);
  constexpr int NC2 = SPLIT ? HALVES * (NV2 + (MSE ? 0 : 1)) : 1;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  constexpr int GT = kTile * U;                        // tokens per group
  const int len = a.seq_len[bi];
  const int64_t start = a.seq_start[bi];
  const int t_begin = IL ? wi * GT : wi * chunk;       // first group's first token
  const int t_end = IL ? len : min(len, t_begin + chunk);   // the wave's tokens end here
  const int step = IL ? wn * GT : GT;                  // from one group to the next
  const int64_t rec_seq = (int64_t)h * a.keys_stride_head + start;
  const uint32_t rec_bytes = (uint32_t)(a.W * NB * 4);
  // word group of this lane's token (g, or g & 1 folded); groups beyond d read
  // out of range (0)
  const int wg = FOLD ? (g & 1) : g;
  const uint32_t goff = wg < a.W ? (uint32_t)(wg * NB * 4) : 0x80000000u;
  const uint32_t rec_bytes2 = SPLIT ? (uint32_t)(a.set2.W * NB2 * 4) : 0u;
  uint32_t goff2 = 0u;
  if constexpr (SPLIT) goff2 = wg < a.set2.W ? (uint32_t)(wg * NB2 * 4) : 0x80000000u;
  // folded bit masks: shifts 4 (g >> 1) + i of every byte
  uint32_t fmk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fmk[i] = 0x01010101u << (4 * (g >> 1) + i);
  auto bits = [&](uint32_t u, int half) -> v4i {
    if constexpr (FOLD) {
      v4i r;
      r[0] = (int)(u & fmk[0]);
      r[1] = (int)(u & fmk[1]);
      r[2] = (int)(u & fmk[2]);
      r[3] = (int)(u & fmk[3]);
      return r;
    } else {
      return bit_lanes(u, half);
    }
  };
  // stores: lane half hf (0/1) writes 32 consecutive tokens of head gs + hf
  // (gs = 0 for the first store of a tile pair, 2 for the second)
  const int hf = lane >> 5, ts = lane & 31;
  float* out_a = a.logits + (int64_t)(h * a.G + hf) * a.logits_stride_head + start;
  float* out_b = a.logits + (int64_t)(h * a.G + 2 + hf) * a.logits_stride_head + start;
  const bool head_a = hf < a.G, head_b = 2 + hf < a.G;
  // source lanes (head g, token n) of the values this lane stores
  const int src_a = 16 * hf + (ts & 15), src_b = 32 + src_a;

  struct Grp {
    uint32_t wd[U][NB];
    uint32_t nr[U];
    uint32_t wd2[U][NBs];
    uint32_t nr2[U];
  };
  // load(gr, tl): the group whose first token is tl (wave-uniform).
  //  * IL: one plane resource per tile (its tokens that exist) keeps a lane's
  //    plane offset the same for every tile of every group, in one register.
  //    The clamps go through readfirstlane: as vector med3 results they would
  //    put the resources in vector registers and every load in a waterfall
  //    loop.
  //  * contiguous: one resource per wave over its chunk.
  const uint32_t voff = (uint32_t)n * rec_bytes + goff;
  const uint32_t voff2 = (uint32_t)n * rec_bytes2 + goff2;
  const int64_t rec_first = rec_seq + t_begin;
  const uint32_t n_tok = (uint32_t)max(0, t_end - t_begin);
  const rsrc_t rp_w = make_rsrc(a.planes + rec_first * a.W * NB, n_tok * rec_bytes);
  const rsrc_t rn_w = make_rsrc(a.norms + rec_first, n_tok * 4u);
  rsrc_t rp2_w = rp_w, rn2_w = rn_w;
  if constexpr (SPLIT) {
    rp2_w = make_rsrc(a.set2.planes + rec_first * a.set2.W * NB2, n_tok * rec_bytes2);
    rn2_w = make_rsrc(a.set2.norms + rec_first, n_tok * 4u);
  }
  auto load = [&](Grp& gr, int tl) {
    if constexpr (IL) {
      const uint32_t nt = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(GT, t_end - tl)));
      const int64_t rec = rec_seq + tl;
      const rsrc_t rn = make_rsrc(a.norms + rec, nt * 4u);
      rsrc_t rn2 = rn;
      if constexpr (SPLIT) rn2 = make_rsrc(a.set2.norms + rec, nt * 4u);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t ntu = (uint32_t)__builtin_amdgcn_readfirstlane(
            max(0, min(kTile, (int)nt - kTile * u)));
        const int64_t ru = rec + kTile * u;
        buf_group<NB>(make_rsrc(a.planes + ru * a.W * NB, ntu * rec_bytes), voff, gr.wd[u]);
        gr.nr[u] =
            __builtin_amdgcn_raw_buffer_load_b32(rn, (uint32_t)(kTile * u + n) * 4u, 0, kNT);
        if constexpr (SPLIT) {
          buf_group<NB2>(make_rsrc(a.set2.planes + ru * a.set2.W * NB2, ntu * rec_bytes2), voff2,
                         gr.wd2[u]);
          gr.nr2[u] =
              __builtin_amdgcn_raw_buffer_load_b32(rn2, (uint32_t)(kTile * u + n) * 4u, 0, kNT);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t t = (uint32_t)(tl - t_begin + kTile * u + n);
        buf_group<NB>(rp_w, t * rec_bytes + goff, gr.wd[u]);
        gr.nr[u] = __builtin_amdgcn_raw_buffer_load_b32(rn_w, t * 4u, 0, kNT);
        if constexpr (SPLIT) {
          buf_group<NB2>(rp2_w, t * rec_bytes2 + goff2, gr.wd2[u]);
          gr.nr2[u] = __builtin_amdgcn_raw_buffer_load_b32(rn2_w, t * 4u, 0, kNT);
        }
      }
    }
  };
  Grp g0, g1;
  int tl = t_begin;
  const bool any = tl < t_end;                // wave-uniform
  if constexpr (PRIME > 0)
    if (any) load(g0, tl);
  pre();
  if (!any) return;

  v4i A[NC], A2[NC2];
#pragma unroll
  for (int c = 0; c < NC; ++c) A[c] = Asm[c * 64 + lane];
  if constexpr (SPLIT) {
#pragma unroll
    for (int c = 0; c < NC2; ++c) A2[c] = Asm[(NC + c) * 64 + lane];
  }
  // per-head constants with the logit scale and the QJL factor folded in:
  // logit = nu * (vm X + Z + gamma (vq Y + W))
  const float4 cst = cstp[g];
  const float cX = a.scale * cst.x, cZ = a.scale * cst.z;
  const float cY = a.scale * a.alpha * cst.y, cW = a.scale * a.alpha * cst.w;
  float cX2 = 0.f, cZ2 = 0.f, cY2 = 0.f, cW2 = 0.f;
  if constexpr (SPLIT) {
    const float4 c2 = cstp2[g];
    cX2 = a.scale * c2.x;
    cZ2 = a.scale * c2.z;
    cY2 = a.scale * a.set2.alpha * c2.y;
    cW2 = a.scale * a.set2.alpha * c2.w;
  }
  // limbs -> float: |limb accumulators| < 2^21.1 (at most 16 NV K-slots per
  // shift, |A| <= 128, |B| <= 2^k), so limb pairs combine exactly in int32
  auto limbs = [](v4i c) {
    const int lo = c[0] + (c[1] << 8), hi = c[2] + (c[3] << 8);
    return fmaf((float)hi, 65536.f, (float)lo);
  };
  auto logit = [&](v4i am, v4i aq, uint32_t nrm, float x, float z, float y, float w) {
    const float ms = fmaf(limbs(am), x, z);
    const float nu = __half2float(__ushort_as_half((unsigned short)(nrm & 0xffffu)));
    if constexpr (MSE) return nu * ms;
    const float qs = fmaf(limbs(aq), y, w);
    const float ga = __half2float(__ushort_as_half((unsigned short)(nrm >> 16)));
    return nu * fmaf(ga, qs, ms);
  };
  // tile pair at local token tl: lane (g, n) holds head g of tokens tl + n
  // (v0) and tl + 16 + n (v1); permuted so each store instruction writes two
  // whole 32-token rows (128 bytes each), streamed (never re-read)
  auto finish2 = [&](float v0, float v1, int tl) {
    const float a0 = __shfl(v0, src_a), a1 = __shfl(v1, src_a);
    const float b0 = __shfl(v0, src_b), b1 = __shfl(v1, src_b);
    const int tok = tl + ts;
    if (tok < t_end) {
      if (head_a) __builtin_nontemporal_store(ts < 16 ? a0 : a1, &out_a[tok]);
      if (head_b) __builtin_nontemporal_store(ts < 16 ? b0 : b1, &out_b[tok]);
    }
  };
  // the MFMA chains of one record set (B words per group) for a tile pair,
  // interleaved so each hides the other's dependent-issue latency
  auto dots = [&](auto nb_c, const v4i* Aop, const uint32_t* w0, const uint32_t* w1, v4i& am0,
                  v4i& aq0, v4i& am1, v4i& aq1) {
    constexpr int B = decltype(nb_c)::value;
    constexpr int cp = MSE ? B : B - 1;
    constexpr int nv = 1 << (cp - 1);
#pragma unroll
    for (int v = 0; v < nv; ++v) {
      uint32_t u0 = 0u, u1 = 0u;
#pragma unroll
      for (int p = 0; p < cp; ++p)
        if ((walsh_mask<cp>(v) >> p) & 1) {
          u0 ^= w0[p];
          u1 ^= w1[p];
        }
#pragma unroll
      for (int h = 0; h < HALVES; ++h) {
        const v4i Ah = Aop[HALVES * v + h];
        am0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ah, bits(u0, h), am0, 0, 0, 0);
        am1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ah, bits(u1, h), am1, 0, 0, 0);
      }
    }
    if constexpr (!MSE) {
      const uint32_t s0 = w0[B - 1], s1 = w1[B - 1];
#pragma unroll
      for (int h = 0; h < HALVES; ++h) {
        const v4i Ah = Aop[HALVES * nv + h];
        aq0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ah, bits(s0, h), aq0, 0, 0, 0);
        aq1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ah, bits(s1, h), aq1, 0, 0, 0);
      }
    }
  };
  auto compute = [&](const Grp& gr, int tl) {
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      if (tl + kTile * u >= t_end) break;
      v4i am0 = {0, 0, 0, 0}, aq0 = {0, 0, 0, 0}, am1 = {0, 0, 0, 0}, aq1 = {0, 0, 0, 0};
      dots(std::integral_constant<int, NB>{}, A, gr.wd[u], gr.wd[u + 1], am0, aq0, am1, aq1);
      float v0 = logit(am0, aq0, gr.nr[u], cX, cZ, cY, cW);
      float v1 = logit(am1, aq1, gr.nr[u + 1], cX, cZ, cY, cW);
      if constexpr (SPLIT) {
        v4i bm0 = {0, 0, 0, 0}, bq0 = {0, 0, 0, 0}, bm1 = {0, 0, 0, 0}, bq1 = {0, 0, 0, 0};
        dots(std::integral_constant<int, NBs>{}, A2, gr.wd2[u], gr.wd2[u + 1], bm0, bq0, bm1,
             bq1);
        v0 += logit(bm0, bq0, gr.nr2[u], cX2, cZ2, cY2, cW2);
        v1 += logit(bm1, bq1, gr.nr2[u + 1], cX2, cZ2, cY2, cW2);
      }
      finish2(v0, v1, tl + kTile * u);
    }
  };
  if constexpr (PRIME == 0) load(g0, tl);
  for (; tl < t_end; tl += 2 * step) {
    load(g1, tl + step);
    compute(g0, tl);
    load(g0, tl + 2 * step);
    compute(g1, tl + step);
  }
}

// Stream over operands prepared beforehand in the workspace.  grid = (token
// chunks, kv heads, batch); the 4 waves of a workgroup share (sequence, kv
// head), so the prepared operands are read from memory once per workgroup.
template <int NB, bool MSE, int U, int NB2, bool FOLD>
__global__ void __launch_bounds__(256) attn_logits_res_kernel(AttnArgs a) {
  constexpr bool SPLIT = NB2 > 0;
  constexpr int HALVES = FOLD ? 1 : 2;
  constexpr int CP = MSE ? NB : NB - 1;
  constexpr int NC = HALVES * ((1 << (CP - 1)) + (MSE ? 0 : 1));
  constexpr int NBs = SPLIT ? NB2 : NB;
  constexpr int CP2 = MSE ? NBs : NBs - 1;
  constexpr int NC2 = SPLIT ? HALVES * ((1 << (CP2 - 1)) + (MSE ? 0 : 1)) : 1;
  const int h = blockIdx.y, bi = blockIdx.z;
  const size_t rbb = (size_t)NC * 64 * 16 + 64;
  const char* wsb = a.ws + ((size_t)bi * a.n_kv + h) * rbb;
  const size_t rbb2 = (size_t)NC2 * 64 * 16 + 64;
  const char* wsb2 = a.set2.ws + ((size_t)bi * a.n_kv + h) * rbb2;
  __shared__ v4i Asm[(NC + (SPLIT ? NC2 : 0)) * 64];
  auto pre = [&]() {
    for (int i = threadIdx.x; i < NC * 64; i += 256) Asm[i] = ((const v4i*)wsb)[i];
    if constexpr (SPLIT)
      for (int i = threadIdx.x; i < NC2 * 64; i += 256) Asm[NC * 64 + i] = ((const v4i*)wsb2)[i];
    __syncthreads();
  };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  res_stream<NB, MSE, U, NB2, FOLD, false, 0>(a, Asm, (const float4*)(wsb + (size_t)NC * 64 * 16),
                                              (const float4*)(wsb2 + (size_t)NC2 * 64 * 16), h,
                                              bi, blockIdx.x * kWaves + wave, gridDim.x * kWaves,
                                              a.tiles_per_wave * kTile, pre);
}

// One launch for a whole call: each workgroup of 16 waves first prepares the
// query operands of its (sequence, kv head) into LDS -- the work and the
// arithmetic of attn_prep_kernel (prep_block), so the operands are bit for
// bit those of the two-launch form -- then its waves stream their tiles.
// Waves 0-3 prepare the code part, waves 4-7 the sign part (two-stage
// records); the rest only meet the barriers.  No workspace, and no wait on
// another workgroup: the preparation is repeated by every workgroup of a
// (sequence, kv head), so the grid is sized to one workgroup per CU.
constexpr int kOneWaves = 16;
template <int NB, bool MSE, bool FOLD>
__global__ void __launch_bounds__(64 * kOneWaves) attn_logits_one_kernel(AttnArgs a, PrepArgs p) {
  constexpr int HALVES = FOLD ? 1 : 2;
  constexpr int CP = MSE ? NB : NB - 1;
  constexpr int NC = HALVES * ((1 << (CP - 1)) + (MSE ? 0 : 1));
  constexpr int kD = 128;                      // d <= 128 (W <= 4) on this path
  __shared__ float qv[4 * kD];                 // coordinate j of slot hh at 4j + hh
  __shared__ float outp[2][4 * kD];            // per part: [slot][Dp]
  __shared__ float red[2][64 * 32];            // per part: [4 waves][16][nq], nq <= 32
  __shared__ int qfix_e[2][4];
  __shared__ __align__(16) char abuf[NC * 64 * 16 + 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int part = tid >> 8, ptid = tid & 255, pwave = ptid >> 6;
  const bool act = part < p.n_parts;           // uniform per wave
  const int d = p.d, Dp = 32 * p.W, nq = p.nq, nj = 256 / nq;
  const float* tab = part ? p.st : p.pit;
  float* out = outp[part & 1];
  float* rd = red[part & 1];

  float* cdst_base = (float*)(abuf + (size_t)NC * 64 * 16);

  // the preparation (every wave runs it, in the stream after its first loads
  // are issued where the stream primes them)
  auto pre = [&]() {
    // Dp <= 4 nq: one chunk of outputs, as prep_block at these sizes; a
    // thread's table rows (at most 16: jl = 16 at d = 128) are all requested
    // before the queries are staged, so the two memory round trips overlap
    const int quad = ptid & (nq - 1), jg = ptid / nq;
    const int jl = (d + nj - 1) / nj;
    const int ja = min(d, jg * jl), jb = min(d, ja + jl);
    const int r = 4 * quad;
    const bool rows = act && r < d;
    float4 t[16];
    if (rows) {
      const float* tr = tab + r;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (ja + u < jb) t[u] = *(const float4*)(tr + (int64_t)(ja + u) * d);
    }
    for (int it = tid; it < 4 * d; it += 64 * kOneWaves) {
      const int hh = it / d, j = it - hh * d;
      qv[4 * j + hh] = hh < p.G
          ? p.q[(int64_t)bi * p.q_stride_batch + (int64_t)(h * p.G + hh) * p.q_stride_head + j]
          : 0.f;
    }
    __syncthreads();
    if (act) {
      float acc[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;
      if (rows) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (ja + u < jb) {
            const float4 qq = *(const float4*)&qv[4 * (ja + u)];
            const float tv[4] = {t[u].x, t[u].y, t[u].z, t[u].w}, qs[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(tv[e], qs[i], acc[i][e]);
          }
        }
      }
      for (int off = nq; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] += __shfl_xor(acc[i][e], off);
      if (lane < nq)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) rd[(pwave * 16 + 4 * i + e) * nq + quad] = acc[i][e];
    }
    __syncthreads();
    if (act) {
      for (int it = ptid; it < 16 * nq; it += 256) {
        const int k = it / nq, qd = it - k * nq;
        const float v = (rd[k * nq + qd] + rd[(16 + k) * nq + qd]) +
                        (rd[(32 + k) * nq + qd] + rd[(48 + k) * nq + qd]);
        const int o = 4 * qd + (k & 3);
        if (o < Dp) out[(k >> 2) * Dp + o] = v;
      }
    }
    __syncthreads();
    if (act) {
      const float* r1 = out + pwave * Dp;
      float m1 = 0.f, t1 = 0.f;
      for (int j = lane; j < Dp; j += 64) {
        m1 = fmaxf(m1, fabsf(r1[j]));
        t1 += r1[j];
      }
      m1 = wave_max(m1);
      t1 = wave_sum(t1);
      if (lane == 0) {
        float wmax = 2.f;
        if (part == 0) {
          wmax = 0.f;
          for (int v = 0; v < p.nv; ++v) wmax = fmaxf(wmax, fabsf(p.wm2[v]));
        }
        const float vmax = wmax * m1;
        int e = 0;
        if (vmax > 0.f) { int ex; frexpf(vmax, &ex); e = min(30 - ex, 120); }
        qfix_e[part][pwave] = e;
        float* cdst = cdst_base + 4 * pwave;
        if (part == 0) {
          cdst[0] = ldexpf(1.f, -e);
          cdst[2] = p.c0 * t1;
          if (p.n_parts == 1) {
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
    {
      // the operands of both parts, spread over all 16 waves
      const int code_calls = p.fold ? p.nv : 2 * p.nv;
      const int sign_calls = p.nc - code_calls;
      const int items0 = 4 * code_calls * 4, items = items0 + (p.n_parts > 1 ? 4 * sign_calls * 4 : 0);
      for (int it = tid; it < items; it += 64 * kOneWaves) {
        const int pt = it >= items0;
        const int n_c = pt ? sign_calls : code_calls;
        const int i = it - (pt ? items0 : 0);
        const int g = i & 3, rest = i >> 2;
        const int cl = rest % n_c, hh = rest / n_c;
        const int c = (pt ? code_calls : 0) + cl;
        const int w = p.fold ? (g & 1) : g;
        const int kbase = p.fold ? 4 * (g >> 1) : (pt ? 4 * cl : 4 * (c % 2));
        const float wv = pt ? 2.f : p.wm2[p.fold ? c : c / 2];
        uint4 o[4];
        limb_operands(outp[pt] + hh * Dp, qfix_e[pt][hh], wv, w, p.W, d, kbase, o);
        uint4* dst = (uint4*)(abuf + ((size_t)c * 64 + 16 * g + 4 * hh) * 16);
#pragma unroll
        for (int L = 0; L < 4; ++L) dst[L] = o[L];
      }
    }
    __syncthreads();
  };
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool IL = NB >= 3;                 // (measured: see res_stream)
  res_stream<NB, MSE, 4, 0, FOLD, IL, IL ? 1 : 0>(a, (const v4i*)abuf, (const float4*)cdst_base,
                                                  (const float4*)cdst_base, h, bi,
                                                  blockIdx.x * kOneWaves + wave,
                                                  gridDim.x * kOneWaves,
                                                  a.tiles_per_wave * kTile, pre);
}

template <typename K>
int resident_blocks_per_cu(K kernel) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, 256, 0) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

}  // namespace

size_t attn_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t n_q_heads,
                            int32_t n_kv_heads) {
  const int G = n_q_heads / n_kv_heads;
  const int n_rb = (G + 3) / 4;
  return (size_t)batch * n_kv_heads * n_rb * rb_bytes(ctx->W, n_calls(ctx->cp, !ctx->mse));
}

hipError_t launch_attn_prepare(const tq_ctx* ctx, const float* q, int32_t batch,
                               int32_t n_q_heads, int64_t q_stride_batch, int32_t n_kv_heads,
                               void* workspace, bool fold, hipStream_t stream) {
  PrepArgs p;
  size_t shm;
  dim3 grid;
  prep_args(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads, workspace, p, shm, grid, fold);
  // raise the dynamic-LDS limit once (never inside a sequence a caller may capture)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)attn_prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(attn_prep_kernel, grid, dim3(256), shm, stream, p);
  return hipGetLastError();
}

namespace {

// Fill the arguments of one record set's stream (everything but the grid).
AttnArgs stream_args(const tq_ctx* ctx, const void* workspace, int32_t n_q_heads,
                     const uint32_t* planes, const uint16_t* norms, int32_t n_kv_heads,
                     int64_t keys_stride_head, const int64_t* seq_start, const int32_t* seq_len,
                     float scale, float* logits, int64_t logits_stride_head) {
  const int G = n_q_heads / n_kv_heads;
  AttnArgs a{};
  a.ws = (const char*)workspace;
  a.planes = planes;
  a.norms = (const uint32_t*)norms;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.logits = logits;
  a.keys_stride_head = keys_stride_head;
  a.logits_stride_head = logits_stride_head;
  a.W = ctx->W;
  a.G = G;
  a.n_kv = n_kv_heads;
  a.n_rb = (G + 3) / 4;
  a.scale = scale;
  a.alpha = (float)(std::sqrt(M_PI / 2.0) / ctx->d);
  for (int v = 0; v < ctx->n_mono; ++v) a.mask[v] = ctx->mono_mask[v];
  return a;
}

// The resident kernel applies: d <= 128, G <= 4 and the Walsh subsets it
// hard-codes (1 / 1,2 / 1,2,4,7).
bool resident_ok(const tq_ctx* ctx, int n_rb) {
  static const int kMasks[3][4] = {{1, 0, 0, 0}, {1, 2, 0, 0}, {1, 2, 4, 7}};
  bool masks_ok = true;
  for (int v = 0; v < ctx->n_mono; ++v) masks_ok &= ctx->mono_mask[v] == kMasks[ctx->cp - 1][v];
  return ctx->W <= 4 && n_rb == 1 && masks_ok;
}

// Grid of a stream with nb resident blocks per CU: one round of resident
// waves over all tiles (each wave takes a contiguous chunk of one sequence),
// so no partial second round is left.  Short chunks (about 8 rounds of
// resident waves) keep many independent read/write streams in flight, which
// measured best on the mixed record-read / logit-write traffic; at least 8
// tiles per wave.
dim3 stream_grid(int n_cu, int nb, int32_t batch, int32_t n_kv_heads, int32_t max_seq_len,
                 int& tiles_per_wave) {
  const int64_t tiles_seq = (max_seq_len + kTile - 1) / kTile;
  const int64_t tiles_total = (int64_t)batch * n_kv_heads * tiles_seq;
  const int64_t resident_waves = (int64_t)n_cu * nb * kWaves;
  int64_t tpw = (tiles_total + 8 * resident_waves - 1) / (8 * resident_waves);
  tpw = std::max<int64_t>(8, std::min<int64_t>(256, tpw));
  tiles_per_wave = (int)tpw;
  const int64_t tok_per_block = (int64_t)kWaves * tpw * kTile;
  return dim3((unsigned)((max_seq_len + tok_per_block - 1) / tok_per_block), n_kv_heads, batch);
}

template <int NB, bool MSE, int NB2, bool FOLD>
hipError_t launch_res(const AttnArgs& a, int n_cu, int32_t batch, int32_t n_kv_heads,
                      int32_t max_seq_len, hipStream_t stream) {
  static const int nb = resident_blocks_per_cu(attn_logits_res_kernel<NB, MSE, 4, NB2, FOLD>);
  AttnArgs b = a;
  const dim3 grid = stream_grid(n_cu, nb, batch, n_kv_heads, max_seq_len, b.tiles_per_wave);
  hipLaunchKernelGGL((attn_logits_res_kernel<NB, MSE, 4, NB2, FOLD>), grid, dim3(256), 0, stream,
                     b);
  return hipGetLastError();
}

template <int NB, bool MSE>
hipError_t launch_general(const AttnArgs& a, int n_cu, int32_t batch, int32_t n_kv_heads,
                          int32_t max_seq_len, hipStream_t stream) {
  AttnArgs b = a;
  const dim3 grid = stream_grid(n_cu, 4, batch, n_kv_heads, max_seq_len, b.tiles_per_wave);
  hipLaunchKernelGGL((attn_logits_kernel<NB, MSE, false>), grid, dim3(256), 0, stream, b);
  return hipGetLastError();
}

// Channel-split preparation: the queries' first d1 channels against the first
// instance and the rest against the second, as disjoint workgroups of one grid.
struct SplitPrepArgs {
  PrepArgs p1, p2;
  uint32_t n1;                    // workgroups of the first preparation
  uint32_t x1, y1, x2, y2;        // the two preparations' grids (x, y); z = batch
};

__global__ void __launch_bounds__(256) split_prep_kernel(SplitPrepArgs a) {
  uint32_t b = blockIdx.x;
  if (b < a.n1) {
    const uint32_t byz = b / a.x1;
    prep_block(a.p1, (int)(b % a.x1), (int)(byz % a.y1), (int)(byz / a.y1));
  } else {
    b -= a.n1;
    const uint32_t byz = b / a.x2;
    prep_block(a.p2, (int)(b % a.x2), (int)(byz % a.y2), (int)(byz / a.y2));
  }
}

size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

}  // namespace

hipError_t launch_attn_stream(const tq_ctx* ctx, const void* workspace, int32_t batch,
                              int32_t n_q_heads, const uint32_t* planes, const uint16_t* norms,
                              int32_t n_kv_heads, int64_t keys_stride_head,
                              const int64_t* seq_start, const int32_t* seq_len,
                              int32_t max_seq_len, float scale, float* logits,
                              int64_t logits_stride_head, hipStream_t stream) {
  const AttnArgs a = stream_args(ctx, workspace, n_q_heads, planes, norms, n_kv_heads,
                                 keys_stride_head, seq_start, seq_len, scale, logits,
                                 logits_stride_head);
  const bool res = resident_ok(ctx, a.n_rb);
  const bool fold = res && ctx->W <= 2;        // as logits_fold()
  const int n_cu = ctx->n_cu;
#define TQ_LOGITS(NB, MSE)                                                                 \
  return !res ? launch_general<NB, MSE>(a, n_cu, batch, n_kv_heads, max_seq_len, stream)   \
         : fold ? launch_res<NB, MSE, 0, true>(a, n_cu, batch, n_kv_heads, max_seq_len, stream) \
                : launch_res<NB, MSE, 0, false>(a, n_cu, batch, n_kv_heads, max_seq_len, stream)
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: TQ_LOGITS(1, true);
      case 2: TQ_LOGITS(2, true);
      default: TQ_LOGITS(3, true);
    }
  }
  switch (ctx->b) {
    case 2: TQ_LOGITS(2, false);
    case 3: TQ_LOGITS(3, false);
    default: TQ_LOGITS(4, false);
  }
#undef TQ_LOGITS
}

namespace {

template <int NB, bool MSE, bool FOLD>
hipError_t launch_one(const AttnArgs& a, const PrepArgs& p, int n_cu, int32_t batch,
                      int32_t n_kv_heads, int32_t max_seq_len, hipStream_t stream) {
  // one workgroup per CU: the tiles per wave that cover every tile in one
  // round (at most 256, beyond which further rounds repeat the preparation)
  AttnArgs b = a;
  const int64_t tiles_seq = (max_seq_len + kTile - 1) / kTile;
  const int64_t tiles_total = (int64_t)batch * n_kv_heads * tiles_seq;
  const int64_t waves = (int64_t)n_cu * kOneWaves;
  const int64_t tpw = std::max<int64_t>(1, std::min<int64_t>(256, (tiles_total + waves - 1) / waves));
  b.tiles_per_wave = (int)tpw;
  const int64_t tok_per_block = (int64_t)kOneWaves * tpw * kTile;
  const dim3 grid((unsigned)((max_seq_len + tok_per_block - 1) / tok_per_block), n_kv_heads,
                  batch);
  hipLaunchKernelGGL((attn_logits_one_kernel<NB, MSE, FOLD>), grid, dim3(64 * kOneWaves), 0,
                     stream, b, p);
  return hipGetLastError();
}

}  // namespace

bool attn_one_applies(const tq_ctx* ctx, int32_t n_q_heads, int32_t n_kv_heads) {
  return ctx->d <= 128 && resident_ok(ctx, (n_q_heads / n_kv_heads + 3) / 4);
}

hipError_t launch_attn_one(const tq_ctx* ctx, const float* q, int32_t batch, int32_t n_q_heads,
                           int64_t q_stride_batch, const uint32_t* planes, const uint16_t* norms,
                           int32_t n_kv_heads, int64_t keys_stride_head,
                           const int64_t* seq_start, const int32_t* seq_len,
                           int32_t max_seq_len, float scale, float* logits,
                           int64_t logits_stride_head, hipStream_t stream) {
  if (!attn_one_applies(ctx, n_q_heads, n_kv_heads)) return hipErrorInvalidValue;
  const bool fold = ctx->W <= 2;
  PrepArgs p;
  size_t shm;
  dim3 pgrid;
  prep_args(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads, nullptr, p, shm, pgrid, fold);
  const AttnArgs a = stream_args(ctx, nullptr, n_q_heads, planes, norms, n_kv_heads,
                                 keys_stride_head, seq_start, seq_len, scale, logits,
                                 logits_stride_head);
  const int n_cu = ctx->n_cu;
#define TQ_ONE(NB, MSE)                                                                        \
  return fold ? launch_one<NB, MSE, true>(a, p, n_cu, batch, n_kv_heads, max_seq_len, stream) \
              : launch_one<NB, MSE, false>(a, p, n_cu, batch, n_kv_heads, max_seq_len, stream)
  if (ctx->mse) {
    switch (ctx->b) {
      case 1: TQ_ONE(1, true);
      case 2: TQ_ONE(2, true);
      default: TQ_ONE(3, true);
    }
  }
  switch (ctx->b) {
    case 2: TQ_ONE(2, false);
    case 3: TQ_ONE(3, false);
    default: TQ_ONE(4, false);
  }
#undef TQ_ONE
}

bool logits_fold(const tq_ctx* ctx, int32_t n_q_heads, int32_t n_kv_heads) {
  return ctx->W <= 2 && resident_ok(ctx, (n_q_heads / n_kv_heads + 3) / 4);
}

size_t split_attn_workspace_bytes(const tq_ctx* c1, const tq_ctx* c2, int32_t batch,
                                  int32_t n_q_heads, int32_t n_kv_heads) {
  return align16(attn_workspace_bytes(c1, batch, n_q_heads, n_kv_heads)) +
         attn_workspace_bytes(c2, batch, n_q_heads, n_kv_heads);
}

bool split_logits_supported(const tq_ctx* c1, const tq_ctx* c2, int32_t n_q_heads,
                            int32_t n_kv_heads) {
  const int n_rb = (n_q_heads / n_kv_heads + 3) / 4;
  return c1->mse == c2->mse && resident_ok(c1, n_rb) && resident_ok(c2, n_rb);
}

hipError_t launch_split_prepare(const tq_ctx* c1, const tq_ctx* c2, const float* q,
                                int32_t batch, int32_t n_q_heads, int64_t q_stride_batch,
                                int32_t n_kv_heads, void* workspace, hipStream_t stream) {
  char* ws1 = (char*)workspace;
  char* ws2 = ws1 + align16(attn_workspace_bytes(c1, batch, n_q_heads, n_kv_heads));
  // q channels [0, d1) against the first instance, [d1, d1 + d2) against the
  // second, head stride d1 + d2
  SplitPrepArgs sp{};
  size_t shm1, shm2;
  dim3 g1, g2;
  const bool fold = c1->W <= 2 && c2->W <= 2;   // as the split stream
  prep_args(c1, q, batch, n_q_heads, q_stride_batch, n_kv_heads, ws1, sp.p1, shm1, g1, fold);
  prep_args(c2, q + c1->d, batch, n_q_heads, q_stride_batch, n_kv_heads, ws2, sp.p2, shm2, g2,
            fold);
  sp.p1.q_stride_head = sp.p2.q_stride_head = c1->d + c2->d;
  sp.n1 = g1.x * g1.y * g1.z;
  sp.x1 = g1.x;
  sp.y1 = g1.y;
  sp.x2 = g2.x;
  sp.y2 = g2.y;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)split_prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(split_prep_kernel, dim3(sp.n1 + g2.x * g2.y * g2.z), dim3(256),
                     std::max(shm1, shm2), stream, sp);
  return hipGetLastError();
}

hipError_t launch_split_stream(const tq_ctx* c1, const tq_ctx* c2, const void* workspace,
                               int32_t batch, int32_t n_q_heads, const uint32_t* planes1,
                               const uint16_t* norms1, const uint32_t* planes2,
                               const uint16_t* norms2, int32_t n_kv_heads,
                               int64_t keys_stride_head, const int64_t* seq_start,
                               const int32_t* seq_len, int32_t max_seq_len, float scale,
                               float* logits, int64_t logits_stride_head, hipStream_t stream) {
  const char* ws1 = (const char*)workspace;
  const char* ws2 = ws1 + align16(attn_workspace_bytes(c1, batch, n_q_heads, n_kv_heads));
  // one stream over both record sets; the set with more words per group is
  // the kernel's first
  const bool swap = c2->b > c1->b;
  const tq_ctx* ca = swap ? c2 : c1;
  const tq_ctx* cb = swap ? c1 : c2;
  AttnArgs a = stream_args(ca, swap ? ws2 : ws1, n_q_heads, swap ? planes2 : planes1,
                           swap ? norms2 : norms1, n_kv_heads, keys_stride_head, seq_start,
                           seq_len, scale, logits, logits_stride_head);
  a.set2.ws = swap ? ws1 : ws2;
  a.set2.planes = swap ? planes1 : planes2;
  a.set2.norms = (const uint32_t*)(swap ? norms1 : norms2);
  a.set2.W = cb->W;
  a.set2.alpha = (float)(std::sqrt(M_PI / 2.0) / cb->d);
  const int n_cu = ca->n_cu;
  const bool fold = c1->W <= 2 && c2->W <= 2;   // as the split preparation
#define TQ_SPLIT(NB, MSE, NB2)                                                                 \
  return fold ? launch_res<NB, MSE, NB2, true>(a, n_cu, batch, n_kv_heads, max_seq_len, stream) \
              : launch_res<NB, MSE, NB2, false>(a, n_cu, batch, n_kv_heads, max_seq_len, stream)
  const int key = 10 * ca->b + cb->b;
  if (ca->mse) {
    switch (key) {
      case 11: TQ_SPLIT(1, true, 1);
      case 21: TQ_SPLIT(2, true, 1);
      case 22: TQ_SPLIT(2, true, 2);
      case 31: TQ_SPLIT(3, true, 1);
      case 32: TQ_SPLIT(3, true, 2);
      default: TQ_SPLIT(3, true, 3);
    }
  }
  switch (key) {
    case 22: TQ_SPLIT(2, false, 2);
    case 32: TQ_SPLIT(3, false, 2);
    case 33: TQ_SPLIT(3, false, 3);
    case 42: TQ_SPLIT(4, false, 2);
    case 43: TQ_SPLIT(4, false, 3);
    default: TQ_SPLIT(4, false, 4);
  }
#undef TQ_SPLIT
}

// ---- static scratch of tq_attn_logits_noalloc ------------------------------
// The prepared query operands of the entry point that allocates nothing live
// in this file-scope device array instead of a caller workspace.  Every GPU
// the library runs on holds its own copy until the process ends.  In host
// code the array's name is only a stand-in: its device address is looked up
// once per device (hipGetSymbolAddress, at context creation with that device
// current) and only that address is ever passed to a kernel.  Calls that
// overlap on one GPU share the array and race.
static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t noalloc_scratch(int device, void** out) {
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  if (out) *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace tq
