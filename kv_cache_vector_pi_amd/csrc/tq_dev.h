// Device helpers shared by the logit, query-preparation, value-output and
// fused decode kernels (the value-side code itself is in tq_vacc.h).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace tq {
namespace dev {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;          // key tokens per MFMA tile
constexpr int kWaves = 4;          // waves per workgroup

// MFMA calls per word step: two per Walsh subset of the cp code planes, and
// two for the sign plane when the records carry the QJL stage
__host__ __device__ inline int n_calls(int cp, bool qjl) { return 2 * (1 << (cp - 1)) + (qjl ? 2 : 0); }
__host__ __device__ inline int n_ws(int W) { return (W + 3) / 4; }                  // word steps of 4 words

// Prepared-query workspace for one (batch, kv head, row block of 4 q heads):
//   int4 frag[n_ws][n_calls][64 lanes]   A operands (16 int8 each)
//   float4 consts[4]                      per q head: mse scale, qjl scale,
//                                         mse offset, qjl offset
__host__ __device__ inline size_t rb_bytes(int W, int nc) {
  return (size_t)n_ws(W) * nc * 64 * 16 + 4 * 16;
}

template <int NB>
__device__ inline void load_group(const uint32_t* p, uint32_t (&w)[NB]) {
  // NB words per record group
  if constexpr (NB == 4) {
    uint4 v = *(const uint4*)p;
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (NB == 2) {
    uint2 v = *(const uint2*)p;
    w[0] = v.x; w[1] = v.y;
  } else {
    for (int i = 0; i < NB; ++i) w[i] = p[i];
  }
}

// masked int8 lanes of a plane word for shifts 4*half .. 4*half+3
__device__ inline v4i bit_lanes(uint32_t u, int half) {
  const uint32_t m = 0x01010101u << (4 * half);
  v4i r;
  r[0] = (int)(u & m);
  r[1] = (int)(u & (m << 1));
  r[2] = (int)(u & (m << 2));
  r[3] = (int)(u & (m << 3));
  return r;
}

// Four balanced base-256 limbs accumulated by the int8 MFMAs -> float.
__device__ inline float limbs_to_float(const v4i& c) {
  return fmaf((float)c[3], 16777216.f, fmaf((float)c[2], 65536.f, fmaf((float)c[1], 256.f, (float)c[0])));
}

// Odd-sized subsets of the cp code planes (Walsh expansion of a symmetric
// codebook), in the order the context lists them: masks 1 / 1, 2 / 1, 2, 4, 7.
template <int CP>
__device__ constexpr int walsh_mask(int v) {
  return CP == 1 ? 1 : (CP == 2 ? (v == 0 ? 1 : 2) : (v == 0 ? 1 : v == 1 ? 2 : v == 2 ? 4 : 7));
}

// rint(Q / 2^k) for k >= 1 (half away from -inf), Q for k == 0
__device__ inline int shift_round(int Q, int k) {
  return k == 0 ? Q : ((Q + (1 << (k - 1))) >> k);
}

}  // namespace dev
}  // namespace tq
