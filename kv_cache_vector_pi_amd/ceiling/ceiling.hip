// Ceiling kernels (declared and described in include/tq_ceiling.h): the
// HBM stream with the logit kernel's read/write mix, a plain copy, and
// matrix-core loops.  Built into libtq_ceiling.so, not libtq.so.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "../../include/tq_ceiling.h"

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTile = 16;

// lane (g = lane / 16, n = lane % 16) loads word group g of token n of a
// tile; tile pairs, then each lane half stores 32 consecutive tokens of one
// of two heads per store (as the logit stream does)
__global__ void __launch_bounds__(256) logit_mix_kernel(const uint32_t* __restrict__ planes,
                                                        const uint32_t* __restrict__ norms,
                                                        int64_t n, float* __restrict__ out,
                                                        int64_t out_stride, int tiles_per_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, nn = lane & 15, hf = lane >> 5, ts = lane & 31;
  const int64_t t_begin = ((int64_t)blockIdx.x * 4 + wave) * tiles_per_wave * kTile;
  const int64_t t_end = std::min<int64_t>(n, t_begin + (int64_t)tiles_per_wave * kTile);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * kTile) {
    uint32_t v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t t = t0 + u * kTile + nn;
      uint32_t x = 0u;
      if (t < t_end) {
        const u4v w = __builtin_nontemporal_load((const u4v*)(planes + t * 16) + g);
        x = w[0] ^ w[1] ^ w[2] ^ w[3] ^ __builtin_nontemporal_load(norms + t);
      }
      v[u] = x;
    }
    // lane (g, n) holds head g's value of tokens t0 + n and t0 + 16 + n
    const int src_a = 16 * hf + (ts & 15), src_b = 32 + src_a;
    const uint32_t a0 = __shfl(v[0], src_a), a1 = __shfl(v[1], src_a);
    const uint32_t b0 = __shfl(v[0], src_b), b1 = __shfl(v[1], src_b);
    const int64_t t = t0 + ts;
    if (t < t_end) {
      __builtin_nontemporal_store((float)(ts < 16 ? a0 : a1), &out[hf * out_stride + t]);
      __builtin_nontemporal_store((float)(ts < 16 ? b0 : b1), &out[(2 + hf) * out_stride + t]);
    }
  }
}

// the same bytes per record in one-shot workgroups of `per` records: thread
// (record tid / 4, part tid % 4) loads 16 bytes of planes and the norm word,
// stores part's float; rounds of 64 records
__global__ void __launch_bounds__(256) logit_mix_blocks_kernel(const u4v* __restrict__ planes,
                                                               const uint32_t* __restrict__ norms,
                                                               int64_t n, float* __restrict__ out,
                                                               int64_t out_stride, int per) {
  const int tid = threadIdx.x, r = tid >> 2, part = tid & 3;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = std::min<int64_t>(n, b0 + per);
  for (int64_t base = b0; base < b1; base += 128) {
    const int64_t i0 = base + r, i1 = base + 64 + r;
    uint32_t x0 = 0u, x1 = 0u;
    if (i0 < b1) {
      const u4v w = __builtin_nontemporal_load(planes + 4 * i0 + part);
      x0 = w[0] ^ w[1] ^ w[2] ^ w[3] ^ __builtin_nontemporal_load(norms + i0);
    }
    if (i1 < b1) {
      const u4v w = __builtin_nontemporal_load(planes + 4 * i1 + part);
      x1 = w[0] ^ w[1] ^ w[2] ^ w[3] ^ __builtin_nontemporal_load(norms + i1);
    }
    if (i0 < b1) __builtin_nontemporal_store((float)x0, &out[part * out_stride + i0]);
    if (i1 < b1) __builtin_nontemporal_store((float)x1, &out[part * out_stride + i1]);
  }
}

__global__ void __launch_bounds__(256) copy_kernel(const u4v* __restrict__ src,
                                                   u4v* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

template <int KIND>
__global__ void __launch_bounds__(256) mfma_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
  if constexpr (KIND == 0) {
    const v4i a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 * lane, lane, 7, 1};
    v4i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, b, c3, 0, 0, 0);
      }
    }
    for (int i = 0; i < 4; ++i) s += (float)(c0[i] ^ c1[i] ^ c2[i] ^ c3[i]);
  } else {
    v8bf a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(1e-3f * (lane + i));
      b[i] = (__bf16)(1e-3f * (i - lane));
    }
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
      }
    }
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  }
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// MFMA / VALU co-issue on one SIMD: a workgroup of 8 waves, waves 4-7 issue
// v_mfma_f32_32x32x16_bf16 on two accumulators (if MFMA_ON), waves 0-3 issue
// VALU work (if VALU_ON): FMA chains (VK = 0) or compare / select /
// add-with-carry sequences like the quantizer's code decisions (VK = 1).
template <bool MFMA_ON, bool VALU_ON, int VK>
__global__ void __launch_bounds__(512, 1) overlap_kernel(int iters, float* out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float s = 0.f;
  if (wave >= 4) {
    if constexpr (MFMA_ON) {
      v8bf a, b;
      for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1e-3f * (lane + i));
        b[i] = (__bf16)(1e-3f * (i - lane));
      }
      v16f c0 = {}, c1 = {};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        }
      }
      for (int i = 0; i < 16; ++i) s += c0[i] + c1[i];
    }
  } else if constexpr (VALU_ON) {
    if constexpr (VK == 0) {
      float v[8];
      for (int i = 0; i < 8; ++i) v[i] = 1e-3f * (lane + i);
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = fmaf(v[i], 1.0001f, v[(i + 3) & 7]);
      }
      for (int i = 0; i < 8; ++i) s += v[i];
    } else {
      float y[8];
      uint32_t acc[4] = {0u, 0u, 0u, 0u};
      for (int i = 0; i < 8; ++i) y[i] = 1e-3f * (lane - 20 + 5 * i);
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float ay = fabsf(y[i]);
            const bool g0 = ay > 0.01f, g1 = ay > 0.02f, g2 = ay > 0.04f, p = y[i] > 0.f;
            float c = g0 ? 0.3f : 0.1f;
            c = g1 ? 0.5f : c;
            c = g2 ? 0.7f : c;
            y[i] = p ? y[i] - c * 1e-3f : y[i] + c * 1e-3f;
            acc[0] = 2u * acc[0] + (uint32_t)g0;
            acc[1] = 2u * acc[1] + (uint32_t)g1;
            acc[2] = 2u * acc[2] + (uint32_t)g2;
            acc[3] = 2u * acc[3] + (uint32_t)p;
          }
      }
      for (int i = 0; i < 8; ++i) s += y[i];
      s += (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
    }
  }
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

int n_cu() {
  static const int cus = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v < 1)
      v = 1;
    return v;
  }();
  return cus;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int tq_ceiling_logit_mix(
    const uint32_t* planes, const uint32_t* norms, int64_t n, float* out, int64_t out_stride,
    void* stream) {
  if (n < 0 || out_stride < n) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  if (!planes || !norms || !out) return (int)hipErrorInvalidValue;
  // the stream kernel's grid rule: about 8 rounds of 4 resident workgroups
  // per CU, at least 8 tiles per wave
  const int64_t tiles = (n + kTile - 1) / kTile;
  const int64_t waves = (int64_t)n_cu() * 4 * 4;
  const int64_t tpw = std::max<int64_t>(8, std::min<int64_t>(256, (tiles + 8 * waves - 1) / (8 * waves)));
  const int64_t blocks = (tiles + 4 * tpw - 1) / (4 * tpw);
  hipLaunchKernelGGL(logit_mix_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     planes, norms, n, out, out_stride, (int)tpw);
  return (int)hipGetLastError();
}

extern "C" __attribute__((visibility("default"))) int tq_ceiling_logit_mix_blocks(
    const uint32_t* planes, const uint32_t* norms, int64_t n, float* out, int64_t out_stride,
    int per_block, void* stream) {
  if (n < 0 || out_stride < n || per_block < 1) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  if (!planes || !norms || !out) return (int)hipErrorInvalidValue;
  const int64_t blocks = (n + per_block - 1) / per_block;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(logit_mix_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, (const u4v*)planes, norms, n, out, out_stride, per_block);
  return (int)hipGetLastError();
}

extern "C" __attribute__((visibility("default"))) int tq_ceiling_copy(const void* src, void* dst,
                                                                      int64_t bytes,
                                                                      void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  if (bytes == 0) return 0;
  if (!src || !dst) return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, (int64_t)n_cu() * 8);
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u4v*)src, (u4v*)dst, n16);
  return (int)hipGetLastError();
}

extern "C" __attribute__((visibility("default"))) int tq_ceiling_mfma(int kind, int blocks,
                                                                      int iters, float* out,
                                                                      void* stream) {
  if (blocks < 0 || iters < 0 || (kind != 0 && kind != 1)) return (int)hipErrorInvalidValue;
  if (blocks == 0) return 0;
  if (!out) return (int)hipErrorInvalidValue;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_kernel<0>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  else
    hipLaunchKernelGGL(mfma_kernel<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}

extern "C" __attribute__((visibility("default"))) int tq_ceiling_overlap(int mode, int kind,
                                                                         int blocks, int iters,
                                                                         float* out,
                                                                         void* stream) {
  if (blocks < 0 || iters < 0 || mode < 0 || mode > 2 || (kind != 0 && kind != 1))
    return (int)hipErrorInvalidValue;
  if (blocks == 0) return 0;
  if (!out) return (int)hipErrorInvalidValue;
  const hipStream_t st = (hipStream_t)stream;
#define TQ_OV(M, V, K) \
  hipLaunchKernelGGL((overlap_kernel<M, V, K>), dim3(blocks), dim3(512), 0, st, iters, out)
  if (kind == 0) {
    if (mode == 0) TQ_OV(true, false, 0); else if (mode == 1) TQ_OV(false, true, 0); else TQ_OV(true, true, 0);
  } else {
    if (mode == 0) TQ_OV(true, false, 1); else if (mode == 1) TQ_OV(false, true, 1); else TQ_OV(true, true, 1);
  }
#undef TQ_OV
  return (int)hipGetLastError();
}
