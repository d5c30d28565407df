// Kernel-launcher stand-ins for a host-only build of tq_host.cpp (the
// sanitizer test in tests/test_sanitizers.py).  Every launch reports
// hipErrorNotSupported, so a call whose arguments pass validation returns
// TQ_ERR_HIP; the sizing functions return fixed sizes so that the workspace
// checks can be driven.  Never part of libtq.
#include "../../kv_cache_vector_pi_amd/csrc/tq_internal.h"

namespace tq {

constexpr size_t kStubBytes = 4096;

hipError_t launch_quantize(const tq_ctx*, const void*, int32_t, int64_t, int32_t, int64_t, int64_t,
                           uint32_t*, uint16_t*, int64_t, int64_t, const int64_t*, hipStream_t) {
  return hipErrorNotSupported;
}
bool quantize_big_applies(const tq_ctx* ctx) { return ctx->Dp >= 512; }
size_t quantize_big_workspace_bytes(const tq_ctx* ctx, int64_t n_rows) {
  return ctx->Dp >= 512 ? kStubBytes * (size_t)(n_rows > 0 ? 1 : 0) : 0;
}
hipError_t launch_quantize_big(const tq_ctx*, const void*, int32_t, int64_t, int32_t, int64_t,
                               int64_t, uint32_t*, uint16_t*, int64_t, int64_t, void*, size_t,
                               hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_quantize128(const tq_ctx*, const void*, int32_t, int64_t, int32_t, int64_t,
                              int64_t, uint32_t*, uint16_t*, int64_t, int64_t, const int64_t*,
                              hipStream_t) {
  return hipErrorNotSupported;
}
bool quantize64_pairs_apply(const tq_ctx*, int64_t, int32_t, int64_t, int64_t, int64_t,
                            const int64_t*) {
  return false;
}
hipError_t launch_quantize64_pairs(const tq_ctx*, const void*, int32_t, int64_t, int32_t, int64_t,
                                   int64_t, uint32_t*, uint16_t*, int64_t, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode_step_prepare(const tq_ctx*, const void*, const void*, int32_t, int64_t,
                                      int32_t, int64_t, int64_t, uint32_t*, uint16_t*, uint32_t*,
                                      uint16_t*, int64_t, int64_t, const int64_t*, const float*,
                                      int32_t, int32_t, int64_t, int32_t, void*, hipStream_t) {
  return hipErrorNotSupported;
}
size_t attn_workspace_bytes(const tq_ctx*, int32_t batch, int32_t, int32_t n_kv) {
  return kStubBytes * (size_t)(batch > 0 ? batch : 0) * (size_t)(n_kv > 0 ? n_kv : 0);
}
hipError_t noalloc_scratch(int, void**) { return hipErrorNotSupported; }
hipError_t launch_attn_prepare(const tq_ctx*, const float*, int32_t, int32_t, int64_t, int32_t,
                               void*, bool, hipStream_t) {
  return hipErrorNotSupported;
}
bool logits_fold(const tq_ctx*, int32_t, int32_t) { return false; }
// the one-launch logit path is never taken here, so the two-launch path's
// validation and launches are what the driver reaches
bool attn_one_applies(const tq_ctx*, int32_t, int32_t) { return false; }
hipError_t launch_attn_one(const tq_ctx*, const float*, int32_t, int32_t, int64_t,
                           const uint32_t*, const uint16_t*, int32_t, int64_t, const int64_t*,
                           const int32_t*, int32_t, float, float*, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_attn_stream(const tq_ctx*, const void*, int32_t, int32_t, const uint32_t*,
                              const uint16_t*, int32_t, int64_t, const int64_t*, const int32_t*,
                              int32_t, float, float*, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
size_t search_workspace_bytes(const tq_ctx*, int64_t, int64_t, int32_t) { return kStubBytes; }
hipError_t launch_search_topk(const tq_ctx*, const float*, int64_t, const uint32_t*,
                              const uint16_t*, int64_t, int32_t, int64_t*, float*, void*,
                              hipStream_t) {
  return hipErrorNotSupported;
}
size_t vout_workspace_bytes(const tq_ctx*, int32_t, int32_t, int32_t, int32_t) {
  return kStubBytes;
}
hipError_t launch_attn_output(const tq_ctx*, const float*, int64_t, int32_t, int32_t,
                              const uint32_t*, const uint16_t*, int32_t, int64_t, const int64_t*,
                              const int32_t*, int32_t, float*, int64_t, int64_t, void*,
                              hipStream_t) {
  return hipErrorNotSupported;
}
size_t split_attn_workspace_bytes(const tq_ctx*, const tq_ctx*, int32_t, int32_t, int32_t) {
  return kStubBytes;
}
bool split_logits_supported(const tq_ctx*, const tq_ctx*, int32_t, int32_t) { return true; }
hipError_t launch_split_prepare(const tq_ctx*, const tq_ctx*, const float*, int32_t, int32_t,
                                int64_t, int32_t, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_split_stream(const tq_ctx*, const tq_ctx*, const void*, int32_t, int32_t,
                               const uint32_t*, const uint16_t*, const uint32_t*,
                               const uint16_t*, int32_t, int64_t, const int64_t*, const int32_t*,
                               int32_t, float, float*, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
size_t decode_workspace_bytes(const tq_ctx*, int32_t, int32_t, int32_t, int32_t) {
  return kStubBytes;
}
hipError_t launch_attn_decode(const tq_ctx*, const float*, int32_t, int32_t, int64_t,
                              const uint32_t*, const uint16_t*, const uint32_t*, const uint16_t*,
                              int32_t, int64_t, const int64_t*, const int32_t*, int32_t, float,
                              float*, int64_t, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_dequantize(const tq_ctx*, const uint32_t*, const uint16_t*, int64_t, float*,
                             int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace tq
