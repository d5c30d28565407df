// Drives the host-side code of libtq (tq_host.cpp, built without the kernels
// and with AddressSanitizer and UndefinedBehaviorSanitizer) through its
// set-up calls and its argument validation.  A context is faked on the host
// (no device), so validation runs in full and a call whose arguments pass it
// reaches a launcher stand-in that reports an error.  Exit status 0 when
// every expectation holds; the sanitizers abort on the first finding.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../kv_cache_vector_pi_amd/csrc/tq_internal.h"

static int g_fail = 0;
#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

static void setup_calls() {
  // rotation: orthogonal rows, sketch filled, bad sizes rejected
  for (int d : {3, 5, 64, 128, 200}) {
    std::vector<float> pi((size_t)d * d), s((size_t)d * d, 0.f);
    EXPECT(tq_make_rotation(d, 7, pi.data(), s.data()) == TQ_OK);
    double worst = 0.0;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += (double)pi[(size_t)i * d + k] * pi[(size_t)j * d + k];
        worst = std::fmax(worst, std::fabs(acc - (i == j ? 1.0 : 0.0)));
      }
    EXPECT(worst < 2e-6);
    double ss = 0.0;
    for (float v : s) ss += (double)v * v;
    EXPECT(ss > 0.5 * d * d && ss < 1.5 * d * d);
    EXPECT(tq_make_rotation(d, 7, pi.data(), nullptr) == TQ_OK);   // either output optional
    EXPECT(tq_make_rotation(d, 7, nullptr, s.data()) == TQ_OK);
  }
  float dummy[9];
  EXPECT(tq_make_rotation(2, 0, dummy, dummy) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_make_rotation(-5, 0, dummy, dummy) == TQ_ERR_INVALID_ARG);
  EXPECT(std::strlen(tq_last_error()) > 0);

  // Lloyd-Max: ascending, symmetric, converged; bad arguments rejected
  for (int d : {3, 64, 128, 200, 1536})
    for (int bits = 1; bits <= 4; ++bits) {
      std::vector<float> c((size_t)1 << bits);
      double dist = -1.0;
      int32_t it = 0;
      EXPECT(tq_lloyd_max(d, bits, 100000, 1e-13, c.data(), &dist, &it) == TQ_OK);
      const int K = 1 << bits;
      for (int k = 0; k + 1 < K; ++k) EXPECT(c[k] < c[k + 1]);
      for (int k = 0; k < K; ++k) EXPECT(c[k] == -c[K - 1 - k]);
      EXPECT(dist > 0.0 && dist < 1.0 && it >= 1);
      EXPECT(tq_lloyd_max(d, bits, 100000, 1e-13, c.data(), nullptr, nullptr) == TQ_OK);
    }
  float c8[16];
  EXPECT(tq_lloyd_max(128, 0, 100, 1e-13, c8, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_lloyd_max(128, 5, 100, 1e-13, c8, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_lloyd_max(2, 2, 100, 1e-13, c8, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_lloyd_max(128, 2, 100, 0.0, c8, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_lloyd_max(128, 2, 0, 1e-13, c8, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_lloyd_max(128, 2, 100, 1e-13, nullptr, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_lloyd_max(128, 3, 1, 1e-13, c8, nullptr, nullptr) == TQ_ERR_NOT_CONVERGED);

  for (int st : {0, -1, -2, -3, -4, -5, 99}) EXPECT(tq_status_string(st) != nullptr);
  EXPECT(tq_words_per_plane(200) == 7 && tq_record_words(200, 3) == 21);
  EXPECT(tq_words_per_plane(0) == 0 && tq_record_words(128, 0) == 0);
}

// A context as tq_ctx_create would describe it, without device tables.
static tq_ctx fake_ctx(int d, int b) {
  tq_ctx c;
  std::memset(&c, 0, sizeof(c));
  c.d = d;
  c.b = b;
  c.W = (d + 31) / 32;
  c.Dp = 32 * c.W;
  c.K = 1 << (b - 1);
  c.cp = b - 1;
  c.n_cu = 256;
  return c;
}

static void validation() {
  tq_ctx ctx = fake_ctx(128, 4);
  alignas(64) static float x[4 * 128];
  alignas(64) static uint32_t planes[4 * 16];
  alignas(64) static uint16_t norms[8];
  alignas(64) static unsigned char ws[8192];
  alignas(64) static int64_t starts[2] = {0, 0};
  alignas(64) static int32_t lens[2] = {4, 4};
  alignas(64) static float logits[16 * 8];
  alignas(64) static int64_t oidx[16];
  alignas(64) static float oscore[16];

  // null context everywhere
  EXPECT(tq_quantize_kv(nullptr, x, TQ_F32, 4, 1, 128, 0, planes, norms, 4, 0, nullptr) ==
         TQ_ERR_INVALID_ARG);
  EXPECT(tq_dequantize(nullptr, planes, norms, 4, x, 128, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_search_topk(nullptr, x, 1, planes, norms, 4, 2, oidx, oscore, ws, sizeof(ws),
                        nullptr) == TQ_ERR_INVALID_ARG);

  // quantize: each argument error, then a valid call that reaches the launcher
  EXPECT(tq_quantize_kv(&ctx, x, 7, 4, 1, 128, 0, planes, norms, 4, 0, nullptr) ==
         TQ_ERR_INVALID_ARG);                                     // dtype
  EXPECT(tq_quantize_kv(&ctx, x, TQ_F32, -1, 1, 128, 0, planes, norms, 4, 0, nullptr) ==
         TQ_ERR_INVALID_ARG);                                     // n < 0
  EXPECT(tq_quantize_kv(&ctx, nullptr, TQ_F32, 4, 1, 128, 0, planes, norms, 4, 0, nullptr) ==
         TQ_ERR_INVALID_ARG);                                     // NULL input
  EXPECT(tq_quantize_kv(&ctx, x, TQ_F32, 4, 1, 64, 0, planes, norms, 4, 0, nullptr) ==
         TQ_ERR_INVALID_ARG);                                     // stride < d
  EXPECT(tq_quantize_kv(&ctx, x + 1, TQ_F32, 4, 1, 128, 0, planes, norms, 4, 0, nullptr) ==
         TQ_ERR_INVALID_ARG);                                     // misaligned
  EXPECT(tq_quantize_kv(&ctx, x, TQ_F32, 0, 1, 128, 0, planes, norms, 4, 0, nullptr) ==
         TQ_OK);                                                  // empty: no-op
  EXPECT(tq_quantize_kv(&ctx, x, TQ_F32, 4, 1, 128, 0, planes, norms, 4, 0, nullptr) ==
         TQ_ERR_HIP);                                             // reaches the launcher

  // logits: GQA divisibility, workspace size, then the launcher
  EXPECT(tq_attn_logits(&ctx, x, 1, 4, 512, planes, norms, 3, 4, starts, lens, 4, 1.f, logits,
                        8, ws, sizeof(ws), nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_attn_logits(&ctx, x, 1, 4, 512, planes, norms, 1, 4, starts, lens, 4, 1.f, logits,
                        8, ws, 16, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_attn_logits(&ctx, x, 1, 4, 512, planes, norms, 1, 4, starts, lens, 4, 1.f, logits,
                        8, ws, sizeof(ws), nullptr) == TQ_ERR_HIP);

  // the entry point without a workspace: too much prepared-query data for
  // the static scratch, then (scratch lookup unavailable here) a HIP error
  EXPECT(tq_attn_logits_noalloc(&ctx, x, 2000, 4, 512, planes, norms, 1, 4, starts, lens, 4, 1.f,
                                logits, 8, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(std::strstr(tq_last_error(), "static scratch") != nullptr);
  EXPECT(tq_attn_logits_noalloc(&ctx, x, 1, 4, 512, planes, norms, 3, 4, starts, lens, 4, 1.f,
                                logits, 8, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_attn_logits_noalloc(&ctx, x, 1, 4, 512, planes, norms, 1, 4, starts, lens, 4, 1.f,
                                logits, 8, nullptr) == TQ_ERR_HIP);

  // search: k out of range, too small a workspace, then the launcher
  EXPECT(tq_search_topk(&ctx, x, 1, planes, norms, 4, 0, oidx, oscore, ws, sizeof(ws),
                        nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_search_topk(&ctx, x, 1, planes, norms, 4, 2, oidx, oscore, ws, 8, nullptr) ==
         TQ_ERR_INVALID_ARG);
  EXPECT(tq_search_topk(&ctx, x, 1, planes, norms, 4, 2, oidx, oscore, ws, sizeof(ws),
                        nullptr) == TQ_ERR_HIP);

  // dequantize: stride below d
  EXPECT(tq_dequantize(&ctx, planes, norms, 4, x, 64, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_dequantize(&ctx, planes, norms, 4, x, 128, nullptr) == TQ_ERR_HIP);

  // attention output and fused decode: workspace and GQA checks
  EXPECT(tq_attn_output(&ctx, x, 4, 1, 4, planes, norms, 3, 4, starts, lens, 4, x, 512, ws,
                        sizeof(ws), nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_attn_decode(&ctx, x, 1, 4, 512, planes, norms, planes, norms, 1, 4, starts, lens, 4,
                        1.f, x, 512, ws, 16, nullptr) == TQ_ERR_INVALID_ARG);

  // the error message of the last failure names the entry point
  EXPECT(tq_dequantize(&ctx, planes, norms, -1, x, 128, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(std::strstr(tq_last_error(), "tq_dequantize") != nullptr);
}

int main() {
  setup_calls();
  validation();
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host driver ok\n");
  return 0;
}
