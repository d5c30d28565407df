// Host side of libtq: status/error reporting, the offline set-up (seeded
// rotation and sketch, Lloyd-Max codebook), the device context, and argument
// validation in front of every kernel launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace {

thread_local char g_last_error[512] = "";

tq_status fail(tq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

tq_status ok() {
  g_last_error[0] = '\0';
  return TQ_OK;
}

tq_status hip_fail(hipError_t e, const char* what) {
  return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// bf16 bits of a finite float, rounded to nearest even, and back
uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float bf16_value(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// ---------------------------------------------------------------------------
// Seeded Gaussians.  SplitMix64 (Steele, Lea & Flood 2014) used as a
// counter-based generator: output i of state s is mix(s + (i+1)*golden).
// The key of (seed, stream) is output `stream` of state `seed`; value i of a
// stream is output i of state key.  Box-Muller turns uniforms 2j, 2j+1
// (each (top 53 bits + 1) * 2^-53, so in (0, 1]) into r*cos, r*sin.
constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

inline uint64_t splitmix_out(uint64_t state, uint64_t i) {
  uint64_t z = state + (i + 1) * kGolden;
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

void gaussians(uint64_t seed, uint64_t stream, std::vector<double>& out) {
  const uint64_t key = splitmix_out(seed, stream);
  const double two_pi = 6.283185307179586476925286766559;
  const double inv53 = 1.0 / 9007199254740992.0;
  const size_t n = out.size();
  for (size_t j = 0; 2 * j < n; ++j) {
    const double u1 = double((splitmix_out(key, 2 * j) >> 11) + 1) * inv53;
    const double u2 = double((splitmix_out(key, 2 * j + 1) >> 11) + 1) * inv53;
    const double rad = std::sqrt(-2.0 * std::log(u1));
    const double ang = two_pi * u2;
    out[2 * j] = rad * std::cos(ang);
    if (2 * j + 1 < n) out[2 * j + 1] = rad * std::sin(ang);
  }
}

// QR by classical Gram-Schmidt with one re-orthogonalisation pass (CGS2), in
// double, on the columns of G.  It yields the unique Q with diag(R) > 0, i.e.
// the sign-fixed (Haar) rotation.  g is row-major d x d; q receives Q
// row-major.
void qr_positive(int d, const std::vector<double>& g, std::vector<double>& q) {
  std::vector<double> cols((size_t)d * d);      // column-major copy, Q built in place
  for (int r = 0; r < d; ++r)
    for (int c = 0; c < d; ++c) cols[(size_t)c * d + r] = g[(size_t)r * d + c];
  std::vector<double> h(d);
  for (int j = 0; j < d; ++j) {
    double* v = &cols[(size_t)j * d];
    for (int pass = 0; pass < 2; ++pass) {
      for (int i = 0; i < j; ++i) {
        const double* qi = &cols[(size_t)i * d];
        double s = 0.0;
        for (int r = 0; r < d; ++r) s += qi[r] * v[r];
        h[i] = s;
      }
      for (int i = 0; i < j; ++i) {
        const double* qi = &cols[(size_t)i * d];
        const double s = h[i];
        for (int r = 0; r < d; ++r) v[r] -= s * qi[r];
      }
    }
    double nrm = 0.0;
    for (int r = 0; r < d; ++r) nrm += v[r] * v[r];
    nrm = std::sqrt(nrm);
    for (int r = 0; r < d; ++r) v[r] /= nrm;
  }
  q.assign((size_t)d * d, 0.0);
  for (int c = 0; c < d; ++c)
    for (int r = 0; r < d; ++r) q[(size_t)r * d + c] = cols[(size_t)c * d + r];
}

// ---------------------------------------------------------------------------
// Coordinate law of a uniform point on S^{d-1}: X = 2B - 1 with
// B ~ Beta(a, a), a = (d-1)/2, whose density is the f_d of the PolarQuant
// section.  P(X <= x) = I_{(1+x)/2}(a, a): regularised incomplete beta from
// its continued fraction (modified Lentz), with the reflection
// I_z(a, b) = 1 - I_{1-z}(b, a) where the fraction converges slowly.
double betacf(double a, double b, double z) {
  const double tiny = 1e-300, eps = 1e-16;
  double c = 1.0, dd = 1.0 - (a + b) * z / (a + 1.0);
  if (std::fabs(dd) < tiny) dd = tiny;
  dd = 1.0 / dd;
  double f = dd;
  for (int m = 1; m < 100000; ++m) {
    const double m2 = 2.0 * m;
    double num = m * (b - m) * z / ((a + m2 - 1.0) * (a + m2));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    f *= dd * c;
    num = -(a + m) * (a + b + m) * z / ((a + m2) * (a + m2 + 1.0));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    const double del = dd * c;
    f *= del;
    if (std::fabs(del - 1.0) < eps) break;
  }
  return f;
}

double inc_beta(double a, double b, double z) {
  if (z <= 0.0) return 0.0;
  if (z >= 1.0) return 1.0;
  const double lfront = a * std::log(z) + b * std::log1p(-z) -
                        (std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b));
  if (z < (a + 1.0) / (a + b + 2.0)) return std::exp(lfront) * betacf(a, b, z) / a;
  return 1.0 - std::exp(lfront) * betacf(b, a, 1.0 - z) / b;
}

// P(lo < X <= hi) and E[X; lo < X <= hi] for the coordinate law.  The first
// moment has a closed form: d/dx (1-x^2)^((d-1)/2) = -(d-1) x (1-x^2)^((d-3)/2).
struct CoordLaw {
  int d;
  double a, log_cd;
  explicit CoordLaw(int dim) : d(dim), a(0.5 * (dim - 1)) {
    log_cd = std::lgamma(0.5 * dim) - 0.5 * std::log(M_PI) - std::lgamma(0.5 * (dim - 1));
  }
  double cdf(double x) const {
    if (x <= -1.0) return 0.0;
    if (x >= 1.0) return 1.0;
    if (x <= 0.0) return inc_beta(a, a, 0.5 * (1.0 + x));
    return 1.0 - inc_beta(a, a, 0.5 * (1.0 - x));
  }
  // C_d (1 - x^2)^((d-1)/2) / (d-1)
  double g(double x) const {
    if (x <= -1.0 || x >= 1.0) return 0.0;
    return std::exp(log_cd + 0.5 * (d - 1) * (std::log1p(-x) + std::log1p(x)) -
                    std::log(double(d - 1)));
  }
  double mass(double lo, double hi) const { return cdf(hi) - cdf(lo); }
  double moment1(double lo, double hi) const { return g(lo) - g(hi); }
};

}  // namespace

// ===========================================================================
extern "C" {

TQ_API const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_NOT_CONVERGED: return "TQ_ERR_NOT_CONVERGED";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
    case TQ_ERR_ALLOC: return "TQ_ERR_ALLOC";
    default: return "TQ_ERR_UNKNOWN";
  }
}

TQ_API const char* tq_last_error(void) { return g_last_error; }

TQ_API int32_t tq_words_per_plane(int32_t d) { return d < 1 ? 0 : (d + 31) / 32; }

TQ_API int32_t tq_record_words(int32_t d, int32_t b) {
  return (d < 1 || b < 1) ? 0 : tq_words_per_plane(d) * b;
}

TQ_API tq_status tq_make_rotation(int32_t d, uint64_t seed, float* pi, float* s) {
  if (d < 3 || d > TQ_MAX_D) return fail(TQ_ERR_INVALID_ARG, "tq_make_rotation: d=%d", d);
  const size_t dd = (size_t)d * d;
  if (pi) {
    std::vector<double> g(dd), q;
    gaussians(seed, 0, g);
    qr_positive(d, g, q);
    for (size_t i = 0; i < dd; ++i) pi[i] = (float)q[i];
  }
  if (s) {
    std::vector<double> g(dd);
    gaussians(seed, 1, g);
    for (size_t i = 0; i < dd; ++i) s[i] = (float)g[i];
  }
  return ok();
}

TQ_API tq_status tq_lloyd_max(int32_t d, int32_t lm_bits, int32_t max_iter, double tol,
                              float* centroids, double* distortion_out, int32_t* iters_out) {
  if (d < 3 || d > TQ_MAX_D || lm_bits < 1 || lm_bits > 4 || max_iter < 1 || !(tol > 0.0) ||
      !centroids)
    return fail(TQ_ERR_INVALID_ARG, "tq_lloyd_max: d=%d lm_bits=%d max_iter=%d tol=%g", d,
                lm_bits, max_iter, tol);
  const int K = 1 << lm_bits;
  const CoordLaw law(d);
  // start from an even spread over +-2.5 standard deviations (1/sqrt(d))
  std::vector<double> c(K), t(K + 1);
  const double spread = std::min(1.0, d == 3 ? 1.0 : 2.5 / std::sqrt((double)d));
  for (int k = 0; k < K; ++k) c[k] = spread * (-1.0 + (2.0 * k + 1.0) / K);
  int it = 0;
  bool converged = false;
  for (it = 1; it <= max_iter; ++it) {
    t[0] = -1.0;
    t[K] = 1.0;
    for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    // positive half only; the negative half mirrors it exactly
    double delta = 0.0;
    for (int k = K / 2; k < K; ++k) {
      const double m0 = law.mass(t[k], t[k + 1]);
      const double nc = m0 > 0.0 ? law.moment1(t[k], t[k + 1]) / m0 : c[k];
      delta = std::max(delta, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    for (int k = 0; k < K / 2; ++k) c[k] = -c[K - 1 - k];
    if (delta < tol) {
      converged = true;
      break;
    }
  }
  if (it > max_iter) it = max_iter;
  for (int k = 0; k < K; ++k) centroids[k] = (float)c[k];
  if (distortion_out) {
    // D = d * E[(X - c(X))^2] = 1 - d * sum_k c_k^2 P_k   (E[X^2] = 1/d,
    // and each c_k is the mean of its cell)
    t[0] = -1.0;
    t[K] = 1.0;
    for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += c[k] * c[k] * law.mass(t[k], t[k + 1]);
    *distortion_out = 1.0 - d * acc;
  }
  if (iters_out) *iters_out = it;
  if (!converged)
    return fail(TQ_ERR_NOT_CONVERGED, "tq_lloyd_max: no convergence in %d iterations", max_iter);
  return ok();
}

// ---------------------------------------------------------------------------
namespace {

// Shared by tq_ctx_create (two-stage records: b-1 code planes + QJL signs)
// and tq_ctx_create_mse (b code planes, no QJL stage; s == NULL).
tq_status create_ctx(int32_t d, int32_t b, const float* pi, const float* s,
                     const float* centroids, bool mse, tq_ctx** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_ctx_create: out is NULL");
  *out = nullptr;
  if (d < 8 || d > TQ_MAX_D || d % 8 != 0)
    return fail(TQ_ERR_UNSUPPORTED, "tq_ctx_create: d=%d (need a multiple of 8 in 8..%d)", d,
                TQ_MAX_D);
  if (!mse && (b < 2 || b > 4)) return fail(TQ_ERR_UNSUPPORTED, "tq_ctx_create: b=%d (need 2..4)", b);
  if (mse && (b < 1 || b > 3))
    return fail(TQ_ERR_UNSUPPORTED, "tq_ctx_create_mse: b=%d (need 1..3)", b);
  if (!pi || (!mse && !s) || !centroids)
    return fail(TQ_ERR_INVALID_ARG, "tq_ctx_create: NULL table");
  const int CP = mse ? b : b - 1;
  const int K = 1 << CP;
  for (int k = 0; k < K; ++k) {
    if (!std::isfinite(centroids[k]))
      return fail(TQ_ERR_INVALID_ARG, "tq_ctx_create: centroid %d not finite", k);
    if (k > 0 && !(centroids[k] > centroids[k - 1]))
      return fail(TQ_ERR_INVALID_ARG, "tq_ctx_create: centroids not strictly ascending");
    if (centroids[k] != -centroids[K - 1 - k])
      return fail(TQ_ERR_INVALID_ARG, "tq_ctx_create: centroids not symmetric");
  }
  const size_t dd = (size_t)d * d;
  std::vector<float> zeros;
  if (mse) {              // no sketch: S (and M = S Pi^T) are zero tables
    zeros.assign(dd, 0.f);
    s = zeros.data();
  }
  for (size_t i = 0; i < dd; ++i)
    if (!std::isfinite(pi[i]) || !std::isfinite(s[i]))
      return fail(TQ_ERR_INVALID_ARG, "tq_ctx_create: non-finite Pi or S entry");

  tq_ctx* ctx = new tq_ctx();
  ctx->d = d;
  ctx->b = b;
  ctx->mse = mse ? 1 : 0;
  ctx->cp = CP;
  ctx->W = (d + 31) / 32;
  ctx->Dp = 32 * ctx->W;
  ctx->K = K;
  for (int k = 0; k < tq::kMaxK; ++k) {
    ctx->cent[k] = k < K ? centroids[k] : 0.f;
    ctx->mid[k] = k + 1 < K ? 0.5f * (centroids[k] + centroids[k + 1]) : 0.f;
  }
  // Walsh expansion over the B code bits: chi_m(beta) = (-1)^(XOR of the
  // bits in m) = 1 - 2 u_m.  c(beta) = sum_m w_m chi_m(beta) with
  // w_m = mean over beta of c(beta) chi_m(beta); a symmetric codebook has
  // w_m = 0 for every even-sized m, and c(beta) = c(0) - 2 sum_{m != 0} w_m u_m.
  {
    const int B = CP;
    ctx->n_mono = 0;
    ctx->c0 = centroids[0];
    for (int m = 1; m < (1 << B); ++m) {
      if (__builtin_popcount(m) % 2 == 0) continue;
      double w = 0.0;
      for (int beta = 0; beta < (1 << B); ++beta) {
        const int par = __builtin_popcount(beta & m) & 1;
        w += (par ? -1.0 : 1.0) * (double)centroids[beta];
      }
      w /= (double)(1 << B);
      ctx->mono_mask[ctx->n_mono] = m;
      ctx->mono_w[ctx->n_mono] = w;
      ctx->n_mono++;
    }
  }
  hipError_t e = hipGetDevice(&ctx->device);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&ctx->n_cu, hipDeviceAttributeMultiprocessorCount, ctx->device);
  if (e != hipSuccess) {
    delete ctx;
    return hip_fail(e, "tq_ctx_create: device query");
  }
  if (ctx->n_cu < 1) ctx->n_cu = 1;
  // the static scratch of tq_attn_logits_noalloc: its address on this device
  e = tq::noalloc_scratch(ctx->device, nullptr);
  if (e != hipSuccess) {
    delete ctx;
    return hip_fail(e, "tq_ctx_create: scratch symbol");
  }
  const int Dp = ctx->Dp;
  const int Rp = (Dp + 63) / 64 * 64;
  const size_t dpp = (size_t)Dp * Dp;
  const size_t rpp = (size_t)Rp * Dp;
  // host staging (fp16, zero padded): pi_hi, pi_lo, m_hi, m_lo [Dp][Dp], then
  // Pi^T hi/lo and S^T hi/lo [Rp][Dp]; then fp32 Pi and S [d][d]
  std::vector<__half> h16(4 * dpp + 4 * rpp, __float2half(0.f));
  {
    std::vector<double> M(dd, 0.0);   // M = S Pi^T in double
    for (int i = 0; i < (mse ? 0 : d); ++i)
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += (double)s[(size_t)i * d + k] * (double)pi[(size_t)j * d + k];
        M[(size_t)i * d + j] = acc;
      }
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        const float p = pi[(size_t)i * d + j];
        const __half ph = __float2half(p);
        const __half pl = __float2half(p - __half2float(ph));
        const float mf = (float)M[(size_t)i * d + j];
        const __half mh = __float2half(mf);
        const __half ml = __float2half(mf - __half2float(mh));
        h16[0 * dpp + (size_t)i * Dp + j] = ph;
        h16[1 * dpp + (size_t)i * Dp + j] = pl;
        h16[2 * dpp + (size_t)i * Dp + j] = mh;
        h16[3 * dpp + (size_t)i * Dp + j] = ml;
        // transposes: row j of Pi^T is column j of Pi
        const float sv = s[(size_t)i * d + j];
        const __half sh = __float2half(sv);
        const __half sl = __float2half(sv - __half2float(sh));
        h16[4 * dpp + 0 * rpp + (size_t)j * Dp + i] = ph;
        h16[4 * dpp + 1 * rpp + (size_t)j * Dp + i] = pl;
        h16[4 * dpp + 2 * rpp + (size_t)j * Dp + i] = sh;
        h16[4 * dpp + 3 * rpp + (size_t)j * Dp + i] = sl;
      }
  }
  // bf16 hi and mid parts of Pi (the raw-bf16 products of the d = 128
  // quantizer): hi = bf16(Pi), mid = bf16(Pi - hi), both rounded to nearest
  // even; Pi - hi is exact in fp32
  std::vector<uint16_t> b16(2 * dpp, 0);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      const float p = pi[(size_t)i * d + j];
      const uint16_t hb = bf16_rne(p);
      const float hv = bf16_value(hb);
      b16[(size_t)i * Dp + j] = hb;
      b16[dpp + (size_t)i * Dp + j] = bf16_rne(p - hv);
    }
  const size_t bytes16 = (4 * dpp + 4 * rpp) * sizeof(__half);
  const size_t bytes32 = 4 * dd * sizeof(float);
  const size_t bytesb = 2 * dpp * sizeof(uint16_t);
  void* blk = nullptr;
  e = hipMalloc(&blk, bytes16 + bytes32 + bytesb);
  if (e != hipSuccess) {
    delete ctx;
    return fail(TQ_ERR_ALLOC, "tq_ctx_create: hipMalloc(%zu): %s", bytes16 + bytes32 + bytesb,
                hipGetErrorString(e));
  }
  char* p = (char*)blk;
  // fp32 tables: Pi^T and S^T for the query projections (one thread per
  // output row reads a contiguous column), Pi and S row-major for the
  // value-output transforms (one thread per output column)
  std::vector<float> t32(4 * dd);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      t32[(size_t)j * d + i] = pi[(size_t)i * d + j];
      t32[dd + (size_t)j * d + i] = s[(size_t)i * d + j];
      t32[2 * dd + (size_t)i * d + j] = pi[(size_t)i * d + j];
      t32[3 * dd + (size_t)i * d + j] = s[(size_t)i * d + j];
    }
  e = hipMemcpy(p, h16.data(), bytes16, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(p + bytes16, t32.data(), 4 * dd * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(p + bytes16 + bytes32, b16.data(), bytesb, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(blk);
    delete ctx;
    return hip_fail(e, "tq_ctx_create: hipMemcpy");
  }
  ctx->dev_block = blk;
  const __half* h = (const __half*)p;
  ctx->t.pi_hi = h;
  ctx->t.pi_lo = h + dpp;
  ctx->t.m_hi = h + 2 * dpp;
  ctx->t.m_lo = h + 3 * dpp;
  ctx->t.pit_hi = h + 4 * dpp;
  ctx->t.pit_lo = h + 4 * dpp + rpp;
  ctx->t.st_hi = h + 4 * dpp + 2 * rpp;
  ctx->t.st_lo = h + 4 * dpp + 3 * rpp;
  ctx->t.pit32 = (const float*)(p + bytes16);
  ctx->t.st32 = (const float*)(p + bytes16) + dd;
  ctx->t.pi32 = (const float*)(p + bytes16) + 2 * dd;
  ctx->t.s32 = (const float*)(p + bytes16) + 3 * dd;
  ctx->t.pib_hi = (const uint16_t*)(p + bytes16 + bytes32);
  ctx->t.pib_mid = ctx->t.pib_hi + dpp;
  *out = ctx;
  return ok();
}

}  // namespace

TQ_API tq_status tq_ctx_create(int32_t d, int32_t b, const float* pi, const float* s,
                               const float* centroids, tq_ctx** out) {
  return create_ctx(d, b, pi, s, centroids, false, out);
}

TQ_API tq_status tq_ctx_create_mse(int32_t d, int32_t b, const float* pi, const float* centroids,
                                   tq_ctx** out) {
  return create_ctx(d, b, pi, nullptr, centroids, true, out);
}

TQ_API int32_t tq_ctx_is_mse(const tq_ctx* ctx) { return ctx ? ctx->mse : 0; }

TQ_API tq_status tq_ctx_destroy(tq_ctx* ctx) {
  if (!ctx) return ok();
  hipError_t e = hipDeviceSynchronize();
  hipError_t e2 = hipFree(ctx->dev_block);
  delete ctx;
  if (e != hipSuccess) return hip_fail(e, "tq_ctx_destroy: hipDeviceSynchronize");
  if (e2 != hipSuccess) return hip_fail(e2, "tq_ctx_destroy: hipFree");
  return ok();
}

TQ_API int32_t tq_ctx_dim(const tq_ctx* ctx) { return ctx ? ctx->d : 0; }
TQ_API int32_t tq_ctx_bits(const tq_ctx* ctx) { return ctx ? ctx->b : 0; }

// ---------------------------------------------------------------------------
static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

namespace {

// Argument checks of one quantize job (fn names the entry point in messages);
// *empty is set for a no-op job.  With slots (per-token destinations) the
// records of a head are addressed by slot alone: dst_token0 must be 0 and
// dst_stride_head, the slot range, at least 1.
tq_status check_quantize(const char* fn, const tq_ctx* ctx, const void* x, int32_t x_dtype,
                         int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                         int64_t x_stride_head, const uint32_t* planes, const uint16_t* norms,
                         int64_t dst_stride_head, int64_t dst_token0, const int64_t* slots,
                         bool* empty) {
  *empty = false;
  if (n_tokens < 0 || n_heads < 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: n_tokens=%lld n_heads=%d", fn, (long long)n_tokens,
                n_heads);
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16)
    return fail(TQ_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, x_dtype);
  if (n_tokens == 0 || n_heads == 0) {
    *empty = true;
    return TQ_OK;
  }
  if (!x || !planes || !norms) return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (x_stride_token < ctx->d || (n_heads > 1 && x_stride_head < 0) || dst_stride_head < 0 ||
      dst_token0 < 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: bad strides", fn);
  if (slots && (dst_token0 != 0 || dst_stride_head < 1 || !aligned(slots, 8)))
    return fail(TQ_ERR_INVALID_ARG,
                "%s: with slots, dst_token0 must be 0, dst_stride_head >= 1 and slots 8-byte "
                "aligned", fn);
  const size_t esz = x_dtype == TQ_F32 ? 4 : 2;
  if (!aligned(planes, 16) || !aligned(norms, 4) || !aligned(x, 16) ||
      (x_stride_token * esz) % 16 != 0 || (x_stride_head * esz) % 16 != 0)
    return fail(TQ_ERR_INVALID_ARG,
                "%s: planes, x and x strides must be 16-byte aligned, norms 4-byte", fn);
  return TQ_OK;
}

// Argument checks of one query preparation; *empty is set for batch == 0.
tq_status check_prepare(const char* fn, const tq_ctx* ctx, const float* q, int32_t batch,
                        int32_t n_q_heads, int64_t q_stride_batch, int32_t n_kv_heads,
                        const void* workspace, size_t workspace_bytes, bool* empty) {
  *empty = false;
  if (batch < 0 || n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: batch=%d n_q=%d n_kv=%d", fn, batch, n_q_heads,
                n_kv_heads);
  if (batch == 0) {
    *empty = true;
    return TQ_OK;
  }
  if (!q || !workspace) return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (q_stride_batch < (int64_t)n_q_heads * ctx->d && batch > 1)
    return fail(TQ_ERR_INVALID_ARG, "%s: q_stride_batch too small", fn);
  if (!aligned(workspace, 16) || !aligned(q, 4))
    return fail(TQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  const size_t need = tq::attn_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads);
  if (workspace_bytes < need)
    return fail(TQ_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  return TQ_OK;
}

}  // namespace

TQ_API tq_status tq_quantize_kv(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                                int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                                int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                                int64_t dst_stride_head, int64_t dst_token0, void* stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "tq_quantize_kv: ctx is NULL");
  bool empty;
  const tq_status st = check_quantize("tq_quantize_kv", ctx, x, x_dtype, n_tokens, n_heads,
                                      x_stride_token, x_stride_head, planes, norms,
                                      dst_stride_head, dst_token0, nullptr, &empty);
  if (st != TQ_OK) return st;
  if (empty) return ok();
  hipError_t e = tq::launch_quantize(ctx, x, x_dtype, n_tokens, n_heads, x_stride_token,
                                     x_stride_head, planes, norms, dst_stride_head, dst_token0,
                                     nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_quantize_kv: launch");
  return ok();
}

TQ_API size_t tq_quantize_workspace_bytes(const tq_ctx* ctx, int64_t n_rows) {
  if (!ctx || n_rows < 0) return 0;
  return tq::quantize_big_workspace_bytes(ctx, n_rows);
}

TQ_API tq_status tq_quantize_kv_ws(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                                   int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                                   int64_t x_stride_head, uint32_t* planes, uint16_t* norms,
                                   int64_t dst_stride_head, int64_t dst_token0, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const char* fn = "tq_quantize_kv_ws";
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
  bool empty;
  const tq_status st = check_quantize(fn, ctx, x, x_dtype, n_tokens, n_heads, x_stride_token,
                                      x_stride_head, planes, norms, dst_stride_head, dst_token0,
                                      nullptr, &empty);
  if (st != TQ_OK) return st;
  if (empty) return ok();
  hipError_t e;
  if (tq::quantize_big_applies(ctx)) {
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < tq::quantize_big_workspace_bytes(ctx, 1))
      return fail(TQ_ERR_INVALID_ARG,
                  "%s: workspace must be 256-byte aligned and hold at least %zu bytes", fn,
                  tq::quantize_big_workspace_bytes(ctx, 1));
    e = tq::launch_quantize_big(ctx, x, x_dtype, n_tokens, n_heads, x_stride_token,
                                x_stride_head, planes, norms, dst_stride_head, dst_token0,
                                workspace, workspace_bytes, (hipStream_t)stream);
  } else {
    e = tq::launch_quantize(ctx, x, x_dtype, n_tokens, n_heads, x_stride_token, x_stride_head,
                            planes, norms, dst_stride_head, dst_token0, nullptr,
                            (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "tq_quantize_kv_ws: launch");
  return ok();
}

TQ_API tq_status tq_quantize_kv_slots(const tq_ctx* ctx, const void* x, int32_t x_dtype,
                                      int64_t n_tokens, int32_t n_heads, int64_t x_stride_token,
                                      int64_t x_stride_head, const int64_t* slots,
                                      uint32_t* planes, uint16_t* norms,
                                      int64_t dst_stride_head, void* stream) {
  const char* fn = "tq_quantize_kv_slots";
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
  if (!slots && n_tokens > 0 && n_heads > 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: slots is NULL", fn);
  bool empty;
  const tq_status st = check_quantize(fn, ctx, x, x_dtype, n_tokens, n_heads, x_stride_token,
                                      x_stride_head, planes, norms, dst_stride_head, 0, slots,
                                      &empty);
  if (st != TQ_OK) return st;
  if (empty) return ok();
  hipError_t e = tq::launch_quantize(ctx, x, x_dtype, n_tokens, n_heads, x_stride_token,
                                     x_stride_head, planes, norms, dst_stride_head, 0, slots,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_quantize_kv_slots: launch");
  return ok();
}

TQ_API tq_status tq_decode_step_prepare(const tq_ctx* ctx, const void* k_new, const void* v_new,
                                        int32_t x_dtype, int64_t n_tokens, int32_t n_heads,
                                        int64_t x_stride_token, int64_t x_stride_head,
                                        uint32_t* k_planes, uint16_t* k_norms,
                                        uint32_t* v_planes, uint16_t* v_norms,
                                        int64_t dst_stride_head, int64_t dst_token0,
                                        const int64_t* dst_slots,
                                        const float* q, int32_t batch, int32_t n_q_heads,
                                        int64_t q_stride_batch, int32_t n_kv_heads,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tq_decode_step_prepare";
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
  bool no_k, no_v, no_q;
  tq_status st = check_quantize(fn, ctx, k_new, x_dtype, n_tokens, n_heads, x_stride_token,
                                x_stride_head, k_planes, k_norms, dst_stride_head, dst_token0,
                                dst_slots, &no_k);
  if (st == TQ_OK)
    st = check_quantize(fn, ctx, v_new, x_dtype, n_tokens, n_heads, x_stride_token,
                        x_stride_head, v_planes, v_norms, dst_stride_head, dst_token0,
                        dst_slots, &no_v);
  if (st == TQ_OK)
    st = check_prepare(fn, ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads, workspace,
                       workspace_bytes, &no_q);
  if (st != TQ_OK) return st;
  if (no_k && no_q) return ok();
  hipError_t e = tq::launch_decode_step_prepare(
      ctx, k_new, v_new, x_dtype, no_k ? 0 : n_tokens, no_k ? 0 : n_heads, x_stride_token,
      x_stride_head, k_planes, k_norms, v_planes, v_norms, dst_stride_head, dst_token0,
      dst_slots, q,
      no_q ? 0 : batch, n_q_heads, q_stride_batch, n_kv_heads, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_decode_step_prepare: launch");
  return ok();
}

TQ_API tq_status tq_dequantize(const tq_ctx* ctx, const uint32_t* planes, const uint16_t* norms,
                               int64_t n, float* out, int64_t out_ld, void* stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "tq_dequantize: ctx is NULL");
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "tq_dequantize: n=%lld", (long long)n);
  if (n == 0) return ok();
  if (!planes || !norms || !out) return fail(TQ_ERR_INVALID_ARG, "tq_dequantize: NULL pointer");
  if (out_ld < ctx->d) return fail(TQ_ERR_INVALID_ARG, "tq_dequantize: out_ld < d");
  if (!aligned(planes, 16) || !aligned(norms, 4) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "tq_dequantize: misaligned pointer");
  hipError_t e = tq::launch_dequantize(ctx, planes, norms, n, out, out_ld, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_dequantize: launch");
  return ok();
}

TQ_API size_t tq_attn_logits_workspace_bytes(const tq_ctx* ctx, int32_t batch, int32_t n_q_heads,
                                             int32_t n_kv_heads) {
  if (!ctx || batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads) return 0;
  return tq::attn_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads);
}

TQ_API tq_status tq_attn_logits(const tq_ctx* ctx, const float* q, int32_t batch,
                                int32_t n_q_heads, int64_t q_stride_batch,
                                const uint32_t* planes, const uint16_t* norms,
                                int32_t n_kv_heads, int64_t keys_stride_head,
                                const int64_t* seq_start, const int32_t* seq_len,
                                int32_t max_seq_len, float scale, float* logits,
                                int64_t logits_stride_head, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits: ctx is NULL");
  if (batch < 0 || max_seq_len < 0 || n_kv_heads < 1 || n_q_heads < 1 ||
      n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits: batch=%d n_q=%d n_kv=%d max_seq_len=%d",
                batch, n_q_heads, n_kv_heads, max_seq_len);
  if (batch == 0 || max_seq_len == 0) return ok();
  if (!q || !planes || !norms || !seq_start || !seq_len || !logits || !workspace)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits: NULL pointer");
  if (q_stride_batch < (int64_t)n_q_heads * ctx->d && batch > 1)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits: q_stride_batch too small");
  if (keys_stride_head < 0 || logits_stride_head < 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits: negative stride");
  if (!aligned(planes, 16) || !aligned(norms, 4) || !aligned(workspace, 16) || !aligned(q, 4))
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits: misaligned pointer");
  const size_t need = tq::attn_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads);
  if (workspace_bytes < need)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits: workspace %zu < %zu bytes", workspace_bytes,
                need);
  if (!std::isfinite(scale)) return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits: scale not finite");
  // one launch where the resident stream applies (the workspace stays unused)
  hipError_t e;
  if (tq::attn_one_applies(ctx, n_q_heads, n_kv_heads)) {
    e = tq::launch_attn_one(ctx, q, batch, n_q_heads, q_stride_batch, planes, norms, n_kv_heads,
                            keys_stride_head, seq_start, seq_len, max_seq_len, scale, logits,
                            logits_stride_head, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "tq_attn_logits: launch");
    return ok();
  }
  e = tq::launch_attn_prepare(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads, workspace,
                              tq::logits_fold(ctx, n_q_heads, n_kv_heads), (hipStream_t)stream);
  if (e == hipSuccess)
    e = tq::launch_attn_stream(ctx, workspace, batch, n_q_heads, planes, norms, n_kv_heads,
                               keys_stride_head, seq_start, seq_len, max_seq_len, scale, logits,
                               logits_stride_head, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_attn_logits: launch");
  return ok();
}

TQ_API tq_status tq_attn_logits_noalloc(const tq_ctx* ctx, const float* q, int32_t batch,
                                        int32_t n_q_heads, int64_t q_stride_batch,
                                        const uint32_t* planes, const uint16_t* norms,
                                        int32_t n_kv_heads, int64_t keys_stride_head,
                                        const int64_t* seq_start, const int32_t* seq_len,
                                        int32_t max_seq_len, float scale, float* logits,
                                        int64_t logits_stride_head, void* stream) {
  static const char* fn = "tq_attn_logits_noalloc";
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
  if (batch < 0 || max_seq_len < 0 || n_kv_heads < 1 || n_q_heads < 1 ||
      n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: batch=%d n_q=%d n_kv=%d max_seq_len=%d", fn, batch,
                n_q_heads, n_kv_heads, max_seq_len);
  if (batch == 0 || max_seq_len == 0) return ok();
  if (!q || !planes || !norms || !seq_start || !seq_len || !logits)
    return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (q_stride_batch < (int64_t)n_q_heads * ctx->d && batch > 1)
    return fail(TQ_ERR_INVALID_ARG, "%s: q_stride_batch too small", fn);
  if (keys_stride_head < 0 || logits_stride_head < 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: negative stride", fn);
  if (!aligned(planes, 16) || !aligned(norms, 4) || !aligned(q, 4))
    return fail(TQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (!std::isfinite(scale)) return fail(TQ_ERR_INVALID_ARG, "%s: scale not finite", fn);
  // one launch where the resident stream applies: no scratch at all
  hipError_t e;
  if (tq::attn_one_applies(ctx, n_q_heads, n_kv_heads)) {
    e = tq::launch_attn_one(ctx, q, batch, n_q_heads, q_stride_batch, planes, norms, n_kv_heads,
                            keys_stride_head, seq_start, seq_len, max_seq_len, scale, logits,
                            logits_stride_head, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "tq_attn_logits_noalloc: launch");
    return ok();
  }
  // otherwise the two launches, with the prepared queries in the static scratch
  const size_t need = tq::attn_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads);
  if (need > (size_t)TQ_NOALLOC_SCRATCH_BYTES)
    return fail(TQ_ERR_INVALID_ARG,
                "%s: %zu bytes of prepared queries exceed the static scratch (%zu bytes); "
                "use tq_attn_logits with a workspace", fn, need,
                (size_t)TQ_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  e = tq::noalloc_scratch(ctx->device, &ws);
  if (e != hipSuccess) return hip_fail(e, "tq_attn_logits_noalloc: scratch symbol");
  e = tq::launch_attn_prepare(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads, ws,
                              tq::logits_fold(ctx, n_q_heads, n_kv_heads), (hipStream_t)stream);
  if (e == hipSuccess)
    e = tq::launch_attn_stream(ctx, ws, batch, n_q_heads, planes, norms, n_kv_heads,
                               keys_stride_head, seq_start, seq_len, max_seq_len, scale, logits,
                               logits_stride_head, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_attn_logits_noalloc: launch");
  return ok();
}

TQ_API tq_status tq_attn_prepare(const tq_ctx* ctx, const float* q, int32_t batch,
                                 int32_t n_q_heads, int64_t q_stride_batch, int32_t n_kv_heads,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "tq_attn_prepare: ctx is NULL");
  bool empty;
  const tq_status st = check_prepare("tq_attn_prepare", ctx, q, batch, n_q_heads, q_stride_batch,
                                     n_kv_heads, workspace, workspace_bytes, &empty);
  if (st != TQ_OK) return st;
  if (empty) return ok();
  hipError_t e = tq::launch_attn_prepare(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads,
                                         workspace, tq::logits_fold(ctx, n_q_heads, n_kv_heads),
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_attn_prepare: launch");
  return ok();
}

TQ_API tq_status tq_attn_logits_prepared(const tq_ctx* ctx, const void* workspace,
                                         size_t workspace_bytes, int32_t batch,
                                         int32_t n_q_heads, const uint32_t* planes,
                                         const uint16_t* norms, int32_t n_kv_heads,
                                         int64_t keys_stride_head, const int64_t* seq_start,
                                         const int32_t* seq_len, int32_t max_seq_len,
                                         float scale, float* logits,
                                         int64_t logits_stride_head, void* stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits_prepared: ctx is NULL");
  if (batch < 0 || max_seq_len < 0 || n_kv_heads < 1 || n_q_heads < 1 ||
      n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits_prepared: batch=%d n_q=%d n_kv=%d", batch,
                n_q_heads, n_kv_heads);
  if (batch == 0 || max_seq_len == 0) return ok();
  if (!workspace || !planes || !norms || !seq_start || !seq_len || !logits)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits_prepared: NULL pointer");
  if (keys_stride_head < 0 || logits_stride_head < 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits_prepared: negative stride");
  if (!aligned(planes, 16) || !aligned(norms, 4) || !aligned(workspace, 16))
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits_prepared: misaligned pointer");
  const size_t need = tq::attn_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads);
  if (workspace_bytes < need)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits_prepared: workspace %zu < %zu bytes",
                workspace_bytes, need);
  if (!std::isfinite(scale))
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_logits_prepared: scale not finite");
  hipError_t e = tq::launch_attn_stream(ctx, workspace, batch, n_q_heads, planes, norms,
                                        n_kv_heads, keys_stride_head, seq_start, seq_len,
                                        max_seq_len, scale, logits, logits_stride_head,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_attn_logits_prepared: launch");
  return ok();
}

TQ_API size_t tq_search_workspace_bytes(const tq_ctx* ctx, int64_t n_queries, int64_t n_db,
                                        int32_t k) {
  if (!ctx || n_queries < 0 || n_db < 0 || k < 1 || k > 64) return 0;
  return tq::search_workspace_bytes(ctx, n_queries, n_db, k);
}

TQ_API size_t tq_attn_output_workspace_bytes(const tq_ctx* ctx, int32_t batch,
                                             int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t max_seq_len) {
  if (!ctx || batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads ||
      max_seq_len < 0)
    return 0;
  return tq::vout_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads, max_seq_len);
}

TQ_API tq_status tq_attn_output(const tq_ctx* ctx, const float* p, int64_t p_stride_head,
                                int32_t batch, int32_t n_q_heads, const uint32_t* planes,
                                const uint16_t* norms, int32_t n_kv_heads,
                                int64_t values_stride_head, const int64_t* seq_start,
                                const int32_t* seq_len, int32_t max_seq_len, float* out,
                                int64_t out_stride_batch, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "tq_attn_output: ctx is NULL");
  if (batch < 0 || max_seq_len < 0 || n_kv_heads < 1 || n_q_heads < 1 ||
      n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_output: batch=%d n_q=%d n_kv=%d max_seq_len=%d",
                batch, n_q_heads, n_kv_heads, max_seq_len);
  if (batch == 0) return ok();
  if (!p || !planes || !norms || !seq_start || !seq_len || !out || !workspace)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_output: NULL pointer");
  if (p_stride_head < 0 || values_stride_head < 0 ||
      (batch > 1 && out_stride_batch < (int64_t)n_q_heads * ctx->d))
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_output: bad stride");
  if (!aligned(planes, 16) || !aligned(norms, 4) || !aligned(workspace, 16) || !aligned(p, 4) ||
      !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_output: misaligned pointer");
  const size_t need =
      tq::vout_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads, max_seq_len);
  if (workspace_bytes < need)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_output: workspace %zu < %zu bytes", workspace_bytes,
                need);
  hipError_t e = tq::launch_attn_output(ctx, p, p_stride_head, batch, n_q_heads, planes, norms,
                                        n_kv_heads, values_stride_head, seq_start, seq_len,
                                        max_seq_len, out, out_stride_batch, ctx->d, workspace,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_attn_output: launch");
  return ok();
}

TQ_API size_t tq_attn_decode_workspace_bytes(const tq_ctx* ctx, int32_t batch,
                                             int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t max_seq_len) {
  if (!ctx || batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads ||
      max_seq_len < 0)
    return 0;
  return tq::decode_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads, max_seq_len);
}

TQ_API tq_status tq_attn_decode(const tq_ctx* ctx, const float* q, int32_t batch,
                                int32_t n_q_heads, int64_t q_stride_batch,
                                const uint32_t* k_planes, const uint16_t* k_norms,
                                const uint32_t* v_planes, const uint16_t* v_norms,
                                int32_t n_kv_heads, int64_t kv_stride_head,
                                const int64_t* seq_start, const int32_t* seq_len,
                                int32_t max_seq_len, float scale, float* out,
                                int64_t out_stride_batch, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "tq_attn_decode: ctx is NULL");
  if (batch < 0 || max_seq_len < 0 || n_kv_heads < 1 || n_q_heads < 1 ||
      n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_decode: batch=%d n_q=%d n_kv=%d max_seq_len=%d",
                batch, n_q_heads, n_kv_heads, max_seq_len);
  if (batch == 0) return ok();
  if (!q || !k_planes || !k_norms || !v_planes || !v_norms || !seq_start || !seq_len || !out ||
      !workspace)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_decode: NULL pointer");
  if ((batch > 1 && q_stride_batch < (int64_t)n_q_heads * ctx->d) || kv_stride_head < 0 ||
      (batch > 1 && out_stride_batch < (int64_t)n_q_heads * ctx->d))
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_decode: bad stride");
  if (!aligned(k_planes, 16) || !aligned(v_planes, 16) || !aligned(k_norms, 4) ||
      !aligned(v_norms, 4) || !aligned(workspace, 16) || !aligned(q, 4) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_decode: misaligned pointer");
  const size_t need = tq::decode_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads, max_seq_len);
  if (workspace_bytes < need)
    return fail(TQ_ERR_INVALID_ARG, "tq_attn_decode: workspace %zu < %zu bytes", workspace_bytes,
                need);
  hipError_t e = tq::launch_attn_decode(ctx, q, batch, n_q_heads, q_stride_batch, k_planes,
                                        k_norms, v_planes, v_norms, n_kv_heads, kv_stride_head,
                                        seq_start, seq_len, max_seq_len, scale, out,
                                        out_stride_batch, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_attn_decode: launch");
  return ok();
}

TQ_API tq_status tq_search_topk(const tq_ctx* ctx, const float* queries, int64_t n_queries,
                                const uint32_t* planes, const uint16_t* norms, int64_t n_db,
                                int32_t k, int64_t* out_idx, float* out_score, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(TQ_ERR_INVALID_ARG, "tq_search_topk: ctx is NULL");
  if (n_queries < 0 || n_db < 0 || k < 1 || k > 64)
    return fail(TQ_ERR_INVALID_ARG, "tq_search_topk: n_queries=%lld n_db=%lld k=%d",
                (long long)n_queries, (long long)n_db, k);
  if (n_queries == 0) return ok();
  if (!queries || !out_idx || !out_score || !workspace || (n_db > 0 && (!planes || !norms)))
    return fail(TQ_ERR_INVALID_ARG, "tq_search_topk: NULL pointer");
  if (!aligned(planes, 16) || !aligned(norms, 4) || !aligned(workspace, 16) ||
      !aligned(queries, 4) || !aligned(out_idx, 8) || !aligned(out_score, 4))
    return fail(TQ_ERR_INVALID_ARG, "tq_search_topk: misaligned pointer");
  const size_t need = tq::search_workspace_bytes(ctx, n_queries, n_db, k);
  if (workspace_bytes < need)
    return fail(TQ_ERR_INVALID_ARG, "tq_search_topk: workspace %zu < %zu bytes",
                workspace_bytes, need);
  hipError_t e = tq::launch_search_topk(ctx, queries, n_queries, planes, norms, n_db, k,
                                        out_idx, out_score, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_search_topk: launch");
  return ok();
}

// ---- fractional bit widths: two instances over a channel split ------------
namespace {

// Both instances present, of one kind (two-stage or MSE-only) and on one device.
tq_status check_split(const char* fn, const tq_ctx* hi, const tq_ctx* lo) {
  if (!hi || !lo) return fail(TQ_ERR_INVALID_ARG, "%s: ctx is NULL", fn);
  if (hi->mse != lo->mse)
    return fail(TQ_ERR_INVALID_ARG, "%s: both instances must be two-stage or both MSE-only", fn);
  if (hi->device != lo->device)
    return fail(TQ_ERR_INVALID_ARG, "%s: instances on different devices", fn);
  return TQ_OK;
}

}  // namespace

TQ_API tq_status tq_split_quantize_kv(const tq_ctx* hi, const tq_ctx* lo, const void* x,
                                      int32_t x_dtype, int64_t n_tokens, int32_t n_heads,
                                      int64_t x_stride_token, int64_t x_stride_head,
                                      uint32_t* hi_planes, uint16_t* hi_norms,
                                      uint32_t* lo_planes, uint16_t* lo_norms,
                                      int64_t dst_stride_head, int64_t dst_token0, void* stream) {
  const char* fn = "tq_split_quantize_kv";
  tq_status st = check_split(fn, hi, lo);
  if (st != TQ_OK) return st;
  bool empty_hi, empty_lo;
  if (n_tokens > 0 && n_heads > 0 && x_stride_token < (int64_t)hi->d + lo->d)
    return fail(TQ_ERR_INVALID_ARG, "%s: x_stride_token < d_hi + d_lo", fn);
  const size_t esz = x_dtype == TQ_F32 ? 4 : 2;
  const void* x_lo = x ? (const void*)((const char*)x + (size_t)hi->d * esz) : nullptr;
  st = check_quantize(fn, hi, x, x_dtype, n_tokens, n_heads, x_stride_token, x_stride_head,
                      hi_planes, hi_norms, dst_stride_head, dst_token0, nullptr, &empty_hi);
  if (st == TQ_OK)
    st = check_quantize(fn, lo, x_lo, x_dtype, n_tokens, n_heads, x_stride_token, x_stride_head,
                        lo_planes, lo_norms, dst_stride_head, dst_token0, nullptr, &empty_lo);
  if (st != TQ_OK) return st;
  if (empty_hi) return ok();
  hipError_t e = tq::launch_quantize(hi, x, x_dtype, n_tokens, n_heads, x_stride_token,
                                     x_stride_head, hi_planes, hi_norms, dst_stride_head,
                                     dst_token0, nullptr, (hipStream_t)stream);
  if (e == hipSuccess)
    e = tq::launch_quantize(lo, x_lo, x_dtype, n_tokens, n_heads, x_stride_token, x_stride_head,
                            lo_planes, lo_norms, dst_stride_head, dst_token0, nullptr,
                            (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_split_quantize_kv: launch");
  return ok();
}

TQ_API tq_status tq_split_dequantize(const tq_ctx* hi, const tq_ctx* lo,
                                     const uint32_t* hi_planes, const uint16_t* hi_norms,
                                     const uint32_t* lo_planes, const uint16_t* lo_norms,
                                     int64_t n, float* out, int64_t out_ld, void* stream) {
  const char* fn = "tq_split_dequantize";
  const tq_status st = check_split(fn, hi, lo);
  if (st != TQ_OK) return st;
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "%s: n=%lld", fn, (long long)n);
  if (n == 0) return ok();
  if (!hi_planes || !hi_norms || !lo_planes || !lo_norms || !out)
    return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (out_ld < (int64_t)hi->d + lo->d)
    return fail(TQ_ERR_INVALID_ARG, "%s: out_ld < d_hi + d_lo", fn);
  if (!aligned(hi_planes, 16) || !aligned(lo_planes, 16) || !aligned(hi_norms, 4) ||
      !aligned(lo_norms, 4) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  hipError_t e = tq::launch_dequantize(hi, hi_planes, hi_norms, n, out, out_ld,
                                       (hipStream_t)stream);
  if (e == hipSuccess)
    e = tq::launch_dequantize(lo, lo_planes, lo_norms, n, out + hi->d, out_ld,
                              (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_split_dequantize: launch");
  return ok();
}

TQ_API size_t tq_split_attn_logits_workspace_bytes(const tq_ctx* hi, const tq_ctx* lo,
                                                   int32_t batch, int32_t n_q_heads,
                                                   int32_t n_kv_heads) {
  if (!hi || !lo || batch < 0 || n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads)
    return 0;
  return tq::split_attn_workspace_bytes(hi, lo, batch, n_q_heads, n_kv_heads);
}

namespace {

// Checks shared by the split logit calls (q == nullptr skips the query checks,
// records == false the record and sequence checks); *empty for no work.
tq_status check_split_logits(const char* fn, const tq_ctx* hi, const tq_ctx* lo, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t max_seq_len,
                             const float* q, int64_t q_stride_batch, bool records,
                             const uint32_t* hi_planes, const uint16_t* hi_norms,
                             const uint32_t* lo_planes, const uint16_t* lo_norms,
                             int64_t keys_stride_head, const int64_t* seq_start,
                             const int32_t* seq_len, float scale, float* logits,
                             int64_t logits_stride_head, const void* workspace,
                             size_t workspace_bytes, bool* empty) {
  *empty = false;
  tq_status st = check_split(fn, hi, lo);
  if (st != TQ_OK) return st;
  if (batch < 0 || max_seq_len < 0 || n_kv_heads < 1 || n_q_heads < 1 ||
      n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: batch=%d n_q=%d n_kv=%d max_seq_len=%d", fn, batch,
                n_q_heads, n_kv_heads, max_seq_len);
  if (!tq::split_logits_supported(hi, lo, n_q_heads, n_kv_heads))
    return fail(TQ_ERR_UNSUPPORTED,
                "%s: needs d <= 128 per instance and at most 4 query heads per kv head", fn);
  if (batch == 0 || (records && max_seq_len == 0)) {
    *empty = true;
    return TQ_OK;
  }
  if (!workspace) return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (q) {
    if (q_stride_batch < (int64_t)n_q_heads * (hi->d + lo->d) && batch > 1)
      return fail(TQ_ERR_INVALID_ARG, "%s: q_stride_batch too small", fn);
    if (!aligned(q, 4)) return fail(TQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  }
  if (records) {
    if (!hi_planes || !hi_norms || !lo_planes || !lo_norms || !seq_start || !seq_len || !logits)
      return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (keys_stride_head < 0 || logits_stride_head < 0)
      return fail(TQ_ERR_INVALID_ARG, "%s: negative stride", fn);
    if (!aligned(hi_planes, 16) || !aligned(lo_planes, 16) || !aligned(hi_norms, 4) ||
        !aligned(lo_norms, 4))
      return fail(TQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if (!std::isfinite(scale)) return fail(TQ_ERR_INVALID_ARG, "%s: scale not finite", fn);
  }
  if (!aligned(workspace, 16)) return fail(TQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  const size_t need = tq::split_attn_workspace_bytes(hi, lo, batch, n_q_heads, n_kv_heads);
  if (workspace_bytes < need)
    return fail(TQ_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  return TQ_OK;
}

}  // namespace

TQ_API tq_status tq_split_attn_logits(const tq_ctx* hi, const tq_ctx* lo, const float* q,
                                      int32_t batch, int32_t n_q_heads, int64_t q_stride_batch,
                                      const uint32_t* hi_planes, const uint16_t* hi_norms,
                                      const uint32_t* lo_planes, const uint16_t* lo_norms,
                                      int32_t n_kv_heads, int64_t keys_stride_head,
                                      const int64_t* seq_start, const int32_t* seq_len,
                                      int32_t max_seq_len, float scale, float* logits,
                                      int64_t logits_stride_head, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const char* fn = "tq_split_attn_logits";
  if (!q && hi && lo && batch > 0 && max_seq_len > 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  bool empty;
  const tq_status st = check_split_logits(
      fn, hi, lo, batch, n_q_heads, n_kv_heads, max_seq_len, q, q_stride_batch, true, hi_planes,
      hi_norms, lo_planes, lo_norms, keys_stride_head, seq_start, seq_len, scale, logits,
      logits_stride_head, workspace, workspace_bytes, &empty);
  if (st != TQ_OK) return st;
  if (empty) return ok();
  hipError_t e = tq::launch_split_prepare(hi, lo, q, batch, n_q_heads, q_stride_batch,
                                          n_kv_heads, workspace, (hipStream_t)stream);
  if (e == hipSuccess)
    e = tq::launch_split_stream(hi, lo, workspace, batch, n_q_heads, hi_planes, hi_norms,
                                lo_planes, lo_norms, n_kv_heads, keys_stride_head, seq_start,
                                seq_len, max_seq_len, scale, logits, logits_stride_head,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_split_attn_logits: launch");
  return ok();
}

TQ_API tq_status tq_split_attn_prepare(const tq_ctx* hi, const tq_ctx* lo, const float* q,
                                       int32_t batch, int32_t n_q_heads, int64_t q_stride_batch,
                                       int32_t n_kv_heads, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const char* fn = "tq_split_attn_prepare";
  if (!q && hi && lo && batch > 0) return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  bool empty;
  const tq_status st = check_split_logits(
      fn, hi, lo, batch, n_q_heads, n_kv_heads, 0, q, q_stride_batch, false, nullptr, nullptr,
      nullptr, nullptr, 0, nullptr, nullptr, 1.f, nullptr, 0, workspace, workspace_bytes, &empty);
  if (st != TQ_OK) return st;
  if (empty) return ok();
  hipError_t e = tq::launch_split_prepare(hi, lo, q, batch, n_q_heads, q_stride_batch,
                                          n_kv_heads, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_split_attn_prepare: launch");
  return ok();
}

TQ_API tq_status tq_split_attn_logits_prepared(
    const tq_ctx* hi, const tq_ctx* lo, const void* workspace, size_t workspace_bytes,
    int32_t batch, int32_t n_q_heads, const uint32_t* hi_planes, const uint16_t* hi_norms,
    const uint32_t* lo_planes, const uint16_t* lo_norms, int32_t n_kv_heads,
    int64_t keys_stride_head, const int64_t* seq_start, const int32_t* seq_len,
    int32_t max_seq_len, float scale, float* logits, int64_t logits_stride_head, void* stream) {
  const char* fn = "tq_split_attn_logits_prepared";
  bool empty;
  const tq_status st = check_split_logits(
      fn, hi, lo, batch, n_q_heads, n_kv_heads, max_seq_len, nullptr, 0, true, hi_planes,
      hi_norms, lo_planes, lo_norms, keys_stride_head, seq_start, seq_len, scale, logits,
      logits_stride_head, workspace, workspace_bytes, &empty);
  if (st != TQ_OK) return st;
  if (empty) return ok();
  hipError_t e = tq::launch_split_stream(hi, lo, workspace, batch, n_q_heads, hi_planes,
                                         hi_norms, lo_planes, lo_norms, n_kv_heads,
                                         keys_stride_head, seq_start, seq_len, max_seq_len,
                                         scale, logits, logits_stride_head, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_split_attn_logits_prepared: launch");
  return ok();
}

TQ_API size_t tq_split_attn_output_workspace_bytes(const tq_ctx* hi, const tq_ctx* lo,
                                                   int32_t batch, int32_t n_q_heads,
                                                   int32_t n_kv_heads, int32_t max_seq_len) {
  if (!hi || !lo || batch < 0 || max_seq_len < 0 || n_kv_heads < 1 || n_q_heads < 1 ||
      n_q_heads % n_kv_heads)
    return 0;
  // the two instances run one after the other on the stream and reuse it
  return std::max(tq::vout_workspace_bytes(hi, batch, n_q_heads, n_kv_heads, max_seq_len),
                  tq::vout_workspace_bytes(lo, batch, n_q_heads, n_kv_heads, max_seq_len));
}

TQ_API tq_status tq_split_attn_output(const tq_ctx* hi, const tq_ctx* lo, const float* p,
                                      int64_t p_stride_head, int32_t batch, int32_t n_q_heads,
                                      const uint32_t* hi_planes, const uint16_t* hi_norms,
                                      const uint32_t* lo_planes, const uint16_t* lo_norms,
                                      int32_t n_kv_heads, int64_t values_stride_head,
                                      const int64_t* seq_start, const int32_t* seq_len,
                                      int32_t max_seq_len, float* out, int64_t out_stride_batch,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tq_split_attn_output";
  const tq_status st = check_split(fn, hi, lo);
  if (st != TQ_OK) return st;
  if (batch < 0 || max_seq_len < 0 || n_kv_heads < 1 || n_q_heads < 1 ||
      n_q_heads % n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: batch=%d n_q=%d n_kv=%d max_seq_len=%d", fn, batch,
                n_q_heads, n_kv_heads, max_seq_len);
  if (batch == 0) return ok();
  if (!p || !hi_planes || !hi_norms || !lo_planes || !lo_norms || !seq_start || !seq_len ||
      !out || !workspace)
    return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  const int64_t d = (int64_t)hi->d + lo->d;
  if (p_stride_head < 0 || values_stride_head < 0 ||
      (batch > 1 && out_stride_batch < (int64_t)n_q_heads * d))
    return fail(TQ_ERR_INVALID_ARG, "%s: bad stride", fn);
  if (!aligned(hi_planes, 16) || !aligned(lo_planes, 16) || !aligned(hi_norms, 4) ||
      !aligned(lo_norms, 4) || !aligned(workspace, 16) || !aligned(p, 4) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  const size_t need =
      tq_split_attn_output_workspace_bytes(hi, lo, batch, n_q_heads, n_kv_heads, max_seq_len);
  if (workspace_bytes < need)
    return fail(TQ_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  // channels [0, d_hi) of every head from the first instance, the rest from
  // the second: head stride d, channel offset d_hi
  hipError_t e = tq::launch_attn_output(hi, p, p_stride_head, batch, n_q_heads, hi_planes,
                                        hi_norms, n_kv_heads, values_stride_head, seq_start,
                                        seq_len, max_seq_len, out, out_stride_batch, d, workspace,
                                        (hipStream_t)stream);
  if (e == hipSuccess)
    e = tq::launch_attn_output(lo, p, p_stride_head, batch, n_q_heads, lo_planes, lo_norms,
                               n_kv_heads, values_stride_head, seq_start, seq_len, max_seq_len,
                               out + hi->d, out_stride_batch, d, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tq_split_attn_output: launch");
  return ok();
}

}  // extern "C"
