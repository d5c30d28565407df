/* Drives the CPU oracle (oracle/tq_oracle.c, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer) through every path the tests use: rotation,
 * density integrals, Lloyd-Max, pack/unpack, two-stage and MSE-only
 * quantize with margins, the second stage on given codes, dequantize,
 * estimate and top-k, at several d (ragged last words included) and b.
 * Exit status 0 when the light consistency checks hold; the sanitizers abort
 * on the first memory or undefined-behaviour finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_make_rotation(int32_t d, uint64_t seed, double* pi64, double* s64, float* pi32, float* s32);
double orc_beta_density(int32_t d, double x);
double orc_beta_integral(int32_t d, int32_t p, double a, double b);
int orc_lloyd_max(int32_t d, int32_t bits, int32_t max_iter, double tol, double* c, double* dist,
                  int32_t* iters, double* hist);
void orc_pack_record(int32_t d, int32_t b, const int32_t* idx, const int32_t* sgn, uint32_t* rec);
void orc_unpack_record(int32_t d, int32_t b, const uint32_t* rec, int32_t* idx, int32_t* sgn);
void orc_quantize(int32_t d, int32_t b, const float* pi, const float* s, const float* cen,
                  int64_t n, const double* x, int64_t ld, uint32_t* planes, uint16_t* norms,
                  double* code_margin, double* sign_margin, double* nu, double* gamma, double* y);
void orc_qjl_given_codes(int32_t d, int32_t b, const float* pi, const float* s, const float* cen,
                         int64_t n, const double* x, int64_t ld, const int32_t* idx,
                         uint32_t* planes, uint16_t* norms, double* sign_margin, double* gamma);
void orc_dequantize(int32_t d, int32_t b, const float* pi, const float* s, const float* cen,
                    int64_t n, const uint32_t* planes, const uint16_t* norms, double* out,
                    int64_t ld);
void orc_estimate(int32_t d, int32_t b, const float* pi, const float* s, const float* cen,
                  int64_t nq, const double* q, int64_t ldq, int64_t n, const uint32_t* planes,
                  const uint16_t* norms, const double* nu_exact, const double* gamma_exact,
                  double scale, double* out);
void orc_quantize_mse(int32_t d, int32_t b, const float* pi, const float* cen, int64_t n,
                      const double* x, int64_t ld, uint32_t* planes, uint16_t* norms,
                      double* code_margin);
void orc_dequantize_mse(int32_t d, int32_t b, const float* pi, const float* cen, int64_t n,
                        const uint32_t* planes, const uint16_t* norms, double* out, int64_t ld);
void orc_estimate_mse(int32_t d, int32_t b, const float* pi, const float* cen, int64_t nq,
                      const double* q, int64_t ldq, int64_t n, const uint32_t* planes,
                      const uint16_t* norms, double scale, double* out);
void orc_topk(int64_t nq, int64_t n, const double* scores, int32_t k, int64_t* idx, double* sc);

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "FAILED %d: %s\n", __LINE__, #c); ++fails; } } while (0)

static double urand(uint64_t* s) {
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((*s >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static void run(int d, int b, int n) {
    int W = (d + 31) / 32, K = 1 << (b - 1);
    size_t dd = (size_t)d * d;
    double* pi64 = malloc(dd * sizeof(double));
    double* s64 = malloc(dd * sizeof(double));
    float* pi = malloc(dd * sizeof(float));
    float* s = malloc(dd * sizeof(float));
    EXPECT(orc_make_rotation(d, 3, pi64, s64, pi, s) == 0);
    double c64[16];
    float c[16], cm[16];
    EXPECT(orc_lloyd_max(d, b - 1, 100000, 1e-13, c64, NULL, NULL, NULL) == 0);
    for (int k = 0; k < K; ++k) c[k] = (float)c64[k];
    EXPECT(orc_lloyd_max(d, b, 100000, 1e-13, c64, NULL, NULL, NULL) == 0);  /* MSE codebook */
    for (int k = 0; k < 2 * K; ++k) cm[k] = (float)c64[k];

    uint64_t st = 1234 + d * 7 + b;
    double* x = malloc((size_t)n * d * sizeof(double));
    for (size_t i = 0; i < (size_t)n * d; ++i) x[i] = urand(&st) - 0.5;
    memset(x + d, 0, d * sizeof(double));                     /* a zero vector */
    uint32_t* planes = malloc((size_t)n * W * b * sizeof(uint32_t));
    uint16_t* norms = malloc((size_t)n * 2 * sizeof(uint16_t));
    double* cmarg = malloc((size_t)n * d * sizeof(double));
    double* smarg = malloc((size_t)n * d * sizeof(double));
    double* y = malloc((size_t)n * d * sizeof(double));
    double nu[64], ga[64];
    orc_quantize(d, b, pi, s, c, n, x, d, planes, norms, cmarg, smarg, nu, ga, y);
    orc_quantize(d, b, pi, s, c, n, x, d, planes, norms, NULL, NULL, NULL, NULL, NULL);

    int32_t* idx = malloc((size_t)n * d * sizeof(int32_t));
    int32_t* sg = malloc((size_t)d * sizeof(int32_t));
    for (int i = 0; i < n; ++i) orc_unpack_record(d, b, planes + (size_t)i * W * b, idx + (size_t)i * d, sg);
    uint32_t* p2 = malloc((size_t)n * W * b * sizeof(uint32_t));
    uint16_t* n2 = malloc((size_t)n * 2 * sizeof(uint16_t));
    orc_qjl_given_codes(d, b, pi, s, c, n, x, d, idx, p2, n2, smarg, ga);
    EXPECT(memcmp(p2, planes, (size_t)n * W * b * sizeof(uint32_t)) == 0);
    EXPECT(memcmp(n2, norms, (size_t)n * 2 * sizeof(uint16_t)) == 0);
    uint32_t rec[256];
    orc_pack_record(d, b, idx, sg, rec);

    double* deq = malloc((size_t)n * d * sizeof(double));
    orc_dequantize(d, b, pi, s, c, n, planes, norms, deq, d);
    double q[3 * 2048];
    for (int i = 0; i < 3 * d; ++i) q[i] = urand(&st) - 0.5;
    double* est = malloc((size_t)3 * n * sizeof(double));
    orc_estimate(d, b, pi, s, c, 3, q, d, n, planes, norms, NULL, NULL, 0.5, est);
    orc_estimate(d, b, pi, s, c, 3, q, d, n, planes, norms, nu, ga, 1.0, est);
    int64_t ti[3 * 5];
    double ts[3 * 5];
    orc_topk(3, n, est, 5, ti, ts);
    for (int a = 0; a < 3; ++a)
        for (int j = 0; j + 1 < 5; ++j) EXPECT(ts[a * 5 + j] >= ts[a * 5 + j + 1]);

    /* MSE-only mode: b code planes */
    orc_quantize_mse(d, b, pi, cm, n, x, d, planes, norms, cmarg);
    orc_dequantize_mse(d, b, pi, cm, n, planes, norms, deq, d);
    orc_estimate_mse(d, b, pi, cm, 3, q, d, n, planes, norms, 2.0, est);

    free(pi64); free(s64); free(pi); free(s); free(x); free(planes); free(norms); free(cmarg);
    free(smarg); free(y); free(idx); free(sg); free(p2); free(n2); free(deq); free(est);
}

int main(void) {
    for (int d = 3; d <= 5; ++d)
        EXPECT(fabs(orc_beta_integral(d, 0, -1.0, 1.0) - 1.0) < 1e-10);
    EXPECT(orc_beta_density(128, 0.0) > 0.0);
    double c[16], dist, hist[200];
    int32_t it;
    EXPECT(orc_lloyd_max(128, 3, 200, 1e-13, c, &dist, &it, hist) == 0);
    run(5, 2, 9);
    run(33, 3, 17);
    run(128, 4, 40);
    run(200, 3, 21);
    run(64, 2, 30);
    if (fails) { fprintf(stderr, "%d expectation(s) failed\n", fails); return 1; }
    printf("oracle driver ok\n");
    return 0;
}
