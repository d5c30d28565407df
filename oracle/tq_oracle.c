/*
 * tq_oracle.c -- TEST INFRASTRUCTURE ONLY (never part of the product path).
 *
 * Plain, slow, double-precision CPU oracle for the TurboQuant hot path:
 * seeded rotation and sketch, the coordinate density of a rotated unit
 * vector, Lloyd-Max centroids of that density, the two-stage quantizer
 * ((b-1)-bit scalar codes + 1-bit QJL signs of the residual), dequantization,
 * the inner-product estimator and top-k.  Only tests/, __graft_entry__.smoke()
 * and the cpu_baseline leg of bench.py may load this library.  It shares no
 * code, header or table with the HIP library; both sides implement the same
 * published random generator (SplitMix64 + Box-Muller) independently.
 *
 * Sources (the pages this oracle follows; each function cites its passage):
 *  [P1] zingnex.cn forum digest "TurboQuant: KV cache quantization close to the
 *       theoretical limit" -- sections "random rotation and Beta distribution",
 *       "two-stage inner-product quantization".
 *  [P2] turboquant.net landing page -- section "PolarQuant" (coordinate density
 *       formula), section "pseudo-code implementation steps" (Lloyd-Max
 *       centroids, QR rotation, quant/dequant, attention integration), section
 *       "potential challenges" (reuse of the rotation, residual norm as one fp16
 *       scalar).
 *  [P3] admirer.cn news article on Google Research's TurboQuant -- paragraphs on
 *       PolarQuant (rotation, Beta coordinates, Lloyd-Max), on QJL (one sign
 *       bit, unbiased inner products) and on the two-stage b-1 + 1 bit split.
 *
 * Readings where the pages are silent:
 *  - the random generator (the pages use numpy's randn, which is not
 *    reproduced): SplitMix64 over a per-(seed, stream) key, Box-Muller;
 *  - Pi is the Q factor with the signs fixed so that R has a positive
 *    diagonal (Haar-distributed rotation); y = Pi x, x = Pi^T y;
 *  - S has m = d rows of iid N(0,1);
 *  - vectors are normalised first (the density lives on the unit sphere) and
 *    ||x|| is stored as fp16 next to ||r||;
 *  - sign(0) = +1; ties in the nearest-centroid search go to the lower index;
 *  - the QJL scale is alpha = sqrt(pi/2)/m, which makes the estimator
 *    unbiased over S: for s ~ N(0, I), E[sign(s.r) s.q] = sqrt(2/pi) <r, q> / ||r||;
 *  - a zero vector stores nu = 0, gamma = 0, codes of y = 0, all signs +1.
 *
 * Canonical packed record (the format both sides read and write):
 *  W = ceil(d/32) groups; group w holds b uint32 words: words 0..b-2 carry bit
 *  p of the code index of coordinates 32w..32w+31 (bit j%32 <-> coordinate j),
 *  word b-1 carries the QJL signs (1 <-> +1).  Bits of coordinates >= d are 0.
 *  norms[2*i] = fp16 bits of ||x||, norms[2*i+1] = fp16 bits of ||r||.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Random numbers.  The pages draw G with numpy's randn ([P2] pseudo-code,
 * "generate random rotation matrix"); we use the published SplitMix64
 * generator (Steele, Lea, Flood 2014; reference code by S. Vigna) as a
 * counter-based generator, and the Box-Muller transform (1958).
 *   key(seed, stream) = SplitMix64 output number `stream` for state `seed`
 *   u64(seed, stream, i) = SplitMix64 output number i for state key
 * where output number i of state s is mix(s + (i+1)*0x9E3779B97F4A7C15).
 * ------------------------------------------------------------------------ */
static uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

ORC_API uint64_t orc_splitmix64(uint64_t state, uint64_t i) {
    return sm64_mix(state + (i + 1ULL) * 0x9E3779B97F4A7C15ULL);
}

ORC_API uint64_t orc_rng_u64(uint64_t seed, uint64_t stream, uint64_t i) {
    uint64_t key = orc_splitmix64(seed, stream);
    return orc_splitmix64(key, i);
}

/* uniform in (0, 1]: the top 53 bits plus one, times 2^-53 */
ORC_API double orc_rng_uniform(uint64_t seed, uint64_t stream, uint64_t i) {
    uint64_t v = orc_rng_u64(seed, stream, i);
    return (double)((v >> 11) + 1ULL) * (1.0 / 9007199254740992.0);
}

/* n standard normals; pair j uses uniforms 2j (radius) and 2j+1 (angle) and
 * yields r*cos(theta) then r*sin(theta). */
ORC_API void orc_rng_normals(uint64_t seed, uint64_t stream, int64_t n, double* out) {
    for (int64_t j = 0; 2 * j < n; ++j) {
        double u1 = orc_rng_uniform(seed, stream, (uint64_t)(2 * j));
        double u2 = orc_rng_uniform(seed, stream, (uint64_t)(2 * j + 1));
        double r = sqrt(-2.0 * log(u1));
        double th = 6.283185307179586476925286766559 * u2;
        out[2 * j] = r * cos(th);
        if (2 * j + 1 < n) out[2 * j + 1] = r * sin(th);
    }
}

/* ------------------------------------------------------------------------ */
/* IEEE binary16, round to nearest even, straight from double.  The residual
 * norm is stored as one fp16 scalar ([P2] "potential challenges", residual
 * norm storage); we store ||x|| the same way. */
ORC_API uint16_t orc_f16_from_double(double v) {
    uint16_t sign = (signbit(v) ? 0x8000u : 0u);
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u); /* rounds to inf */
    if (a == 0.0) return sign;
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;           /* a = (2m) * 2^E, 2m in [1, 2) */
    if (E < -14) {
        /* subnormal: value = k * 2^-24 */
        double k = a * 16777216.0;      /* exact scaling by 2^24 */
        double fl = floor(k);
        double fr = k - fl;
        uint32_t ki = (uint32_t)fl;
        if (fr > 0.5 || (fr == 0.5 && (ki & 1u))) ki += 1u;
        /* ki may reach 1024 = smallest normal, which the bit pattern encodes */
        return (uint16_t)(sign | ki);
    }
    double sig = a / ldexp(1.0, E) * 1024.0; /* in [1024, 2048) */
    double fl = floor(sig);
    double fr = sig - fl;
    uint32_t si = (uint32_t)fl;
    if (fr > 0.5 || (fr == 0.5 && (si & 1u))) si += 1u;
    if (si == 2048u) { si = 1024u; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | ((uint32_t)(E + 15) << 10) | (si - 1024u));
}

ORC_API double orc_f16_to_double(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(f + 1024), e - 25);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Rotation Pi and sketch S.  [P2] pseudo-code "generate random rotation
 * matrix": G = randn(d, d), Pi = Q of the QR decomposition; [P2] "potential
 * challenges": generate once and reuse.  Householder QR in double; the signs
 * of Q's columns are fixed so that diag(R) > 0.  S (m = d rows) is a Gaussian
 * JL matrix ([P3] QJL paragraph).  G uses stream 0, S stream 1, row-major. */
ORC_API int orc_make_rotation(int32_t d, uint64_t seed, double* pi64, double* s64,
                              float* pi32, float* s32) {
    if (d < 1) return -1;
    int64_t dd = (int64_t)d * d;
    double* A = (double*)malloc(sizeof(double) * dd);   /* becomes R / reflectors */
    double* V = (double*)malloc(sizeof(double) * dd);   /* Householder vectors */
    double* beta = (double*)malloc(sizeof(double) * d);
    double* Q = (double*)malloc(sizeof(double) * dd);
    if (!A || !V || !beta || !Q) { free(A); free(V); free(beta); free(Q); return -2; }
    orc_rng_normals(seed, 0, dd, A);
    /* A is row-major: A[r*d + c].  Householder on columns k = 0..d-1. */
    for (int k = 0; k < d; ++k) {
        double norm2 = 0.0;
        for (int r = k; r < d; ++r) norm2 += A[(int64_t)r * d + k] * A[(int64_t)r * d + k];
        double norm = sqrt(norm2);
        double a0 = A[(int64_t)k * d + k];
        double alpha = (a0 >= 0.0) ? -norm : norm;  /* R[k][k] = alpha */
        for (int r = 0; r < d; ++r) V[(int64_t)k * d + r] = 0.0;
        double vnorm2 = 0.0;
        for (int r = k; r < d; ++r) {
            double v = A[(int64_t)r * d + k] - (r == k ? alpha : 0.0);
            V[(int64_t)k * d + r] = v;
            vnorm2 += v * v;
        }
        beta[k] = (vnorm2 > 0.0) ? 2.0 / vnorm2 : 0.0;
        /* apply H_k = I - beta v v^T to columns k..d-1 */
        for (int c = k; c < d; ++c) {
            double dot = 0.0;
            for (int r = k; r < d; ++r) dot += V[(int64_t)k * d + r] * A[(int64_t)r * d + c];
            dot *= beta[k];
            for (int r = k; r < d; ++r) A[(int64_t)r * d + c] -= dot * V[(int64_t)k * d + r];
        }
    }
    /* Q = H_0 H_1 ... H_{d-1}: start from I and apply from the right end */
    for (int64_t i = 0; i < dd; ++i) Q[i] = 0.0;
    for (int i = 0; i < d; ++i) Q[(int64_t)i * d + i] = 1.0;
    for (int k = d - 1; k >= 0; --k) {
        for (int c = 0; c < d; ++c) {
            double dot = 0.0;
            for (int r = k; r < d; ++r) dot += V[(int64_t)k * d + r] * Q[(int64_t)r * d + c];
            dot *= beta[k];
            for (int r = k; r < d; ++r) Q[(int64_t)r * d + c] -= dot * V[(int64_t)k * d + r];
        }
    }
    /* sign fix: column c of Q times sign(R[c][c]) */
    for (int c = 0; c < d; ++c) {
        double rc = A[(int64_t)c * d + c];
        if (rc < 0.0)
            for (int r = 0; r < d; ++r) Q[(int64_t)r * d + c] = -Q[(int64_t)r * d + c];
    }
    for (int64_t i = 0; i < dd; ++i) {
        if (pi64) pi64[i] = Q[i];
        if (pi32) pi32[i] = (float)Q[i];
    }
    double* S = A; /* reuse */
    orc_rng_normals(seed, 1, dd, S);
    for (int64_t i = 0; i < dd; ++i) {
        if (s64) s64[i] = S[i];
        if (s32) s32[i] = (float)S[i];
    }
    free(A); free(V); free(beta); free(Q);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Coordinate density of a uniformly random point on the unit sphere in R^d
 * ([P2] "PolarQuant" section, coordinate distribution formula):
 *   f_d(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - x^2)^((d-3)/2),
 * x in [-1, 1].  Evaluated through lgamma / log1p so that large d does not
 * overflow. */
ORC_API double orc_beta_density(int32_t d, double x) {
    if (d < 2 || x <= -1.0 || x >= 1.0) {
        if (d == 3 && (x == -1.0 || x == 1.0)) return 0.5;
        return 0.0;
    }
    double lc = lgamma(0.5 * d) - 0.5 * log(M_PI) - lgamma(0.5 * (d - 1));
    /* log(1 - x^2) as log1p(-x) + log1p(x): no cancellation near |x| = 1 */
    return exp(lc + 0.5 * (d - 3) * (log1p(-x) + log1p(x)));
}

/* Adaptive Gauss-Kronrod (7, 15) quadrature of x^p f_d(x) (p = 0, 1, 2) or
 * of (x - c)^2 f_d(x) (p = 3) on [a, b]. */
static const double gk_x[8] = {
    0.991455371120812639206854697526329, 0.949107912342758524526189684047851,
    0.864864423359769072789712788640926, 0.741531185599394439863864773280788,
    0.586087235467691130294144845693013, 0.405845151377397166906606412076961,
    0.207784955007898467600689403773245, 0.000000000000000000000000000000000};
static const double gk_wk[8] = {
    0.022935322010529224963732008058970, 0.063092092629978553290700663189204,
    0.104790010322250183839876322541518, 0.140653259715525918745189590510238,
    0.169004726639267902826583426598550, 0.190350578064785409913256402421014,
    0.204432940075298892414161999234649, 0.209482141084727828012999174891714};
static const double gk_wg[4] = {
    0.129484966168869693270611432679082, 0.279705391489276667901467771423780,
    0.381830050505118944950369775488975, 0.417959183673469387755102040816327};

typedef struct { int32_t d; int p; double c; } orc_integrand;

static double integrand(const orc_integrand* it, double x) {
    double f = orc_beta_density(it->d, x);
    switch (it->p) {
        case 0: return f;
        case 1: return x * f;
        case 2: return x * x * f;
        default: return (x - it->c) * (x - it->c) * f;
    }
}

static void gk15(const orc_integrand* it, double a, double b, double* res, double* err) {
    double c = 0.5 * (a + b), h = 0.5 * (b - a);
    double fc = integrand(it, c);
    double rk = fc * gk_wk[7], rg = fc * gk_wg[3];
    for (int j = 0; j < 7; ++j) {
        double dx = h * gk_x[j];
        double f1 = integrand(it, c - dx), f2 = integrand(it, c + dx);
        rk += gk_wk[j] * (f1 + f2);
        if (j % 2 == 1) rg += gk_wg[j / 2] * (f1 + f2);
    }
    *res = rk * h;
    *err = fabs((rk - rg) * h);
}

static double gk_adapt(const orc_integrand* it, double a, double b, double tol, int depth) {
    double r, e;
    gk15(it, a, b, &r, &e);
    /* stop at the requested absolute tolerance, at rounding level relative
     * to this panel's value, or at depth 30 */
    if (depth >= 30 || e <= tol || e <= 1e-15 * fabs(r) || (b - a) < 1e-300) return r;
    double m = 0.5 * (a + b);
    return gk_adapt(it, a, m, 0.5 * tol, depth + 1) + gk_adapt(it, m, b, 0.5 * tol, depth + 1);
}

/* integral over [a, b] of x^p f_d (p = 0, 1, 2), absolute tolerance ~1e-16 of
 * the total mass; the interval is first cut at multiples of 1/sqrt(d) so the
 * narrow peak of f_d at large d is resolved. */
static double beta_integral(int32_t d, int p, double c, double a, double b) {
    if (b <= a) return 0.0;
    orc_integrand it = {d, p, c};
    double s = 1.0 / sqrt((double)d);
    double cuts[64];
    int nc = 0;
    cuts[nc++] = a;
    for (int k = -24; k <= 24; ++k) {
        double t = k * 0.5 * s;
        if (t > a && t < b) cuts[nc++] = t;
    }
    cuts[nc++] = b;
    double total = 0.0;
    for (int i = 0; i + 1 < nc; ++i) total += gk_adapt(&it, cuts[i], cuts[i + 1], 1e-17, 0);
    return total;
}

ORC_API double orc_beta_integral(int32_t d, int32_t p, double a, double b) {
    return beta_integral(d, p, 0.0, a, b);
}

/* ------------------------------------------------------------------------ */
/* Lloyd-Max scalar quantizer with K = 2^bits levels for f_d ([P2] pseudo-code
 * "precompute Lloyd-Max centroids", offline and reused; [P3] PolarQuant
 * paragraph: the optimal scalar quantizer is found with the Lloyd-Max
 * algorithm, i.e. continuous 1-D k-means).  Iteration: thresholds at the
 * midpoints of neighbouring centroids, then each centroid moves to the mean
 * of f_d over its cell; both cell integrals are computed by adaptive
 * Gauss-Kronrod quadrature (one plain code path for every d).  Symmetry
 * c_k = -c_{K-1-k} is imposed after every step (f_d is even).
 * Returns 0 on convergence (max |delta c| < tol), 1 if max_iter was reached.
 * distortion_out = d * sum_k int_cell (x - c_k)^2 f_d  (per-vector MSE of a
 * unit vector).  history (nullable, max_iter entries) receives the distortion
 * after each iteration. */
ORC_API int orc_lloyd_max(int32_t d, int32_t bits, int32_t max_iter, double tol,
                          double* centroids, double* distortion_out, int32_t* iters_out,
                          double* history) {
    if (d < 3 || bits < 1 || bits > 8 || max_iter < 1) return -1;
    int K = 1 << bits;
    double* c = centroids;
    double* t = (double*)malloc(sizeof(double) * (K + 1));
    double s = 1.0 / sqrt((double)d);
    double spread = (d == 3) ? 1.0 : 2.5 * s;
    if (spread > 1.0) spread = 1.0;
    for (int k = 0; k < K; ++k) c[k] = spread * (-1.0 + (2.0 * k + 1.0) / K);
    int it = 0, converged = 0;
    for (it = 0; it < max_iter; ++it) {
        t[0] = -1.0;
        t[K] = 1.0;
        for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        double maxd = 0.0;
        double nc[256];
        for (int k = 0; k < K; ++k) {
            double m0 = beta_integral(d, 0, 0.0, t[k], t[k + 1]);
            double m1 = beta_integral(d, 1, 0.0, t[k], t[k + 1]);
            nc[k] = (m0 > 0.0) ? m1 / m0 : c[k];
        }
        for (int k = 0; k < K / 2; ++k) {
            double v = 0.5 * (nc[K - 1 - k] - nc[k]);
            nc[k] = -v;
            nc[K - 1 - k] = v;
        }
        for (int k = 0; k < K; ++k) {
            double dd = fabs(nc[k] - c[k]);
            if (dd > maxd) maxd = dd;
            c[k] = nc[k];
        }
        if (history) {
            double D = 0.0;
            for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
            for (int k = 0; k < K; ++k) D += beta_integral(d, 3, c[k], t[k], t[k + 1]);
            history[it] = d * D;
        }
        if (maxd < tol) { converged = 1; ++it; break; }
    }
    if (distortion_out) {
        t[0] = -1.0;
        t[K] = 1.0;
        for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        double D = 0.0;
        for (int k = 0; k < K; ++k) D += beta_integral(d, 3, c[k], t[k], t[k + 1]);
        *distortion_out = d * D;
    }
    if (iters_out) *iters_out = it;
    free(t);
    return converged ? 0 : 1;
}

/* ------------------------------------------------------------------------ */
/* Packed record helpers (canonical layout in the header comment). */
ORC_API int32_t orc_words_per_plane(int32_t d) { return (d + 31) / 32; }

ORC_API void orc_pack_record(int32_t d, int32_t b, const int32_t* idx, const int32_t* sgn,
                             uint32_t* rec) {
    int W = (d + 31) / 32;
    memset(rec, 0, sizeof(uint32_t) * (size_t)W * b);
    for (int j = 0; j < d; ++j) {
        int w = j / 32, bit = j % 32;
        for (int p = 0; p < b - 1; ++p)
            if ((idx[j] >> p) & 1) rec[w * b + p] |= (1u << bit);
        if (sgn[j] > 0) rec[w * b + (b - 1)] |= (1u << bit);
    }
}

ORC_API void orc_unpack_record(int32_t d, int32_t b, const uint32_t* rec, int32_t* idx,
                               int32_t* sgn) {
    for (int j = 0; j < d; ++j) {
        int w = j / 32, bit = j % 32;
        int v = 0;
        for (int p = 0; p < b - 1; ++p) v |= (int)((rec[w * b + p] >> bit) & 1u) << p;
        idx[j] = v;
        sgn[j] = ((rec[w * b + (b - 1)] >> bit) & 1u) ? 1 : -1;
    }
}

/* ------------------------------------------------------------------------ */
/* Quantize n vectors ([P2] pseudo-code "Quant / DeQuant": rotate by Pi, find
 * the nearest centroid per coordinate; [P1] "two-stage inner-product
 * quantization" and [P3]: (b-1)-bit scalar stage, then a 1-bit QJL sign of
 * the residual; [P2] "potential challenges": the residual norm is one fp16
 * scalar; no per-block constants anywhere ([P2] PolarQuant section).
 *   nu = ||x||, xh = x / nu
 *   y = Pi xh, idx_j = argmin_k |y_j - c_k|  (ties: lower k)
 *   r = xh - Pi^T c[idx], gamma = ||r||
 *   z = S r, s_i = +1 iff z_i >= 0
 * pi, s, cen are the canonical fp32 tables (used in double).  x is double,
 * row i at x + i*ld.  Optional outputs: code_margin[n*d] = min_k |y_j - t_k|
 * over the midpoints t_k; sign_margin[n*d] = |z_i|; nu_out/gamma_out are the
 * unrounded norms; y_out[n*d] the rotated coordinates. */
ORC_API void orc_quantize(int32_t d, int32_t b, const float* pi, const float* s,
                          const float* cen, int64_t n, const double* x, int64_t ld,
                          uint32_t* planes, uint16_t* norms, double* code_margin,
                          double* sign_margin, double* nu_out, double* gamma_out,
                          double* y_out) {
    int K = 1 << (b - 1);
    int W = (d + 31) / 32;
    double c[256], t[256];
    for (int k = 0; k < K; ++k) c[k] = (double)cen[k];
    for (int k = 0; k + 1 < K; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
#pragma omp parallel
    {
        double* xh = (double*)malloc(sizeof(double) * d);
        double* y = (double*)malloc(sizeof(double) * d);
        double* r = (double*)malloc(sizeof(double) * d);
        double* z = (double*)malloc(sizeof(double) * d);
        int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * d);
        int32_t* sg = (int32_t*)malloc(sizeof(int32_t) * d);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            const double* xi = x + i * ld;
            double nu2 = 0.0;
            for (int j = 0; j < d; ++j) nu2 += xi[j] * xi[j];
            double nu = sqrt(nu2);
            for (int j = 0; j < d; ++j) xh[j] = (nu > 0.0) ? xi[j] / nu : 0.0;
            for (int jr = 0; jr < d; ++jr) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += (double)pi[(int64_t)jr * d + j] * xh[j];
                y[jr] = acc;
            }
            for (int j = 0; j < d; ++j) {
                int best = 0;
                double bd = fabs(y[j] - c[0]);
                for (int k = 1; k < K; ++k) {
                    double dk = fabs(y[j] - c[k]);
                    if (dk < bd) { bd = dk; best = k; }
                }
                idx[j] = best;
                if (code_margin) {
                    double m = INFINITY;
                    for (int k = 0; k + 1 < K; ++k) {
                        double mk = fabs(y[j] - t[k]);
                        if (mk < m) m = mk;
                    }
                    code_margin[i * d + j] = m;
                }
                if (y_out) y_out[i * d + j] = y[j];
            }
            double g2 = 0.0;
            for (int j = 0; j < d; ++j) {
                double back = 0.0;
                for (int jr = 0; jr < d; ++jr) back += (double)pi[(int64_t)jr * d + j] * c[idx[jr]];
                r[j] = (nu > 0.0) ? xh[j] - back : 0.0;
                g2 += r[j] * r[j];
            }
            double gamma = sqrt(g2);
            for (int ir = 0; ir < d; ++ir) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += (double)s[(int64_t)ir * d + j] * r[j];
                z[ir] = acc;
                sg[ir] = (acc >= 0.0) ? 1 : -1;
                if (sign_margin) sign_margin[i * d + ir] = fabs(acc);
            }
            orc_pack_record(d, b, idx, sg, planes + i * (int64_t)W * b);
            norms[2 * i] = orc_f16_from_double(nu);
            norms[2 * i + 1] = orc_f16_from_double(gamma);
            if (nu_out) nu_out[i] = nu;
            if (gamma_out) gamma_out[i] = gamma;
        }
        free(xh); free(y); free(r); free(z); free(idx); free(sg);
    }
}

/* ------------------------------------------------------------------------ */
/* The second stage for codes chosen elsewhere ([P1] two-stage section and
 * [P3] QJL paragraph: 1-bit signs of the sketch of the residual that the
 * codes leave; [P2] "potential challenges": its norm as one fp16 scalar):
 *   nu = ||x||, xh = x / nu, r = xh - Pi^T c[idx], gamma = ||r||,
 *   z = S r, s_i = +1 iff z_i >= 0,
 * with idx[n*d] given rather than the nearest centroids.  Used to check the
 * signs and gamma of a vector whose codes differ from orc_quantize's only at
 * coordinates on a decision boundary: the residual depends on the codes.
 * Outputs: packed records (the given codes and these signs), fp16 norms,
 * sign_margin[n*d] = |z_i| and the unrounded gamma (both optional).
 * A zero vector gets r = 0: gamma = 0 and all signs +1. */
ORC_API void orc_qjl_given_codes(int32_t d, int32_t b, const float* pi, const float* s,
                                 const float* cen, int64_t n, const double* x, int64_t ld,
                                 const int32_t* idx_in, uint32_t* planes, uint16_t* norms,
                                 double* sign_margin, double* gamma_out) {
    int W = (d + 31) / 32;
#pragma omp parallel
    {
        double* xh = (double*)malloc(sizeof(double) * d);
        double* r = (double*)malloc(sizeof(double) * d);
        int32_t* sg = (int32_t*)malloc(sizeof(int32_t) * d);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            const double* xi = x + i * ld;
            const int32_t* idx = idx_in + i * (int64_t)d;
            double nu2 = 0.0;
            for (int j = 0; j < d; ++j) nu2 += xi[j] * xi[j];
            double nu = sqrt(nu2);
            for (int j = 0; j < d; ++j) xh[j] = (nu > 0.0) ? xi[j] / nu : 0.0;
            double g2 = 0.0;
            for (int j = 0; j < d; ++j) {
                double back = 0.0;
                for (int jr = 0; jr < d; ++jr) back += (double)pi[(int64_t)jr * d + j] * (double)cen[idx[jr]];
                r[j] = (nu > 0.0) ? xh[j] - back : 0.0;
                g2 += r[j] * r[j];
            }
            for (int ir = 0; ir < d; ++ir) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += (double)s[(int64_t)ir * d + j] * r[j];
                sg[ir] = (acc >= 0.0) ? 1 : -1;
                if (sign_margin) sign_margin[i * d + ir] = fabs(acc);
            }
            orc_pack_record(d, b, idx, sg, planes + i * (int64_t)W * b);
            norms[2 * i] = orc_f16_from_double(nu);
            norms[2 * i + 1] = orc_f16_from_double(sqrt(g2));
            if (gamma_out) gamma_out[i] = sqrt(g2);
        }
        free(xh); free(r); free(sg);
    }
}

/* ------------------------------------------------------------------------ */
/* Dequantize ([P2] pseudo-code "dequant": y = centroids[idx], x = Pi^T y),
 * with the QJL term included so that <q, xt> equals the estimator below:
 *   xt = nu16 * (Pi^T c[idx] + alpha * gamma16 * S^T s),  alpha = sqrt(pi/2)/d.
 * out row i at out + i*ld. */
ORC_API void orc_dequantize(int32_t d, int32_t b, const float* pi, const float* s,
                            const float* cen, int64_t n, const uint32_t* planes,
                            const uint16_t* norms, double* out, int64_t ld) {
    int W = (d + 31) / 32;
    double alpha = sqrt(M_PI / 2.0) / (double)d;
#pragma omp parallel
    {
        int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * d);
        int32_t* sg = (int32_t*)malloc(sizeof(int32_t) * d);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            orc_unpack_record(d, b, planes + i * (int64_t)W * b, idx, sg);
            double nu = orc_f16_to_double(norms[2 * i]);
            double ga = orc_f16_to_double(norms[2 * i + 1]);
            for (int j = 0; j < d; ++j) {
                double a1 = 0.0, a2 = 0.0;
                for (int jr = 0; jr < d; ++jr) {
                    a1 += (double)pi[(int64_t)jr * d + j] * (double)cen[idx[jr]];
                    a2 += (double)s[(int64_t)jr * d + j] * (double)sg[jr];
                }
                out[i * ld + j] = nu * (a1 + alpha * ga * a2);
            }
        }
        free(idx); free(sg);
    }
}

/* ------------------------------------------------------------------------ */
/* Inner-product estimator ([P1] two-stage section: MSE stage then QJL on the
 * residual gives an unbiased inner-product quantizer; [P2] "integrate into
 * attention": inner products estimated with QJL; [P3] QJL paragraph):
 *   est(q, rec) = nu * ( <Pi q, c[idx]> + alpha * gamma * <S q, s> )
 * out[a * n + i] = scale * est(q_a, rec_i).  q row a at q + a*ldq.
 * If nu_exact / gamma_exact are non-null they replace the stored fp16 norms
 * (used to test unbiasedness without fp16 rounding). */
ORC_API void orc_estimate(int32_t d, int32_t b, const float* pi, const float* s,
                          const float* cen, int64_t nq, const double* q, int64_t ldq,
                          int64_t n, const uint32_t* planes, const uint16_t* norms,
                          const double* nu_exact, const double* gamma_exact, double scale,
                          double* out) {
    int W = (d + 31) / 32;
    double alpha = sqrt(M_PI / 2.0) / (double)d;
    double* qr = (double*)malloc(sizeof(double) * (size_t)nq * d);
    double* qp = (double*)malloc(sizeof(double) * (size_t)nq * d);
    for (int64_t a = 0; a < nq; ++a)
        for (int jr = 0; jr < d; ++jr) {
            double acc1 = 0.0, acc2 = 0.0;
            for (int j = 0; j < d; ++j) {
                acc1 += (double)pi[(int64_t)jr * d + j] * q[a * ldq + j];
                acc2 += (double)s[(int64_t)jr * d + j] * q[a * ldq + j];
            }
            qr[a * d + jr] = acc1;
            qp[a * d + jr] = acc2;
        }
#pragma omp parallel
    {
        int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * d);
        int32_t* sg = (int32_t*)malloc(sizeof(int32_t) * d);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            orc_unpack_record(d, b, planes + i * (int64_t)W * b, idx, sg);
            double nu = nu_exact ? nu_exact[i] : orc_f16_to_double(norms[2 * i]);
            double ga = gamma_exact ? gamma_exact[i] : orc_f16_to_double(norms[2 * i + 1]);
            for (int64_t a = 0; a < nq; ++a) {
                double m1 = 0.0, m2 = 0.0;
                for (int j = 0; j < d; ++j) {
                    m1 += qr[a * d + j] * (double)cen[idx[j]];
                    m2 += qp[a * d + j] * (double)sg[j];
                }
                out[a * n + i] = scale * nu * (m1 + alpha * ga * m2);
            }
        }
        free(idx); free(sg);
    }
    free(qr); free(qp);
}

/* ------------------------------------------------------------------------ */
/* MSE-only variant ([P2] pseudo-code "quant" / "dequant" as printed: b-bit
 * Lloyd-Max codes of the rotated coordinates, no QJL stage; [P1] notes that
 * this stage alone biases inner products).  Record: W groups of b code-plane
 * words (bit p of idx in word p), fp16 nu, and 0 in the gamma slot.
 *   quantize:   nu = ||x||, y = Pi x / nu, idx_j = argmin_k |y_j - c_k|
 *   dequantize: xt = nu16 * Pi^T c[idx]
 *   estimate:   est(q, rec) = nu16 * <Pi q, c[idx]>                            */
static void unpack_codes(int32_t d, int32_t b, const uint32_t* rec, int32_t* idx) {
    for (int j = 0; j < d; ++j) {
        int w = j / 32, bit = j % 32, v = 0;
        for (int p = 0; p < b; ++p) v |= (int)((rec[w * b + p] >> bit) & 1u) << p;
        idx[j] = v;
    }
}

ORC_API void orc_quantize_mse(int32_t d, int32_t b, const float* pi, const float* cen, int64_t n,
                              const double* x, int64_t ld, uint32_t* planes, uint16_t* norms,
                              double* code_margin) {
    int K = 1 << b;
    int W = (d + 31) / 32;
    double c[256], t[256];
    for (int k = 0; k < K; ++k) c[k] = (double)cen[k];
    for (int k = 0; k + 1 < K; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
#pragma omp parallel
    {
        double* y = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            const double* xi = x + i * ld;
            double nu2 = 0.0;
            for (int j = 0; j < d; ++j) nu2 += xi[j] * xi[j];
            double nu = sqrt(nu2);
            for (int jr = 0; jr < d; ++jr) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j)
                    acc += (double)pi[(int64_t)jr * d + j] * ((nu > 0.0) ? xi[j] / nu : 0.0);
                y[jr] = acc;
            }
            uint32_t* rec = planes + i * (int64_t)W * b;
            memset(rec, 0, sizeof(uint32_t) * (size_t)W * b);
            for (int j = 0; j < d; ++j) {
                int best = 0;
                double bd = fabs(y[j] - c[0]);
                for (int k = 1; k < K; ++k) {
                    double dk = fabs(y[j] - c[k]);
                    if (dk < bd) { bd = dk; best = k; }
                }
                for (int p = 0; p < b; ++p)
                    if ((best >> p) & 1) rec[(j / 32) * b + p] |= 1u << (j % 32);
                if (code_margin) {
                    double m = INFINITY;
                    for (int k = 0; k + 1 < K; ++k) m = fmin(m, fabs(y[j] - t[k]));
                    code_margin[i * d + j] = m;
                }
            }
            norms[2 * i] = orc_f16_from_double(nu);
            norms[2 * i + 1] = 0;
        }
        free(y);
    }
}

ORC_API void orc_dequantize_mse(int32_t d, int32_t b, const float* pi, const float* cen,
                                int64_t n, const uint32_t* planes, const uint16_t* norms,
                                double* out, int64_t ld) {
    int W = (d + 31) / 32;
#pragma omp parallel
    {
        int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * d);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            unpack_codes(d, b, planes + i * (int64_t)W * b, idx);
            double nu = orc_f16_to_double(norms[2 * i]);
            for (int j = 0; j < d; ++j) {
                double a1 = 0.0;
                for (int jr = 0; jr < d; ++jr)
                    a1 += (double)pi[(int64_t)jr * d + j] * (double)cen[idx[jr]];
                out[i * ld + j] = nu * a1;
            }
        }
        free(idx);
    }
}

ORC_API void orc_estimate_mse(int32_t d, int32_t b, const float* pi, const float* cen,
                              int64_t nq, const double* q, int64_t ldq, int64_t n,
                              const uint32_t* planes, const uint16_t* norms, double scale,
                              double* out) {
    int W = (d + 31) / 32;
    double* qr = (double*)malloc(sizeof(double) * (size_t)nq * d);
    for (int64_t a = 0; a < nq; ++a)
        for (int jr = 0; jr < d; ++jr) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j) acc += (double)pi[(int64_t)jr * d + j] * q[a * ldq + j];
            qr[a * d + jr] = acc;
        }
#pragma omp parallel
    {
        int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * d);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            unpack_codes(d, b, planes + i * (int64_t)W * b, idx);
            double nu = orc_f16_to_double(norms[2 * i]);
            for (int64_t a = 0; a < nq; ++a) {
                double m1 = 0.0;
                for (int j = 0; j < d; ++j) m1 += qr[a * d + j] * (double)cen[idx[j]];
                out[a * n + i] = scale * nu * m1;
            }
        }
        free(idx);
    }
    free(qr);
}

/* ------------------------------------------------------------------------ */
/* Top-k over a score matrix ([P1] nearest-neighbour section; [P3] vector
 * search paragraph): for each query row, the k largest scores, ordered by
 * (score descending, index ascending).  scores[a * n + i]. */
ORC_API void orc_topk(int64_t nq, int64_t n, const double* scores, int32_t k, int64_t* out_idx,
                      double* out_score) {
#pragma omp parallel for schedule(static)
    for (int64_t a = 0; a < nq; ++a) {
        const double* row = scores + a * n;
        int64_t* bi = out_idx + a * k;
        double* bs = out_score + a * k;
        int cnt = 0;
        for (int64_t i = 0; i < n; ++i) {
            double v = row[i];
            /* position where (v, i) goes: before the first entry it beats */
            int pos = cnt;
            while (pos > 0 && (v > bs[pos - 1] || (v == bs[pos - 1] && i < bi[pos - 1]))) --pos;
            if (pos >= k) continue;
            int last = (cnt < k) ? cnt : k - 1;
            for (int p = last; p > pos; --p) { bs[p] = bs[p - 1]; bi[p] = bi[p - 1]; }
            bs[pos] = v;
            bi[pos] = i;
            if (cnt < k) ++cnt;
        }
        for (int p = cnt; p < k; ++p) { bs[p] = -INFINITY; bi[p] = -1; }
    }
}

/* number of OpenMP threads the oracle runs with */
ORC_API int32_t orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
