/*
 * nvfp4_oracle.c -- plain, slow, obviously-correct CPU oracle for the NVFP4
 * weight-only projection GEMV of batched LLM decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The HIP product library
 * shares no code, header, table or constant generator with this file, and this
 * file includes nothing from the product.
 *
 * What it computes (the method of the pages, restated):
 *   Atlas PR #266, "What it does" (PR description) and the GPU A/B section:
 *   for n concurrent decode tokens each projection reads one NVFP4 weight
 *   matrix W (N rows x K columns) and produces y[t][r] = sum_k x[t][k]*W[r][k].
 *   Tiling the n tokens only changes the accumulation order, never the result
 *   (same page, "Numeric identity" caveat), so the oracle evaluates the plain
 *   definition, in fp64, with k ascending.
 *
 * Number formats (the pages only name NVFP4; the bit-level definitions are the
 * OCP Microscaling FP4 E2M1 and OCP FP8 E4M3 "FN" encodings):
 *   E2M1 code c (4 bits): sign = bit 3, magnitude = {0,.5,1,1.5,2,3,4,6}[c&7].
 *   E4M3 byte b: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
 *     exponent 0 is subnormal m/8 * 2^-6; 0x7F/0xFF are NaN; no infinities;
 *     largest finite value 448 (0x7E).
 *
 * Canonical packed layout (the pages are silent; this is the layout every
 * entry point of the oracle reads):
 *   codes  [N][K/2] bytes: element (r,k) is byte r*K/2 + k/2, low nibble for
 *          even k, high nibble for odd k;
 *   scales [N][K/16] bytes: one E4M3 byte per 16 consecutive k of one row;
 *   gscale: fp32 multiplier applied to every weight;
 *   X      [n][K] bf16 bit patterns; Y / A outputs [n][N] fp64.
 *
 * Parity pins for every function here live in tests/test_oracle.py.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stddef.h>
#include <string.h>

/* ---- decode tables ----------------------------------------------------- */

/* E2M1 magnitudes and signs written out code by code (OCP FP4 E2M1). */
static const double E2M1_TABLE[16] = {
    0.0,  0.5,  1.0,  1.5,  2.0,  3.0,  4.0,  6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

/* E4M3FN value of every byte, filled once from the field definition. */
static double E4M3_TABLE[256];
static int e4m3_ready = 0;

static void e4m3_fill(void)
{
    if (e4m3_ready)
        return;
    for (int b = 0; b < 256; ++b) {
        int sign = (b >> 7) & 1;
        int expo = (b >> 3) & 15;
        int mant = b & 7;
        double v;
        if ((b & 0x7F) == 0x7F)
            v = NAN;
        else if (expo == 0)
            v = ldexp((double)mant / 8.0, -6);
        else
            v = ldexp(1.0 + (double)mant / 8.0, expo - 7);
        E4M3_TABLE[b] = sign ? -v : v;
    }
    e4m3_ready = 1;
}

double oracle_e2m1(int code) { return E2M1_TABLE[code & 15]; }

double oracle_e4m3(int byte)
{
    e4m3_fill();
    return E4M3_TABLE[byte & 255];
}

/* ---- bf16 helpers -------------------------------------------------------- */

/* bf16 bit pattern -> exact fp64 value (bf16 is the top half of an fp32). */
static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round an fp64 value to the nearest bf16 (ties to even), directly from fp64.
 * bf16: 8 significant bits, exponent range of fp32 (normal >= 2^-126,
 * subnormal step 2^-133), overflow to +-inf above the largest finite value. */
uint16_t oracle_bf16_rne(double v)
{
    if (isnan(v))
        return 0x7FC0;
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    uint16_t sign = (uint16_t)(neg << 15);
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                   /* quantum for 8 significant bits */
    if (q < -133)
        q = -133;                    /* subnormal bf16 quantum */
    double m = nearbyint(ldexp(a, -q)); /* default FP env rounds ties to even */
    double r = ldexp(m, q);
    if (r > 0x1.FEp127)              /* rounds past the largest finite bf16 */
        return (uint16_t)(sign | 0x7F80);
    float f = (float)r;              /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

void oracle_bf16_rne_array(const double *v, size_t count, uint16_t *out)
{
    for (size_t i = 0; i < count; ++i)
        out[i] = oracle_bf16_rne(v[i]);
}

/* ---- quantiser (input recipe) ------------------------------------------ */

/* Nearest E2M1 magnitude index for q >= 0, ties to the even index, values
 * beyond 6 saturate to index 7.  Plain scan of the 8 grid points. */
int oracle_e2m1_rne_index(double q)
{
    int best = 0;
    double best_err = fabs(q - E2M1_TABLE[0]);
    for (int i = 1; i < 8; ++i) {
        double err = fabs(q - E2M1_TABLE[i]);
        if (err < best_err || (err == best_err && (i % 2) == 0)) {
            best = i;
            best_err = err;
        }
    }
    return best;
}

/* Nearest non-negative finite E4M3 byte for v >= 0, ties to even mantissa
 * (even byte), saturating at 448 (0x7E).  Plain scan of bytes 0x00..0x7E. */
int oracle_e4m3_rne(double v)
{
    e4m3_fill();
    if (v >= E4M3_TABLE[0x7E])
        return 0x7E;
    int best = 0;
    double best_err = fabs(v - E4M3_TABLE[0]);
    for (int b = 1; b <= 0x7E; ++b) {
        double err = fabs(v - E4M3_TABLE[b]);
        if (err < best_err || (err == best_err && (b % 2) == 0)) {
            best = b;
            best_err = err;
        }
    }
    return best;
}

/* Tensor scale of the recipe: fp32(amax / (6 * 448)), amax = max |w|. */
float oracle_tensor_scale(const float *W, size_t count)
{
    float amax = 0.0f;
    for (size_t i = 0; i < count; ++i) {
        float a = fabsf(W[i]);
        if (a > amax)
            amax = a;
    }
    return (float)((double)amax / (6.0 * 448.0));
}

/* Quantise W [N][K] fp32 (finite) to the canonical layout.
 *   g = fp32(amax_tensor / 2688)
 *   per 16-block: s = E4M3_RNE(amax_block / (6 g)), d = E4M3[s] * g
 *   per element: code = sign(w) | E2M1_RNE(|w| / d), or magnitude 0 if d == 0.
 * All-zero tensors give g = 0, scale bytes 0 and magnitude-0 codes. */
void oracle_quantize(const float *W, int N, int K, uint8_t *codes,
                     uint8_t *scales, float *gscale_out)
{
    e4m3_fill();
    float g = oracle_tensor_scale(W, (size_t)N * (size_t)K);
    *gscale_out = g;
    int nb = K / 16;
    memset(codes, 0, (size_t)N * (size_t)(K / 2));
#pragma omp parallel for schedule(static)
    for (int r = 0; r < N; ++r) {
        for (int b = 0; b < nb; ++b) {
            const float *w = W + (size_t)r * K + (size_t)b * 16;
            double amax_b = 0.0;
            for (int i = 0; i < 16; ++i)
                if (fabs((double)w[i]) > amax_b)
                    amax_b = fabs((double)w[i]);
            int s = 0;
            if (g > 0.0f)
                s = oracle_e4m3_rne(amax_b / (6.0 * (double)g));
            scales[(size_t)r * nb + b] = (uint8_t)s;
            double d = E4M3_TABLE[s] * (double)g;
            for (int i = 0; i < 16; ++i) {
                int k = b * 16 + i;
                int mag = d > 0.0 ? oracle_e2m1_rne_index(fabs((double)w[i]) / d) : 0;
                int code = (signbit(w[i]) ? 8 : 0) | mag;
                size_t byte = (size_t)r * (K / 2) + (size_t)(k / 2);
                if (k % 2 == 0)
                    codes[byte] = (uint8_t)((codes[byte] & 0xF0) | code);
                else
                    codes[byte] = (uint8_t)((codes[byte] & 0x0F) | (code << 4));
            }
        }
    }
}

/* ---- dequant and GEMV ---------------------------------------------------- */

/* Element (r,k) of the canonical codes array. */
static int code_at(const uint8_t *codes, int K, int r, int k)
{
    uint8_t byte = codes[(size_t)r * (K / 2) + (size_t)(k / 2)];
    return (k % 2 == 0) ? (byte & 15) : (byte >> 4);
}

/* Dense fp64 weight: Wd[r][k] = E2M1[code] * E4M3[scale] * gscale (exact). */
void oracle_dequant(const uint8_t *codes, const uint8_t *scales, float gscale,
                    int N, int K, double *Wd)
{
    e4m3_fill();
    for (int r = 0; r < N; ++r)
        for (int k = 0; k < K; ++k)
            Wd[(size_t)r * K + k] = E2M1_TABLE[code_at(codes, K, r, k)] *
                                    E4M3_TABLE[scales[(size_t)r * (K / 16) + k / 16]] *
                                    (double)gscale;
}

/* y[t][r] = sum_{k ascending} w(r,k) * x[t][k] in fp64, and
 * A[t][r] = sum_k |w(r,k) * x[t][k]| (the error-bound scale).
 * nthreads <= 0 uses the OpenMP default. */
void oracle_gemv(const uint8_t *codes, const uint8_t *scales, float gscale,
                 const uint16_t *X, int n, int N, int K, double *Y, double *A,
                 int nthreads)
{
    e4m3_fill();
    /* nthreads > 0 sets this call's thread count only (a clause on the
       region, not the process-wide setting). */
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    const int nt = 1;
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int r = 0; r < N; ++r) {
        for (int t = 0; t < n; ++t) {
            double acc = 0.0, mag = 0.0;
            for (int k = 0; k < K; ++k) {
                double w = E2M1_TABLE[code_at(codes, K, r, k)] *
                           E4M3_TABLE[scales[(size_t)r * (K / 16) + k / 16]] *
                           (double)gscale;
                double p = w * bf16_bits_to_double(X[(size_t)t * K + k]);
                acc += p;
                mag += fabs(p);
            }
            Y[(size_t)t * N + r] = acc;
            A[(size_t)t * N + r] = mag;
        }
    }
}

/* Same sum for a single output element; used to check sampled outputs of the
 * full-size workloads one by one. */
double oracle_gemv_one(const uint8_t *codes, const uint8_t *scales, float gscale,
                       const uint16_t *X, int K, int t, int r, double *A_out)
{
    e4m3_fill();
    double acc = 0.0, mag = 0.0;
    for (int k = 0; k < K; ++k) {
        double w = E2M1_TABLE[code_at(codes, K, r, k)] *
                   E4M3_TABLE[scales[(size_t)r * (K / 16) + k / 16]] *
                   (double)gscale;
        double p = w * bf16_bits_to_double(X[(size_t)t * K + k]);
        acc += p;
        mag += fabs(p);
    }
    if (A_out)
        *A_out = mag;
    return acc;
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
