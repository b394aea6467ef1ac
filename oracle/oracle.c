/*
 * CPU reference ("the oracle") for the deterministic Split-K LoRA shrink and
 * the LoRA expand.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may load,
 * link or call this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * Everything here is the plain definition written out, in double precision,
 * with loops a reader can check against the paper by eye.  Source:
 * "Reproducible LoRA Inference Through Deterministic Split-K Reduction"
 * (Balusamy & Mohan, arXiv 2611.10334), abbreviated RLI below.
 *
 * Operand layouts follow RLI Eq. 1 (Y = X W^T + s (X A^T) B^T):
 *   x  bf16 [M][K]   (X in R^{M x H}, K = H)
 *   A  bf16 [r][K]   (A in R^{r x H})
 *   B  bf16 [N][r]   (B in R^{H_out x r}, N = H_out)
 *   h  [M][r]        shrink output X A^T
 *   y  bf16 [M][N]   the output the expand adds into
 * bf16 values are passed as their uint16 bit patterns.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC oracle.c -lm
 * (no fast-math: every double operation is IEEE round-to-nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> double.                                                      */
/* bf16 is the upper 16 bits of an IEEE binary32: 1 sign, 8 exponent and 7    */
/* stored significand bits (8 significant bits).                            */
/* ------------------------------------------------------------------------ */

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint16_t float_bits_hi(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/*
 * Round a double to the nearest bf16 value, ties to even, in ONE rounding
 * (RLI section 6.2 and Fig. 5 rely on this conversion: fp32 shrink values on
 * either side of, or exactly on, a bf16 midpoint become different bf16 values).
 *
 * Method: the bf16 quantum (distance between neighbouring bf16 values) at v is
 * 2^(e-8) where v = m * 2^e with 0.5 <= |m| < 1 (8 significant bits), but never
 * below 2^-133, the spacing of bf16 subnormals (min normal 2^-126, 7 stored
 * bits).  v / quantum is then rounded to an integer with rint(), which under
 * the default floating-point environment rounds half to even.  Division and
 * multiplication by a power of two are exact in double.
 */
uint16_t oracle_bf16_rne_from_double(double v)
{
    if (isnan(v))
        return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    if (isinf(v) || v == 0.0)
        return float_bits_hi((float)v);          /* exact: +-inf, +-0 */
    int e;
    (void)frexp(v, &e);                           /* |v| = m 2^e, m in [0.5,1) */
    int qexp = e - 8;
    if (qexp < -133)
        qexp = -133;
    double q = ldexp(1.0, qexp);
    double rounded = rint(v / q) * q;             /* exact scaling, one RNE */
    /* Largest finite bf16 is (2 - 2^-7) * 2^127; anything rounding beyond it
       becomes infinity (IEEE overflow under round-to-nearest). */
    const double bf16_max = ldexp(255.0, 120);
    if (fabs(rounded) > bf16_max)
        return (uint16_t)(rounded > 0 ? 0x7F80u : 0xFF80u);
    if (rounded == 0.0)
        return (uint16_t)(signbit(v) ? 0x8000u : 0x0000u);
    /* `rounded` is a bf16 value, hence exactly a float whose low 16 bits are 0 */
    return float_bits_hi((float)rounded);
}

uint16_t oracle_bf16_rne_from_float(float f)
{
    return oracle_bf16_rne_from_double((double)f);  /* float -> double is exact */
}

void oracle_bf16_rne_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne_from_double(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Shrink (RLI Eq. 1, the X A^T term, and Eq. 3 summed over all partitions).  */
/*   h[i][j] = scale * sum_{k=0}^{K-1} x[i][k] * A[j][k]                      */
/* Products of two bf16 values are exact in double; the sum runs k ascending  */
/* in double.                                                                */
/* ------------------------------------------------------------------------ */
void oracle_shrink(const uint16_t* x, const uint16_t* A, int64_t M, int64_t K, int64_t r,
                   double scale, double* h)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += oracle_bf16_to_double(x[i * K + k]) * oracle_bf16_to_double(A[j * K + k]);
            h[i * r + j] = scale * acc;
        }
    }
}

/* Sum of |x[i][k] A[j][k]| (for rounding-error bounds) and the two Euclidean
   norms ||x_i|| and ||A_j|| used by the shrink tolerance. */
void oracle_shrink_bounds(const uint16_t* x, const uint16_t* A, int64_t M, int64_t K, int64_t r,
                          double* abs_sum, double* xnorm, double* anorm)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = oracle_bf16_to_double(x[i * K + k]);
            s += v * v;
        }
        xnorm[i] = sqrt(s);
        for (int64_t j = 0; j < r; ++j) {
            double t = 0.0;
            for (int64_t k = 0; k < K; ++k)
                t += fabs(oracle_bf16_to_double(x[i * K + k]) * oracle_bf16_to_double(A[j * K + k]));
            abs_sum[i * r + j] = t;
        }
    }
    for (int64_t j = 0; j < r; ++j) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = oracle_bf16_to_double(A[j * K + k]);
            s += v * v;
        }
        anorm[j] = sqrt(s);
    }
}

/* ------------------------------------------------------------------------ */
/* Split-K partials (RLI Eq. 3): the reduction dimension is cut into S       */
/* subsets; here, as drawn in RLI Fig. 1 (K0..K7), S contiguous chunks of     */
/* K/S.  P[s][i][j] = sum_{k in K_s} x[i][k] A[j][k], in double.             */
/* ------------------------------------------------------------------------ */
void oracle_split_partials(const uint16_t* x, const uint16_t* A, int64_t M, int64_t K, int64_t r,
                           int64_t S, double* P)
{
    int64_t Kc = K / S;
    for (int64_t s = 0; s < S; ++s)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < r; ++j) {
                double acc = 0.0;
                for (int64_t k = s * Kc; k < (s + 1) * Kc; ++k)
                    acc += oracle_bf16_to_double(x[i * K + k]) * oracle_bf16_to_double(A[j * K + k]);
                P[(s * M + i) * r + j] = acc;
            }
}

/* ------------------------------------------------------------------------ */
/* Fixed-order combine of S fp32 partials, in fp32 (float) arithmetic.       */
/*                                                                          */
/* Pairwise tree (RLI section 4.3 describes an earlier deterministic design  */
/* whose second kernel summed the Split-K partials along a fixed pairwise     */
/* tree): level 1 adds neighbours (P0+P1), (P2+P3), ...; each                 */
/* further level adds neighbouring results of the level before, until one    */
/* value is left; then one multiply by the scale (RLI Alg. 1 applies the      */
/* scale after the sum).  S must be a power of two.                          */
/*                                                                          */
/* Sequential fold (RLI Alg. 1 as printed): total = 0; total += P_j for       */
/* j = 0..S-1 in increasing partition order; then times the scale.           */
/*                                                                          */
/* P is laid out [S][n]; out[n].                                             */
/* ------------------------------------------------------------------------ */
void oracle_combine_tree_f32(const float* P, int64_t S, int64_t n, float scale, float* out)
{
    float level[64];
    for (int64_t e = 0; e < n; ++e) {
        for (int64_t s = 0; s < S; ++s)
            level[s] = P[s * n + e];
        int64_t width = S;
        while (width > 1) {
            for (int64_t q = 0; q < width / 2; ++q) {
                volatile float sum = level[2 * q] + level[2 * q + 1];   /* one fp32 rounding */
                level[q] = sum;
            }
            width /= 2;
        }
        volatile float scaled = level[0] * scale;
        out[e] = scaled;
    }
}

void oracle_combine_sequential_f32(const float* P, int64_t S, int64_t n, float scale, float* out)
{
    for (int64_t e = 0; e < n; ++e) {
        volatile float total = 0.0f;
        for (int64_t s = 0; s < S; ++s)
            total = total + P[s * n + e];
        volatile float scaled = total * scale;
        out[e] = scaled;
    }
}

/* ------------------------------------------------------------------------ */
/* Expand (RLI Eq. 1, the s (X A^T) B^T term added to Y).                    */
/* The fp32 shrink output is converted to bf16 (round to nearest even) before */
/* it meets B: RLI section 6.2 traces how two fp32 shrink values that round  */
/* to different bf16 values change the next layer's input.                   */
/*   hb[i][j] = bf16_rne(h[i][j])                                           */
/*   e[i][n]  = y[i][n] + scale * sum_{j<r} hb[i][j] * B[n][j]   (double)     */
/*   out[i][n] = bf16_rne(e[i][n])   (one rounding, straight from double)    */
/* Also returns sum_j |hb B| per element for error bounds.                   */
/* ------------------------------------------------------------------------ */
void oracle_expand(const float* h, const uint16_t* B, const uint16_t* y_in, int64_t M, int64_t r,
                   int64_t N, double scale, double* e_out, uint16_t* y_out, double* abs_sum)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double hb[256];
        for (int64_t j = 0; j < r; ++j)
            hb[j] = oracle_bf16_to_double(oracle_bf16_rne_from_float(h[i * r + j]));
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t j = 0; j < r; ++j) {
                double p = hb[j] * oracle_bf16_to_double(B[n * r + j]);
                acc += p;
                aacc += fabs(p);
            }
            double e = oracle_bf16_to_double(y_in[i * N + n]) + scale * acc;
            e_out[i * N + n] = e;
            y_out[i * N + n] = oracle_bf16_rne_from_double(e);
            if (abs_sum)
                abs_sum[i * N + n] = fabs(scale) * aacc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Compensated expand ("Demystifying Numerical Instability in LLM Inference  */
/* ... with HEAL", section 3, GEMM algebraic compensation, Eq. 10): the      */
/* fp32 input of a 16-bit product is written as a leading 16-bit value plus  */
/* a 16-bit residual, and the product is the sum of the two products.  Read  */
/* here with bf16 halves (bf16 has the fp32 exponent range, so the residual  */
/* needs no 2^10 shift):                                                     */
/*   hi = bf16_rne(h),  lo = bf16_rne(h - hi)      (h - hi is exact)          */
/*   e[i][n]  = y[i][n] + scale * sum_{j<r} (hi_j + lo_j) * B[n][j]  (double) */
/*   out[i][n] = bf16_rne(e[i][n])                                           */
/* Also returns sum_j (|hi B| + |lo B|) per element for error bounds.       */
/* ------------------------------------------------------------------------ */
void oracle_expand_compensated(const float* h, const uint16_t* B, const uint16_t* y_in, int64_t M, int64_t r,
                               int64_t N, double scale, double* e_out, uint16_t* y_out, double* abs_sum)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double hi[256], lo[256];
        for (int64_t j = 0; j < r; ++j) {
            const double hv = (double)h[i * r + j];
            hi[j] = oracle_bf16_to_double(oracle_bf16_rne_from_float(h[i * r + j]));
            lo[j] = oracle_bf16_to_double(oracle_bf16_rne_from_double(hv - hi[j]));
        }
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t j = 0; j < r; ++j) {
                const double b = oracle_bf16_to_double(B[n * r + j]);
                acc += hi[j] * b + lo[j] * b;
                aacc += fabs(hi[j] * b) + fabs(lo[j] * b);
            }
            double e = oracle_bf16_to_double(y_in[i * N + n]) + scale * acc;
            e_out[i * N + n] = e;
            y_out[i * N + n] = oracle_bf16_rne_from_double(e);
            if (abs_sum)
                abs_sum[i * N + n] = fabs(scale) * aacc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Multi-adapter (SGMV) shrink and expand.  RLI section 5.2 replays shrink   */
/* operations together with the token-to-adapter mapping: which adapter each */
/* token uses.  Per token i with a = ids[i]:                                 */
/*   a outside [0, n_adapters): no LoRA - h row is 0, y row is unchanged.    */
/*   otherwise the single-adapter definitions with A_a, B_a, r_a, scale_a;   */
/*   h columns j >= r_a are 0.                                              */
/* A_a is [r_a][K]; B_a is [N][r_a]; h is [M][r_max].                        */
/* ------------------------------------------------------------------------ */
void oracle_sgmv_shrink(const uint16_t* x, const uint16_t* const* A_list, const int32_t* ranks,
                        const float* scales, const int32_t* ids, int32_t n_adapters,
                        int64_t M, int64_t K, int64_t r_max, double* h)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        int32_t a = ids[i];
        for (int64_t j = 0; j < r_max; ++j)
            h[i * r_max + j] = 0.0;
        if (a < 0 || a >= n_adapters)
            continue;
        const uint16_t* A = A_list[a];
        double scale = scales ? (double)scales[a] : 1.0;
        for (int64_t j = 0; j < ranks[a]; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += oracle_bf16_to_double(x[i * K + k]) * oracle_bf16_to_double(A[j * K + k]);
            h[i * r_max + j] = scale * acc;
        }
    }
}

void oracle_sgmv_expand(const float* h, const uint16_t* const* B_list, const int32_t* ranks,
                        const float* scales, const int32_t* ids, int32_t n_adapters,
                        const uint16_t* y_in, int64_t M, int64_t N, int64_t r_max,
                        double* e_out, uint16_t* y_out, double* abs_sum)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        int32_t a = ids[i];
        if (a < 0 || a >= n_adapters) {
            for (int64_t n = 0; n < N; ++n) {
                y_out[i * N + n] = y_in[i * N + n];
                e_out[i * N + n] = oracle_bf16_to_double(y_in[i * N + n]);
                if (abs_sum)
                    abs_sum[i * N + n] = 0.0;
            }
            continue;
        }
        int64_t r = ranks[a];
        const uint16_t* B = B_list[a];
        double scale = scales ? (double)scales[a] : 1.0;
        double hb[256];
        for (int64_t j = 0; j < r; ++j)
            hb[j] = oracle_bf16_to_double(oracle_bf16_rne_from_float(h[i * r_max + j]));
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t j = 0; j < r; ++j) {
                double p = hb[j] * oracle_bf16_to_double(B[n * r + j]);
                acc += p;
                aacc += fabs(p);
            }
            double e = oracle_bf16_to_double(y_in[i * N + n]) + scale * acc;
            e_out[i * N + n] = e;
            y_out[i * N + n] = oracle_bf16_rne_from_double(e);
            if (abs_sum)
                abs_sum[i * N + n] = fabs(scale) * aacc;
        }
    }
}

/* Sets the number of OpenMP threads later calls run with (n >= 1) and returns
   the previous setting, so a timing run can take one thread and restore the
   host's default afterwards. */
int oracle_set_threads(int n)
{
#ifdef _OPENMP
    const int prev = omp_get_max_threads();
    omp_set_num_threads(n > 0 ? n : 1);
    return prev;
#else
    (void)n;
    return 1;
#endif
}

/* Number of OpenMP threads this library runs with (for reporting). */
int oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
    #pragma omp parallel
    {
        #pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
