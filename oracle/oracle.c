/*
 * CPU oracle for the factorized linear layer  Y = (X . A) . B.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * reference that the GPU path is checked against.  It shares no code with the
 * HIP library and must never be linked into it or called from it.
 *
 * What it computes (the plain definition):
 *   "Why Smaller Is Slower? Dimensional Misalignment in Compressed LLMs",
 *   section 1 / Figure 1: Y = X.W with W replaced by two factors A.B whose
 *   inner dimension is the rank r, i.e. two smaller GEMMs;
 *   "LowRankArena ...", Prerequisites, Figure A: the forward pass y = Wx
 *   becomes y = A(Bx) (column-vector orientation of the same product).
 * With X[M x K], A[K x r], B[r x N] (row-major):
 *     T[m][j] = sum_{k=0}^{K-1} X[m][k] * A[k][j]
 *     Y[m][n] = sum_{j=0}^{r-1} T[m][j] * B[j][n]
 *
 * Arithmetic rule (fixed so results are reproducible and padding-invariant):
 *   - float64 throughout; T is never rounded to a narrower type;
 *   - every product is rounded to float64 and then added (no fused
 *     multiply-add: build with -ffp-contract=off);
 *   - every sum starts from +0.0 and runs over its reduction index in
 *     increasing order.  The loops below are ordered m, then reduction index,
 *     then output column, which accumulates each output element in exactly
 *     that sequential order.
 * bf16 inputs are decoded exactly (a bf16 value is the upper half of an
 * IEEE float32, and every float32 is exactly a float64).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 bit pattern -> float64, exact. */
static double bf16_to_f64(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_bf16_decode(const uint16_t* src, double* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = bf16_to_f64(src[i]);
}

/* C[rows x cols] = P[rows x inner] . Q[inner x cols], sequential sums. */
static void matmul_seq(const double* P, const double* Q, double* C,
                       int64_t rows, int64_t inner, int64_t cols, int nthreads) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i) {
        double* c = C + i * cols;
        for (int64_t n = 0; n < cols; ++n) c[n] = 0.0;
        for (int64_t k = 0; k < inner; ++k) {
            const double p = P[i * inner + k];
            const double* q = Q + k * cols;
            for (int64_t n = 0; n < cols; ++n) {
                double prod = p * q[n];
                c[n] = c[n] + prod;
            }
        }
    }
    (void)nthreads;
}

/* Y = (X.A).B in float64; T[M x r] is caller-provided scratch. */
void oracle_lowrank_f64(const double* X, const double* A, const double* B,
                        int64_t M, int64_t K, int64_t r, int64_t N,
                        double* T, double* Y, int nthreads) {
    matmul_seq(X, A, T, M, K, r, nthreads);
    matmul_seq(T, B, Y, M, r, N, nthreads);
}

/* Same, from bf16 bit patterns. */
int oracle_lowrank_bf16(const uint16_t* Xb, const uint16_t* Ab, const uint16_t* Bb,
                        int64_t M, int64_t K, int64_t r, int64_t N,
                        double* Y, int nthreads) {
    double* X = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
    double* A = (double*)malloc(sizeof(double) * (size_t)(K * r + 1));
    double* B = (double*)malloc(sizeof(double) * (size_t)(r * N + 1));
    double* T = (double*)malloc(sizeof(double) * (size_t)(M * r + 1));
    if (!X || !A || !B || !T) {
        free(X); free(A); free(B); free(T);
        return 1;
    }
    oracle_bf16_decode(Xb, X, M * K);
    oracle_bf16_decode(Ab, A, K * r);
    oracle_bf16_decode(Bb, B, r * N);
    oracle_lowrank_f64(X, A, B, M, K, r, N, T, Y, nthreads);
    free(X); free(A); free(B); free(T);
    return 0;
}

/*
 * Selected outputs only: Y[rows[a]][cols[b]] -> Yout[a * ncols + b].
 * For each selected row the full T row is formed (sequential over k), then
 * each selected output sums T[m][j] * B[j][n] sequentially over j.
 */
int oracle_lowrank_bf16_sampled(const uint16_t* Xb, const uint16_t* Ab, const uint16_t* Bb,
                                int64_t M, int64_t K, int64_t r, int64_t N,
                                const int64_t* rows, int64_t nrows,
                                const int64_t* cols, int64_t ncols,
                                double* Yout, int nthreads) {
    (void)M; (void)N;
    int status = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t a = 0; a < nrows; ++a) {
        const int64_t m = rows[a];
        double* T = (double*)malloc(sizeof(double) * (size_t)r);
        if (!T) { status = 1; continue; }
        for (int64_t j = 0; j < r; ++j) T[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double x = bf16_to_f64(Xb[m * K + k]);
            const uint16_t* arow = Ab + k * r;
            for (int64_t j = 0; j < r; ++j) {
                double prod = x * bf16_to_f64(arow[j]);
                T[j] = T[j] + prod;
            }
        }
        for (int64_t b = 0; b < ncols; ++b) {
            const int64_t n = cols[b];
            double s = 0.0;
            for (int64_t j = 0; j < r; ++j) {
                double prod = T[j] * bf16_to_f64(Bb[j * N + n]);
                s = s + prod;
            }
            Yout[a * ncols + b] = s;
        }
        free(T);
    }
    (void)nthreads;
    return status;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
