/*
 * CPU oracle for dense row-major GEMM, C[M x N] = A[M x K] * B[K x N].
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the GPU library and includes
 * no HIP header.
 *
 * What it computes (plain definition, no blocking, no reordering):
 *   C_ref[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]          (k ascending)
 *   D[i][j]     = sum_{k=0}^{K-1} |A[i][k]| * |B[k][j]|      (error scale)
 * Sources: the row-major problem statement C = A x B with 2MNK flops in
 * "GEMM: from naive to shared memory tiling and register blocking"
 * (quant67.com, introduction and section 1, the one-thread-per-output
 * kernel); the per-element K loop of the naive kernel in "sgemm - beyond
 * cuBLAS" (wingedge777.com, section 1); the 2MNK operation count in the
 * lqnn.cn SGEMM article (section 1.1); C = A x B with A of size M x K in
 * "hgemm_naive_kernel explained" (yuyanqi.com, section 1.1).
 *
 * Arithmetic: every input is widened to double before use.  An FP32 x FP32
 * product carries at most 48 significant bits and an FP16 x FP16 product at
 * most 22, so each product is exact in double and only the K-1 additions
 * round.  The loop order is i, k, j with k ascending for every element, so
 * each C_ref[i][j] is accumulated in exactly the order of the textbook
 * i-j-k triple loop; FMA contraction cannot change a bit because the product
 * is exact.  Build without -ffast-math (no reassociation).
 *
 * FP16 inputs arrive as IEEE binary16 bit patterns and are decoded by this
 * file's own bit-level decoder (exact, including subnormals, signed zeros,
 * infinities and NaN).  BF16 inputs (bfloat16: the upper 16 bits of a
 * binary32, the 16-bit type the GB300 GEMM article lists beside FP16 in
 * sections 1.1 and 5.1) arrive as bit patterns too and have a decoder of
 * their own; a BF16 x BF16 product carries at most 16 significant bits, so
 * it is exact in double as well.  FP8 inputs (OCP E4M3: the 8-bit type the
 * GB300 GEMM article puts a tier above FP16 in section 1.1) arrive as byte
 * patterns with a decoder of their own (4 significant bits, products exact);
 * so do FP8 E5M2 inputs (OCP E5M2, the other 8-bit encoding of that tier:
 * 3 significant bits, products exact).
 *
 * Parity status: pinned.  The pins (identity, permutation, all-ones closed
 * form C_ij = K, rank-1 outer products, K = 0 and K = 1, brute force against
 * exact rational arithmetic on tiny shapes, float64 library matmul, the
 * exhaustive binary16 decode table) live in the test suite.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_VERSION 1

int oracle_version(void) { return ORACLE_VERSION; }

/* ---------------------------------------------------------------------- */
/* IEEE 754 binary16 -> binary64, exact.                                   */
/* Layout: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.        */
/* ---------------------------------------------------------------------- */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        /* zero or subnormal: frac * 2^(1 - 15 - 10) */
        mag = ldexp((double)frac, -24);
    } else if (expo == 0x1f) {
        mag = frac ? NAN : INFINITY;
    } else {
        /* normal: (1024 + frac) * 2^(expo - 15 - 10) */
        mag = ldexp((double)(0x400 | frac), expo - 25);
    }
    return sign ? -mag : mag;
}

void oracle_f16_array_to_f64(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t t = 0; t < n; ++t)
        dst[t] = oracle_f16_to_f64(src[t]);
}

/* ---------------------------------------------------------------------- */
/* bfloat16 -> binary64, exact.                                            */
/* Layout: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.        */
/* ---------------------------------------------------------------------- */
double oracle_bf16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 7) & 0xff;
    const int frac = h & 0x7f;
    double mag;
    if (expo == 0) {
        /* zero or subnormal: frac * 2^(1 - 127 - 7) */
        mag = ldexp((double)frac, -133);
    } else if (expo == 0xff) {
        mag = frac ? NAN : INFINITY;
    } else {
        /* normal: (128 + frac) * 2^(expo - 127 - 7) */
        mag = ldexp((double)(0x80 | frac), expo - 134);
    }
    return sign ? -mag : mag;
}

void oracle_bf16_array_to_f64(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t t = 0; t < n; ++t)
        dst[t] = oracle_bf16_to_f64(src[t]);
}

/* ---------------------------------------------------------------------- */
/* FP8 E4M3 (OCP) -> binary64, exact.                                      */
/* Layout: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; no       */
/* infinities: exponent 15 with fraction 7 is NaN, the rest are finite     */
/* (largest 448); exponent 0 holds zeros and subnormals (fraction * 2^-9). */
/* ---------------------------------------------------------------------- */
double oracle_e4m3_to_f64(uint8_t b)
{
    const int sign = (b >> 7) & 1;
    const int expo = (b >> 3) & 0xf;
    const int frac = b & 0x7;
    double mag;
    if (expo == 0xf && frac == 0x7)
        mag = NAN;
    else if (expo == 0)
        mag = ldexp((double)frac, -9);
    else
        mag = ldexp((double)(0x8 | frac), expo - 10);
    return sign ? -mag : mag;
}

void oracle_e4m3_array_to_f64(const uint8_t *src, double *dst, int64_t n)
{
    for (int64_t t = 0; t < n; ++t)
        dst[t] = oracle_e4m3_to_f64(src[t]);
}

/* ---------------------------------------------------------------------- */
/* FP8 E5M2 (OCP) -> binary64, exact.                                      */
/* Layout: 1 sign bit, 5 exponent bits (bias 15), 2 fraction bits;         */
/* exponent 31 holds the infinities (fraction 0) and NaN (fraction != 0);  */
/* exponent 0 holds zeros and subnormals (fraction * 2^-16).               */
/* ---------------------------------------------------------------------- */
double oracle_e5m2_to_f64(uint8_t b)
{
    const int sign = (b >> 7) & 1;
    const int expo = (b >> 2) & 0x1f;
    const int frac = b & 0x3;
    double mag;
    if (expo == 0x1f)
        mag = frac ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)frac, -16);
    else
        mag = ldexp((double)(0x4 | frac), expo - 17);
    return sign ? -mag : mag;
}

void oracle_e5m2_array_to_f64(const uint8_t *src, double *dst, int64_t n)
{
    for (int64_t t = 0; t < n; ++t)
        dst[t] = oracle_e5m2_to_f64(src[t]);
}

/* ---------------------------------------------------------------------- */
/* Input access: element (i, k) of a row-major matrix with leading         */
/* dimension ld lives at base[i * ld + k].                                  */
/* ---------------------------------------------------------------------- */
enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_E4M3 = 3, ORACLE_E5M2 = 4 };

static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    if (dtype == ORACLE_E4M3)
        return oracle_e4m3_to_f64(((const uint8_t *)base)[idx]);
    if (dtype == ORACLE_E5M2)
        return oracle_e5m2_to_f64(((const uint8_t *)base)[idx]);
    if (dtype == ORACLE_BF16)
        return oracle_bf16_to_f64(((const uint16_t *)base)[idx]);
    return oracle_f16_to_f64(((const uint16_t *)base)[idx]);
}

typedef struct {
    int dtype;
    int64_t N, K;
    const void *A; int64_t lda;
    const void *B; int64_t ldb;
    const int64_t *rows;   /* which rows of C to produce (NULL: 0..nrows-1) */
    int64_t r_begin, r_end; /* slice of the row list this worker owns */
    double *C; int64_t ldr; /* output row t of the list goes to C + t*ldr   */
    double *D; int64_t ldd; /* same for the error scale                      */
} rows_job;

/* One worker: for each owned row i of C, acc[:] = 0, then for k ascending
 * acc[j] += A[i][k] * B[k][j] and den[j] += |A[i][k]| * |B[k][j]|. */
static void *rows_worker(void *arg)
{
    const rows_job *jb = (const rows_job *)arg;
    for (int64_t t = jb->r_begin; t < jb->r_end; ++t) {
        const int64_t i = jb->rows ? jb->rows[t] : t;
        double *acc = jb->C + t * jb->ldr;
        double *den = jb->D + t * jb->ldd;
        for (int64_t j = 0; j < jb->N; ++j) {
            acc[j] = 0.0;
            den[j] = 0.0;
        }
        for (int64_t k = 0; k < jb->K; ++k) {
            const double a = load_elem(jb->A, jb->dtype, i * jb->lda + k);
            const double abs_a = fabs(a);
            const int64_t brow = k * jb->ldb;
            for (int64_t j = 0; j < jb->N; ++j) {
                const double b = load_elem(jb->B, jb->dtype, brow + j);
                acc[j] += a * b;
                den[j] += abs_a * fabs(b);
            }
        }
    }
    return NULL;
}

static int run_rows(int dtype, int64_t nrows, int64_t N, int64_t K,
                    const void *A, int64_t lda, const void *B, int64_t ldb,
                    const int64_t *rows, double *C, int64_t ldr,
                    double *D, int64_t ldd, int nthreads)
{
    if (nrows < 0 || N < 0 || K < 0 || ldr < N || ldd < N)
        return -1;
    if (nrows == 0 || N == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nrows)
        nthreads = (int)nrows;
    rows_job *jobs = (rows_job *)calloc((size_t)nthreads, sizeof(rows_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    int rc = 0;
    int started = 0;
    for (int w = 0; w < nthreads; ++w) {
        rows_job *jb = &jobs[w];
        jb->dtype = dtype;
        jb->N = N; jb->K = K;
        jb->A = A; jb->lda = lda;
        jb->B = B; jb->ldb = ldb;
        jb->rows = rows;
        jb->r_begin = nrows * w / nthreads;
        jb->r_end = nrows * (w + 1) / nthreads;
        jb->C = C; jb->ldr = ldr;
        jb->D = D; jb->ldd = ldd;
        if (w == 0)
            continue; /* worker 0 runs on the calling thread */
        if (pthread_create(&tids[w], NULL, rows_worker, jb) != 0) {
            rc = -3;
            break;
        }
        started = w;
    }
    if (rc == 0)
        rows_worker(&jobs[0]);
    for (int w = 1; w <= started; ++w)
        pthread_join(tids[w], NULL);
    free(jobs);
    free(tids);
    return rc;
}

/*
 * Rows of C_ref and D.
 *   rows == NULL : produce rows 0..nrows-1 (nrows is then M)
 *   rows != NULL : produce rows rows[0..nrows-1]; output row t is rows[t]
 * C and D are caller-owned double arrays with leading dimensions ldr, ldd.
 * Returns 0 on success, a negative value on bad arguments or thread failure.
 */
int oracle_gemm_rows_f32(int64_t nrows, int64_t N, int64_t K,
                         const float *A, int64_t lda, const float *B, int64_t ldb,
                         const int64_t *rows, double *C, int64_t ldr,
                         double *D, int64_t ldd, int nthreads)
{
    return run_rows(ORACLE_F32, nrows, N, K, A, lda, B, ldb, rows, C, ldr, D, ldd,
                    nthreads);
}

int oracle_gemm_rows_f16(int64_t nrows, int64_t N, int64_t K,
                         const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                         const int64_t *rows, double *C, int64_t ldr,
                         double *D, int64_t ldd, int nthreads)
{
    return run_rows(ORACLE_F16, nrows, N, K, A, lda, B, ldb, rows, C, ldr, D, ldd,
                    nthreads);
}

int oracle_gemm_rows_bf16(int64_t nrows, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                          const int64_t *rows, double *C, int64_t ldr,
                          double *D, int64_t ldd, int nthreads)
{
    return run_rows(ORACLE_BF16, nrows, N, K, A, lda, B, ldb, rows, C, ldr, D, ldd,
                    nthreads);
}

int oracle_gemm_rows_f8(int64_t nrows, int64_t N, int64_t K,
                        const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                        const int64_t *rows, double *C, int64_t ldr,
                        double *D, int64_t ldd, int nthreads)
{
    return run_rows(ORACLE_E4M3, nrows, N, K, A, lda, B, ldb, rows, C, ldr, D, ldd,
                    nthreads);
}

int oracle_gemm_rows_e5m2(int64_t nrows, int64_t N, int64_t K,
                          const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                          const int64_t *rows, double *C, int64_t ldr,
                          double *D, int64_t ldd, int nthreads)
{
    return run_rows(ORACLE_E5M2, nrows, N, K, A, lda, B, ldb, rows, C, ldr, D, ldd,
                    nthreads);
}

/*
 * Rows of C_ref and D for B given transposed: Bt is the N x K row-major
 * matrix with Bt[j][k] = B[k][j] (B column-major, the layout of the
 * baseline kernel in the lqnn.cn SGEMM article, section 3.1), so
 *   C_ref[i][j] = sum_k A[i][k] * Bt[j][k],  D[i][j] = sum_k |A[i][k]| |Bt[j][k]|
 * with the same i-k-j order (k ascending) as oracle_gemm_rows_*.
 */
static void *rows_worker_bt(void *arg)
{
    const rows_job *jb = (const rows_job *)arg;
    for (int64_t t = jb->r_begin; t < jb->r_end; ++t) {
        const int64_t i = jb->rows ? jb->rows[t] : t;
        double *acc = jb->C + t * jb->ldr;
        double *den = jb->D + t * jb->ldd;
        for (int64_t j = 0; j < jb->N; ++j) {
            acc[j] = 0.0;
            den[j] = 0.0;
        }
        for (int64_t k = 0; k < jb->K; ++k) {
            const double a = load_elem(jb->A, jb->dtype, i * jb->lda + k);
            for (int64_t j = 0; j < jb->N; ++j) {
                const double bt = load_elem(jb->B, jb->dtype, j * jb->ldb + k);
                acc[j] += a * bt;
                den[j] += fabs(a) * fabs(bt);
            }
        }
    }
    return NULL;
}

static int run_rows_bt(int dtype, int64_t nrows, int64_t N, int64_t K, const void *A, int64_t lda,
                       const void *Bt, int64_t ldbt, const int64_t *rows, double *C, int64_t ldr,
                       double *D, int64_t ldd)
{
    if (nrows < 0 || N < 0 || K < 0 || ldr < N || ldd < N)
        return -1;
    rows_job jb;
    jb.dtype = dtype;
    jb.N = N; jb.K = K;
    jb.A = A; jb.lda = lda;
    jb.B = Bt; jb.ldb = ldbt;
    jb.rows = rows;
    jb.r_begin = 0;
    jb.r_end = nrows;
    jb.C = C; jb.ldr = ldr;
    jb.D = D; jb.ldd = ldd;
    rows_worker_bt(&jb);
    return 0;
}

int oracle_gemm_rows_bt_f32(int64_t nrows, int64_t N, int64_t K, const float *A, int64_t lda,
                            const float *Bt, int64_t ldbt, const int64_t *rows, double *C,
                            int64_t ldr, double *D, int64_t ldd)
{
    return run_rows_bt(ORACLE_F32, nrows, N, K, A, lda, Bt, ldbt, rows, C, ldr, D, ldd);
}

int oracle_gemm_rows_bt_f16(int64_t nrows, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                            const uint16_t *Bt, int64_t ldbt, const int64_t *rows, double *C,
                            int64_t ldr, double *D, int64_t ldd)
{
    return run_rows_bt(ORACLE_F16, nrows, N, K, A, lda, Bt, ldbt, rows, C, ldr, D, ldd);
}

int oracle_gemm_rows_bt_bf16(int64_t nrows, int64_t N, int64_t K, const uint16_t *A,
                             int64_t lda, const uint16_t *Bt, int64_t ldbt, const int64_t *rows,
                             double *C, int64_t ldr, double *D, int64_t ldd)
{
    return run_rows_bt(ORACLE_BF16, nrows, N, K, A, lda, Bt, ldbt, rows, C, ldr, D, ldd);
}

int oracle_gemm_rows_bt_f8(int64_t nrows, int64_t N, int64_t K, const uint8_t *A,
                           int64_t lda, const uint8_t *Bt, int64_t ldbt, const int64_t *rows,
                           double *C, int64_t ldr, double *D, int64_t ldd)
{
    return run_rows_bt(ORACLE_E4M3, nrows, N, K, A, lda, Bt, ldbt, rows, C, ldr, D, ldd);
}

int oracle_gemm_rows_bt_e5m2(int64_t nrows, int64_t N, int64_t K, const uint8_t *A,
                             int64_t lda, const uint8_t *Bt, int64_t ldbt, const int64_t *rows,
                             double *C, int64_t ldr, double *D, int64_t ldd)
{
    return run_rows_bt(ORACLE_E5M2, nrows, N, K, A, lda, Bt, ldbt, rows, C, ldr, D, ldd);
}

/*
 * Rows of C_ref and D with either operand given transposed, the four BLAS
 * layouts: A element (i, k) is A[i*lda + k], or A[k*lda + i] when trans_a
 * (A passed as its K x M transpose, i.e. column-major A); B element (k, j)
 * is B[k*ldb + j], or B[j*ldb + k] when trans_b (column-major B, the layout
 * of the lqnn.cn SGEMM article's baseline, section 3.1).  Same i-k-j order
 * (k ascending) as oracle_gemm_rows_*.  Single-threaded (test sizes).
 */
static int run_rows_trans(int dtype, int64_t nrows, int64_t N, int64_t K, const void *A,
                          int64_t lda, const void *B, int64_t ldb, int trans_a, int trans_b,
                          const int64_t *rows, double *C, int64_t ldr, double *D, int64_t ldd)
{
    if (nrows < 0 || N < 0 || K < 0 || ldr < N || ldd < N)
        return -1;
    for (int64_t t = 0; t < nrows; ++t) {
        const int64_t i = rows ? rows[t] : t;
        double *acc = C + t * ldr;
        double *den = D + t * ldd;
        for (int64_t j = 0; j < N; ++j) {
            acc[j] = 0.0;
            den[j] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_elem(A, dtype, trans_a ? k * lda + i : i * lda + k);
            for (int64_t j = 0; j < N; ++j) {
                const double b = load_elem(B, dtype, trans_b ? j * ldb + k : k * ldb + j);
                acc[j] += a * b;
                den[j] += fabs(a) * fabs(b);
            }
        }
    }
    return 0;
}

#define ORACLE_TRANS(SUFFIX, DT, T)                                                            \
    int oracle_gemm_rows_trans_##SUFFIX(int64_t nrows, int64_t N, int64_t K, const T *A,      \
                                        int64_t lda, const T *B, int64_t ldb, int trans_a,    \
                                        int trans_b, const int64_t *rows, double *C,          \
                                        int64_t ldr, double *D, int64_t ldd)                  \
    {                                                                                         \
        return run_rows_trans(DT, nrows, N, K, A, lda, B, ldb, trans_a, trans_b, rows, C,     \
                              ldr, D, ldd);                                                   \
    }
ORACLE_TRANS(f32, ORACLE_F32, float)
ORACLE_TRANS(f16, ORACLE_F16, uint16_t)
ORACLE_TRANS(bf16, ORACLE_BF16, uint16_t)
ORACLE_TRANS(f8, ORACLE_E4M3, uint8_t)
ORACLE_TRANS(e5m2, ORACLE_E5M2, uint8_t)

/*
 * Fused epilogue, applied to rows of C_ref and D produced by
 * oracle_gemm_rows_* (in place):
 *   C[t][j] <- act(alpha * C[t][j] + beta * C0[i][j] + bias[j])
 *   D[t][j] <- |alpha| * D[t][j] + |beta * C0[i][j]| + |bias[j]|
 * with i = rows[t] (t when rows is NULL).  D stays a bound on the rounding
 * error scale: the activation (act 1: max(x, 0)) is 1-Lipschitz.
 * Sources: the alpha and beta parameters of the tiled kernel in the lqnn.cn
 * SGEMM article (section 3.3), read with their usual BLAS meaning, since the
 * page leaves beta unapplied; bias and activation fused into the GEMM's
 * epilogue as the GB300 GEMM article proposes (section 7.1).
 * beta == 0: C0 is not read (it may be NULL or hold NaN).  bias == NULL: no
 * bias term.  Returns 0, or -1 on bad arguments.
 */
static int run_epilogue(int dtype, int64_t nrows, int64_t N, double alpha, double beta,
                        const void *C0, int64_t ldc0, const float *bias, int act,
                        const int64_t *rows, double *C, int64_t ldr, double *D, int64_t ldd)
{
    if (nrows < 0 || N < 0 || ldr < N || ldd < N || (act != 0 && act != 1))
        return -1;
    if (beta != 0.0 && (!C0 || ldc0 < N))
        return -1;
    for (int64_t t = 0; t < nrows; ++t) {
        const int64_t i = rows ? rows[t] : t;
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * C[t * ldr + j];
            double d = fabs(alpha) * D[t * ldd + j];
            if (beta != 0.0) {
                const double c0 = beta * load_elem(C0, dtype, i * ldc0 + j);
                v += c0;
                d += fabs(c0);
            }
            if (bias) {
                v += (double)bias[j];
                d += fabs((double)bias[j]);
            }
            if (act == 1 && v < 0.0)
                v = 0.0;
            C[t * ldr + j] = v;
            D[t * ldd + j] = d;
        }
    }
    return 0;
}

int oracle_epilogue_rows_f32(int64_t nrows, int64_t N, double alpha, double beta,
                             const float *C0, int64_t ldc0, const float *bias, int act,
                             const int64_t *rows, double *C, int64_t ldr, double *D, int64_t ldd)
{
    return run_epilogue(ORACLE_F32, nrows, N, alpha, beta, C0, ldc0, bias, act, rows, C, ldr,
                        D, ldd);
}

int oracle_epilogue_rows_f16(int64_t nrows, int64_t N, double alpha, double beta,
                             const uint16_t *C0, int64_t ldc0, const float *bias, int act,
                             const int64_t *rows, double *C, int64_t ldr, double *D, int64_t ldd)
{
    return run_epilogue(ORACLE_F16, nrows, N, alpha, beta, C0, ldc0, bias, act, rows, C, ldr,
                        D, ldd);
}

int oracle_epilogue_rows_bf16(int64_t nrows, int64_t N, double alpha, double beta,
                              const uint16_t *C0, int64_t ldc0, const float *bias, int act,
                              const int64_t *rows, double *C, int64_t ldr, double *D, int64_t ldd)
{
    return run_epilogue(ORACLE_BF16, nrows, N, alpha, beta, C0, ldc0, bias, act, rows, C, ldr,
                        D, ldd);
}

/*
 * INT8 quantisation of an epilogue value v (the output of the fused
 * epilogue, whose alpha carries the quantisation scale): round to the
 * nearest integer with ties to even, then saturate to [-128, 127].  The
 * GB300 GEMM article (section 7.1) fuses this FP32-to-INT8 conversion with
 * its scaling into the GEMM's epilogue.  The rounding is IEEE
 * roundTiesToEven applied to an integer result; NaN maps to 0.
 */
int oracle_quantize_i8(double v)
{
    if (v != v)
        return 0;
    if (v >= 127.0)
        return 127;
    if (v <= -128.0)
        return -128;
    const double f = floor(v);
    const double frac = v - f;
    double r;
    if (frac > 0.5)
        r = f + 1.0;
    else if (frac < 0.5)
        r = f;
    else
        r = (fmod(f, 2.0) == 0.0) ? f : f + 1.0; /* tie: the even neighbour */
    return (int)r;
}

void oracle_quantize_i8_array(const double *v, int8_t *q, int64_t n)
{
    for (int64_t t = 0; t < n; ++t)
        q[t] = (int8_t)oracle_quantize_i8(v[t]);
}

/*
 * Single entries C_ref[ii[t]][jj[t]] and D[ii[t]][jj[t]], each one a plain
 * dot product over k ascending (the same order as the row routine).
 */
static int run_entries(int dtype, int64_t K, const void *A, int64_t lda,
                       const void *B, int64_t ldb, const int64_t *ii,
                       const int64_t *jj, int64_t n, double *c, double *d)
{
    if (K < 0 || n < 0)
        return -1;
    for (int64_t t = 0; t < n; ++t) {
        double acc = 0.0, den = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_elem(A, dtype, ii[t] * lda + k);
            const double b = load_elem(B, dtype, k * ldb + jj[t]);
            acc += a * b;
            den += fabs(a) * fabs(b);
        }
        c[t] = acc;
        d[t] = den;
    }
    return 0;
}

int oracle_gemm_entries_f32(int64_t K, const float *A, int64_t lda,
                            const float *B, int64_t ldb, const int64_t *ii,
                            const int64_t *jj, int64_t n, double *c, double *d)
{
    return run_entries(ORACLE_F32, K, A, lda, B, ldb, ii, jj, n, c, d);
}

int oracle_gemm_entries_f16(int64_t K, const uint16_t *A, int64_t lda,
                            const uint16_t *B, int64_t ldb, const int64_t *ii,
                            const int64_t *jj, int64_t n, double *c, double *d)
{
    return run_entries(ORACLE_F16, K, A, lda, B, ldb, ii, jj, n, c, d);
}

int oracle_gemm_entries_bf16(int64_t K, const uint16_t *A, int64_t lda,
                             const uint16_t *B, int64_t ldb, const int64_t *ii,
                             const int64_t *jj, int64_t n, double *c, double *d)
{
    return run_entries(ORACLE_BF16, K, A, lda, B, ldb, ii, jj, n, c, d);
}

int oracle_gemm_entries_f8(int64_t K, const uint8_t *A, int64_t lda,
                           const uint8_t *B, int64_t ldb, const int64_t *ii,
                           const int64_t *jj, int64_t n, double *c, double *d)
{
    return run_entries(ORACLE_E4M3, K, A, lda, B, ldb, ii, jj, n, c, d);
}

int oracle_gemm_entries_e5m2(int64_t K, const uint8_t *A, int64_t lda,
                             const uint8_t *B, int64_t ldb, const int64_t *ii,
                             const int64_t *jj, int64_t n, double *c, double *d)
{
    return run_entries(ORACLE_E5M2, K, A, lda, B, ldb, ii, jj, n, c, d);
}

/* ---------------------------------------------------------------------- */
/* Error metric.                                                           */
/*   r_ij = |C_gpu[i][j] - C_ref[i][j]| / D[i][j]                           */
/*   r_ij = 0 when numerator and D are both 0; +inf when only D is 0.      */
/*   e = max r_ij.  A NaN or Inf in C_gpu is counted as non-finite.         */
/* C_gpu is widened exactly (FP32) or decoded exactly (FP16 or BF16 bit     */
/* patterns), i.e. a 16-bit result is judged after its own output rounding.*/
/* out[0] = e, out[1] = max |C_gpu - C_ref|, out[2] = i of e, out[3] = j.   */
/* cnt[0] = #(r_ij > tol), cnt[1] = #non-finite C_gpu entries.              */
/* ---------------------------------------------------------------------- */
static void check_common(int dtype, int64_t M, int64_t N, const void *C, int64_t ldc,
                         const double *R, int64_t ldr, const double *D, int64_t ldd,
                         double tol, double *out, int64_t *cnt)
{
    double worst = 0.0, worst_abs = 0.0;
    int64_t wi = -1, wj = -1, n_bad = 0, n_nonfinite = 0;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            const double g = load_elem(C, dtype, i * ldc + j);
            const double ref = R[i * ldr + j];
            const double den = D[i * ldd + j];
            double r;
            if (!isfinite(g)) {
                ++n_nonfinite;
                r = INFINITY;
            } else {
                const double diff = fabs(g - ref);
                if (diff > worst_abs)
                    worst_abs = diff;
                if (den == 0.0)
                    r = (diff == 0.0) ? 0.0 : INFINITY;
                else
                    r = diff / den;
            }
            if (r > tol)
                ++n_bad;
            if (r > worst || wi < 0) {
                if (r > worst || (wi < 0 && r >= worst)) {
                    worst = r;
                    wi = i;
                    wj = j;
                }
            }
        }
    }
    out[0] = worst;
    out[1] = worst_abs;
    out[2] = (double)wi;
    out[3] = (double)wj;
    cnt[0] = n_bad;
    cnt[1] = n_nonfinite;
}

void oracle_check_f32(int64_t M, int64_t N, const float *C, int64_t ldc,
                      const double *R, int64_t ldr, const double *D, int64_t ldd,
                      double tol, double *out, int64_t *cnt)
{
    check_common(ORACLE_F32, M, N, C, ldc, R, ldr, D, ldd, tol, out, cnt);
}

void oracle_check_f16(int64_t M, int64_t N, const uint16_t *C, int64_t ldc,
                      const double *R, int64_t ldr, const double *D, int64_t ldd,
                      double tol, double *out, int64_t *cnt)
{
    check_common(ORACLE_F16, M, N, C, ldc, R, ldr, D, ldd, tol, out, cnt);
}

void oracle_check_bf16(int64_t M, int64_t N, const uint16_t *C, int64_t ldc,
                       const double *R, int64_t ldr, const double *D, int64_t ldd,
                       double tol, double *out, int64_t *cnt)
{
    check_common(ORACLE_BF16, M, N, C, ldc, R, ldr, D, ldd, tol, out, cnt);
}
