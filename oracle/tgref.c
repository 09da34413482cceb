/*
 * tgref.c — plain fp64 CPU oracle for the tiled fp16 GEMM and its fused
 * bias + ReLU variant.  TEST INFRASTRUCTURE ONLY: nothing on the product path
 * may link, load or call this file; only the tests, the smoke check and the
 * bench's CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * What it computes (the plain definition, written out):
 *   C[i][j] = sum_{k<K} A[i][k] * B[k][j]
 * for fp16 A (M x K) and B (K x N), both row-major with leading dimensions
 * lda and ldb, accumulated in fp64 -- the GEMM of the lqnn.cn TileLang
 * walkthrough, section 2.1 (matmul listing: fp16 operands, fp32 fragment
 * accumulator) and section 4.2 (the runnable FP16-in / FP32-accumulate GEMM),
 * and of the codechina.net TileLang article, section 3.2 (float32 C).
 * The fused variant is the one sketched in the xdnf.cn TileLang article,
 * section 4.2 (GEMM, then per element max(acc + Bias[column], 0)):
 *   C[i][j] = max(sum_k A[i][k] * B[k][j] + bias[j], 0)
 * The _ex entry points take either operand transposed (the backward products
 * of a linear layer, codechina.net TileLang article, section 5.1): with
 * op_a = 1, A is stored K x M and the product uses A[k*lda + i] for element
 * (i, k); with op_b = 1, B is stored N x K and uses B[j*ldb + k] for (k, j).
 *
 * Arithmetic, step by step:
 *  1. every fp16 bit pattern is decoded to a double exactly (subnormals too);
 *  2. each output is one dot product: s = +0.0, then s += a_ik * b_kj for
 *     k = 0, 1, ..., K-1 in ascending order.  A product of two fp16 values
 *     has at most 22 significant bits, so each product is exact in double and
 *     only the additions round (FMA contraction therefore changes nothing);
 *  3. fused: s = s + (double)bias[j] (fp32 is exact in double), then
 *     s = (s > 0) ? s : +0.0;
 *  4. the unrounded double s is the reference value; the output-typed value is
 *     (float)s for fp32 output, or a direct double -> fp16 round-to-nearest-
 *     even (never through float, which would round twice) for fp16 output.
 *
 * Build: gcc -O2 -fPIC -shared -pthread (never -ffast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- fp16 codec (IEEE 754 binary16: 1 sign, 5 exponent, 10 fraction bits) */

double tgref_f16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)            /* zero or subnormal: frac * 2^-24 */
        v = ldexp((double)frac, -24);
    else if (expo == 31)      /* infinity or NaN */
        v = frac ? NAN : INFINITY;
    else                      /* normal: (1024 + frac) * 2^(expo - 25) */
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* Direct double -> fp16, round to nearest, ties to even.  Overflow gives
 * +-Inf, underflow gives a subnormal or a signed zero, NaN gives a quiet NaN. */
uint16_t tgref_f16_encode(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7e00;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7c00;
    int e2;
    frexp(a, &e2);            /* a = f * 2^e2 with f in [0.5, 1) */
    int E = e2 - 1;           /* floor(log2(a)) */
    if (E > 15)
        return sign | 0x7c00;
    if (E < -14)              /* subnormal range shares the 2^-24 quantum */
        E = -14;
    double q = ldexp(1.0, E - 10);          /* spacing of fp16 values here */
    double n = rint(a / q);                 /* a / q is exact; rint is RNE */
    if (n >= 2048.0) {                      /* rounded up into the next binade */
        n = 1024.0;
        E += 1;
        if (E > 15)
            return sign | 0x7c00;
    }
    if (n < 1024.0)                         /* subnormal (only when E == -14) */
        return sign | (uint16_t)n;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)n - 1024));
}

void tgref_decode_array(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        dst[i] = tgref_f16_decode(src[i]);
}

void tgref_to_f32(const double *src, float *dst, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        dst[i] = (float)src[i];
}

void tgref_to_f16(const double *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        dst[i] = tgref_f16_encode(src[i]);
}

/* ---- one output entry: the dot product in ascending k, then the epilogue */

static double dot_entry(const double *arow, const double *bcol, int64_t K,
                        const float *bias, int64_t j)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; k++)
        s += arow[k] * bcol[k];
    if (bias) {
        s = s + (double)bias[j];
        s = (s > 0.0) ? s : 0.0;
    }
    return s;
}

/* ---- full GEMM, rows split over threads ---------------------------------- */

typedef struct {
    const double *a;   /* decoded A, M x K, dense */
    const double *bt;  /* decoded B transposed, N x K, dense (column j of B is row j) */
    const float *bias;
    double *c;
    int64_t N, K, ldc;
    int64_t row_begin, row_end;
} gemm_job;

static void *gemm_worker(void *p)
{
    gemm_job *jb = (gemm_job *)p;
    for (int64_t i = jb->row_begin; i < jb->row_end; i++)
        for (int64_t j = 0; j < jb->N; j++)
            jb->c[i * jb->ldc + j] =
                dot_entry(jb->a + i * jb->K, jb->bt + j * jb->K, jb->K, jb->bias, j);
    return NULL;
}

/* Element (i, k) of op(A) and (k, j) of op(B), as fp16 bits. */
static uint16_t elem_a(const uint16_t *A, int op_a, int64_t lda, int64_t i, int64_t k)
{
    return op_a ? A[k * lda + i] : A[i * lda + k];
}

static uint16_t elem_b(const uint16_t *B, int op_b, int64_t ldb, int64_t k, int64_t j)
{
    return op_b ? B[j * ldb + k] : B[k * ldb + j];
}

/* C_ref (double, row-major, leading dimension ldc) for all M x N entries of
 * op(A).op(B).  bias == NULL gives the plain GEMM; otherwise the fused
 * bias + ReLU.  Returns 0 on success, -1 on bad arguments or allocation
 * failure. */
int tgref_gemm_ex(int op_a, int op_b, const uint16_t *A, const uint16_t *B, const float *bias,
                  double *C, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                  int64_t ldc, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || ldc < N || (op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1))
        return -1;
    if (lda < (op_a ? M : K) || ldb < (op_b ? K : N))
        return -1;
    if (M == 0 || N == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *bt = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!a || !bt) {
        free(a);
        free(bt);
        return -1;
    }
    for (int64_t i = 0; i < M; i++)
        for (int64_t k = 0; k < K; k++)
            a[i * K + k] = tgref_f16_decode(elem_a(A, op_a, lda, i, k));
    for (int64_t k = 0; k < K; k++)
        for (int64_t j = 0; j < N; j++)
            bt[j * K + k] = tgref_f16_decode(elem_b(B, op_b, ldb, k, j));

    if (nthreads > M)
        nthreads = (int)M;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    gemm_job *jobs = (gemm_job *)malloc(sizeof(gemm_job) * (size_t)nthreads);
    int rc = 0;
    if (!th || !jobs) {
        rc = -1;
    } else {
        char *started = (char *)calloc((size_t)nthreads, 1);
        for (int t = 0; t < nthreads; t++) {
            jobs[t] = (gemm_job){a, bt, bias, C, N, K, ldc,
                                 M * t / nthreads, M * (t + 1) / nthreads};
            if (started && pthread_create(&th[t], NULL, gemm_worker, &jobs[t]) == 0)
                started[t] = 1;
            else
                gemm_worker(&jobs[t]);      /* run inline if a thread cannot start */
        }
        for (int t = 0; t < nthreads; t++)
            if (started && started[t])
                pthread_join(th[t], NULL);
        free(started);
    }
    free(th);
    free(jobs);
    free(a);
    free(bt);
    return rc;
}

/* The plain row-major product: tgref_gemm_ex with both operands as stored. */
int tgref_gemm(const uint16_t *A, const uint16_t *B, const float *bias, double *C,
               int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
               int64_t ldc, int nthreads)
{
    return tgref_gemm_ex(0, 0, A, B, bias, C, M, N, K, lda, ldb, ldc, nthreads);
}

/* Selected entries only (rows[t], cols[t]) -> out[t]; for checks at sizes where
 * the full product is too slow on the CPU.  Same arithmetic as tgref_gemm_ex. */
int tgref_gemm_entries_ex(int op_a, int op_b, const uint16_t *A, const uint16_t *B,
                          const float *bias, const int64_t *rows, const int64_t *cols,
                          int64_t count, double *out, int64_t K, int64_t lda, int64_t ldb)
{
    if (K < 0 || (op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1))
        return -1;
    double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double *bcol = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!arow || !bcol) {
        free(arow);
        free(bcol);
        return -1;
    }
    for (int64_t t = 0; t < count; t++) {
        int64_t i = rows[t], j = cols[t];
        for (int64_t k = 0; k < K; k++) {
            arow[k] = tgref_f16_decode(elem_a(A, op_a, lda, i, k));
            bcol[k] = tgref_f16_decode(elem_b(B, op_b, ldb, k, j));
        }
        out[t] = dot_entry(arow, bcol, K, bias, j);
    }
    free(arow);
    free(bcol);
    return 0;
}

int tgref_gemm_entries(const uint16_t *A, const uint16_t *B, const float *bias,
                       const int64_t *rows, const int64_t *cols, int64_t count,
                       double *out, int64_t K, int64_t lda, int64_t ldb)
{
    return tgref_gemm_entries_ex(0, 0, A, B, bias, rows, cols, count, out, K, lda, ldb);
}

/* ---- int8 operands, exact integer product (the quantized variant of the
 * pwwt.cn article, section 5.3).  Each output is the exact sum
 *   C[i][j] = sum_{k<K} op(A)[i][k] * op(B)[k][j]
 * of int8 products in int64 (no rounding, no overflow for K < 2^47). */

static void *gemm_i8_worker(void *p);

typedef struct {
    const int8_t *A, *B;
    int op_a, op_b;
    int64_t *C;
    int64_t N, K, lda, ldb, ldc;
    int64_t row_begin, row_end;
} gemm_i8_job;

static int64_t dot_i8(const int8_t *A, const int8_t *B, int op_a, int op_b, int64_t lda,
                      int64_t ldb, int64_t K, int64_t i, int64_t j)
{
    int64_t s = 0;
    for (int64_t k = 0; k < K; k++) {
        const int64_t a = op_a ? A[k * lda + i] : A[i * lda + k];
        const int64_t b = op_b ? B[j * ldb + k] : B[k * ldb + j];
        s += a * b;
    }
    return s;
}

/* The worker sees op(A) as M x K and op(B) as N x K (k contiguous in both):
 * the caller copies the operands into that layout first, so each dot product
 * runs over two contiguous rows.  The sums are the same exact ascending-k
 * sums as dot_i8 on the operands as stored. */
static void *gemm_i8_worker(void *p)
{
    gemm_i8_job *jb = (gemm_i8_job *)p;
    for (int64_t i = jb->row_begin; i < jb->row_end; i++)
        for (int64_t j = 0; j < jb->N; j++)
            jb->C[i * jb->ldc + j] = dot_i8(jb->A, jb->B, 0, 1, jb->K, jb->K, jb->K, i, j);
    return NULL;
}

/* All M x N entries of op(A).op(B) for int8 A, B into int64 C (leading
 * dimension ldc).  Returns 0, or -1 on bad arguments. */
int tgref_gemm_i8_ex(int op_a, int op_b, const int8_t *A, const int8_t *B, int64_t *C,
                     int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                     int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || ldc < N || (op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1))
        return -1;
    if (lda < (op_a ? M : K) || ldb < (op_b ? K : N))
        return -1;
    if (M == 0 || N == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > M)
        nthreads = (int)M;
    /* op(A) as M x K and op(B) as N x K, both k-contiguous */
    int8_t *a = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    int8_t *bt = (int8_t *)malloc((size_t)(N * K > 0 ? N * K : 1));
    if (!a || !bt) {
        free(a);
        free(bt);
        return -1;
    }
    for (int64_t i = 0; i < M; i++)
        for (int64_t k = 0; k < K; k++)
            a[i * K + k] = op_a ? A[k * lda + i] : A[i * lda + k];
    for (int64_t k = 0; k < K; k++)
        for (int64_t j = 0; j < N; j++)
            bt[j * K + k] = op_b ? B[j * ldb + k] : B[k * ldb + j];
    pthread_t th[64];
    gemm_i8_job jobs[64];
    if (nthreads > 64)
        nthreads = 64;
    int started[64] = {0};
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = (gemm_i8_job){a, bt, 0, 1, C, N, K, K, K, ldc,
                                M * t / nthreads, M * (t + 1) / nthreads};
        if (pthread_create(&th[t], NULL, gemm_i8_worker, &jobs[t]) == 0)
            started[t] = 1;
        else
            gemm_i8_worker(&jobs[t]);
    }
    for (int t = 0; t < nthreads; t++)
        if (started[t])
            pthread_join(th[t], NULL);
    free(a);
    free(bt);
    return 0;
}

/* Selected entries (rows[t], cols[t]) of the int8 product. */
int tgref_gemm_i8_entries_ex(int op_a, int op_b, const int8_t *A, const int8_t *B,
                             const int64_t *rows, const int64_t *cols, int64_t count,
                             int64_t *out, int64_t K, int64_t lda, int64_t ldb)
{
    if (K < 0 || (op_a != 0 && op_a != 1) || (op_b != 0 && op_b != 1))
        return -1;
    for (int64_t t = 0; t < count; t++)
        out[t] = dot_i8(A, B, op_a, op_b, lda, ldb, K, rows[t], cols[t]);
    return 0;
}
