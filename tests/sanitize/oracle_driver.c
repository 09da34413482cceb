/* Exercises the CPU oracle (oracle/tgref.c, oracle/tgref_attention.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer: every operand buffer is
 * allocated at exactly its footprint ((rows - 1) * ld + cols elements), so a
 * read one element past the last stored element is reported.  Shapes cover
 * padded leading dimensions, all four orientations, K = 0, empty outputs,
 * more threads than rows, int8 operands, selected entries and attention with
 * grouped heads, causal masks and Lq != Lk.  Exits 0 when every call returned
 * its expected status and the integer results equal a direct sum here. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double tgref_f16_decode(uint16_t h);
uint16_t tgref_f16_encode(double x);
void tgref_decode_array(const uint16_t *src, double *dst, int64_t n);
void tgref_to_f32(const double *src, float *dst, int64_t n);
void tgref_to_f16(const double *src, uint16_t *dst, int64_t n);
int tgref_gemm_ex(int op_a, int op_b, const uint16_t *A, const uint16_t *B, const float *bias,
                  double *C, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                  int64_t ldc, int nthreads);
int tgref_gemm_entries_ex(int op_a, int op_b, const uint16_t *A, const uint16_t *B,
                          const float *bias, const int64_t *rows, const int64_t *cols,
                          int64_t count, double *out, int64_t K, int64_t lda, int64_t ldb);
int tgref_gemm_i8_ex(int op_a, int op_b, const int8_t *A, const int8_t *B, int64_t *C, int64_t M,
                     int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int nthreads);
int tgref_gemm_i8_entries_ex(int op_a, int op_b, const int8_t *A, const int8_t *B,
                             const int64_t *rows, const int64_t *cols, int64_t count,
                             int64_t *out, int64_t K, int64_t lda, int64_t ldb);
int tgref_attention(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B,
                    int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d, const int64_t *qs,
                    const int64_t *ks, const int64_t *vs, double scale, int causal, double *O,
                    double *lse, double *A, int nthreads);
int tgref_attention_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B,
                         int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                         const int64_t *qs, const int64_t *ks, const int64_t *vs, double scale,
                         int causal, const int64_t *rows, int64_t n, double *O, double *lse,
                         double *A, int nthreads);

static int failures;
#define EXPECT(c)                                                                      \
    do {                                                                               \
        if (!(c)) {                                                                    \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c);           \
            failures++;                                                                \
        }                                                                              \
    } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static int small_int(void)   /* -4 .. 4 */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (int)(rng % 9) - 4;
}

static int64_t footprint(int64_t rows, int64_t cols, int64_t ld)
{
    return rows > 0 && cols > 0 ? (rows - 1) * ld + cols : 0;
}

/* An fp16 operand of rows x cols stored with leading dimension ld, integer
 * values, allocated at its exact footprint (at least one element). */
static uint16_t *f16_operand(int64_t rows, int64_t cols, int64_t ld, int *vals)
{
    int64_t n = footprint(rows, cols, ld);
#ifdef TG_PLANT_SHORT_BUFFER
    /* a deliberately short operand: the sanitizer must report the oracle's
     * read of its last element */
    uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n > 1 ? n - 1 : 1));
    for (int64_t i = 0; i + 1 < n; i++) {
        p[i] = 0;
        if (vals)
            vals[i] = 0;
    }
    if (vals && n > 0)
        vals[n - 1] = 0;
    return p;
#else
    uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; i++) {
        int v = small_int();
        p[i] = tgref_f16_encode((double)v);
        if (vals)
            vals[i] = v;
    }
    return p;
#endif
}

static void gemm_case(int op_a, int op_b, int64_t M, int64_t N, int64_t K, int pa, int pb,
                      int pc, int fused, int threads)
{
    int64_t ar = op_a ? K : M, ac = op_a ? M : K, br = op_b ? N : K, bc = op_b ? K : N;
    int64_t lda = ac + pa, ldb = bc + pb, ldc = N + pc;
    int64_t na = footprint(ar, ac, lda), nb = footprint(br, bc, ldb);
    int *av = (int *)malloc(sizeof(int) * (size_t)(na > 0 ? na : 1));
    int *bv = (int *)malloc(sizeof(int) * (size_t)(nb > 0 ? nb : 1));
    uint16_t *A = f16_operand(ar, ac, lda, av);
    uint16_t *B = f16_operand(br, bc, ldb, bv);
    float *bias = NULL;
    if (fused) {
        bias = (float *)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
        for (int64_t j = 0; j < N; j++)
            bias[j] = (float)small_int();
    }
    int64_t nc = footprint(M, N, ldc);
    double *C = (double *)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
    EXPECT(tgref_gemm_ex(op_a, op_b, A, B, bias, C, M, N, K, lda, ldb, ldc, threads) == 0);
    for (int64_t i = 0; i < M; i++)
        for (int64_t j = 0; j < N; j++) {
            long s = 0;
            for (int64_t k = 0; k < K; k++)
                s += (long)av[op_a ? k * lda + i : i * lda + k] *
                     bv[op_b ? j * ldb + k : k * ldb + j];
            double want = (double)s;
            if (fused) {
                want += bias[j];
                want = want > 0 ? want : 0.0;
            }
            EXPECT(C[i * ldc + j] == want);
        }
    /* the same entries one by one */
    if (M > 0 && N > 0) {
        int64_t rows[3] = {0, M - 1, M / 2}, cols[3] = {N - 1, 0, N / 2};
        double out[3];
        EXPECT(tgref_gemm_entries_ex(op_a, op_b, A, B, bias, rows, cols, 3, out, K, lda, ldb) == 0);
        for (int t = 0; t < 3; t++)
            EXPECT(out[t] == C[rows[t] * ldc + cols[t]]);
    }
    free(A);
    free(B);
    free(av);
    free(bv);
    free(bias);
    free(C);
}

static void i8_case(int op_a, int op_b, int64_t M, int64_t N, int64_t K, int pa, int pb)
{
    int64_t ar = op_a ? K : M, ac = op_a ? M : K, br = op_b ? N : K, bc = op_b ? K : N;
    int64_t lda = ac + pa, ldb = bc + pb;
    int64_t na = footprint(ar, ac, lda), nb = footprint(br, bc, ldb);
    int8_t *A = (int8_t *)malloc((size_t)(na > 0 ? na : 1));
    int8_t *B = (int8_t *)malloc((size_t)(nb > 0 ? nb : 1));
    for (int64_t i = 0; i < na; i++)
        A[i] = (int8_t)(small_int() * 31);
    for (int64_t i = 0; i < nb; i++)
        B[i] = (int8_t)(small_int() * 32);
    int64_t *C = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M * N > 0 ? M * N : 1));
    EXPECT(tgref_gemm_i8_ex(op_a, op_b, A, B, C, M, N, K, lda, ldb, N, 3) == 0);
    if (M > 0 && N > 0) {
        int64_t rows[2] = {M - 1, 0}, cols[2] = {0, N - 1}, out[2];
        EXPECT(tgref_gemm_i8_entries_ex(op_a, op_b, A, B, rows, cols, 2, out, K, lda, ldb) == 0);
        for (int t = 0; t < 2; t++) {
            long s = 0;
            for (int64_t k = 0; k < K; k++)
                s += (long)A[op_a ? k * lda + rows[t] : rows[t] * lda + k] *
                     B[op_b ? cols[t] * ldb + k : k * ldb + cols[t]];
            EXPECT(out[t] == s && C[rows[t] * N + cols[t]] == s);
        }
    }
    free(A);
    free(B);
    free(C);
}

static void attention_case(int64_t Bt, int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                           int causal, int blhd)
{
    int64_t qs[3], ks[3], vs[3];
    if (blhd) {   /* [B, L, H, d] */
        qs[0] = Lq * H * d, qs[1] = d, qs[2] = H * d;
        ks[0] = Lk * Hkv * d, ks[1] = d, ks[2] = Hkv * d;
    } else {      /* [B, H, L, d] */
        qs[0] = H * Lq * d, qs[1] = Lq * d, qs[2] = d;
        ks[0] = Hkv * Lk * d, ks[1] = Lk * d, ks[2] = d;
    }
    memcpy(vs, ks, sizeof(vs));
    int64_t nq = (Bt - 1) * qs[0] + (H - 1) * qs[1] + (Lq - 1) * qs[2] + d;
    int64_t nk = Lk > 0 ? (Bt - 1) * ks[0] + (Hkv - 1) * ks[1] + (Lk - 1) * ks[2] + d : 1;
    uint16_t *Q = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)nq);
    uint16_t *K = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)nk);
    uint16_t *V = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)nk);
    for (int64_t i = 0; i < nq; i++)
        Q[i] = tgref_f16_encode(small_int() * 0.25);
    for (int64_t i = 0; i < nk; i++) {
        K[i] = tgref_f16_encode(small_int() * 0.25);
        V[i] = tgref_f16_encode((double)small_int());
    }
    int64_t rows_out = Bt * H * Lq;
    double *O = (double *)malloc(sizeof(double) * (size_t)(rows_out * d));
    double *lse = (double *)malloc(sizeof(double) * (size_t)rows_out);
    double *Aw = (double *)malloc(sizeof(double) * (size_t)(rows_out * d));
    EXPECT(tgref_attention(Q, K, V, Bt, H, Hkv, Lq, Lk, d, qs, ks, vs, 0.125, causal, O, lse, Aw,
                           4) == 0);
    int64_t sel[6] = {Bt - 1, H - 1, Lq - 1, 0, 0, 0};
    double O2[2 * 128], l2[2], A2[2 * 128];
    EXPECT(tgref_attention_rows(Q, K, V, Bt, H, Hkv, Lq, Lk, d, qs, ks, vs, 0.125, causal, sel, 2,
                                O2, l2, A2, 2) == 0);
    int64_t last = ((Bt - 1) * H + (H - 1)) * Lq + (Lq - 1);
    EXPECT(l2[0] == lse[last] || (l2[0] != l2[0] && lse[last] != lse[last]));
    for (int64_t c = 0; c < d; c++)
        EXPECT(O2[c] == O[last * d + c]);
    int64_t bad[3] = {Bt, 0, 0};
    EXPECT(tgref_attention_rows(Q, K, V, Bt, H, Hkv, Lq, Lk, d, qs, ks, vs, 0.125, causal, bad, 1,
                                O2, l2, A2, 1) != 0);
    free(Q);
    free(K);
    free(V);
    free(O);
    free(lse);
    free(Aw);
}

int main(void)
{
    /* fp16 codec over every pattern and some doubles */
    for (uint32_t h = 0; h < 65536; h++) {
        double x = tgref_f16_decode((uint16_t)h);
        if (x == x && !(h == 0x8000))
            EXPECT(tgref_f16_encode(x) == (uint16_t)h);
    }
    double xs[5] = {1e-30, -7e-8, 65519.0, 65520.0, 1e300};
    uint16_t hs[5];
    float fs[5];
    double back[5];
    tgref_to_f16(xs, hs, 5);
    tgref_to_f32(xs, fs, 5);
    tgref_decode_array(hs, back, 5);
    EXPECT(hs[3] == 0x7C00 && back[2] == 65504.0);

    const int64_t dims[][3] = {{1, 1, 1}, {4, 4, 4}, {7, 5, 3}, {3, 7, 5}, {17, 33, 65},
                               {64, 1, 129}, {1, 64, 31}, {9, 9, 0}, {0, 5, 5}, {5, 0, 5}};
    for (size_t t = 0; t < sizeof(dims) / sizeof(dims[0]); t++)
        for (int op = 0; op < 4; op++)
            for (int fused = 0; fused < 2; fused++)
                gemm_case(op >> 1, op & 1, dims[t][0], dims[t][1], dims[t][2], (int)t % 3,
                          (int)(t + op) % 4, (int)t % 2, fused, 1 + (int)t % 5);
    /* more threads than rows */
    gemm_case(0, 0, 3, 40, 20, 0, 0, 0, 1, 16);
    /* argument errors */
    uint16_t one = 0;
    double c1 = 0;
    EXPECT(tgref_gemm_ex(0, 0, &one, &one, NULL, &c1, 1, 1, 1, 0, 1, 1, 1) == -1);
    EXPECT(tgref_gemm_ex(2, 0, &one, &one, NULL, &c1, 1, 1, 1, 1, 1, 1, 1) == -1);
    EXPECT(tgref_gemm_ex(0, 0, &one, &one, NULL, &c1, -1, 1, 1, 1, 1, 1, 1) == -1);

    for (int op = 0; op < 4; op++) {
        i8_case(op >> 1, op & 1, 9, 13, 70, op, 3 - op);
        i8_case(op >> 1, op & 1, 1, 1, 1, 0, 0);
        i8_case(op >> 1, op & 1, 6, 4, 0, 1, 0);
    }

    attention_case(1, 2, 2, 5, 7, 64, 0, 0);
    attention_case(2, 4, 2, 9, 4, 64, 1, 0);    /* grouped heads, Lk < Lq: some rows see nothing */
    attention_case(1, 2, 1, 3, 11, 128, 1, 1);  /* [B, L, H, d] strides */
    attention_case(1, 1, 1, 4, 0, 64, 0, 0);    /* no keys */

    if (failures)
        fprintf(stderr, "%d failures\n", failures);
    else
        printf("oracle driver ok\n");
    return failures ? 1 : 0;
}
