/*
 * tgref_attention.c — plain fp64 CPU oracle for scaled dot-product attention
 * (forward).  TEST INFRASTRUCTURE ONLY: nothing on the product path may link,
 * load or call this file; only the tests, the smoke check and the bench's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * The pages name the operation but print no formula for it: the lqnn.cn
 * TileLang walkthrough (section 3.2) and the xdnf.cn article (section 3.2,
 * the operator table) describe flash attention as loading K and V block by
 * block and folding each block into a running softmax held in registers.
 * That fold reproduces the softmax over all keys at once, so this oracle is
 * that plain definition, written out (the block-wise online form is the GPU
 * kernel's business, not the oracle's):
 *
 *   s_ij    = scale * sum_{c<d} Q[i][c] * K[j][c]        for every visible key j
 *   m_i     = max_j s_ij
 *   w_ij    = exp(s_ij - m_i)
 *   l_i     = sum_j w_ij
 *   O[i][c] = (sum_j w_ij * V[j][c]) / l_i
 *   lse_i   = m_i + log(l_i)
 *   A[i][c] = (sum_j w_ij * |V[j][c]|) / l_i    (the softmax-weighted mean
 *                                                magnitude: it bounds the error
 *                                                of rounding the weights)
 *
 * Visible keys: j < Lk; with `causal`, also j <= i + (Lk - Lq), so that the
 * last query sees every key (the mask aligned at the bottom right; with
 * Lq == Lk this is j <= i).  A query that sees no key gets O = A = 0 and
 * lse = -inf.  Query head h reads key/value head h / (H / Hkv) (grouped
 * heads; Hkv == H is plain multi-head attention).
 *
 * Layout: element (b, h, i, c) of Q is Q[b*qs[0] + h*qs[1] + i*qs[2] + c]
 * (strides in elements, the head dimension contiguous); likewise K and V with
 * their key/value head index, and the outputs are dense: O and A as
 * [B][H][Lq][d], lse as [B][H][Lq].
 *
 * Arithmetic: fp16 inputs decode exactly to double; every sum runs in
 * ascending index order in double; exp and log are the C library's.
 *
 * Build: together with tgref.c (gcc -O2, never -ffast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double tgref_f16_decode(uint16_t h);

typedef struct {
    const uint16_t *Q, *K, *V;
    int64_t B, H, Hkv, Lq, Lk, d;
    int64_t qs[3], ks[3], vs[3];
    double scale;
    int causal;
    double *O, *lse, *A;
    /* the (b, h, i) query rows to compute: rows[3*r .. 3*r+2]; NULL = all */
    const int64_t *rows;
    int64_t nrows;
    int64_t first, step;   /* this worker's share of the rows */
    int err;
} attn_job;

/* Last visible key + 1 for query i. */
static int64_t visible_keys(const attn_job *J, int64_t i)
{
    if (!J->causal)
        return J->Lk;
    int64_t n = i + (J->Lk - J->Lq) + 1;
    if (n < 0)
        n = 0;
    return n < J->Lk ? n : J->Lk;
}

/* One query row; out_O / out_A point at its d outputs, out_lse at its lse. */
static void attn_row(const attn_job *J, int64_t b, int64_t h, int64_t i, double *q, double *s,
                     double *out_O, double *out_lse, double *out_A)
{
    const int64_t d = J->d;
    const int64_t hk = h / (J->H / J->Hkv);
    const uint16_t *qrow = J->Q + b * J->qs[0] + h * J->qs[1] + i * J->qs[2];
    const uint16_t *kbase = J->K + b * J->ks[0] + hk * J->ks[1];
    const uint16_t *vbase = J->V + b * J->vs[0] + hk * J->vs[1];
    for (int64_t c = 0; c < d; c++)
        q[c] = tgref_f16_decode(qrow[c]);
    const int64_t n = visible_keys(J, i);
    for (int64_t c = 0; c < d; c++) {
        out_O[c] = 0.0;
        if (out_A)
            out_A[c] = 0.0;
    }
    if (n == 0) {
        *out_lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n; j++) {
        const uint16_t *krow = kbase + j * J->ks[2];
        double acc = 0.0;
        for (int64_t c = 0; c < d; c++)
            acc += q[c] * tgref_f16_decode(krow[c]);
        s[j] = J->scale * acc;
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; j++) {
        s[j] = exp(s[j] - m);   /* s now holds the weight w_ij */
        l += s[j];
    }
    for (int64_t j = 0; j < n; j++) {
        const uint16_t *vrow = vbase + j * J->vs[2];
        for (int64_t c = 0; c < d; c++) {
            const double v = tgref_f16_decode(vrow[c]);
            out_O[c] += s[j] * v;
            if (out_A)
                out_A[c] += s[j] * fabs(v);
        }
    }
    for (int64_t c = 0; c < d; c++) {
        out_O[c] /= l;
        if (out_A)
            out_A[c] /= l;
    }
    *out_lse = m + log(l);
}

static void *attn_worker(void *p)
{
    attn_job *J = (attn_job *)p;
    double *q = malloc(sizeof(double) * (size_t)(J->d > 0 ? J->d : 1));
    double *s = malloc(sizeof(double) * (size_t)(J->Lk > 0 ? J->Lk : 1));
    if (!q || !s) {
        J->err = 1;
        free(q);
        free(s);
        return NULL;
    }
    const int64_t total = J->rows ? J->nrows : J->B * J->H * J->Lq;
    for (int64_t r = J->first; r < total; r += J->step) {
        int64_t b, h, i;
        if (J->rows) {
            b = J->rows[3 * r];
            h = J->rows[3 * r + 1];
            i = J->rows[3 * r + 2];
        } else {
            i = r % J->Lq;
            h = (r / J->Lq) % J->H;
            b = r / (J->Lq * J->H);
        }
        attn_row(J, b, h, i, q, s, J->O + r * J->d, J->lse + r, J->A ? J->A + r * J->d : NULL);
    }
    free(q);
    free(s);
    return NULL;
}

static int attn_run(attn_job *proto, int nthreads)
{
    if (proto->B < 0 || proto->H <= 0 || proto->Hkv <= 0 || proto->H % proto->Hkv ||
        proto->Lq < 0 || proto->Lk < 0 || proto->d <= 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t tid[256];
    attn_job jobs[256];
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = *proto;
        jobs[t].first = t;
        jobs[t].step = nthreads;
        jobs[t].err = 0;
    }
    for (int t = 1; t < nthreads; t++)
        if (pthread_create(&tid[t], NULL, attn_worker, &jobs[t]) != 0)
            return -2;
    attn_worker(&jobs[0]);
    int err = jobs[0].err;
    for (int t = 1; t < nthreads; t++) {
        pthread_join(tid[t], NULL);
        err |= jobs[t].err;
    }
    return err ? -3 : 0;
}

/* All B*H*Lq rows.  qs, ks, vs: {batch, head, row} strides in elements.
 * Returns 0, or negative for invalid sizes / resource failure. */
int tgref_attention(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B,
                    int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d, const int64_t *qs,
                    const int64_t *ks, const int64_t *vs, double scale, int causal, double *O,
                    double *lse, double *A, int nthreads)
{
    attn_job J;
    memset(&J, 0, sizeof(J));
    J.Q = Q;
    J.K = K;
    J.V = V;
    J.B = B;
    J.H = H;
    J.Hkv = Hkv;
    J.Lq = Lq;
    J.Lk = Lk;
    J.d = d;
    memcpy(J.qs, qs, sizeof(J.qs));
    memcpy(J.ks, ks, sizeof(J.ks));
    memcpy(J.vs, vs, sizeof(J.vs));
    J.scale = scale;
    J.causal = causal;
    J.O = O;
    J.lse = lse;
    J.A = A;
    return attn_run(&J, nthreads);
}

/* Only the listed query rows (rows: n triples b, h, i); outputs are packed
 * per listed row: O and A n x d, lse n. */
int tgref_attention_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B,
                         int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                         const int64_t *qs, const int64_t *ks, const int64_t *vs, double scale,
                         int causal, const int64_t *rows, int64_t n, double *O, double *lse,
                         double *A, int nthreads)
{
    for (int64_t r = 0; r < n; r++)
        if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 ||
            rows[3 * r + 1] >= H || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= Lq)
            return -1;
    attn_job J;
    memset(&J, 0, sizeof(J));
    J.Q = Q;
    J.K = K;
    J.V = V;
    J.B = B;
    J.H = H;
    J.Hkv = Hkv;
    J.Lq = Lq;
    J.Lk = Lk;
    J.d = d;
    memcpy(J.qs, qs, sizeof(J.qs));
    memcpy(J.ks, ks, sizeof(J.ks));
    memcpy(J.vs, vs, sizeof(J.vs));
    J.scale = scale;
    J.causal = causal;
    J.O = O;
    J.lse = lse;
    J.A = A;
    J.rows = rows;
    J.nrows = n;
    return attn_run(&J, nthreads);
}
