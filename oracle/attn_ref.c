/*
 * Plain fp64 CPU oracle for the forward pass of scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the GPU library.
 *
 * What it computes.  Page "GPU注意力算子性能优化" (QiMeng-Attention), section 1:
 * the formula softmax(Q K^T / sqrt(d_k)) V.  Page "注意力机制的本质与计算挑战",
 * section 1: the three steps, scores -> softmax -> probability-weighted sum of
 * V.  Page "AVO算法优化Transformer注意力机制性能解析", section 3.1 item 2: the
 * max-subtracted softmax with the 1/sqrt(d_k) scale folded into the scores.
 * For every batch b, query head h and query row i:
 *
 *     g    = H_q / H_kv,  kv = h / g          (contiguous GQA groups; MQA when
 *                                              H_kv = 1, MHA when H_kv = H_q;
 *                                              QiMeng page, section 3.2)
 *     J_i  = {0..N-1}, or {0..i} when causal  (lower-triangular mask)
 *     s_j  = scale * sum_d Q[b,h,i,d] K[b,kv,j,d]            for j in J_i
 *     m    = max_j s_j
 *     l    = sum_j exp(s_j - m)
 *     O[d] = (sum_j exp(s_j - m) V[b,kv,j,d]) / l
 *     LSE  = m + ln(l)
 *
 * Everything after the bf16 -> double widening (exact) is done in double, in
 * the order written above, with no blocking, no online rescaling and no
 * reordering: the fused/tiled method reaches this same value up to rounding.
 *
 * Parity pins (closed forms, invariants, library special cases, brute force)
 * live in the test suite; see tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> double, exact: the bf16 bits are the top half of an fp32. */
static double widen_bf16(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v;
    double *o, *lse;
    int B, Hq, Hkv, N, D, causal;
    double scale;
    const int64_t *rows;   /* NULL: every row in [B, Hq, N] order */
    int64_t n_rows;
    int64_t first, last;   /* this worker's half-open slice of the row list */
    int status;
} job_t;

/* One query row, straight from the definition above. */
static int one_row(const job_t *jb, int64_t r, double *o_row, double *lse_out,
                   double *qrow, double *s)
{
    const int N = jb->N, D = jb->D;
    const int64_t i = r % N;
    const int64_t bh = r / N;
    const int64_t h = bh % jb->Hq;
    const int64_t b = bh / jb->Hq;
    const int64_t group = jb->Hq / jb->Hkv;
    const int64_t kvh = h / group;
    const uint16_t *qp = jb->q + ((b * jb->Hq + h) * (int64_t)N + i) * D;
    const uint16_t *kp = jb->k + (b * jb->Hkv + kvh) * (int64_t)N * D;
    const uint16_t *vp = jb->v + (b * jb->Hkv + kvh) * (int64_t)N * D;
    const int64_t nkeys = jb->causal ? i + 1 : N;

    for (int d = 0; d < D; ++d) qrow[d] = widen_bf16(qp[d]);

    /* step 1: scores */
    for (int64_t j = 0; j < nkeys; ++j) {
        const uint16_t *kj = kp + j * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qrow[d] * widen_bf16(kj[d]);
        s[j] = jb->scale * dot;
    }
    /* step 2: softmax, max-subtracted */
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* step 3: probability-weighted sum of V rows */
    for (int d = 0; d < D; ++d) o_row[d] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        const uint16_t *vj = vp + j * D;
        const double p = s[j];
        for (int d = 0; d < D; ++d) o_row[d] += p * widen_bf16(vj[d]);
    }
    for (int d = 0; d < D; ++d) o_row[d] /= l;
    *lse_out = m + log(l);
    return 0;
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    double *qrow = (double *)malloc(sizeof(double) * (size_t)jb->D);
    double *s = (double *)malloc(sizeof(double) * (size_t)jb->N);
    if (!qrow || !s) {
        free(qrow);
        free(s);
        jb->status = -2;
        return NULL;
    }
    for (int64_t t = jb->first; t < jb->last; ++t) {
        const int64_t r = jb->rows ? jb->rows[t] : t;
        one_row(jb, r, jb->o + t * (int64_t)jb->D, jb->lse + t, qrow, s);
    }
    free(qrow);
    free(s);
    jb->status = 0;
    return NULL;
}

/*
 * q: bf16 bits [B, H_q, N, D]; k, v: bf16 bits [B, H_kv, N, D] (host memory).
 * rows == NULL: o is [B, H_q, N, D] doubles and lse is [B, H_q, N] doubles.
 * rows != NULL: n_rows flat row ids ((b*H_q + h)*N + i); o is [n_rows, D] and
 * lse is [n_rows], in the order given.
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int attn_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                 double *o, double *lse,
                 int B, int H_q, int H_kv, int N, int D, int causal, double scale,
                 int n_threads, const int64_t *rows, int64_t n_rows)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0) return -1;
    if (H_q % H_kv != 0) return -1;
    const int64_t total = (int64_t)B * H_q * N;
    if (!rows) n_rows = total;
    if (n_rows < 0) return -1;
    if (rows)
        for (int64_t t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= total) return -1;
    if (n_rows == 0) return 0;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    if ((int64_t)n_threads > n_rows) n_threads = (int)n_rows;

    job_t jobs[256];
    pthread_t tids[256];
    for (int t = 0; t < n_threads; ++t) {
        job_t *jb = &jobs[t];
        jb->q = q; jb->k = k; jb->v = v; jb->o = o; jb->lse = lse;
        jb->B = B; jb->Hq = H_q; jb->Hkv = H_kv; jb->N = N; jb->D = D;
        jb->causal = causal ? 1 : 0;
        jb->scale = scale;
        jb->rows = rows;
        jb->n_rows = n_rows;
        /* interleaved slices would balance causal rows better, but contiguous
         * slices keep each worker's output writes private and simple. */
        jb->first = n_rows * t / n_threads;
        jb->last = n_rows * (t + 1) / n_threads;
        jb->status = -3;
    }
    int started = 0;
    for (int t = 1; t < n_threads; ++t) {
        if (pthread_create(&tids[t], NULL, worker, &jobs[t]) != 0) break;
        started = t;
    }
    worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    /* any slice whose thread could not start runs here */
    for (int t = started + 1; t < n_threads; ++t) worker(&jobs[t]);
    for (int t = 0; t < n_threads; ++t)
        if (jobs[t].status != 0) return jobs[t].status;
    return 0;
}
