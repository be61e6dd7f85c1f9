/*
 * Plain fp64 CPU oracle for the backward pass of scaled dot-product attention:
 * the gradients dQ, dK, dV of a scalar loss L whose gradient with respect to
 * the forward output O is dO.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the GPU library.
 *
 * What it computes.  The forward is the one in attn_ref.c (page "GPU注意力算子
 * 性能优化" (QiMeng-Attention), section 1; page "AVO算法优化Transformer注意力
 * 机制性能解析", section 3.1).  The backward is named, not written out, by the
 * AVO page (section 2.2: a backward pass that reuses gradients and recomputes
 * instead of storing) and by the QiMeng page (section 2.2.2: gradient
 * computation in the backward pass).  The plain reading is the chain rule
 * through the three forward steps, for every batch b, query head h, row i:
 *
 *     kv      = h / (H_q / H_kv),  J_i = {0..N-1}, or {0..i} when causal
 *     s_ij    = scale * Q_i . K_j                          (j in J_i)
 *     P_ij    = exp(s_ij - max_j s_ij) / sum_j exp(...)     (row softmax)
 *     dV_j   += P_ij dO_i                  (O_i = sum_j P_ij V_j)
 *     dP_ij   = dO_i . V_j
 *     delta_i = sum_j P_ij dP_ij           (softmax Jacobian: dS = P (dP - delta))
 *     dS_ij   = P_ij (dP_ij - delta_i)
 *     dQ_i    = scale * sum_j dS_ij K_j
 *     dK_j   += scale * dS_ij Q_i
 *
 * dK and dV of a shared K/V head sum over every query head of its group.  The
 * work runs in two phases so that each output element has exactly one writer:
 * phase 1 goes row by row (softmax, delta, dQ) and keeps each row's log-sum-exp
 * and delta; phase 2 goes key by key and recomputes P_ij = exp(s_ij - lse_i)
 * from them (the same number, by the definition of the log-sum-exp).
 *
 * Error-scale sums (optional outputs).  For the parity tolerance only, not
 * part of the method: for each gradient element the same sum with every term
 * replaced by its magnitude, with |dP - delta| widened by
 * a_i = sum_j P_ij sum_d |dO_id| |V_jd| (the size a rounding error in a
 * low-precision O can give delta_i):
 *     mag_dQ_id = scale * sum_j P_ij (|dP_ij - delta_i| + a_i) |K_jd|
 *     mag_dK_jd = scale * sum_i P_ij (|dP_ij - delta_i| + a_i) |Q_id|
 *     mag_dV_jd =         sum_i P_ij |dO_id|
 *
 * Parity pins (finite differences of the forward oracle, a library autograd,
 * closed forms, invariants) live in tests/test_oracle_bwd_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> double, exact: the bf16 bits are the top half of an fp32. */
static double bwd_widen(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v, *dout;
    double *dq, *dk, *dv, *mdq, *mdk, *mdv;
    double *lse, *delta, *amag;   /* per row of [B, H_q, N], written by phase 1 */
    int B, Hq, Hkv, N, D, causal;
    double scale;
    const int64_t *rows;          /* phase 1: NULL = every row */
    int rows_give_dq;             /* phase 1: write dQ (row list order) or only the stats */
    const int64_t *keys;          /* phase 2: NULL = every key row */
} bctx_t;

typedef struct {
    const bctx_t *c;
    int phase;
    int64_t first, last;
    int status;
} bjob_t;

/* Phase 1: softmax row, delta, dQ (and its error-scale sum) for row r. */
static void bwd_row(const bctx_t *c, int64_t r, double *dq_row, double *mdq_row,
                    int64_t slot, double *qrow, double *dorow, double *p, double *dp)
{
    const int N = c->N, D = c->D;
    const int64_t i = r % N;
    const int64_t bh = r / N;
    const int64_t h = bh % c->Hq;
    const int64_t b = bh / c->Hq;
    const int64_t kvh = h / (c->Hq / c->Hkv);
    const uint16_t *kp = c->k + (b * c->Hkv + kvh) * (int64_t)N * D;
    const uint16_t *vp = c->v + (b * c->Hkv + kvh) * (int64_t)N * D;
    const int64_t nkeys = c->causal ? i + 1 : N;

    for (int d = 0; d < D; ++d) {
        qrow[d] = bwd_widen(c->q[r * D + d]);
        dorow[d] = bwd_widen(c->dout[r * D + d]);
    }
    /* softmax of the scaled scores */
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qrow[d] * bwd_widen(kp[j * D + d]);
        p[j] = c->scale * dot;
        if (p[j] > m) m = p[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int64_t j = 0; j < nkeys; ++j) p[j] /= l;
    /* dP and the Jacobian's row term */
    double delta = 0.0, a = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        double dot = 0.0, mag = 0.0;
        for (int d = 0; d < D; ++d) {
            const double vjd = bwd_widen(vp[j * D + d]);
            dot += dorow[d] * vjd;
            mag += fabs(dorow[d]) * fabs(vjd);
        }
        dp[j] = dot;
        delta += p[j] * dot;
        a += p[j] * mag;
    }
    if (slot >= 0) {
        c->lse[slot] = m + log(l);
        c->delta[slot] = delta;
        c->amag[slot] = a;
    }
    if (!dq_row) return;
    /* dQ_i = scale * sum_j P_ij (dP_ij - delta_i) K_j */
    for (int d = 0; d < D; ++d) {
        dq_row[d] = 0.0;
        if (mdq_row) mdq_row[d] = 0.0;
    }
    for (int64_t j = 0; j < nkeys; ++j) {
        const double ds = p[j] * (dp[j] - delta);
        const double w = p[j] * (fabs(dp[j] - delta) + a);
        for (int d = 0; d < D; ++d) {
            const double kjd = bwd_widen(kp[j * D + d]);
            dq_row[d] += ds * kjd;
            if (mdq_row) mdq_row[d] += w * fabs(kjd);
        }
    }
    for (int d = 0; d < D; ++d) {
        dq_row[d] *= c->scale;
        if (mdq_row) mdq_row[d] *= fabs(c->scale);
    }
}

/* Phase 2: dK_j and dV_j (and their error-scale sums) for key row t of
 * [B, H_kv, N], summed over the query heads of the group and the rows that
 * see key j. */
static void bwd_key(const bctx_t *c, int64_t out, int64_t t, double *qrow, double *dorow)
{
    const int N = c->N, D = c->D;
    const int64_t j = t % N;
    const int64_t bk = t / N;
    const int64_t kvh = bk % c->Hkv;
    const int64_t b = bk / c->Hkv;
    const int64_t group = c->Hq / c->Hkv;
    const uint16_t *kj = c->k + t * D;
    const uint16_t *vj = c->v + t * D;
    double *dk = c->dk + out * D, *dv = c->dv + out * D;
    double *mdk = c->mdk ? c->mdk + out * D : NULL;
    double *mdv = c->mdv ? c->mdv + out * D : NULL;

    for (int d = 0; d < D; ++d) {
        dk[d] = 0.0;
        dv[d] = 0.0;
        if (mdk) mdk[d] = 0.0;
        if (mdv) mdv[d] = 0.0;
    }
    for (int64_t h = kvh * group; h < (kvh + 1) * group; ++h) {
        const int64_t first_row = c->causal ? j : 0;
        for (int64_t i = first_row; i < N; ++i) {
            const int64_t r = (b * c->Hq + h) * (int64_t)N + i;
            double s = 0.0, dp = 0.0;
            for (int d = 0; d < D; ++d) {
                qrow[d] = bwd_widen(c->q[r * D + d]);
                dorow[d] = bwd_widen(c->dout[r * D + d]);
                s += qrow[d] * bwd_widen(kj[d]);
                dp += dorow[d] * bwd_widen(vj[d]);
            }
            const double p = exp(c->scale * s - c->lse[r]);
            const double ds = p * (dp - c->delta[r]);
            const double w = p * (fabs(dp - c->delta[r]) + c->amag[r]);
            for (int d = 0; d < D; ++d) {
                dk[d] += ds * qrow[d];
                dv[d] += p * dorow[d];
                if (mdk) mdk[d] += w * fabs(qrow[d]);
                if (mdv) mdv[d] += p * fabs(dorow[d]);
            }
        }
    }
    for (int d = 0; d < D; ++d) {
        dk[d] *= c->scale;
        if (mdk) mdk[d] *= fabs(c->scale);
    }
}

static void *bwd_worker(void *arg)
{
    bjob_t *jb = (bjob_t *)arg;
    const bctx_t *c = jb->c;
    const int64_t n = c->N > c->D ? c->N : c->D;
    double *buf = (double *)malloc(sizeof(double) * (size_t)(2 * c->D + 2 * n));
    if (!buf) {
        jb->status = -2;
        return NULL;
    }
    double *qrow = buf, *dorow = buf + c->D, *p = buf + 2 * c->D, *dp = p + n;
    for (int64_t t = jb->first; t < jb->last; ++t) {
        if (jb->phase == 1) {
            const int64_t r = c->rows ? c->rows[t] : t;
            double *dq = c->rows_give_dq ? c->dq + t * c->D : NULL;
            double *mdq = (c->rows_give_dq && c->mdq) ? c->mdq + t * c->D : NULL;
            bwd_row(c, r, dq, mdq, c->lse ? r : -1, qrow, dorow, p, dp);
        } else {
            bwd_key(c, t, c->keys ? c->keys[t] : t, qrow, dorow);
        }
    }
    free(buf);
    jb->status = 0;
    return NULL;
}

/* Per-row statistics (lse, delta, a) of [B, H_q, N] rows, filled with NaN so
 * that a row phase 1 did not visit poisons every result that reads it. */
static double *bwd_stats_alloc(int64_t total)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)(3 * total));
    if (s)
        for (int64_t t = 0; t < 3 * total; ++t) s[t] = NAN;
    return s;
}

static int bwd_par_for(const bctx_t *c, int phase, int64_t n, int n_threads)
{
    if (n == 0) return 0;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    if ((int64_t)n_threads > n) n_threads = (int)n;
    bjob_t jobs[256];
    pthread_t tids[256];
    for (int t = 0; t < n_threads; ++t) {
        jobs[t].c = c;
        jobs[t].phase = phase;
        jobs[t].first = n * t / n_threads;
        jobs[t].last = n * (t + 1) / n_threads;
        jobs[t].status = -3;
    }
    int started = 0;
    for (int t = 1; t < n_threads; ++t) {
        if (pthread_create(&tids[t], NULL, bwd_worker, &jobs[t]) != 0) break;
        started = t;
    }
    bwd_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    for (int t = started + 1; t < n_threads; ++t) bwd_worker(&jobs[t]);
    for (int t = 0; t < n_threads; ++t)
        if (jobs[t].status != 0) return jobs[t].status;
    return 0;
}

/*
 * q, dout: bf16 bits [B, H_q, N, D]; k, v: bf16 bits [B, H_kv, N, D] (host).
 * rows == NULL: dq [B, H_q, N, D], dk and dv [B, H_kv, N, D] doubles.
 * rows != NULL: only dQ, for n_rows flat row ids ((b*H_q + h)*N + i): dq is
 * [n_rows, D] in the order given; dk, dv, mag_dk, mag_dv are not touched.
 * mag_*: optional error-scale sums of the same shapes (NULL to skip).
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int attn_bwd_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const uint16_t *dout, double *dq, double *dk, double *dv,
                     double *mag_dq, double *mag_dk, double *mag_dv,
                     int B, int H_q, int H_kv, int N, int D, int causal, double scale,
                     int n_threads, const int64_t *rows, int64_t n_rows)
{
    if (!q || !k || !v || !dout || !dq) return -1;
    if (!rows && (!dk || !dv)) return -1;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0) return -1;
    if (H_q % H_kv != 0) return -1;
    const int64_t total = (int64_t)B * H_q * N;
    if (rows) {
        if (n_rows < 0) return -1;
        for (int64_t t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= total) return -1;
    }
    bctx_t c;
    memset(&c, 0, sizeof c);
    c.q = q; c.k = k; c.v = v; c.dout = dout;
    c.dq = dq; c.dk = dk; c.dv = dv;
    c.mdq = mag_dq; c.mdk = rows ? NULL : mag_dk; c.mdv = rows ? NULL : mag_dv;
    c.B = B; c.Hq = H_q; c.Hkv = H_kv; c.N = N; c.D = D;
    c.causal = causal ? 1 : 0;
    c.scale = scale;
    c.rows = rows;
    c.rows_give_dq = 1;
    if (rows) return bwd_par_for(&c, 1, n_rows, n_threads);

    double *stats = bwd_stats_alloc(total);
    if (!stats) return -2;
    c.lse = stats;
    c.delta = stats + total;
    c.amag = stats + 2 * total;
    int rc = bwd_par_for(&c, 1, total, n_threads);
    if (rc == 0) rc = bwd_par_for(&c, 2, (int64_t)B * H_kv * N, n_threads);
    free(stats);
    return rc;
}

/*
 * dK and dV of a subset of key rows: n_keys flat key ids ((b*H_kv + kv)*N + j).
 * dk, dv (and the optional mag_dk, mag_dv) are [n_keys, D] doubles in the order
 * given.  Phase 1 runs, without dQ, over the rows of the query heads whose
 * group contains a listed key that phase 2 reads: every row, or with the causal
 * mask only rows i >= the smallest listed key of that (b, kv) panel (row i sees
 * key j only when j <= i).  Phase 2 runs only for the listed keys.  Same
 * arithmetic as attn_bwd_ref_f64, so the rows agree with its full result.
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int attn_bwd_ref_keys_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const uint16_t *dout, double *dk, double *dv,
                          double *mag_dk, double *mag_dv,
                          int B, int H_q, int H_kv, int N, int D, int causal, double scale,
                          int n_threads, const int64_t *keys, int64_t n_keys)
{
    if (!q || !k || !v || !dout || !dk || !dv || !keys || n_keys < 0) return -1;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0) return -1;
    if (H_q % H_kv != 0) return -1;
    const int64_t total = (int64_t)B * H_q * N;
    const int64_t nkv = (int64_t)B * H_kv;
    for (int64_t t = 0; t < n_keys; ++t)
        if (keys[t] < 0 || keys[t] >= nkv * N) return -1;
    if (n_keys == 0) return 0;

    /* the (b, kv) panels that hold a listed key, the first row of each that
     * phase 2 reads (causal: the panel's smallest listed key; else row 0), and
     * those rows of every query head of the panel's group */
    int64_t *first = (int64_t *)malloc(sizeof(int64_t) * (size_t)nkv);
    double *stats = bwd_stats_alloc(total);
    int64_t *rows = NULL;
    int rc = -2;
    if (!first || !stats) goto done;
    for (int64_t u = 0; u < nkv; ++u) first[u] = N;   /* N: panel unused */
    for (int64_t t = 0; t < n_keys; ++t) {
        const int64_t u = keys[t] / N, j = keys[t] % N;
        const int64_t f = causal ? j : 0;
        if (f < first[u]) first[u] = f;
    }
    const int64_t group = H_q / H_kv;
    int64_t n_need = 0;
    for (int64_t u = 0; u < nkv; ++u) n_need += group * (N - first[u]);
    rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_need > 0 ? n_need : 1));
    if (!rows) goto done;
    int64_t n_rows = 0;
    for (int64_t u = 0; u < nkv; ++u) {
        const int64_t b = u / H_kv, kvh = u % H_kv;
        for (int64_t h = kvh * group; h < (kvh + 1) * group; ++h)
            for (int64_t i = first[u]; i < N; ++i) rows[n_rows++] = (b * H_q + h) * N + i;
    }
    bctx_t c;
    memset(&c, 0, sizeof c);
    c.q = q; c.k = k; c.v = v; c.dout = dout;
    c.dk = dk; c.dv = dv; c.mdk = mag_dk; c.mdv = mag_dv;
    c.B = B; c.Hq = H_q; c.Hkv = H_kv; c.N = N; c.D = D;
    c.causal = causal ? 1 : 0;
    c.scale = scale;
    c.lse = stats;
    c.delta = stats + total;
    c.amag = stats + 2 * total;
    c.rows = rows;
    c.rows_give_dq = 0;
    c.keys = keys;
    rc = bwd_par_for(&c, 1, n_rows, n_threads);
    if (rc == 0) rc = bwd_par_for(&c, 2, n_keys, n_threads);
done:
    free(first);
    free(stats);
    free(rows);
    return rc;
}
