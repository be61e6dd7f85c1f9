/*
 * Plain fp64 CPU oracle for the attention forward over a packed batch of
 * variable-length sequences with an optional sliding-window mask.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the GPU library.
 *
 * Packed batch.  Sequences are concatenated along the token axis: q is
 * [H_q, total, D], k and v [H_kv, total, D]; sequence s occupies tokens
 * cu[s] .. cu[s+1]-1.  Attention never crosses a sequence boundary (support
 * for variable sequence lengths is future work on page "AVO算法优化Transformer
 * 注意力机制性能解析", section 6).
 *
 * Window.  Page "注意力机制的本质与计算挑战", section 2.1, describes local-window
 * attention (each token attends to neighbours within a fixed radius) and band
 * attention (a band around the diagonal).  Both are the rule: row i (a token
 * of sequence s) sees key j of the same sequence when
 *
 *     i - left <= j <= i + right        (left, right < 0: no bound on that side)
 *
 * and, with the causal mask, also j <= i.  Each row's result is the forward's
 * definition (page "GPU注意力算子性能优化" (QiMeng-Attention), section 1) over
 * those keys; query head h reads K/V head h / (H_q / H_kv).
 *
 * Pins live in tests/oracle_varlen_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double vl_widen(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * cu: n_seq + 1 non-decreasing token offsets, cu[0] = 0, cu[n_seq] = total.
 * o: [H_q, total, D] doubles, lse: [H_q, total] doubles.  A row with no allowed
 * key (impossible unless the window excludes the row's own position) gets O = 0
 * and LSE = -inf.
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int attn_varlen_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        double *o, double *lse, const int32_t *cu, int n_seq, int H_q,
                        int H_kv, int D, int causal, int left, int right, double scale)
{
    if (!q || !k || !v || !o || !lse || !cu) return -1;
    if (n_seq <= 0 || H_q <= 0 || H_kv <= 0 || D <= 0 || H_q % H_kv != 0) return -1;
    if (cu[0] != 0) return -1;
    for (int s = 0; s < n_seq; ++s)
        if (cu[s + 1] < cu[s]) return -1;
    const int64_t total = cu[n_seq];
    /* one score per key of the whole batch: a row never needs more */
    double *e = (double *)malloc(sizeof(double) * (size_t)(total > 0 ? total : 1));
    if (!e) return -2;
    const int group = H_q / H_kv;
    for (int h = 0; h < H_q; ++h) {
        const int kvh = h / group;
        const uint16_t *kp = k + (size_t)kvh * total * D;
        const uint16_t *vp = v + (size_t)kvh * total * D;
        for (int s = 0; s < n_seq; ++s) {
            const int64_t s0 = cu[s], s1 = cu[s + 1];
            for (int64_t i = s0; i < s1; ++i) {
                int64_t lo = s0, hi = s1 - 1;
                if (left >= 0 && i - left > lo) lo = i - left;
                if (right >= 0 && i + right < hi) hi = i + right;
                if (causal && i < hi) hi = i;
                const uint16_t *qr = q + ((size_t)h * total + i) * D;
                double *orow = o + ((size_t)h * total + i) * D;
                for (int d = 0; d < D; ++d) orow[d] = 0.0;
                if (lo > hi) {
                    lse[(size_t)h * total + i] = -INFINITY;
                    continue;
                }
                double m = -INFINITY;
                for (int64_t j = lo; j <= hi; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += vl_widen(qr[d]) * vl_widen(kp[j * D + d]);
                    e[j - lo] = scale * dot;
                    if (e[j - lo] > m) m = e[j - lo];
                }
                double l = 0.0;
                for (int64_t j = lo; j <= hi; ++j) {
                    e[j - lo] = exp(e[j - lo] - m);
                    l += e[j - lo];
                }
                for (int64_t j = lo; j <= hi; ++j)
                    for (int d = 0; d < D; ++d) orow[d] += e[j - lo] * vl_widen(vp[j * D + d]);
                for (int d = 0; d < D; ++d) orow[d] /= l;
                lse[(size_t)h * total + i] = m + log(l);
            }
        }
    }
    free(e);
    return 0;
}
