/*
 * Plain fp64 CPU oracle for split-KV decode attention and for the merge of
 * partial attention results by their log-sum-exp.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the GPU library.
 *
 * Decode.  M query rows per (batch, query head) attend to a cache of L keys and
 * values; query head h reads K/V head h / (H_q / H_kv) (page "GPU注意力算子性能
 * 优化" (QiMeng-Attention), section 3.2).  The rows are the last M positions of
 * the sequence, so with the causal mask row i (0 <= i < M) sees keys
 * 0 .. L - M + i; without it, every row sees all L keys.  For each row the
 * result is the forward's definition (the QiMeng page, section 1):
 *
 *     s_j = scale * q . k_j,  O = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),
 *     LSE = m + ln sum_j exp(s_j - m),  m = max_j s_j
 *
 * Merge.  The QiMeng page, section 3.1.1, splits attention into local
 * computations whose results a global reduction combines.  Partial results
 * (O_p, LSE_p) over disjoint key sets combine exactly as
 *
 *     LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p
 *
 * (the softmax weights of each part are rescaled by its share of the total
 * normaliser).  A part with LSE_p = -inf (no keys) has weight 0.
 *
 * Pins live in tests/oracle_decode_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double dec_widen(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * q: bf16 bits [B, H_q, M, D]; k, v: bf16 bits [B, H_kv, L, D] (host).
 * o: [B, H_q, M, D] doubles, lse: [B, H_q, M] doubles.
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int attn_decode_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        double *o, double *lse, int B, int H_q, int H_kv, int M, int L,
                        int D, int causal, double scale)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || M <= 0 || L <= 0 || D <= 0) return -1;
    if (H_q % H_kv != 0) return -1;
    if (causal && M > L) return -1;
    double *s = (double *)malloc(sizeof(double) * (size_t)L);
    if (!s) return -2;
    const int group = H_q / H_kv;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H_q; ++h) {
            const int kvh = h / group;
            const uint16_t *kp = k + ((size_t)b * H_kv + kvh) * (size_t)L * D;
            const uint16_t *vp = v + ((size_t)b * H_kv + kvh) * (size_t)L * D;
            for (int i = 0; i < M; ++i) {
                const size_t r = ((size_t)b * H_q + h) * (size_t)M + i;
                const uint16_t *qr = q + r * D;
                const int nkeys = causal ? L - M + i + 1 : L;
                double m = -INFINITY;
                for (int j = 0; j < nkeys; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += dec_widen(qr[d]) * dec_widen(kp[(size_t)j * D + d]);
                    s[j] = scale * dot;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int j = 0; j < nkeys; ++j) {
                    s[j] = exp(s[j] - m);
                    l += s[j];
                }
                double *orow = o + r * D;
                for (int d = 0; d < D; ++d) orow[d] = 0.0;
                for (int j = 0; j < nkeys; ++j)
                    for (int d = 0; d < D; ++d) orow[d] += s[j] * dec_widen(vp[(size_t)j * D + d]);
                for (int d = 0; d < D; ++d) orow[d] /= l;
                lse[r] = m + log(l);
            }
        }
    free(s);
    return 0;
}

/*
 * o_part: [rows, n_parts, D] doubles; lse_part: [rows, n_parts] doubles (-inf
 * marks an empty part).  o: [rows, D], lse: [rows] doubles.  A row whose parts
 * are all empty gets O = 0 and LSE = -inf.  A NaN LSE_p makes the row NaN, as
 * ln sum_p exp(LSE_p) is NaN then.
 * Returns 0, -1 on bad arguments.
 */
int attn_lse_merge_ref_f64(const double *o_part, const double *lse_part, int64_t rows,
                           int n_parts, int D, double *o, double *lse)
{
    if (!o_part || !lse_part || !o || !lse || rows < 0 || n_parts <= 0 || D <= 0) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *lp = lse_part + r * n_parts;
        double m = -INFINITY;
        int nan_part = 0;
        for (int p = 0; p < n_parts; ++p) {
            if (isnan(lp[p])) nan_part = 1;
            if (lp[p] > m) m = lp[p];
        }
        double *orow = o + r * D;
        if (nan_part) {
            for (int d = 0; d < D; ++d) orow[d] = NAN;
            lse[r] = NAN;
            continue;
        }
        for (int d = 0; d < D; ++d) orow[d] = 0.0;
        if (m == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double total = 0.0;
        for (int p = 0; p < n_parts; ++p) total += exp(lp[p] - m);
        const double L = m + log(total);
        for (int p = 0; p < n_parts; ++p) {
            const double w = exp(lp[p] - L);
            const double *op = o_part + (r * n_parts + p) * D;
            for (int d = 0; d < D; ++d) orow[d] += w * op[d];
        }
        lse[r] = L;
    }
    return 0;
}
