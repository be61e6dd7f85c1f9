/*
 * Plain fp64 CPU oracle for the attention forward on FP8 (e4m3) inputs with
 * per-tensor scales.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the GPU library.
 *
 * Inputs.  q8, k8, v8 hold 8-bit e4m3 codes (sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 is subnormal; the all-ones exponent with
 * all-ones mantissa is NaN and there is no infinity, so the largest finite
 * value is 448).  The tensors they stand for are
 *
 *     Q = s_q * dec(q8),  K = s_k * dec(k8),  V = s_v * dec(v8)
 *
 * with fp32 scales (the FP8 matrix products of page "注意力机制的本质与计算挑战",
 * section 3, and the QiMeng-Attention page, section 3.1.1, with softmax and
 * accumulation kept in fp32).  The result is the forward's definition (the
 * QiMeng page, section 1) on those exact values, in double precision.
 *
 * Error-scale sum (optional output, for the parity tolerance only).  If every
 * softmax weight p_j = exp(s_j - max_k s_k) is replaced by p_j (1 + e_j) in a
 * format with relative rounding w_rel and, below its normal range, absolute
 * rounding w_floor (both in units of the row's largest weight), and O is then
 * normalised by the sum of the replaced weights, the change of O_d is, to first
 * order, sum_j e_j p_j (V_jd - O_d) / l with l = sum_j p_j.  Its bound
 *
 *     mag_d = sum_j max(w_rel p_j, min(p_j, w_floor)) |V_jd - O_d| / l
 *
 * is returned per output element.  With independent roundings of at most
 * that size, the typical size of the change is the quadrature sum
 *
 *     rms_d = sqrt( sum_j (max(w_rel p_j, min(p_j, w_floor)) |V_jd - O_d|)^2 ) / l
 *
 * which is returned too (optional).
 *
 * Pins live in tests/oracle_fp8_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* e4m3 code -> value, exact in double. */
double e4m3_decode(uint8_t c)
{
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return s ? -mag : mag;
}

/*
 * q8: [B, H_q, N, D] codes; k8, v8: [B, H_kv, N, D] codes (host).
 * rows: optional flat row ids ((b * H_q + h) * N + i), n_rows of them; then o,
 * lse and mag hold just those rows ([n_rows, D], [n_rows]), else all rows
 * (o: [B, H_q, N, D], lse: [B, H_q, N]).  mag, rms: optional, like o (w_rel
 * and w_floor are only read when one of them is given).
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int attn_fp8_ref_f64(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8, double s_q,
                     double s_k, double s_v, double *o, double *lse, double *mag, double *rms, int B, int H_q,
                     int H_kv, int N, int D, int causal, double scale, double w_rel,
                     double w_floor, const int64_t *rows, int64_t n_rows)
{
    if (!q8 || !k8 || !v8 || !o || !lse) return -1;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0 || H_q % H_kv != 0) return -1;
    const int64_t all = (int64_t)B * H_q * N;
    const int64_t count = rows ? n_rows : all;
    for (int64_t t = 0; rows && t < n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= all) return -1;
    double *p = (double *)malloc(sizeof(double) * (size_t)N);
    double *qr = (double *)malloc(sizeof(double) * (size_t)D);
    if (!p || !qr) {
        free(p);
        free(qr);
        return -2;
    }
    const int group = H_q / H_kv;
    for (int64_t t = 0; t < count; ++t) {
        const int64_t r = rows ? rows[t] : t;
        const int i = (int)(r % N);
        const int h = (int)((r / N) % H_q);
        const int b = (int)(r / ((int64_t)N * H_q));
        const int kvh = h / group;
        const uint8_t *kp = k8 + ((size_t)b * H_kv + kvh) * (size_t)N * D;
        const uint8_t *vp = v8 + ((size_t)b * H_kv + kvh) * (size_t)N * D;
        for (int d = 0; d < D; ++d) qr[d] = s_q * e4m3_decode(q8[(size_t)r * D + d]);
        const int nkeys = causal ? i + 1 : N;
        double m = -INFINITY;
        for (int j = 0; j < nkeys; ++j) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qr[d] * (s_k * e4m3_decode(kp[(size_t)j * D + d]));
            p[j] = scale * dot;
            if (p[j] > m) m = p[j];
        }
        double l = 0.0;
        for (int j = 0; j < nkeys; ++j) {
            p[j] = exp(p[j] - m);
            l += p[j];
        }
        double *orow = o + (size_t)t * D;
        for (int d = 0; d < D; ++d) orow[d] = 0.0;
        for (int j = 0; j < nkeys; ++j)
            for (int d = 0; d < D; ++d) orow[d] += p[j] * (s_v * e4m3_decode(vp[(size_t)j * D + d]));
        for (int d = 0; d < D; ++d) orow[d] /= l;
        lse[t] = m + log(l);
        if (mag || rms) {
            double *mrow = mag ? mag + (size_t)t * D : NULL;
            double *rrow = rms ? rms + (size_t)t * D : NULL;
            for (int d = 0; d < D; ++d) {
                if (mrow) mrow[d] = 0.0;
                if (rrow) rrow[d] = 0.0;
            }
            for (int j = 0; j < nkeys; ++j) {
                const double small = p[j] < w_floor ? p[j] : w_floor;
                const double w = (w_rel * p[j] > small ? w_rel * p[j] : small) / l;
                for (int d = 0; d < D; ++d) {
                    const double dev = w * fabs(s_v * e4m3_decode(vp[(size_t)j * D + d]) - orow[d]);
                    if (mrow) mrow[d] += dev;
                    if (rrow) rrow[d] += dev * dev;
                }
            }
            for (int d = 0; rrow && d < D; ++d) rrow[d] = sqrt(rrow[d]);
        }
    }
    free(p);
    free(qr);
    return 0;
}
