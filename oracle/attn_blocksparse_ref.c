/*
 * Plain fp64 CPU oracle for the attention forward with a block-sparse mask.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the GPU library.
 *
 * Mask.  The query rows and the keys are cut into blocks of `block` tokens
 * (the last block of each may be short).  For query block qb of mask head mh,
 * the key blocks it attends to are listed, in block-compressed-row form, as
 * kb_idx[kb_ptr[mh * n_qb + qb] .. kb_ptr[mh * n_qb + qb + 1] - 1] (block-sparse
 * patterns and a compressed storage format for them are future work on page
 * "AVO算法优化Transformer注意力机制性能解析", section 6).  Row i of query head h
 * sees key j when block j / block is listed for query block i / block of mask
 * head (mask_heads == 1 ? 0 : h), and, with the causal mask, j <= i.  The
 * result is the forward's definition (page "GPU注意力算子性能优化"
 * (QiMeng-Attention), section 1) over those keys.  A row that sees no key gets
 * O = 0 and LSE = -inf.  Listed indices outside [0, n_kb) are ignored; an index
 * listed twice counts once.  The mask is shared by every batch entry.
 *
 * Pins live in tests/oracle_blocksparse_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bs_widen(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * q: [B, H_q, N, D] bf16 bits; k, v: [B, H_kv, N, D].  kb_ptr: mask_heads * n_qb + 1
 * offsets (non-decreasing, kb_ptr[0] = 0), kb_idx: kb_ptr[last] key-block indices,
 * with n_qb = n_kb = ceil(N / block).  mask_heads is 1 or H_q.
 * rows: optional flat row ids ((b * H_q + h) * N + i); then o and lse hold just
 * those rows ([n_rows, D], [n_rows]), else all rows.
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int attn_blocksparse_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *o,
                             double *lse, const int32_t *kb_ptr, const int32_t *kb_idx,
                             int mask_heads, int block, int B, int H_q, int H_kv, int N, int D,
                             int causal, double scale, const int64_t *rows, int64_t n_rows)
{
    if (!q || !k || !v || !o || !lse || !kb_ptr) return -1;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0 || block <= 0 || H_q % H_kv != 0)
        return -1;
    if (mask_heads != 1 && mask_heads != H_q) return -1;
    const int n_blocks = (N + block - 1) / block;
    const int64_t n_lists = (int64_t)mask_heads * n_blocks;
    if (kb_ptr[0] != 0) return -1;
    for (int64_t t = 0; t < n_lists; ++t)
        if (kb_ptr[t + 1] < kb_ptr[t]) return -1;
    if (kb_ptr[n_lists] > 0 && !kb_idx) return -1;
    const int64_t all = (int64_t)B * H_q * N;
    const int64_t count = rows ? n_rows : all;
    for (int64_t t = 0; rows && t < n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= all) return -1;
    double *e = (double *)malloc(sizeof(double) * (size_t)N);
    char *allowed = (char *)malloc((size_t)n_blocks);
    char *sees = (char *)malloc((size_t)N);   /* row i sees key j */
    if (!e || !allowed || !sees) {
        free(e);
        free(allowed);
        free(sees);
        return -2;
    }
    const int group = H_q / H_kv;
    for (int64_t t = 0; t < count; ++t) {
        const int64_t r = rows ? rows[t] : t;
        const int i = (int)(r % N);
        const int h = (int)((r / N) % H_q);
        const int b = (int)(r / ((int64_t)N * H_q));
        const int kvh = h / group;
        const int64_t list = (int64_t)(mask_heads == 1 ? 0 : h) * n_blocks + i / block;
        memset(allowed, 0, (size_t)n_blocks);
        for (int32_t x = kb_ptr[list]; x < kb_ptr[list + 1]; ++x)
            if (kb_idx[x] >= 0 && kb_idx[x] < n_blocks) allowed[kb_idx[x]] = 1;
        const uint16_t *qr = q + (size_t)r * D;
        const uint16_t *kp = k + ((size_t)b * H_kv + kvh) * (size_t)N * D;
        const uint16_t *vp = v + ((size_t)b * H_kv + kvh) * (size_t)N * D;
        double *orow = o + (size_t)t * D;
        for (int d = 0; d < D; ++d) orow[d] = 0.0;
        double m = -INFINITY;
        int seen = 0;
        for (int j = 0; j < N; ++j) {
            e[j] = -INFINITY;
            sees[j] = 0;
            if (!allowed[j / block] || (causal && j > i)) continue;
            sees[j] = 1;
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += bs_widen(qr[d]) * bs_widen(kp[(size_t)j * D + d]);
            e[j] = scale * dot;
            if (e[j] > m) m = e[j];
            seen = 1;
        }
        if (!seen) {
            lse[t] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int j = 0; j < N; ++j) {
            if (!sees[j]) continue;
            const double p = exp(e[j] - m);
            l += p;
            for (int d = 0; d < D; ++d) orow[d] += p * bs_widen(vp[(size_t)j * D + d]);
        }
        for (int d = 0; d < D; ++d) orow[d] /= l;
        lse[t] = m + log(l);
    }
    free(e);
    free(allowed);
    free(sees);
    return 0;
}
