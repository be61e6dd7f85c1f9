/*
 * Test driver for the oracle under AddressSanitizer and UndefinedBehavior-
 * Sanitizer (built and run by tests/test_oracle_sanitize.py, CPU only).
 *
 * Calls every C entry point of oracle/ on small ragged shapes, in full and in
 * row/key-subset modes, with several thread counts and with special values
 * (NaN, +-inf, empty masks), into buffers of exactly the documented sizes.
 * The sanitizers report any out-of-bounds access, use of freed memory or
 * undefined arithmetic; the driver itself checks the return codes and a few
 * properties that hold for any correct result (finite outputs where the
 * inputs are finite, LSE -inf exactly where a row sees no key).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int attn_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *o, double *lse,
                 int B, int H_q, int H_kv, int N, int D, int causal, double scale, int n_threads,
                 const int64_t *rows, int64_t n_rows);
int attn_bwd_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                     double *dq, double *dk, double *dv, double *mag_dq, double *mag_dk,
                     double *mag_dv, int B, int H_q, int H_kv, int N, int D, int causal,
                     double scale, int n_threads, const int64_t *rows, int64_t n_rows);
int attn_bwd_ref_keys_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const uint16_t *dout, double *dk, double *dv, double *mag_dk,
                          double *mag_dv, int B, int H_q, int H_kv, int N, int D, int causal,
                          double scale, int n_threads, const int64_t *keys, int64_t n_keys);
int attn_decode_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *o,
                        double *lse, int B, int H_q, int H_kv, int M, int L, int D, int causal,
                        double scale);
int attn_lse_merge_ref_f64(const double *o_part, const double *lse_part, int64_t rows,
                           int n_parts, int D, double *o, double *lse);
double e4m3_decode(uint8_t c);
int attn_fp8_ref_f64(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8, double s_q,
                     double s_k, double s_v, double *o, double *lse, double *mag, double *rms,
                     int B, int H_q, int H_kv, int N, int D, int causal, double scale,
                     double w_rel, double w_floor, const int64_t *rows, int64_t n_rows);
int attn_varlen_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *o,
                        double *lse, const int32_t *cu, int n_seq, int H_q, int H_kv, int D,
                        int causal, int left, int right, double scale);
int attn_blocksparse_ref_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *o,
                             double *lse, const int32_t *kb_ptr, const int32_t *kb_idx,
                             int mask_heads, int block, int B, int H_q, int H_kv, int N, int D,
                             int causal, double scale, const int64_t *rows, int64_t n_rows);

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
            ++failures;                                    \
        }                                                  \
    } while (0)

/* xorshift64*: deterministic inputs, no library generator */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
/* a bf16 value in about [-2, 2): sign, exponent 126..127 or smaller, random mantissa */
static uint16_t rand_bf16(void) {
    const uint64_t r = next_u64();
    const uint16_t sign = (uint16_t)((r & 1) << 15);
    const uint16_t exp = (uint16_t)(120 + (r >> 1) % 8);
    const uint16_t man = (uint16_t)((r >> 8) & 0x7F);
    return (uint16_t)(sign | (exp << 7) | man);
}
static uint16_t *bf16_buf(size_t n) {
    uint16_t *p = malloc(n * sizeof(uint16_t) + 1);
    for (size_t i = 0; i < n; ++i) p[i] = rand_bf16();
    return p;
}
static double *f64_buf(size_t n) { return malloc(n * sizeof(double) + 1); }
static int all_finite(const double *x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static void forward(void) {
    const int shapes[][5] = {{1, 2, 2, 1, 128}, {1, 4, 2, 37, 128}, {2, 3, 1, 65, 64}, {1, 2, 1, 130, 128}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        const int B = shapes[s][0], Hq = shapes[s][1], Hkv = shapes[s][2], N = shapes[s][3],
                  D = shapes[s][4];
        const size_t nq = (size_t)B * Hq * N * D, nk = (size_t)B * Hkv * N * D;
        uint16_t *q = bf16_buf(nq), *k = bf16_buf(nk), *v = bf16_buf(nk), *dout = bf16_buf(nq);
        for (int causal = 0; causal < 2; ++causal)
            for (int nt = 1; nt <= 3; nt += 2) {
                double *o = f64_buf(nq), *lse = f64_buf((size_t)B * Hq * N);
                CHECK(attn_ref_f64(q, k, v, o, lse, B, Hq, Hkv, N, D, causal, 0.088, nt, NULL, 0) == 0,
                      "attn_ref full");
                CHECK(all_finite(o, nq) && all_finite(lse, (size_t)B * Hq * N), "attn_ref finite");
                const int64_t rows[3] = {0, (int64_t)B * Hq * N - 1, N / 2};
                double *o3 = f64_buf(3 * (size_t)D), *l3 = f64_buf(3);
                CHECK(attn_ref_f64(q, k, v, o3, l3, B, Hq, Hkv, N, D, causal, -0.5, nt, rows, 3) == 0,
                      "attn_ref rows");
                free(o3); free(l3); free(o); free(lse);

                double *dq = f64_buf(nq), *dk = f64_buf(nk), *dv = f64_buf(nk);
                double *mq = f64_buf(nq), *mk = f64_buf(nk), *mv = f64_buf(nk);
                CHECK(attn_bwd_ref_f64(q, k, v, dout, dq, dk, dv, mq, mk, mv, B, Hq, Hkv, N, D,
                                       causal, 0.088, nt, NULL, 0) == 0, "bwd full");
                CHECK(all_finite(dq, nq) && all_finite(dk, nk) && all_finite(dv, nk), "bwd finite");
                CHECK(attn_bwd_ref_f64(q, k, v, dout, dq, dk, dv, NULL, NULL, NULL, B, Hq, Hkv, N, D,
                                       causal, 0.088, nt, NULL, 0) == 0, "bwd full, no mags");
                double *dq3 = f64_buf(3 * (size_t)D), *mq3 = f64_buf(3 * (size_t)D);
                CHECK(attn_bwd_ref_f64(q, k, v, dout, dq3, NULL, NULL, mq3, NULL, NULL, B, Hq, Hkv, N,
                                       D, causal, 0.088, nt, rows, 3) == 0, "bwd rows");
                const int64_t keys[3] = {(int64_t)B * Hkv * N - 1, 0, N - 1};
                double *dk3 = f64_buf(3 * (size_t)D), *dv3 = f64_buf(3 * (size_t)D);
                double *mk3 = f64_buf(3 * (size_t)D), *mv3 = f64_buf(3 * (size_t)D);
                CHECK(attn_bwd_ref_keys_f64(q, k, v, dout, dk3, dv3, mk3, mv3, B, Hq, Hkv, N, D,
                                            causal, 0.088, nt, keys, 3) == 0, "bwd keys");
                free(dq3); free(mq3); free(dk3); free(dv3); free(mk3); free(mv3);
                free(dq); free(dk); free(dv); free(mq); free(mk); free(mv);
            }
        /* special values: a NaN in V, +inf in K, -inf in K */
        k[3] = 0x7F80; k[nk - 1] = 0xFF80; v[D + 1] = 0x7FC1;
        double *o = f64_buf(nq), *lse = f64_buf((size_t)B * Hq * N);
        CHECK(attn_ref_f64(q, k, v, o, lse, B, Hq, Hkv, N, D, 1, 0.088, 2, NULL, 0) == 0, "attn_ref nonfinite");
        free(o); free(lse);
        free(q); free(k); free(v); free(dout);
    }
}

static void decode_and_merge(void) {
    const int shapes[][6] = {{1, 2, 2, 1, 1, 128}, {2, 8, 2, 3, 70, 128}, {1, 4, 1, 5, 5, 128}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        const int B = shapes[s][0], Hq = shapes[s][1], Hkv = shapes[s][2], M = shapes[s][3],
                  L = shapes[s][4], D = shapes[s][5];
        uint16_t *q = bf16_buf((size_t)B * Hq * M * D);
        uint16_t *k = bf16_buf((size_t)B * Hkv * L * D), *v = bf16_buf((size_t)B * Hkv * L * D);
        for (int causal = 0; causal < 2; ++causal) {
            double *o = f64_buf((size_t)B * Hq * M * D), *lse = f64_buf((size_t)B * Hq * M);
            CHECK(attn_decode_ref_f64(q, k, v, o, lse, B, Hq, Hkv, M, L, D, causal, 0.088) == 0,
                  "decode");
            CHECK(all_finite(o, (size_t)B * Hq * M * D), "decode finite");
            free(o); free(lse);
        }
        free(q); free(k); free(v);
    }
    /* merge: random parts, some empty (-inf), one row with all parts empty */
    const int64_t rows = 5;
    const int P = 3, D = 128;
    double *op = f64_buf((size_t)rows * P * D), *lp = f64_buf((size_t)rows * P);
    for (int64_t i = 0; i < rows * P * D; ++i) op[i] = (double)(next_u64() % 1000) / 500.0 - 1.0;
    for (int64_t i = 0; i < rows * P; ++i) lp[i] = (double)(next_u64() % 100) / 10.0 - 5.0;
    lp[1] = -INFINITY;
    for (int p = 0; p < P; ++p) lp[4 * P + p] = -INFINITY;
    double *o = f64_buf((size_t)rows * D), *lse = f64_buf((size_t)rows);
    CHECK(attn_lse_merge_ref_f64(op, lp, rows, P, D, o, lse) == 0, "merge");
    CHECK(isinf(lse[4]) && lse[4] < 0 && isfinite(lse[0]), "merge empty row");
    free(op); free(lp); free(o); free(lse);
}

static void fp8(void) {
    for (int c = 0; c < 256; ++c) {
        const double x = e4m3_decode((uint8_t)c);
        CHECK(isnan(x) == ((c & 0x7F) == 0x7F), "e4m3 NaN codes");
    }
    const int B = 1, Hq = 4, Hkv = 2, N = 67, D = 128;
    const size_t nq = (size_t)B * Hq * N * D, nk = (size_t)B * Hkv * N * D;
    uint8_t *q = malloc(nq), *k = malloc(nk), *v = malloc(nk);
    for (size_t i = 0; i < nq; ++i) q[i] = (uint8_t)(next_u64() % 0x70) | (uint8_t)((next_u64() & 1) << 7);
    for (size_t i = 0; i < nk; ++i) k[i] = (uint8_t)(next_u64() % 0x70) | (uint8_t)((next_u64() & 1) << 7);
    for (size_t i = 0; i < nk; ++i) v[i] = (uint8_t)(next_u64() % 0x70) | (uint8_t)((next_u64() & 1) << 7);
    for (int causal = 0; causal < 2; ++causal) {
        double *o = f64_buf(nq), *lse = f64_buf((size_t)B * Hq * N);
        double *mag = f64_buf(nq), *rms = f64_buf(nq);
        CHECK(attn_fp8_ref_f64(q, k, v, 0.5, 0.25, 2.0, o, lse, mag, rms, B, Hq, Hkv, N, D, causal,
                               0.088, 0.0625, 1e-5, NULL, 0) == 0, "fp8 full");
        CHECK(all_finite(o, nq) && all_finite(mag, nq) && all_finite(rms, nq), "fp8 finite");
        CHECK(attn_fp8_ref_f64(q, k, v, 0.5, 0.25, 2.0, o, lse, NULL, NULL, B, Hq, Hkv, N, D,
                               causal, 0.088, 0.0, 0.0, NULL, 0) == 0, "fp8 no mags");
        const int64_t rows[2] = {(int64_t)B * Hq * N - 1, 3};
        double *o2 = f64_buf(2 * (size_t)D), *l2 = f64_buf(2), *m2 = f64_buf(2 * (size_t)D),
               *r2 = f64_buf(2 * (size_t)D);
        CHECK(attn_fp8_ref_f64(q, k, v, 0.5, 0.25, 2.0, o2, l2, m2, r2, B, Hq, Hkv, N, D, causal,
                               0.088, 0.0625, 1e-5, rows, 2) == 0, "fp8 rows");
        free(o2); free(l2); free(m2); free(r2);
        free(o); free(lse); free(mag); free(rms);
    }
    v[5] = 0x7F; /* a NaN code */
    double *o = f64_buf(nq), *lse = f64_buf((size_t)B * Hq * N);
    CHECK(attn_fp8_ref_f64(q, k, v, 1.0, 1.0, 1.0, o, lse, NULL, NULL, B, Hq, Hkv, N, D, 1, 0.088,
                           0.0, 0.0, NULL, 0) == 0, "fp8 NaN code");
    free(o); free(lse); free(q); free(k); free(v);
}

static void varlen(void) {
    const int32_t cu[] = {0, 1, 40, 40, 171, 200};
    const int n_seq = 5, Hq = 4, Hkv = 2, D = 128, total = 200;
    uint16_t *q = bf16_buf((size_t)Hq * total * D);
    uint16_t *k = bf16_buf((size_t)Hkv * total * D), *v = bf16_buf((size_t)Hkv * total * D);
    const int windows[][2] = {{-1, -1}, {16, -1}, {3, 5}, {0, 0}};
    for (int causal = 0; causal < 2; ++causal)
        for (size_t w = 0; w < sizeof windows / sizeof windows[0]; ++w) {
            double *o = f64_buf((size_t)Hq * total * D), *lse = f64_buf((size_t)Hq * total);
            CHECK(attn_varlen_ref_f64(q, k, v, o, lse, cu, n_seq, Hq, Hkv, D, causal, windows[w][0],
                                      windows[w][1], 0.088) == 0, "varlen");
            CHECK(all_finite(o, (size_t)Hq * total * D), "varlen finite");
            free(o); free(lse);
        }
    free(q); free(k); free(v);
}

static void blocksparse(void) {
    const int B = 2, Hq = 4, Hkv = 2, N = 300, D = 128, block = 128;
    const int nqb = (N + block - 1) / block; /* 3 */
    /* mask head 0: query block 0 sees {0}, block 1 sees nothing, block 2 sees {2, 0} */
    const int32_t ptr1[] = {0, 1, 1, 3};
    const int32_t idx1[] = {0, 2, 0};
    uint16_t *q = bf16_buf((size_t)B * Hq * N * D);
    uint16_t *k = bf16_buf((size_t)B * Hkv * N * D), *v = bf16_buf((size_t)B * Hkv * N * D);
    for (int causal = 0; causal < 2; ++causal) {
        double *o = f64_buf((size_t)B * Hq * N * D), *lse = f64_buf((size_t)B * Hq * N);
        CHECK(attn_blocksparse_ref_f64(q, k, v, o, lse, ptr1, idx1, 1, block, B, Hq, Hkv, N, D,
                                       causal, 0.088, NULL, 0) == 0, "blocksparse shared");
        CHECK(isinf(lse[128]) && lse[128] < 0, "blocksparse empty query block has LSE -inf");
        CHECK(all_finite(o, (size_t)B * Hq * N * D), "blocksparse finite");
        /* one list per head: 4 heads x 3 query blocks */
        int32_t ptr4[4 * 3 + 1], idx4[4 * 3 * 3];
        int n = 0;
        ptr4[0] = 0;
        for (int h = 0; h < Hq; ++h)
            for (int qb = 0; qb < nqb; ++qb) {
                for (int kb = 0; kb <= (h + qb) % nqb; ++kb) idx4[n++] = kb;
                ptr4[h * nqb + qb + 1] = n;
            }
        const int64_t rows[2] = {(int64_t)B * Hq * N - 1, 7};
        double *o2 = f64_buf(2 * (size_t)D), *l2 = f64_buf(2);
        CHECK(attn_blocksparse_ref_f64(q, k, v, o2, l2, ptr4, idx4, Hq, block, B, Hq, Hkv, N, D,
                                       causal, 0.088, rows, 2) == 0, "blocksparse per head rows");
        free(o2); free(l2); free(o); free(lse);
    }
    free(q); free(k); free(v);
}

int main(void) {
    forward();
    decode_and_merge();
    fp8();
    varlen();
    blocksparse();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
