// Split-KV decode attention and the log-sum-exp merge of partial results for
// MI355X (gfx950, CDNA4).
//
// Decode: M query rows per (batch, query head) -- the last M positions of a
// sequence -- attend to a cache of L keys and values, with K/V heads shared by
// groups of query heads (page "GPU注意力算子性能优化" (QiMeng-Attention),
// sections 1 and 3.2).  The key range is cut into splits that run in parallel
// ("local computation"), each producing a partial O and LSE; a second kernel
// combines them exactly by their log-sum-exp ("global reduction", the same
// page, section 3.1.1):
//
//     LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p
//
// The work is bound by reading the K/V cache once from HBM: per key, 4*D
// flops for each of the group's g*M query rows against 4*D bytes of K and V.
//
// attn_decode_split_kernel: one wave = one (batch, K/V head, block of 32 query
// columns, key split).  The 32 columns are the group's query rows (column
// j*M + i = row i of the group's j-th query head), so every K/V byte the wave
// reads serves all of them.  Q^T lives in VGPRs as the MFMA B operand; 32-key
// blocks of K and V are copied by LDS DMA into a private ring of the wave (no
// workgroup barriers: each wave waits for its own DMA with vmcnt).
// Per block, S^T = K Q^T, an online softmax per column (one column per lane),
// and O^T += V^T P^T with V^T read by the transposing LDS read.  The partial
// O (fp32, divided by the sum of the bf16 weights the PV product applied) and
// LSE go to the workspace.
//
// attn_lse_merge_kernel: one workgroup per output row, parts spread over its
// threads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn.h"
#include "cdna4.h"
#include "tile.h"

namespace {

using namespace cdna4;
using tile::BLK_BYTES;
using tile::HD;
using tile::KB;
using tile::ROW_BYTES;

// One wave per workgroup with a 2-block ring (32 KiB of LDS) lets 5 waves
// share a CU, the most bytes in flight per CU of the shapes measured (2- to
// 4-block rings with 1, 2 or 4 waves per workgroup); and about 1024 waves (one
// round, each streaming a long key range) beat both fewer and more splits.
constexpr int DC_WAVES = 1;                       // independent waves per workgroup
constexpr int DC_THREADS = DC_WAVES * 64;
constexpr int DC_RING = 2;                        // K and V blocks of a wave in flight
constexpr int DC_WAVE_LDS = 2 * DC_RING * BLK_BYTES;   // per wave: K ring, then V ring
constexpr int DC_LDS = DC_WAVES * DC_WAVE_LDS;
constexpr int DC_DMA_PER_BLOCK = 16;              // 8 four-row DMAs for K, 8 for V
constexpr int DC_TARGET_WAVES = 1024;

struct DecParams {
    const uint16_t *q, *k, *v;
    float* o_part;     // [rows, n_splits, HD]
    float* lse_part;   // [rows, n_splits]
    int B, Hq, Hkv, M, L;
    int group;         // Hq / Hkv
    int gm;            // group * M query rows per K/V head
    int n_cb;          // ceil(gm / 32) blocks of query columns
    int n_splits;      // split s covers 32-key blocks [s*n_blocks/n_splits, (s+1)*n_blocks/n_splits)
    int n_blocks;      // ceil(L / 32)
    int total_waves;   // B * Hkv * n_cb * n_splits
    int causal;
    int q_mode;        // 0: Q as given, 1: Q negated, 2: Q replaced by zeros
    float c;           // |scale| * log2(e)
    float lse_scale;   // |scale|
};

// NaN-propagating maximum over the wave
__device__ __forceinline__ float wave_maximum_all(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = __builtin_elementwise_maximum(x, __shfl_xor(x, s));
    return x;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ float wave_sum_all(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
    return x;
}
__device__ __forceinline__ float swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                              false, false);
    return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}

__global__ __launch_bounds__(DC_THREADS, 1) void attn_decode_split_kernel(DecParams p) {
    __shared__ __attribute__((aligned(1024))) char lds[DC_LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int gw = blockIdx.x * DC_WAVES + wave;
    if (gw >= p.total_waves) return;   // wave-uniform; the kernel has no barriers

    const int split = gw % p.n_splits;
    const int unit = gw / p.n_splits;
    const int cb = unit % p.n_cb;
    const int bk = unit / p.n_cb;
    const int b = bk / p.Hkv;
    const int kvh = bk % p.Hkv;
    const int L = p.L, M = p.M;

    // this lane's query column: row i of the group's j-th query head
    const int col = cb * 32 + l32;
    const bool col_ok = col < p.gm;
    const int jh = col_ok ? col / M : 0;
    const int i = col_ok ? col % M : 0;
    const int h = kvh * p.group + jh;
    const int klim = !col_ok ? -1 : (p.causal ? L - M + i : L - 1);   // last key it sees
    const int lo = (int)((int64_t)split * p.n_blocks / p.n_splits) * KB;
    const int hi = min(L, (int)((int64_t)(split + 1) * p.n_blocks / p.n_splits) * KB);
    // keys any column of the wave sees end at kmax; blocks past it are skipped.
    // Keys up to kmin are seen by every column of the wave; a key past kmin is
    // hidden from some column (bottom-right causal mask, or past the cache).
    // The wave's columns c0..c1 hold rows col % M: one run of residues, all
    // of them once it has M columns or wraps past a multiple of M.
    int kmin = L - 1, kmax = L - 1;
    if (p.causal) {
        const int c0 = cb * 32, c1 = min(c0 + 31, p.gm - 1);
        const bool all_rows = c1 - c0 + 1 >= M || c0 / M != c1 / M;
        kmin = L - M + (all_rows ? 0 : c0 % M);
        kmax = L - M + (all_rows ? M - 1 : c1 % M);
    }
    const int last = min(hi - 1, kmax);
    const int nb = last >= lo ? (last - lo) / KB + 1 : 0;

    const size_t kv_panel = ((size_t)b * p.Hkv + kvh) * (size_t)L * HD;
    const uint16_t* kbase = p.k + kv_panel;
    const uint16_t* vbase = p.v + kv_panel;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    const uint32_t wlds = (uint32_t)(wave * DC_WAVE_LDS);   // this wave's region

    // Q^T as the B operand: head dims 16ks + 8hh .. +7 of this column's row
    bf16x8 qf[8];
    {
        const size_t row = ((size_t)b * p.Hq + h) * (size_t)M + i;
        const u32x4 keep = (col_ok && p.q_mode != 2) ? u32x4{~0u, ~0u, ~0u, ~0u} : u32x4{0u, 0u, 0u, 0u};
        const u32x4 flip = p.q_mode == 1 ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}
                                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (col_ok) x = *(const u32x4*)(p.q + row * HD + 16 * ks + 8 * hh);
            qf[ks] = __builtin_bit_cast(bf16x8, (x & keep) ^ (flip & keep));
        }
    }
    // Keys past kmin in the wave's blocks meet a 0 weight for some column, and
    // the matrix core makes 0 * inf and 0 * NaN NaN, a product the formula
    // never takes.  Their V rows (the last ones of a causal cache, or past
    // the wave's last key) are checked here; only when one holds a non-finite
    // element does the wave take them out of the product (exact).
    bool exact = false;
    {
        const int j0 = max(lo, kmin + 1);
        const int j1 = min(lo + nb * KB, L) - 1;
        uint32_t bad = 0u;
        for (int idx = lane; idx < (j1 - j0 + 1) * 16; idx += 64) {
            const u32x4 x = *(const u32x4*)(vbase + (size_t)(j0 + (idx >> 4)) * HD + 8 * (idx & 15));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bad |= (uint32_t)((x[e] & 0x7F80u) == 0x7F80u) | (uint32_t)((x[e] & 0x7F800000u) == 0x7F800000u);
        }
        exact = __builtin_amdgcn_ballot_w64(bad != 0u) != 0;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // Q and check loads done: only DMA counts in vmcnt below

    uint32_t dsrc[8];
#pragma unroll
    for (int r4 = 0; r4 < 8; ++r4) dsrc[r4] = tile::dma_src(4 * r4, lane);
    static_assert(DC_DMA_PER_BLOCK == 16 && DC_RING >= 1 && DC_RING <= 4,
                  "the vmcnt waits below count 16 DMAs per block, at most 3 blocks ahead");
    // block g (keys lo + 32g ..) -> ring slot g % DC_RING.  One K and one V
    // descriptor for the whole panel, the block offset in soffset: the buffer
    // unit range-checks voffset + soffset against the panel's L rows, and lanes
    // past them write zeros to LDS, so the rows past L of a ragged last block
    // arrive as zeros.
    const u32x4 rk = sgpr_rsrc(kbase, (uint32_t)L * ROW_BYTES);
    const u32x4 rv = sgpr_rsrc(vbase, (uint32_t)L * ROW_BYTES);
    const uint32_t ring0 = lds_base + wlds;
    auto issue_slot = [&](auto slot_t, uint32_t soff) {
        constexpr uint32_t KS = decltype(slot_t)::value * BLK_BYTES;
        constexpr uint32_t VS = KS + DC_RING * BLK_BYTES;
        lds_dma16_at<KS + 0 * 4 * ROW_BYTES>(rk, ring0, dsrc[0], soff);
        lds_dma16_at<KS + 1 * 4 * ROW_BYTES>(rk, ring0, dsrc[1], soff);
        lds_dma16_at<KS + 2 * 4 * ROW_BYTES>(rk, ring0, dsrc[2], soff);
        lds_dma16_at<KS + 3 * 4 * ROW_BYTES>(rk, ring0, dsrc[3], soff);
        lds_dma16_at<KS + 4 * 4 * ROW_BYTES>(rk, ring0, dsrc[4], soff);
        lds_dma16_at<KS + 5 * 4 * ROW_BYTES>(rk, ring0, dsrc[5], soff);
        lds_dma16_at<KS + 6 * 4 * ROW_BYTES>(rk, ring0, dsrc[6], soff);
        lds_dma16_at<KS + 7 * 4 * ROW_BYTES>(rk, ring0, dsrc[7], soff);
        lds_dma16_at<VS + 0 * 4 * ROW_BYTES>(rv, ring0, dsrc[0], soff);
        lds_dma16_at<VS + 1 * 4 * ROW_BYTES>(rv, ring0, dsrc[1], soff);
        lds_dma16_at<VS + 2 * 4 * ROW_BYTES>(rv, ring0, dsrc[2], soff);
        lds_dma16_at<VS + 3 * 4 * ROW_BYTES>(rv, ring0, dsrc[3], soff);
        lds_dma16_at<VS + 4 * 4 * ROW_BYTES>(rv, ring0, dsrc[4], soff);
        lds_dma16_at<VS + 5 * 4 * ROW_BYTES>(rv, ring0, dsrc[5], soff);
        lds_dma16_at<VS + 6 * 4 * ROW_BYTES>(rv, ring0, dsrc[6], soff);
        lds_dma16_at<VS + 7 * 4 * ROW_BYTES>(rv, ring0, dsrc[7], soff);
    };
    static_assert(DC_RING == 2, "issue() picks one of two ring slots");
    auto issue = [&](int g) {
        const uint32_t soff = (uint32_t)(lo + g * KB) * ROW_BYTES;
        if (g & 1) issue_slot(std::integral_constant<uint32_t, 1>{}, soff);
        else issue_slot(std::integral_constant<uint32_t, 0>{}, soff);
    };

    tile::Reads rd;
    rd.init(lane);
    const float c = p.c;
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    float m = -INFINITY;   // running max of this column's raw scores
    float l = 0.f;         // sum of fp32 p (this half of the keys): the LSE
    float lb = 0.f;        // sum of bf16 p, the weights the PV MFMA applies: O's divisor

#pragma unroll
    for (int g = 0; g < DC_RING; ++g)
        if (g < nb) issue(g);
    // One pass over block g.  EX: the exact form for a block with keys past
    // kmin (a separate copy, so the common loop body stays one basic block).
    auto block = [&](int g, auto ex_t) {
        constexpr bool EX = decltype(ex_t)::value;
        // block g has landed once at most (blocks issued after it) * 16 DMAs are pending
        const int ahead = min(nb - 1 - g, DC_RING - 1);
        if (ahead >= 3) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
        else if (ahead == 2) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const uint32_t ks = wlds + (uint32_t)(g % DC_RING) * BLK_BYTES;
        const uint32_t vs = ks + DC_RING * BLK_BYTES;
        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.row(lds, ks, kk), qf[kk], s, 0, 0, 0);
        const int kb = lo + g * KB;
        const int kb0 = kb + 4 * hh;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kb0 + 8 * (r >> 2) + (r & 3);
            s[r] = (key > klim || key >= hi) ? -INFINITY : s[r];
            mx = fmaxf(mx, s[r]);
        }
        mx = swap_max(mx);
        const float m_new = fmaxf(m, mx);
        const bool none = m_new == -INFINITY;   // no key of this column so far
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f((m - m_new) * c);
        const float mb = none ? 0.f : m_new * c;
        u32x4 pw[2];
        float ls = 0.f, lbs = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * t], c, -mb));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * t + 1], c, -mb));
                const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
                ls += e0 + e1;
                lbs += (float)pr[0] + (float)pr[1];
                pw[kk][t] = __builtin_bit_cast(uint32_t, pr);
            }
        l = l * alpha + ls;
        lb = lb * alpha + lbs;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        // exact: in a block with keys past kmin (rows r0.. of the block) their
        // V rows are cleared in this wave's LDS before the product and their
        // weights taken out of O's divisor; the epilogue adds their terms for
        // the columns that see them.
        if constexpr (EX) {
            const int r0 = max(0, kmin + 1 - kb);
            for (int idx = (r0 << 4) + lane; idx < KB * 16; idx += 64)
                *(u32x4*)(lds + vs + 16 * idx) = u32x4{0u, 0u, 0u, 0u};
            float hid = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kr = 8 * (r >> 2) + 4 * hh + (r & 3);
                const uint32_t w2 = pw[r >> 3][(r & 7) >> 1];
                const float w = bf16_bits_to_f32((uint16_t)((r & 1) ? (w2 >> 16) : (w2 & 0xFFFFu)));
                hid += kr >= r0 ? w : 0.f;
            }
            lb -= hid;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.tr(lds, vs, db, kk),
                                                                __builtin_bit_cast(bf16x8, pw[kk]),
                                                                o[db], 0, 0, 0);
        m = m_new;
        // the ring slot of block g is free once its MFMAs have their operands
        if (g + DC_RING < nb) issue(g + DC_RING);
    };
    // an exact wave runs the blocks from the first one with a key past kmin
    // in the exact form (the blocks wholly at or below kmin come first)
    const int n_common = exact ? min(nb, max(0, kmin + 1 - lo) / KB) : nb;
    for (int g = 0; g < n_common; ++g) block(g, std::false_type{});
    for (int g = n_common; g < nb; ++g) block(g, std::true_type{});

    // exact: the terms of the keys past kmin that a column sees, against the
    // final reference: the raw score again on the vector unit (this lane's 64
    // head dims of q, the partner lane's other 64), its weight rounded to bf16
    // as the product's weights are, counted in O's divisor.
    const int j_end = min(hi - 1, kmax);
    if (exact && nb > 0 && kmin < j_end) {   // wave-uniform
        const float mbf = m == -INFINITY ? 0.f : m * c;
        for (int j = max(lo, kmin + 1); j <= j_end; ++j) {
            const uint16_t* krow = kbase + (size_t)j * HD;
            float sd = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4 x = *(const u32x4*)(krow + 16 * ks + 8 * hh);
                const u32x4 y = __builtin_bit_cast(u32x4, qf[ks]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sd = fmaf(bf16_bits_to_f32((uint16_t)(y[e] & 0xFFFFu)),
                              bf16_bits_to_f32((uint16_t)(x[e] & 0xFFFFu)), sd);
                    sd = fmaf(bf16_bits_to_f32((uint16_t)(y[e] >> 16)),
                              bf16_bits_to_f32((uint16_t)(x[e] >> 16)), sd);
                }
            }
            sd = wave_swap_sum(sd);
            const bool sees = klim >= j;
            const float pb = (float)(__bf16)__builtin_amdgcn_exp2f(fmaf(sd, c, -mbf));
            if (sees && hh == 0) lb += pb;
            const uint16_t* vrow = vbase + (size_t)j * HD + 4 * hh;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const uint2 x = *(const uint2*)(vrow + 32 * db + 8 * r4);
                    const int r = 4 * r4;
                    const float v0 = bf16_bits_to_f32((uint16_t)(x.x & 0xFFFFu));
                    const float v1 = bf16_bits_to_f32((uint16_t)(x.x >> 16));
                    const float v2 = bf16_bits_to_f32((uint16_t)(x.y & 0xFFFFu));
                    const float v3 = bf16_bits_to_f32((uint16_t)(x.y >> 16));
                    o[db][r + 0] = sees ? fmaf(pb, v0, o[db][r + 0]) : o[db][r + 0];
                    o[db][r + 1] = sees ? fmaf(pb, v1, o[db][r + 1]) : o[db][r + 1];
                    o[db][r + 2] = sees ? fmaf(pb, v2, o[db][r + 2]) : o[db][r + 2];
                    o[db][r + 3] = sees ? fmaf(pb, v3, o[db][r + 3]) : o[db][r + 3];
                }
        }
    }

    // partial O = O^T / sum bf16(p) and LSE = m*|scale| + ln(sum p).  A column
    // with no key in this split gets O = 0 and LSE = -inf; one whose keys all
    // scored -inf gets LSE = -inf and O = sum 0 * v (0, or NaN where such a
    // key's V is not finite: the formula's terms); a NaN or +inf score makes
    // the sum, so the LSE and O, NaN.
    const float l_tot = wave_swap_sum(l);
    const float lb_tot = wave_swap_sum(lb);
    if (col_ok) {
        const size_t row = ((size_t)b * p.Hq + h) * (size_t)M + i;
        const size_t part = row * p.n_splits + split;
        const bool any = !(l_tot == 0.f);
        const float inv = any ? 1.0f / lb_tot : 0.f;
        float* orow = p.o_part + part * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 ov;
#pragma unroll
                for (int t = 0; t < 4; ++t) ov[t] = o[db][4 * r4 + t] * inv;
                *(f32x4*)(orow + 32 * db + 8 * r4 + 4 * hh) = ov;
            }
        if (hh == 0) p.lse_part[part] = any ? m * p.lse_scale + logf(l_tot) : -INFINITY;
    }
}

// One workgroup per output row: LSE = max + ln sum exp(LSE_p - max) and
// O = sum exp(LSE_p - LSE) O_p.  Thread t accumulates head dims
// 4(t%32) .. +3 over the parts p = t/32 (mod 8); the 8 partial sums are then
// added in a fixed order, so the result is reproducible.
constexpr int MG_THREADS = 256;
constexpr int MG_GROUPS = MG_THREADS / 32;

// is_max: NaN-propagating maximum (a NaN LSE_p makes the row NaN)
__device__ __forceinline__ float block_reduce(float x, float* red, bool is_max) {
    x = is_max ? wave_maximum_all(x) : wave_sum_all(x);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < MG_THREADS / 64; ++i)
        r = is_max ? __builtin_elementwise_maximum(r, red[i]) : r + red[i];
    __syncthreads();
    return r;
}

// keyed_rows: every row has at least one allowed key (decode), so parts that
// all have LSE -inf mean keys that all scored -inf: the formula's NaN.
// Without it such a row counts as having no keys: O = 0, LSE = -inf.
__global__ __launch_bounds__(MG_THREADS) void attn_lse_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int n_parts,
    uint16_t* __restrict__ o, float* __restrict__ lse, int keyed_rows) {
    __shared__ float red[MG_THREADS / 64];
    __shared__ f32x4 part[MG_GROUPS][32];
    const int t = threadIdx.x;
    const size_t row = blockIdx.x;
    const float* lp = lse_part + row * n_parts;
    float mx = -INFINITY;
    for (int s = t; s < n_parts; s += MG_THREADS) mx = __builtin_elementwise_maximum(mx, lp[s]);
    mx = block_reduce(mx, red, true);
    uint16_t* orow = o + row * HD;
    if (mx == -INFINITY) {
        const uint32_t fill = keyed_rows ? 0x7FC07FC0u : 0u;   // bf16 NaN pairs, or zeros
        if (t < HD / 2) *(uint32_t*)(orow + 2 * t) = fill;
        if (t == 0 && lse) lse[row] = keyed_rows ? __builtin_nanf("") : -INFINITY;
        return;
    }
    float tot = 0.f;
    for (int s = t; s < n_parts; s += MG_THREADS) tot += expf(lp[s] - mx);
    tot = block_reduce(tot, red, false);
    const float L = mx + logf(tot);
    const int d4 = t & 31, sg = t >> 5;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    const float* op = o_part + row * (size_t)n_parts * HD + 4 * d4;
#pragma unroll 4
    for (int s = sg; s < n_parts; s += MG_GROUPS) {
        const float w = expf(lp[s] - L);
        const f32x4 x = *(const f32x4*)(op + (size_t)s * HD);
        a[0] = fmaf(w, x[0], a[0]);
        a[1] = fmaf(w, x[1], a[1]);
        a[2] = fmaf(w, x[2], a[2]);
        a[3] = fmaf(w, x[3], a[3]);
    }
    part[sg][d4] = a;
    __syncthreads();
    if (sg == 0) {
        f32x4 r = part[0][d4];
#pragma unroll
        for (int g = 1; g < MG_GROUPS; ++g) r += part[g][d4];
        *(uint32_t*)(orow + 4 * d4) = tile::pack_bf16(r[0], r[1]);
        *(uint32_t*)(orow + 4 * d4 + 2) = tile::pack_bf16(r[2], r[3]);
    }
    if (t == 0 && lse) lse[row] = L;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Plan {
    int gm, n_cb, n_splits, n_blocks;
    int64_t rows;
};

// Splits: about DC_TARGET_WAVES waves in all, unless the
// caller fixes the count; chosen automatically, at most L / (8 g M) splits so
// the partial results (g*M rows of D+1 floats per split) stay within about an
// eighth of the K/V bytes; never more than one split per 32-key block.
Plan make_plan(int B, int H_q, int H_kv, int M, int L, int n_splits) {
    Plan pl;
    pl.gm = (H_q / H_kv) * M;
    pl.n_cb = (pl.gm + 31) / 32;
    pl.rows = (int64_t)B * H_q * M;
    pl.n_blocks = (L + KB - 1) / KB;
    const int64_t units = (int64_t)B * H_kv * pl.n_cb;
    int64_t s = n_splits;
    if (s <= 0) {
        s = (DC_TARGET_WAVES + units - 1) / units;
        s = std::min<int64_t>(s, (int64_t)L / (8 * (int64_t)pl.gm));
        s = std::max<int64_t>(s, 1);
    }
    pl.n_splits = (int)std::min<int64_t>(s, pl.n_blocks);
    return pl;
}

size_t part_o_bytes(const Plan& pl) { return (size_t)pl.rows * pl.n_splits * HD * 4; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
size_t workspace_bytes(const Plan& pl) {
    return align_up(part_o_bytes(pl), 256) + (size_t)pl.rows * pl.n_splits * 4;
}

attn_status check_decode_shape(int B, int H_q, int H_kv, int M, int L, int D, int causal,
                               float scale) {
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || M <= 0 || L <= 0 || D <= 0) return ATTN_ERR_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_GQA;
    if (D != HD) return ATTN_ERR_HEAD_DIM;
    if (causal && M > L) return ATTN_ERR_SHAPE;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    // a K/V panel is addressed with 32-bit byte offsets; counts fit in int
    if ((int64_t)L * ROW_BYTES >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    if ((int64_t)B * H_q * M > INT32_MAX / 2) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

attn_status launch_merge(const float* o_part, const float* lse_part, int rows, int n_parts,
                         void* o, float* lse, bool keyed_rows, hipStream_t s) {
    if (rows == 0) return ATTN_OK;
    hipLaunchKernelGGL(attn_lse_merge_kernel, dim3((unsigned)rows), dim3(MG_THREADS), 0, s,
                       o_part, lse_part, n_parts, (uint16_t*)o, lse, keyed_rows ? 1 : 0);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Validates the decode arguments shared by attn_decode and attn_decode_partial
// (the outputs listed in outs/out_bytes must not overlap q, k, v or each
// other) and fills the split kernel's parameters.
attn_status prepare_split(const void* q, const void* k, const void* v, const void* const* outs,
                          const size_t* out_bytes, int n_out, int B, int H_q, int H_kv, int M,
                          int L, int D, int causal, float scale, const Plan& pl, DecParams& p) {
    const int64_t total_waves = (int64_t)B * H_kv * pl.n_cb * pl.n_splits;
    if (total_waves > INT32_MAX - DC_WAVES) return ATTN_ERR_SHAPE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15) return ATTN_ERR_ALIGN;
    const size_t qb = (size_t)B * H_q * M * HD * 2;
    const size_t kvb = (size_t)B * H_kv * L * HD * 2;
    const void* ins[3] = {q, k, v};
    const size_t in_bytes[3] = {qb, kvb, kvb};
    for (int a = 0; a < n_out; ++a) {
        for (int j = 0; j < 3; ++j)
            if (ranges_overlap(outs[a], out_bytes[a], ins[j], in_bytes[j])) return ATTN_ERR_ALIAS;
        for (int j = a + 1; j < n_out; ++j)
            if (ranges_overlap(outs[a], out_bytes[a], outs[j], out_bytes[j])) return ATTN_ERR_ALIAS;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev)) return ATTN_ERR_DEVICE;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.M = M;
    p.L = L;
    p.group = H_q / H_kv;
    p.gm = pl.gm;
    p.n_cb = pl.n_cb;
    p.n_splits = pl.n_splits;
    p.n_blocks = pl.n_blocks;
    p.total_waves = (int)total_waves;
    p.causal = causal ? 1 : 0;
    const float mag = std::fabs(scale);
    p.q_mode = scale > 0.f ? 0 : (scale < 0.f ? 1 : 2);
    p.c = (float)((double)(mag > 0.f ? mag : 1.0f) * 1.4426950408889634);
    p.lse_scale = mag;
    return ATTN_OK;
}

attn_status launch_split(const DecParams& p, hipStream_t s) {
    const int grid = (p.total_waves + DC_WAVES - 1) / DC_WAVES;
    hipLaunchKernelGGL(attn_decode_split_kernel, dim3((unsigned)grid), dim3(DC_THREADS), 0, s, p);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// attn_decode_noalloc's partial results: one array per GPU, shared by every
// call on that GPU.  Host code never uses the name `scratch` as an address (on
// the host it is only a stand-in for the device symbol): the device address
// comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

// Device address of this device's copy of `scratch` (dev must be current), or
// nullptr if the runtime cannot give it.
void* scratch_on(int dev) {
    constexpr int MAX_DEVICES = 64;
    static std::atomic<void*> cache[MAX_DEVICES];
    if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
    void* ptr = cache[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return nullptr;
        cache[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

extern "C" size_t attn_decode_workspace_bytes(int B, int H_q, int H_kv, int M, int L, int D,
                                              int n_splits) {
    if (check_decode_shape(B, H_q, H_kv, M, L, D, 0, 1.0f) != ATTN_OK) return 0;
    return workspace_bytes(make_plan(B, H_q, H_kv, M, L, n_splits));
}

extern "C" int attn_decode_splits(int B, int H_q, int H_kv, int M, int L, int D, int n_splits) {
    if (check_decode_shape(B, H_q, H_kv, M, L, D, 0, 1.0f) != ATTN_OK) return 0;
    return make_plan(B, H_q, H_kv, M, L, n_splits).n_splits;
}

extern "C" attn_status attn_decode(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int H_q, int H_kv, int M, int L, int D,
                                   int causal, float scale, int n_splits, void* workspace,
                                   size_t workspace_size, void* stream) {
    if (!q || !k || !v || !o || !workspace) return ATTN_ERR_NULL;
    attn_status st = check_decode_shape(B, H_q, H_kv, M, L, D, causal, scale);
    if (st != ATTN_OK) return st;
    const Plan pl = make_plan(B, H_q, H_kv, M, L, n_splits);
    const size_t ws = workspace_bytes(pl);
    if (workspace_size < ws) return ATTN_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 15) || ((uintptr_t)o & 3) || ((uintptr_t)lse & 3))
        return ATTN_ERR_ALIGN;
    const void* outs[3] = {o, lse, workspace};
    const size_t out_bytes[3] = {(size_t)pl.rows * HD * 2, lse ? (size_t)pl.rows * 4 : 0, ws};
    DecParams p;
    st = prepare_split(q, k, v, outs, out_bytes, 3, B, H_q, H_kv, M, L, D, causal, scale, pl, p);
    if (st != ATTN_OK) return st;
    p.o_part = (float*)workspace;
    p.lse_part = (float*)((char*)workspace + align_up(part_o_bytes(pl), 256));
    const hipStream_t s = (hipStream_t)stream;
    st = launch_split(p, s);
    if (st != ATTN_OK) return st;
    return launch_merge(p.o_part, p.lse_part, (int)pl.rows, pl.n_splits, o, lse, true, s);
}

extern "C" attn_status attn_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                           float* lse, int B, int H_q, int H_kv, int M, int L,
                                           int D, int causal, float scale, int n_splits,
                                           void* stream) {
    if (!q || !k || !v || !o) return ATTN_ERR_NULL;
    attn_status st = check_decode_shape(B, H_q, H_kv, M, L, D, causal, scale);
    if (st != ATTN_OK) return st;
    const Plan pl = make_plan(B, H_q, H_kv, M, L, n_splits);
    if (workspace_bytes(pl) > ATTN_DECODE_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    if (((uintptr_t)o & 3) || ((uintptr_t)lse & 3)) return ATTN_ERR_ALIGN;
    const void* outs[2] = {o, lse};
    const size_t out_bytes[2] = {(size_t)pl.rows * HD * 2, lse ? (size_t)pl.rows * 4 : 0};
    DecParams p;
    st = prepare_split(q, k, v, outs, out_bytes, 2, B, H_q, H_kv, M, L, D, causal, scale, pl, p);
    if (st != ATTN_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_DEVICE;
    char* const ws = (char*)scratch_on(dev);
    if (ws == nullptr) return ATTN_ERR_LAUNCH;
    p.o_part = (float*)ws;
    p.lse_part = (float*)(ws + align_up(part_o_bytes(pl), 256));
    const hipStream_t s = (hipStream_t)stream;
    st = launch_split(p, s);
    if (st != ATTN_OK) return st;
    return launch_merge(p.o_part, p.lse_part, (int)pl.rows, pl.n_splits, o, lse, true, s);
}

extern "C" attn_status attn_decode_partial(const void* q, const void* k, const void* v,
                                           float* o_part, float* lse_part, int B, int H_q,
                                           int H_kv, int M, int L, int D, int causal, float scale,
                                           int n_splits, void* stream) {
    if (!q || !k || !v || !o_part || !lse_part) return ATTN_ERR_NULL;
    attn_status st = check_decode_shape(B, H_q, H_kv, M, L, D, causal, scale);
    if (st != ATTN_OK) return st;
    if (n_splits < 1 || n_splits > (L + KB - 1) / KB) return ATTN_ERR_SHAPE;
    const Plan pl = make_plan(B, H_q, H_kv, M, L, n_splits);
    if (((uintptr_t)o_part & 15) || ((uintptr_t)lse_part & 3)) return ATTN_ERR_ALIGN;
    const void* outs[2] = {o_part, lse_part};
    const size_t out_bytes[2] = {part_o_bytes(pl), (size_t)pl.rows * pl.n_splits * 4};
    DecParams p;
    st = prepare_split(q, k, v, outs, out_bytes, 2, B, H_q, H_kv, M, L, D, causal, scale, pl, p);
    if (st != ATTN_OK) return st;
    p.o_part = o_part;
    p.lse_part = lse_part;
    return launch_split(p, (hipStream_t)stream);
}

extern "C" attn_status attn_lse_merge(const float* o_part, const float* lse_part, int rows,
                                      int n_parts, int D, void* o, float* lse, void* stream) {
    if (!o_part || !lse_part || !o) return ATTN_ERR_NULL;
    if (rows < 0 || n_parts <= 0 || D <= 0) return ATTN_ERR_SHAPE;
    if (D != HD) return ATTN_ERR_HEAD_DIM;
    if ((int64_t)rows * n_parts > INT32_MAX) return ATTN_ERR_SHAPE;
    if ((((uintptr_t)o_part) & 15) != 0 || (((uintptr_t)lse_part | (uintptr_t)o | (uintptr_t)lse) & 3) != 0)
        return ATTN_ERR_ALIGN;
    const size_t opb = (size_t)rows * n_parts * HD * 4, lpb = (size_t)rows * n_parts * 4;
    const size_t ob = (size_t)rows * HD * 2, lb = lse ? (size_t)rows * 4 : 0;
    if (ranges_overlap(o, ob, o_part, opb) || ranges_overlap(o, ob, lse_part, lpb) ||
        ranges_overlap(lse, lb, o_part, opb) || ranges_overlap(lse, lb, lse_part, lpb) ||
        ranges_overlap(o, ob, lse, lb))
        return ATTN_ERR_ALIAS;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev)) return ATTN_ERR_DEVICE;
    return launch_merge(o_part, lse_part, rows, n_parts, o, lse, false, (hipStream_t)stream);
}

extern "C" double attn_decode_flops(int B, int H_q, int M, int L, int D, int causal) {
    // 4*D flops per allowed (query row, key) pair
    double pairs = (double)M * L;
    if (causal) pairs = (double)M * L - 0.5 * (double)M * (M - 1);
    return 4.0 * B * H_q * D * pairs;
}
