// Fused scaled dot-product attention backward for MI355X (gfx950, CDNA4).
//
// Given Q, K, V, the forward's output O and per-row LSE, and the output
// gradient dO, computes dQ, dK, dV by recomputing the probabilities from the
// saved LSE instead of storing them (page "AVO算法优化Transformer注意力机制性能
// 解析", section 2.2: recomputation in the backward pass; page "GPU注意力算子
// 性能优化" (QiMeng-Attention), section 2.2.2: the backward's gradients).  With
// c = scale * log2(e) and the chain rule through softmax:
//
//     P_ij    = exp2(c * q_i.k_j - LSE_i * log2(e))
//     delta_i = dO_i . O_i                   (= sum_j P_ij dP_ij)
//     dP_ij   = dO_i . v_j,   dS_ij = P_ij (dP_ij - delta_i)
//     dV_j    = sum_i P_ij dO_i
//     dK_j    = scale * sum_i dS_ij q_i,   dQ_i = scale * sum_j dS_ij k_j
//
// dK and dV of a shared K/V head sum over the query heads of its group.
//
// Two kernels, no atomics (results are bitwise reproducible):
//   * attn_bwd_dq: one workgroup = 8 waves = 256 query rows of one head; the
//     structure of the forward kernel.  Each wave keeps its 32 rows of Q and dO
//     in VGPRs as MFMA B operands and streams 32-key blocks of K and V through
//     LDS (LDS DMA, double-buffered 64-key tiles).  Per block it computes
//     S^T = K Q^T and dP^T = V dO^T, turns them into dS^T (one query per lane,
//     so LSE and delta are per-lane scalars) and accumulates
//     dQ^T += K^T dS^T, reading K^T with the transposing LDS read.  It also
//     computes delta_i from O and dO once per row and writes it out.
//   * attn_bwd_dkdv: one workgroup = 8 waves = 128 keys of one K/V head,
//     as 4 pairs of waves that own 32 keys each.  Wave A of a pair keeps K of
//     its keys in VGPRs (MFMA B operand) and the fp32 dV^T accumulator; wave B
//     keeps V and dK^T.  64-row tiles of Q, dO, LSE and delta of every query
//     head of the group stream through LDS.  Per tile, wave A computes S = Q K^T
//     (one key per lane), P, and dV^T += dO^T P, and leaves P (bf16) in LDS;
//     one tile later wave B computes dP = dO V^T, dS = P (dP - delta) and
//     dK^T += Q^T dS.  dO^T and Q^T are read with the transposing LDS read.
//     The two waves of a pair share a SIMD, so A's softmax overlaps B's MFMAs.
//   * attn_bwd_ws may split each group's query heads into parts in the dK/dV
//     step, so that few K/V heads still give one workgroup per CU: each part
//     writes fp32 dV and dK sums to a workspace and attn_bwd_reduce_kernel adds
//     the parts in part order (still reproducible bitwise) and rounds to bf16.
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
// 32-row tiles of 128 head dims (256-byte rows) in the shared swizzled LDS layout
using tile::BLK_BYTES;
using tile::HD;
using tile::KB;
using tile::ROW_BYTES;
using tile::pack_bf16;
using tile::swz;
using TileReads = tile::Reads;
constexpr float LOG2E = 1.4426950408889634f;

// attn_bwd_dq: 8 waves, rings of 4 K blocks and 4 V blocks
constexpr int DQ_WAVES = 8;                // 8-wave dQ workgroups (4 for short sequences and small grids)
constexpr int DQ_K_RING = 0;
constexpr int DQ_V_RING = 4 * BLK_BYTES;
constexpr int DQ_LDS = 8 * BLK_BYTES;      // 64 KiB

// attn_bwd_dkdv: 8 waves = 4 pairs x 32 keys.  In a pair, wave A (waves 0-3)
// computes S, P and dV; wave B (waves 4-7) computes dP, dS and dK one tile
// later, reading A's P from LDS.  Three stages of (Q, dO, LSE, delta) x 64
// rows (A's tile, B's tile, the tile in flight), each with its set of P slots.
constexpr int KV_PAIRS = 4;
constexpr int KV_WAVES = 2 * KV_PAIRS;
constexpr int KV_THREADS = KV_WAVES * 64;
constexpr int KV_KEYS = KV_PAIRS * 32;
constexpr int KV_QROWS = 64;
constexpr int KV_TILE = KV_QROWS * ROW_BYTES;           // 16 KiB
constexpr int KV_LSE = 2 * KV_TILE;                     // offset of LSE in a stage
constexpr int KV_DELTA = KV_LSE + KV_QROWS * 4;         // offset of delta in a stage
constexpr int KV_STAGE = KV_DELTA + KV_QROWS * 4;
constexpr int KV_NSTAGE = 3;
constexpr int KV_PSUB = 2 * 1024;                       // bf16 P of one 32x32 sub-block
constexpr int KV_PSET = KV_PAIRS * (KV_QROWS / 32) * KV_PSUB;
constexpr int KV_P = KV_NSTAGE * KV_STAGE;              // offset of the P slots
constexpr int KV_LDS = KV_P + KV_NSTAGE * KV_PSET;   // P slots per stage

struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;
    const float* lse;
    uint16_t *dq, *dk, *dv;
    float* delta;
    int B, Hq, Hkv, N;
    int group;              // Hq / Hkv
    int n_qtiles, total_q;  // attn_bwd_dq grid: B * Hq * ceil(N / (32 * dq_waves))
    int dq_waves;           // attn_bwd_dq workgroup: 8 waves, or 4 for short sequences
    int cgroup;             // attn_bwd_dq, causal: heads whose tiles are interleaved
    int kgroup;             // attn_bwd_dkdv, causal: (batch, K/V head, part)s interleaved
    int n_ktiles, total_k;  // attn_bwd_dkdv grid: B * Hkv * ceil(N / 128) * n_split
    int n_split;            // dK/dV: parts of each group's query heads (1: write dk, dv)
    int dealt_q, dealt_k;   // causal: the dealt grid order (dealt_tile) instead of the plain one
    Deal deal_q, deal_k;    // its sizes for the dQ and dK/dV grids
    float* ws;              // n_split > 1: fp32 partials [n_split][dV, dK][B * Hkv * N][D]
    float c;                // scale * log2(e)
    float scale;
};

__device__ __forceinline__ void store_row_f32(float* row, const f32x16 (&acc)[4], float mul, int hh) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[db][4 * r4 + i] * mul;
            *(f32x4*)(row + 32 * db + 8 * r4 + 4 * hh) = v;
        }
}

__device__ __forceinline__ void store_row_bf16(uint16_t* row, const f32x16 (&acc)[4], float mul,
                                               int hh) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (__bf16)(acc[db][4 * r4 + i] * mul);
            *(bf16x4*)(row + 32 * db + 8 * r4 + 4 * hh) = v;
        }
}

// ---------------------------------------------------------------------------
// dQ (and delta)
// ---------------------------------------------------------------------------
template <bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_bwd_dq_kernel(BwdParams p) {
    static_assert(NW == 8 || NW == 4, "dQ workgroups of 4 or 8 waves");
    constexpr int DQ_THREADS = NW * 64;
    constexpr int DQ_ROWS = NW * 32;
    constexpr int DPW = 8 / NW;   // 4-row DMA instructions per wave per key block
    __shared__ __attribute__((aligned(1024))) char lds[DQ_LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;   // query column owned by this lane
    const int hh = lane >> 5;

    // causal: groups of cgroup heads one after another (a group's tiles share K
    // and V in one XCD's L2), tile-major and heaviest tile first within a group;
    // a group holds at least an XCD's worth of workgroup slots, so light tiles
    // of one group, not heavy tiles of the next, end each XCD's share
    const int logical = xcd_remap(blockIdx.x, p.total_q);
    int bh, qt;
    if (CAUSAL && p.dealt_q) {
        // head groups that do not split evenly over the 8 XCDs: slices of
        // groups dealt to the XCDs in turn, each a strided share of its
        // group's heaviest-first list (whole workgroup, no barrier yet)
        if (!dealt_tile(blockIdx.x, p.B * p.Hq, p.cgroup > 1 ? p.cgroup : 1, p.n_qtiles, p.deal_q, bh, qt))
            return;   // padding of the grid
    } else if (CAUSAL) {
        const int per = p.B * p.Hq;
        const int G = p.cgroup > 1 ? p.cgroup : 1;
        const int grp = logical / (G * p.n_qtiles);
        const int r = logical - grp * G * p.n_qtiles;
        const int gh = min(G, per - grp * G);
        qt = p.n_qtiles - 1 - r / gh;
        bh = grp * G + r % gh;
    } else {
        bh = logical / p.n_qtiles;
        qt = logical % p.n_qtiles;
    }
    const int b = bh / p.Hq;
    const int h = bh % p.Hq;
    const int kvh = h / p.group;
    const int N = p.N;
    const int q0 = qt * DQ_ROWS;
    const int wq0 = q0 + wave * 32;
    const int myq = wq0 + l32;

    const size_t row_panel = ((size_t)b * p.Hq + h) * (size_t)N;
    const size_t qo_panel = row_panel * HD;
    const size_t kv_panel = ((size_t)b * p.Hkv + kvh) * (size_t)N * HD;
    const uint16_t* kbase = p.k + kv_panel;
    const uint16_t* vbase = p.v + kv_panel;

    // key blocks streamed by the workgroup (n_blk_wg) and used by this wave (n_blk)
    const int n_blk_all = (N + KB - 1) / KB;
    int n_blk_wg = n_blk_all, n_blk = n_blk_all;
    if (CAUSAL) {
        n_blk_wg = min(n_blk_all, (min(q0 + DQ_ROWS, N) - 1) / KB + 1);
        n_blk = min(n_blk_all, wq0 / KB + 1);
    }
    if (wq0 >= N) n_blk = 0;

    // LDS DMA: block g of K (V) goes to slot g % 4 of the K (V) ring; wave w
    // copies rows 4*DPW*w .. +4*DPW-1 with DPW 16-byte-per-lane DMAs of 4 rows.
    // The swizzle is applied on the global side: a lane fetches the chunk that
    // belongs at its LDS position.
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    uint32_t dma_off[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int drow = 4 * DPW * wave + 4 * i + (lane >> 4);
        dma_off[i] = (uint32_t)(drow * ROW_BYTES + (((lane & 15) ^ swz(drow)) << 4));
    }
    auto dma_block = [&](const uint16_t* panel, int ring, int g) {
        if (g < n_blk_wg) {
            const u32x4 r = sgpr_rsrc(panel + (size_t)g * KB * HD, (uint32_t)(N - g * KB) * ROW_BYTES);
            const uint32_t dst = lds_base + ring + (g & 3) * BLK_BYTES + 4 * DPW * wave * ROW_BYTES;
#pragma unroll
            for (int i = 0; i < DPW; ++i) lds_dma16(r, dst + 4 * i * ROW_BYTES, dma_off[i]);
        }
    };

    TileReads rd;
    rd.init(lane);

    if (N % KB != 0) {
        // rows past N of the tail block must read as finite values (zeros)
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < DQ_LDS / (16 * DQ_THREADS); ++i)
            *(u32x4*)(lds + 16 * (tid + DQ_THREADS * i)) = z;
        __syncthreads();
    }
    dma_block(kbase, DQ_K_RING, 0);
    dma_block(vbase, DQ_V_RING, 0);
    dma_block(kbase, DQ_K_RING, 1);
    dma_block(vbase, DQ_V_RING, 1);

    // this lane's half row (head dims 16ks + 8hh .. +7) of Q and dO as B
    // operands; delta from O and dO; the row's LSE in base 2
    bf16x8 qf[8], df[8];
    float delta, lse2;
    {
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.q + qo_panel, (uint32_t)N * ROW_BYTES);
        const __amdgpu_buffer_rsrc_t dr = make_rsrc(p.dout + qo_panel, (uint32_t)N * ROW_BYTES);
        const __amdgpu_buffer_rsrc_t orr = make_rsrc(p.o + qo_panel, (uint32_t)N * ROW_BYTES);
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const uint32_t off = (uint32_t)myq * ROW_BYTES + (16 * ks + 8 * hh) * 2;
            qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(qr, off));
            df[ks] = __builtin_bit_cast(bf16x8, buf_load16(dr, off));
            const bf16x8 ov = __builtin_bit_cast(bf16x8, buf_load16(orr, off));
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = fmaf((float)df[ks][i], (float)ov[i], acc);
        }
        delta = wave_swap_sum(acc);
        const __amdgpu_buffer_rsrc_t lr = make_rsrc(p.lse + row_panel, (uint32_t)N * 4);
        lse2 = buf_load_f32(lr, (uint32_t)myq * 4) * LOG2E;
    }
    if (hh == 0 && myq < N) p.delta[row_panel + myq] = delta;
    const float c = p.c;

    f32x16 dq[4];   // dQ^T: 4 blocks of 32 head dims x 32 query columns
#pragma unroll
    for (int db = 0; db < 4; ++db) dq[db] = f32x16{};

    // Key block g from ring slot SLOT.
    auto step = [&](auto slot_t, int g) __attribute__((always_inline)) {
        constexpr uint32_t KS = DQ_K_RING + decltype(slot_t)::value * BLK_BYTES;
        constexpr uint32_t VS = DQ_V_RING + decltype(slot_t)::value * BLK_BYTES;
        if (g >= n_blk) return;
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.row(lds, KS, ks), qf[ks], s, 0, 0, 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.row(lds, VS, ks), df[ks], dp, 0, 0, 0);
        const bool mask = (CAUSAL && g * KB + KB - 1 > wq0) || (g * KB + KB > N);
        u32x4 dsw[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float d2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 8 * kk + 2 * i + e;
                    float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
                    if (mask) {
                        const int key = g * KB + 8 * (r >> 2) + 4 * hh + (r & 3);
                        pr = (key >= N || (CAUSAL && key > myq)) ? 0.f : pr;
                    }
                    d2[e] = pr * (dp[r] - delta);
                }
                dsw[kk][i] = pack_bf16(d2[0], d2[1]);
            }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.tr(lds, KS, db, kk),
                                                                 __builtin_bit_cast(bf16x8, dsw[kk]),
                                                                 dq[db], 0, 0, 0);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    // vmcnt(0) through the builtin: the compiler then knows every VGPR load
    // above is complete and never waits on vmcnt (which counts the DMA) later
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // Tile t = blocks 2t, 2t+1 in slots (2t)%4, (2t+1)%4.  At its start the
    // workgroup prefetches tile t+1 into the slots tile t-1 used.
    const int n_tiles = (n_blk_wg + 1) / 2;
    for (int t = 0; t < n_tiles; t += 2) {
        dma_block(kbase, DQ_K_RING, 2 * t + 2);
        dma_block(vbase, DQ_V_RING, 2 * t + 2);
        dma_block(kbase, DQ_K_RING, 2 * t + 3);
        dma_block(vbase, DQ_V_RING, 2 * t + 3);
        step(I0{}, 2 * t);
        step(I1{}, 2 * t + 1);
        wait_dma();
        __syncthreads();
        if (t + 1 >= n_tiles) break;
        dma_block(kbase, DQ_K_RING, 2 * t + 4);
        dma_block(vbase, DQ_V_RING, 2 * t + 4);
        dma_block(kbase, DQ_K_RING, 2 * t + 5);
        dma_block(vbase, DQ_V_RING, 2 * t + 5);
        step(I2{}, 2 * t + 2);
        step(I3{}, 2 * t + 3);
        wait_dma();
        __syncthreads();
    }

    if (myq < N) store_row_bf16(p.dq + qo_panel + (size_t)myq * HD, dq, p.scale, hh);
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __launch_bounds__(KV_THREADS, 2) void attn_bwd_dkdv_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char lds[KV_LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave % KV_PAIRS;
    const bool is_a = wave < KV_PAIRS;   // A: S, P, dV.  B: dP, dS, dK.
    const int l32 = lane & 31;           // key column owned by this lane
    const int hh = lane >> 5;

    // with a causal mask the first key tiles of a head see the most rows, and
    // they come first in this order.  With n_split parts, part sp covers query
    // heads [sp*gh, (sp+1)*gh) of the group, and the key tiles of one (batch,
    // K/V head, part) stay consecutive.
    // Causal grids interleave the key tiles of kgroup such units (enough tiles
    // for one XCD's workgroup slots), tile by tile, so light tiles of one group,
    // not heavy tiles of the next, end each XCD's share.
    const int ns = p.n_split > 1 ? p.n_split : 1;
    const int logical = xcd_remap(blockIdx.x, p.total_k);
    int bks, kt;
    if (CAUSAL && p.dealt_k) {
        // units that do not split evenly over the 8 XCDs: dealt slices, as
        // for dQ; the heaviest key tile is the first
        int t;
        if (!dealt_tile(blockIdx.x, p.B * p.Hkv * ns, p.kgroup > 1 ? p.kgroup : 1, p.n_ktiles, p.deal_k, bks, t))
            return;   // padding of the grid (whole workgroup, no barrier yet)
        kt = p.n_ktiles - 1 - t;
    } else if (CAUSAL) {
        const int per = p.B * p.Hkv * ns;
        const int G = p.kgroup > 1 ? p.kgroup : 1;
        const int grp = logical / (G * p.n_ktiles);
        const int r = logical - grp * G * p.n_ktiles;
        const int gu = min(G, per - grp * G);
        kt = r / gu;
        bks = grp * G + r % gu;
    } else {
        bks = logical / p.n_ktiles;
        kt = logical % p.n_ktiles;
    }
    const int bk = bks / ns;
    const int sp = bks % ns;
    const int gh = p.group / ns;
    const int b = bk / p.Hkv;
    const int kvh = bk % p.Hkv;
    const int N = p.N;
    const int k0 = kt * KV_KEYS;
    const int wk0 = k0 + 32 * pair;      // first key of this pair
    const int myk = wk0 + l32;
    const size_t kv_panel = ((size_t)b * p.Hkv + kvh) * (size_t)N * HD;

    // query tiles of 64 rows: t0..n_qt-1 for each query head of the part
    const int n_qt = (N + KV_QROWS - 1) / KV_QROWS;
    const int t0 = CAUSAL ? k0 / KV_QROWS : 0;
    const int n_t = n_qt - t0;
    const int n_it = gh * n_t;

    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    uint32_t dma_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 8 * wave + 4 * i + (lane >> 4);
        dma_off[i] = (uint32_t)(row * ROW_BYTES + (((lane & 15) ^ swz(row)) << 4));
    }
    // stage it % 3 <- Q, dO, LSE, delta of iteration it
    auto issue = [&](int it) {
        if (it >= n_it) return;
        const int hq = kvh * p.group + sp * gh + it / n_t;
        const int t = t0 + it % n_t;
        const size_t r0 = ((size_t)b * p.Hq + hq) * (size_t)N + (size_t)t * KV_QROWS;
        const uint32_t left = (uint32_t)(N - t * KV_QROWS);
        const uint32_t st = lds_base + (uint32_t)(it % KV_NSTAGE) * KV_STAGE;
        const u32x4 qr = sgpr_rsrc(p.q + r0 * HD, left * ROW_BYTES);
        const u32x4 dr = sgpr_rsrc(p.dout + r0 * HD, left * ROW_BYTES);
        const uint32_t wrow = (uint32_t)(8 * wave) * ROW_BYTES;
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_dma16(qr, st + wrow + 4 * i * ROW_BYTES, dma_off[i]);
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_dma16(dr, st + KV_TILE + wrow + 4 * i * ROW_BYTES, dma_off[i]);
        if (wave == 0) lds_dma4(sgpr_rsrc(p.lse + r0, left * 4), st + KV_LSE, (uint32_t)lane * 4);
        if (wave == 1) lds_dma4(sgpr_rsrc(p.delta + r0, left * 4), st + KV_DELTA, (uint32_t)lane * 4);
    };
    // first row of iteration it's tile, and whether the pair computes it
    auto tile_row = [&](int it) { return (t0 + it % n_t) * KV_QROWS; };
    auto tile_live = [&](int rt) { return !(CAUSAL && rt + KV_QROWS - 1 < wk0); };
    auto tile_mask = [&](int rt) { return (CAUSAL && rt < wk0 + 31) || rt + KV_QROWS > N; };

    TileReads rd;
    rd.init(lane);

    if (N % KV_QROWS != 0) {
        // rows past N of the tail tile must read as finite values (zeros)
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int i = tid; i < KV_P / 16; i += KV_THREADS) *(u32x4*)(lds + 16 * i) = z;
        __syncthreads();
    }
    issue(0);

    // K (wave A) or V (wave B) of this lane's key as MFMA B operands, head
    // dims 16ks + 8hh .. +7; zeros past N
    bf16x8 kv[8];
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc((is_a ? p.k : p.v) + kv_panel, (uint32_t)N * ROW_BYTES);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            kv[ks] = __builtin_bit_cast(bf16x8, buf_load16(r, (uint32_t)myk * ROW_BYTES + (16 * ks + 8 * hh) * 2));
    }
    const float c = p.c;

    f32x16 acc[4];   // dV^T (wave A) or dK^T (wave B): 4 blocks of 32 head dims x 32 keys
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = f32x16{};

    // X = R K^T or R V^T for the 32 rows of R at LDS offset rs (S or dP)
    auto rows_x_kv = [&](uint32_t rs, f32x16& x) __attribute__((always_inline)) {
        x = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.row(lds, rs, ks), kv[ks], x, 0, 0, 0);
    };
    // acc^T += T^T W for the 32 rows of T at LDS offset ts, W in accumulator order
    auto accumulate = [&](uint32_t ts, const u32x4 (&w)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd.tr(lds, ts, db, kk),
                                                                  __builtin_bit_cast(bf16x8, w[kk]),
                                                                  acc[db], 0, 0, 0);
    };
    // P slot of (stage, pair, sub-block): lane-major, two 16-byte halves
    auto pslot = [&](uint32_t stage, int sb) {
        return (uint32_t)(KV_P + stage * KV_PSET + (pair * 2 + sb) * KV_PSUB + 16 * lane);
    };

    // Wave A, one tile in LDS stage STAGE: S -> P (bf16, also to LDS for wave
    // B) -> dV^T += dO^T P.  MASKED: rows past N, or (causal) before this lane's key.
    auto tile_a = [&](auto stage_t, auto mask_t, int rt) __attribute__((always_inline)) {
        constexpr uint32_t STAGE = decltype(stage_t)::value;
        constexpr bool MASKED = decltype(mask_t)::value;
        constexpr uint32_t st = STAGE * KV_STAGE;
        f32x16 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            rows_x_kv(st + 32 * sb * ROW_BYTES, s[sb]);
            const uint32_t ls = st + KV_LSE + (uint32_t)(32 * sb * 4);
            // register r holds row base + 8(r/4) + r%4 with base = rt + 32sb + 4hh; the
            // allowed rows are [myk (causal) or 0, N), i.e. offsets [lo, lo + span]
            int lo = 0, span = 0;
            if constexpr (MASKED) {
                const int base = rt + 32 * sb + 4 * hh;
                lo = CAUSAL ? myk - base : -base;
                span = (N - 1 - base) - lo;
                if (span < 0) { lo = 1 << 20; span = 0; }
            }
            u32x4 pw[2];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                // rows 8a + 4hh .. +3 of the sub-block are registers 4a .. 4a+3
                const f32x4 l4 = *(const f32x4*)(lds + ls + (8 * a + 4 * hh) * 4);
                float pv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float e = __builtin_amdgcn_exp2f(fmaf(s[sb][4 * a + i], c, -l4[i] * LOG2E));
                    if constexpr (MASKED) e = (uint32_t)(8 * a + i - lo) <= (uint32_t)span ? e : 0.f;
                    pv[i] = e;
                }
                pw[a >> 1][2 * (a & 1)] = pack_bf16(pv[0], pv[1]);
                pw[a >> 1][2 * (a & 1) + 1] = pack_bf16(pv[2], pv[3]);
            }
            const uint32_t ps = pslot(STAGE, sb);
            *(u32x4*)(lds + ps) = pw[0];
            *(u32x4*)(lds + ps + 1024) = pw[1];
            accumulate(st + KV_TILE + (uint32_t)(32 * sb * ROW_BYTES), pw);
        }
    };
    // Wave B, one tile in LDS stage STAGE (A's tile of the previous iteration):
    // dP, then dS = P (dP - delta) with A's bf16 P, then dK^T += Q^T dS.
    auto tile_b = [&](auto stage_t) __attribute__((always_inline)) {
        constexpr uint32_t STAGE = decltype(stage_t)::value;
        constexpr uint32_t st = STAGE * KV_STAGE;
        f32x16 dp[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            rows_x_kv(st + KV_TILE + 32 * sb * ROW_BYTES, dp[sb]);
            const uint32_t ps = pslot(STAGE, sb);
            const u32x4 pw[2] = {*(const u32x4*)(lds + ps), *(const u32x4*)(lds + ps + 1024)};
            const uint32_t ls = st + KV_DELTA + (uint32_t)(32 * sb * 4);
            u32x4 dsw[2];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 d4 = *(const f32x4*)(lds + ls + (8 * a + 4 * hh) * 4);
                float dsv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * a + i;
                    const uint32_t w = pw[r >> 3][(r & 7) >> 1];
                    const float pr = __builtin_bit_cast(float, (r & 1) ? (w & 0xFFFF0000u) : (w << 16));
                    dsv[i] = pr * (dp[sb][r] - d4[i]);
                }
                dsw[a >> 1][2 * (a & 1)] = pack_bf16(dsv[0], dsv[1]);
                dsw[a >> 1][2 * (a & 1) + 1] = pack_bf16(dsv[2], dsv[3]);
            }
            accumulate(st + (uint32_t)(32 * sb * ROW_BYTES), dsw);
        }
    };

    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // Iteration it: the DMA fills tile it+1 (stage (it+1)%3), wave A works on
    // tile it (stage it%3) and wave B on tile it-1 (stage (it-1)%3); one extra
    // iteration drains wave B.  The loop is unrolled by 3 so that every LDS
    // offset is a constant.  Each role runs its own copy of the loop (one shared
    // loop made the register allocator keep both roles' temporaries); both pass
    // the same n_it + 1 barriers.
    using S0 = std::integral_constant<uint32_t, 0>;
    using S1 = std::integral_constant<uint32_t, 1>;
    using S2 = std::integral_constant<uint32_t, 2>;
    if (is_a) {
        auto iter_a = [&](auto stage_t, int it) __attribute__((always_inline)) {
            issue(it + 1);
            if (it < n_it) {
                const int rt = tile_row(it);
                if (tile_live(rt)) {
                    if (tile_mask(rt)) tile_a(stage_t, std::true_type{}, rt);
                    else tile_a(stage_t, std::false_type{}, rt);
                }
            }
            wait_dma();
            __syncthreads();
        };
        for (int it = 0; it <= n_it; it += 3) {
            iter_a(S0{}, it);
            if (it + 1 > n_it) break;
            iter_a(S1{}, it + 1);
            if (it + 2 > n_it) break;
            iter_a(S2{}, it + 2);
        }
    } else {
        auto iter_b = [&](auto prev_stage_t, int it) __attribute__((always_inline)) {
            issue(it + 1);
            if (it > 0 && tile_live(tile_row(it - 1))) tile_b(prev_stage_t);
            wait_dma();
            __syncthreads();
        };
        for (int it = 0; it <= n_it; it += 3) {
            iter_b(S2{}, it);
            if (it + 1 > n_it) break;
            iter_b(S0{}, it + 1);
            if (it + 2 > n_it) break;
            iter_b(S1{}, it + 2);
        }
    }

    if (myk < N) {
        if (ns == 1) {
            if (is_a) store_row_bf16(p.dv + kv_panel + (size_t)myk * HD, acc, 1.0f, hh);
            else store_row_bf16(p.dk + kv_panel + (size_t)myk * HD, acc, p.scale, hh);
        } else {
            // this part's fp32 sums; attn_bwd_reduce_kernel adds the parts
            const size_t rows = (size_t)p.B * p.Hkv * N;
            const size_t part = (size_t)(2 * sp + (is_a ? 0 : 1)) * rows;
            store_row_f32(p.ws + (part + ((size_t)b * p.Hkv + kvh) * N + myk) * HD, acc,
                          is_a ? 1.0f : p.scale, hh);
        }
    }
}

// dV and dK from n_split fp32 partials: summed in part order (so the result is
// reproducible), rounded once to bf16.  One thread per 4 elements.
__global__ __launch_bounds__(256) void attn_bwd_reduce_kernel(const float* ws, uint16_t* dk,
                                                              uint16_t* dv, size_t rows, int ns) {
    const size_t n4 = rows * HD / 4;   // 4-element groups of one tensor
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n4; i += (size_t)gridDim.x * 256) {
        const size_t t = i >= n4 ? 1 : 0;   // 0: dV, 1: dK
        const size_t j = i - t * n4;
        f32x4 acc = ((const f32x4*)(ws + t * rows * HD))[j];
        for (int sp = 1; sp < ns; ++sp) {
            const f32x4 x = ((const f32x4*)(ws + (2 * (size_t)sp + t) * rows * HD))[j];
            acc[0] += x[0];
            acc[1] += x[1];
            acc[2] += x[2];
            acc[3] += x[3];
        }
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[e];
        ((bf16x4*)(t ? dk : dv))[j] = o;
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Buf {
    const void* ptr;
    size_t bytes;
    unsigned align;
};

// Checks the sizes, the pointers (non-NULL, aligned, outputs disjoint from
// inputs and from each other) and the device, then fills the kernel
// parameters.  Nothing is launched unless the result is ATTN_OK.
attn_status prepare(const Buf* ins, int n_in, const Buf* outs, int n_out, int B, int H_q,
                    int H_kv, int N, int D, int causal, float scale, BwdParams& p,
                    bool ws_short = false) {
    for (int i = 0; i < n_in; ++i)
        if (!ins[i].ptr) return ATTN_ERR_NULL;
    for (int i = 0; i < n_out; ++i)
        if (!outs[i].ptr) return ATTN_ERR_NULL;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0) return ATTN_ERR_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_GQA;
    if (D != HD) return ATTN_ERR_HEAD_DIM;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    // one head panel is addressed with 32-bit byte offsets
    if ((int64_t)N * ROW_BYTES >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    // 4-wave dQ workgroups (128 rows, two per CU) for short sequences and for
    // grids of 256-row tiles that do not fill the chip (a causal tile counting
    // as half), as in the forward: twice the workgroups balance the grid
    // better.  Measured (whole backward): causal N = 2048 +4%, 4096 +1%,
    // 8192 +1.4%; non-causal N = 2048 +0-1.5%, 4096 -1.5%; one head N = 32768
    // +8.6%, causal two heads N = 32768 +4.5%.
    const int64_t dq_tiles8 = (int64_t)B * H_q * (((int64_t)N + 255) / 256);
    const bool dq_short = (causal ? N <= 8192 : N <= 2048) || dq_tiles8 < (causal ? 512 : 256);
    const int dq_rows = (dq_short ? 4 : DQ_WAVES) * 32;
    const int64_t n_qtiles = ((int64_t)N + dq_rows - 1) / dq_rows;
    const int64_t n_ktiles = ((int64_t)N + KV_KEYS - 1) / KV_KEYS;
    const int64_t total_q = (int64_t)B * H_q * n_qtiles;
    const int64_t total_k = (int64_t)B * H_kv * n_ktiles;
    if (total_q > INT32_MAX || total_k > INT32_MAX || (int64_t)B * H_q > INT32_MAX)
        return ATTN_ERR_SHAPE;
    for (int i = 0; i < n_in; ++i)
        if ((uintptr_t)ins[i].ptr % ins[i].align != 0) return ATTN_ERR_ALIGN;
    for (int i = 0; i < n_out; ++i)
        if ((uintptr_t)outs[i].ptr % outs[i].align != 0) return ATTN_ERR_ALIGN;
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j)
            if (ranges_overlap(outs[i].ptr, outs[i].bytes, ins[j].ptr, ins[j].bytes))
                return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < n_out; ++j)
            if (ranges_overlap(outs[i].ptr, outs[i].bytes, outs[j].ptr, outs[j].bytes))
                return ATTN_ERR_ALIAS;
    }
    if (ws_short) return ATTN_ERR_WORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev)) return ATTN_ERR_DEVICE;

    p = BwdParams{};
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.N = N;
    p.group = H_q / H_kv;
    p.n_qtiles = (int)n_qtiles;
    p.total_q = (int)total_q;
    p.dq_waves = dq_short ? 4 : DQ_WAVES;
    // XCD workgroup slots: 32 CUs x 2 four-wave or 1 eight-wave dQ workgroups;
    // one dK/dV workgroup per CU
    const int64_t dq_slots = dq_short ? 64 : 32;
    p.cgroup = (int)std::min<int64_t>((int64_t)B * H_q, (dq_slots + n_qtiles - 1) / n_qtiles);
    p.kgroup = (int)std::min<int64_t>((int64_t)B * H_kv, (32 + n_ktiles - 1) / n_ktiles);
    p.n_ktiles = (int)n_ktiles;
    p.total_k = (int)total_k;
    p.c = (float)((double)scale * 1.4426950408889634);
    p.scale = scale;
    return ATTN_OK;
}

size_t q_bytes(int B, int H_q, int N) { return (size_t)B * H_q * N * HD * 2; }
size_t kv_bytes(int B, int H_kv, int N) { return (size_t)B * H_kv * N * HD * 2; }
size_t row_bytes(int B, int H_q, int N) { return (size_t)B * H_q * N * 4; }

// Causal grids whose groups do not split evenly over the 8 XCDs take the
// dealt order (causal_deal); the launch grid is then its padded size.
void deal_dq(BwdParams& p) {
    int64_t G = p.cgroup > 1 ? p.cgroup : 1, grid = 0;
    const int64_t slots = p.dq_waves == 4 ? 64 : 32;
    if (causal_deal((int64_t)p.B * p.Hq, G, p.n_qtiles, slots, p.deal_q, grid) && grid <= INT32_MAX) {
        p.dealt_q = 1;
        p.cgroup = (int)G;
        p.total_q = (int)grid;
    }
}
void deal_dkdv(BwdParams& p) {
    const int64_t ns = p.n_split > 1 ? p.n_split : 1;
    int64_t G = p.kgroup > 1 ? p.kgroup : 1, grid = 0;
    if (causal_deal((int64_t)p.B * p.Hkv * ns, G, p.n_ktiles, 32, p.deal_k, grid) && grid <= INT32_MAX) {
        p.dealt_k = 1;
        p.kgroup = (int)G;
        p.total_k = (int)grid;
    }
}

void launch_dq(BwdParams p, bool causal, hipStream_t s) {
    if (causal) deal_dq(p);
    if (p.dq_waves == 4) {
        if (causal)
            hipLaunchKernelGGL((attn_bwd_dq_kernel<true, 4>), dim3((unsigned)p.total_q), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((attn_bwd_dq_kernel<false, 4>), dim3((unsigned)p.total_q), dim3(256), 0, s, p);
    } else {
        if (causal)
            hipLaunchKernelGGL((attn_bwd_dq_kernel<true, 8>), dim3((unsigned)p.total_q), dim3(512), 0, s, p);
        else
            hipLaunchKernelGGL((attn_bwd_dq_kernel<false, 8>), dim3((unsigned)p.total_q), dim3(512), 0, s, p);
    }
}
void launch_dkdv(BwdParams p, bool causal, hipStream_t s) {
    if (causal) deal_dkdv(p);
    if (causal)
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<true>, dim3((unsigned)p.total_k), dim3(KV_THREADS), 0, s, p);
    else
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<false>, dim3((unsigned)p.total_k), dim3(KV_THREADS), 0, s, p);
}
void launch_reduce(const BwdParams& p, hipStream_t s) {
    const size_t rows = (size_t)p.B * p.Hkv * p.N;
    const size_t groups = 2 * rows * HD / 4;
    const unsigned grid = (unsigned)std::min<size_t>((groups + 255) / 256, 8192);
    hipLaunchKernelGGL(attn_bwd_reduce_kernel, dim3(grid), dim3(256), 0, s, (const float*)p.ws, p.dk,
                       p.dv, rows, p.n_split);
}

// Parts of each group's query heads for the dK/dV step of attn_bwd_ws: a
// divisor of the group size.  n_splits <= 0: the smallest divisor that gives
// at least one dK/dV workgroup per compute unit of an MI355X (256; one
// workgroup fits per CU), or four per CU when causal and eight from 8192 keys
// (a causal key tile's work falls with its index; smaller parts let the
// heaviest-first order even it out, and long sequences have the heaviest
// tiles), or the largest divisor up to 16 when none does.  n_splits > 0: the
// largest divisor of the group size not above n_splits.
int bwd_splits(int B, int H_q, int H_kv, int N, bool causal, int n_splits) {
    const int group = H_q / H_kv;
    const int64_t base = (int64_t)B * H_kv * (((int64_t)N + KV_KEYS - 1) / KV_KEYS);
    const int64_t target = causal ? (N >= 8192 ? 8 : 4) * 256 : 256;
    int best = 1;
    for (int s = 1; s <= std::min(group, 16); ++s) {
        if (group % s != 0) continue;
        if (n_splits > 0) {
            if (s <= n_splits) best = s;
            continue;
        }
        best = s;
        if (base * s >= target) break;
    }
    return best;
}
size_t bwd_ws_bytes(int B, int H_kv, int N, int ns) {
    return ns > 1 ? (size_t)ns * 2 * B * H_kv * (size_t)N * HD * sizeof(float) : 0;
}
bool bwd_shape_ok(int B, int H_q, int H_kv, int N, int D) {
    return B > 0 && H_q > 0 && H_kv > 0 && N > 0 && D == HD && H_q % H_kv == 0;
}

}  // namespace

extern "C" attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, float* delta,
                                   int B, int H_q, int H_kv, int N, int D, int causal, float scale,
                                   void* stream) {
    const Buf ins[6] = {{q, q_bytes(B, H_q, N), 16}, {k, kv_bytes(B, H_kv, N), 16},
                        {v, kv_bytes(B, H_kv, N), 16}, {o, q_bytes(B, H_q, N), 16},
                        {dout, q_bytes(B, H_q, N), 16}, {lse, row_bytes(B, H_q, N), 4}};
    const Buf outs[2] = {{dq, q_bytes(B, H_q, N), 16}, {delta, row_bytes(B, H_q, N), 4}};
    BwdParams p;
    const attn_status st = prepare(ins, 6, outs, 2, B, H_q, H_kv, N, D, causal, scale, p);
    if (st != ATTN_OK) return st;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (const uint16_t*)o;
    p.dout = (const uint16_t*)dout;
    p.lse = lse;
    p.dq = (uint16_t*)dq;
    p.delta = delta;
    launch_dq(p, causal != 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v,
                                     const void* dout, const float* lse, const float* delta,
                                     void* dk, void* dv, int B, int H_q, int H_kv, int N, int D,
                                     int causal, float scale, void* stream) {
    const Buf ins[6] = {{q, q_bytes(B, H_q, N), 16}, {k, kv_bytes(B, H_kv, N), 16},
                        {v, kv_bytes(B, H_kv, N), 16}, {dout, q_bytes(B, H_q, N), 16},
                        {lse, row_bytes(B, H_q, N), 4}, {delta, row_bytes(B, H_q, N), 4}};
    const Buf outs[2] = {{dk, kv_bytes(B, H_kv, N), 16}, {dv, kv_bytes(B, H_kv, N), 16}};
    BwdParams p;
    const attn_status st = prepare(ins, 6, outs, 2, B, H_q, H_kv, N, D, causal, scale, p);
    if (st != ATTN_OK) return st;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.dout = (const uint16_t*)dout;
    p.lse = lse;
    p.delta = const_cast<float*>(delta);   // only read by this kernel
    p.dk = (uint16_t*)dk;
    p.dv = (uint16_t*)dv;
    launch_dkdv(p, causal != 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                float* delta, int B, int H_q, int H_kv, int N, int D, int causal,
                                float scale, void* stream) {
    const Buf ins[6] = {{q, q_bytes(B, H_q, N), 16}, {k, kv_bytes(B, H_kv, N), 16},
                        {v, kv_bytes(B, H_kv, N), 16}, {o, q_bytes(B, H_q, N), 16},
                        {dout, q_bytes(B, H_q, N), 16}, {lse, row_bytes(B, H_q, N), 4}};
    const Buf outs[4] = {{dq, q_bytes(B, H_q, N), 16}, {dk, kv_bytes(B, H_kv, N), 16},
                         {dv, kv_bytes(B, H_kv, N), 16}, {delta, row_bytes(B, H_q, N), 4}};
    BwdParams p;
    const attn_status st = prepare(ins, 6, outs, 4, B, H_q, H_kv, N, D, causal, scale, p);
    if (st != ATTN_OK) return st;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (const uint16_t*)o;
    p.dout = (const uint16_t*)dout;
    p.lse = lse;
    p.dq = (uint16_t*)dq;
    p.dk = (uint16_t*)dk;
    p.dv = (uint16_t*)dv;
    p.delta = delta;
    // delta is written by the dQ kernel and read by the dK/dV kernel: same
    // stream, in this order
    const hipStream_t s = (hipStream_t)stream;
    launch_dq(p, causal != 0, s);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
    launch_dkdv(p, causal != 0, s);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" int attn_bwd_splits(int B, int H_q, int H_kv, int N, int D, int causal, int n_splits) {
    return bwd_shape_ok(B, H_q, H_kv, N, D) ? bwd_splits(B, H_q, H_kv, N, causal != 0, n_splits) : 0;
}

extern "C" size_t attn_bwd_workspace_bytes(int B, int H_q, int H_kv, int N, int D, int causal,
                                           int n_splits) {
    if (!bwd_shape_ok(B, H_q, H_kv, N, D)) return 0;
    return bwd_ws_bytes(B, H_kv, N, bwd_splits(B, H_q, H_kv, N, causal != 0, n_splits));
}

extern "C" attn_status attn_bwd_ws(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   float* delta, int B, int H_q, int H_kv, int N, int D, int causal,
                                   float scale, int n_splits, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    const int ns = bwd_shape_ok(B, H_q, H_kv, N, D) ? bwd_splits(B, H_q, H_kv, N, causal != 0, n_splits) : 1;
    if (ns == 1)
        return attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H_q, H_kv, N, D, causal, scale,
                        stream);
    const size_t need = bwd_ws_bytes(B, H_kv, N, ns);
    const Buf ins[6] = {{q, q_bytes(B, H_q, N), 16}, {k, kv_bytes(B, H_kv, N), 16},
                        {v, kv_bytes(B, H_kv, N), 16}, {o, q_bytes(B, H_q, N), 16},
                        {dout, q_bytes(B, H_q, N), 16}, {lse, row_bytes(B, H_q, N), 4}};
    const Buf outs[5] = {{dq, q_bytes(B, H_q, N), 16}, {dk, kv_bytes(B, H_kv, N), 16},
                         {dv, kv_bytes(B, H_kv, N), 16}, {delta, row_bytes(B, H_q, N), 4},
                         {workspace, std::min(need, workspace_bytes), 16}};
    BwdParams p;
    const attn_status st = prepare(ins, 6, outs, 5, B, H_q, H_kv, N, D, causal, scale, p, workspace_bytes < need);
    if (st != ATTN_OK) return st;
    if ((int64_t)p.total_k * ns > INT32_MAX) return ATTN_ERR_SHAPE;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (const uint16_t*)o;
    p.dout = (const uint16_t*)dout;
    p.lse = lse;
    p.dq = (uint16_t*)dq;
    p.dk = (uint16_t*)dk;
    p.dv = (uint16_t*)dv;
    p.delta = delta;
    p.n_split = ns;
    p.ws = (float*)workspace;
    p.total_k *= ns;
    p.kgroup = (int)std::min<int64_t>((int64_t)B * H_kv * ns, (32 + p.n_ktiles - 1) / p.n_ktiles);
    // dQ (writes delta), dK/dV parts (read delta, write the workspace), then
    // the sum of the parts: one stream, in this order
    const hipStream_t s = (hipStream_t)stream;
    launch_dq(p, causal != 0, s);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
    launch_dkdv(p, causal != 0, s);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
    launch_reduce(p, s);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" double attn_bwd_flops(int B, int H_q, int N, int D, int causal) {
    // five N x N x D products (S, dP, dV, dK, dQ) of 2 flops per multiply-add
    const double f = 10.0 * B * H_q * (double)N * (double)N * D;
    return causal ? 0.5 * f : f;
}
