// Fused attention forward on FP8 (e4m3) Q, K, V with per-tensor descales, for
// MI355X (gfx950, CDNA4).
//
// Q = dq * Q8, K = dk * K8, V = dv * V8 (Q8, K8, V8 hold OCP e4m3 codes);
// O = softmax(scale * Q K^T [causal]) V in bf16 and the per-row natural-log LSE.
//   * formula: page "GPU注意力算子性能优化" (QiMeng-Attention), section 1;
//   * precision split: both matrix products in FP8, softmax and accumulation in
//     fp32 (page "注意力机制的本质与计算挑战", section 3; the QiMeng page,
//     section 3.1.1); the probabilities are stored in FP8 for the second
//     product and the sums are kept wider (page "从硬件视角看注意力机制优化",
//     section 2.3);
//   * tiling, online softmax across key tiles and the shared K/V of a GQA group
//     as in the bf16 forward (same pages, sections cited there).
//
// Matrix core: v_mfma_scale_f32_32x32x64_f8f6f4 with both block scales at the
// neutral exponent (2^0), i.e. a plain e4m3 x e4m3 product with fp32
// accumulation, 64 contraction values per lane pair.
//
// Work decomposition (one workgroup = NW waves = 32 NW query rows of one head;
// launched with 4 waves, two workgroups per CU):
//   * each wave owns 32 query rows; its Q rows (128 bytes each) stay in VGPRs as
//     the B operand of S^T = K Q^T;
//   * key blocks of 64 rows of K and V (8 KiB each) are copied HBM -> LDS by the
//     buffer unit's LDS DMA; K runs one block ahead of V so the score MFMAs of
//     block g+1 and the PV MFMAs of block g-1 overlap the softmax of block g;
//   * scores are computed transposed (each lane owns one query column); the
//     fp32 scores become e4m3 weights packed in the order the accumulator
//     holds them, and that packing is directly the B operand of O^T += V^T P^T;
//   * the A operand V^T is read from the row-major V tile with the gfx950
//     transposing byte read ds_read_b64_tr_b8: in a 16-lane group every lane
//     names one 8-byte row piece and receives one byte column, so each lane
//     can fetch exactly the 8 keys its P bytes stand for;
//   * O's divisor is the sum of the e4m3 weights the MFMA actually applied,
//     taken by one more MFMA against a tile of ones (exact fp32 sums of
//     products), so the rounding of a dominant weight cancels in O; the LSE
//     uses the fp32 weights;
//   * softmax in base 2 against a lagging reference m: e = 2^(s*c - m*c),
//     c = |scale*dq*dk|*log2(e).  A row's weights of a block are multiplied by
//     the power of two 2^k that puts their largest one in (224, 448], the top
//     binade of e4m3 below its largest value, then rounded to e4m3; the matrix
//     core's E8M0 scale of the P operand applies 2^-k back, exactly.  In the
//     32x32x64 operand layout bytes 0-15 of both lanes of a column form the
//     first 32-value k block and bytes 16-31 the second (checked on the GPU),
//     and the scale of block b comes from lane column + 32b; both lanes of a
//     row hold the same k.  No weight can overflow e4m3 and none is rounded
//     more coarsely than the row's largest weight of the block allows.  The
//     reference only moves (rare, wave-uniform branch) when a lane's fp32
//     block sum passes 2^64 or is not finite.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn.h"
#include "cdna4.h"

namespace {

using namespace cdna4;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int HD = 128;                      // head dimension handled by this kernel
constexpr int ROW8 = HD;                     // bytes per e4m3 row
// Workgroups of 4 waves (128 query rows, two per CU).  The kernel is written
// for NW waves; measured against 8-wave workgroups (same-process sweeps,
// 256-32768 tokens, 1-1024 heads, causal and not) 4 waves won or tied on every
// shape but one (-1.5%), by up to 40% on grids of a few heads.
constexpr int NW_LAUNCH = 4;
constexpr int KB = 64;                       // keys per pipeline step (one MFMA k extent)
constexpr int BLK_BYTES = KB * ROW8;         // 8 KiB per K or V block
constexpr int K_RING = 0;                    // LDS: a ring of 4 K blocks, then 4 V blocks
constexpr int V_RING = 4 * BLK_BYTES;
constexpr int LDS_BYTES = 8 * BLK_BYTES;     // 64 KiB
constexpr float LOG2_448 = 8.80735492205760410f;   // log2 of the largest e4m3 value
constexpr float K_CLAMP = 100.0f;            // |k| of a lane's weight scale 2^k (E8M0: 127 - k)
constexpr float MOVE_SUM = 18446744073709551616.0f;   // 2^64: a lane's block sum above this moves the reference
// Exact kernel (a NaN code in a masked block's V): a zero block, and per wave up
// to MAX_SAVED masked blocks' weights (32 rows x 64 keys, e4m3 times 2^-k,
// exact in bf16), the factor each block's weights have been rescaled by since
// (one per lane) and its index.  A wave has at most two masked blocks with a
// visible key (its causal diagonal block, the ragged last block).
constexpr int MAX_SAVED = 2;
constexpr int SAVE_P = 32 * KB * 2;
constexpr int SAVE_WAVE_BYTES = MAX_SAVED * (SAVE_P + 64 * 4) + 16;
// Mark the fast kernel leaves in the first output row of a workgroup it hands
// to the exact kernel: eight signalling-NaN bf16 codes (0x7F81 .. 0x7F88),
// which arithmetic never produces (every NaN it makes is quiet).
__constant__ const uint32_t NF_MARK[4] = {0x7F827F81u, 0x7F847F83u, 0x7F867F85u, 0x7F887F87u};
constexpr int ONE4 = 0x38383838;             // four e4m3 ones

struct Params {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    uint16_t* o;
    float* lse;
    int B, Hq, Hkv, N;
    int group;        // Hq / Hkv
    int n_qtiles;     // ceil(N / (32 NW))
    int total;        // B * Hq * n_qtiles workgroups
    int q_mode;       // 0: Q as given, 1: Q negated, 2: Q replaced by zeros
    int cgroup;       // causal: heads whose tiles are interleaved (<= 1: one head)
    int dealt;        // causal: the dealt grid order (dealt_tile) instead of the plain one
    Deal deal;        // its sizes
    float c;          // |scale*dq*dk| * log2(e), > 0
    float lse_scale;  // |scale*dq*dk|
    float dv;         // V descale, applied to O
};

// 16-byte chunk c of row r of a K tile sits at chunk position c ^ ((r >> 1) & 7):
// the 16 rows one read phase touches (same logical chunk) then cover all 16
// 16-byte bank groups of a 256-byte LDS line.
__device__ __forceinline__ int k_swz(int r) { return (r >> 1) & 7; }
// V tile: chunk c of row r at c ^ (2*((r>>1)&1) + 4*((r>>3)&1) + ((r>>2)&1)).
// A transposing read names 8 rows {b, b+1, b+2, b+3, b+8, .., b+11} (b = 16t +
// 4*half) in two adjacent chunks; this spreads them over distinct bank groups.
__device__ __forceinline__ int v_swz(int r) {
    return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const char* lds, uint32_t off) {
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds + off));
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
    // format 0 (e4m3) for both operands, block scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// The same with an E8M0 scale byte for B.  B's k extent of 64 is two blocks
// of 32: block b is bytes 16b .. 16b+15 of lanes L and L+32 (column L % 32),
// and lane L + 32b supplies its scale (byte 0 of sb).
__device__ __forceinline__ f32x16 mfma8_sb(const i32x8& a, const i32x8& b, const f32x16& c, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// Which (batch, head, query tile) workgroup id bid computes; false: bid is
// padding of the grid.
template <bool CAUSAL, int NW>
__device__ __forceinline__ bool tile_of(const Params& p, int bid, int& b, int& h, int& qt) {
    const int logical = xcd_remap(bid, p.total);
    int bh;
    if (CAUSAL && p.dealt) {
        // head groups that do not split evenly over the 8 XCDs: slices of
        // groups dealt to the XCDs in turn, each a strided share of its
        // group's heaviest-first list, so the XCDs receive equal work
        if (!dealt_tile(bid, p.B * p.Hq, p.cgroup > 1 ? p.cgroup : 1, p.n_qtiles, p.deal, bh, qt))
            return false;
    } else if (CAUSAL) {
        // groups of cgroup heads one after another (a group's tiles share K/V in
        // one XCD's L2), tile-major and heaviest tile first within a group; a
        // group holds at least an XCD's worth of workgroup slots, so light tiles
        // of one group, not heavy tiles of the next, end each XCD's share
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
    b = bh / p.Hq;
    h = bh % p.Hq;
    return true;
}

// One query tile (workgroup id bid).  NW waves per workgroup.
// SAFE = false: the fast kernel's body; SAFE = true: the exact form, for the
// tiles the fast kernel marked (a NaN code in the V rows of a masked block;
// see NF_MARK).
template <bool CAUSAL, int NW, bool SAFE>
__device__ __forceinline__ void fwd8_tile(const Params& p, const int bid) {
    constexpr int BRW = 32 * NW;      // query rows of this workgroup
    constexpr int NTH = NW * 64;
    constexpr int DPW = 8 / NW;       // 8-row DMA instructions per wave per key block
    constexpr int ZERO_OFF = LDS_BYTES;                 // exact kernel: a block of zeros
    constexpr int SAVE_OFF = ZERO_OFF + BLK_BYTES;      // exact kernel: per-wave saved blocks
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES + (SAFE ? BLK_BYTES + NW * SAVE_WAVE_BYTES : 0)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;   // query column owned by this lane
    const int hh = lane >> 5;    // which half of the wave

    int b, h, qt;
    if (!tile_of<CAUSAL, NW>(p, bid, b, h, qt)) return;   // whole workgroup, no barrier yet
    // workgroup-uniform (said so, so the copy descriptors stay scalar)
    b = __builtin_amdgcn_readfirstlane(b);
    h = __builtin_amdgcn_readfirstlane(h);
    qt = __builtin_amdgcn_readfirstlane(qt);
    const int kvh = h / p.group;
    const int N = p.N;
    const int q0 = qt * BRW;
    const int wq0 = q0 + wave * 32;
    const int myq = wq0 + l32;

    const size_t q_panel = ((size_t)b * p.Hq + h) * (size_t)N * HD;     // elements (bytes for Q8)
    const size_t kv_panel = ((size_t)b * p.Hkv + kvh) * (size_t)N * HD;
    uint16_t* const mark = p.o + q_panel + (size_t)q0 * HD;   // the workgroup's first output row
    if constexpr (SAFE) {
        // only the workgroups the fast kernel marked (every thread reads the
        // same 16 bytes, so the exit is workgroup-uniform)
        const u32x4 w = *(const u32x4*)mark;
        if (w[0] != NF_MARK[0] || w[1] != NF_MARK[1] || w[2] != NF_MARK[2] || w[3] != NF_MARK[3]) return;
    }

    // key blocks: n_blk_wg streamed through LDS, n_blk used by this wave (a
    // causal wave stops at the block holding its last row's diagonal)
    const int n_blk_all = (N + KB - 1) / KB;
    int n_blk_wg = n_blk_all, n_blk = n_blk_all;
    if (CAUSAL) {
        n_blk_wg = min(n_blk_all, (min(q0 + BRW, N) - 1) / KB + 1);
        n_blk = min(n_blk_all, (wq0 + 31) / KB + 1);
    }
    if (wq0 >= N) n_blk = 0;
    const uint8_t* kbase = p.k + kv_panel;
    const uint8_t* vbase = p.v + kv_panel;

    // ---- LDS DMA: each wave copies rows 8*DPW*wave .. of a block with DPW
    // instructions of 8 rows (64 lanes x 16 bytes, lane order); lane L fetches
    // the logical chunk that belongs at its physical position.
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    uint32_t k_dma[DPW], v_dma[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int row = 8 * DPW * wave + 8 * i + (lane >> 3);
        const int pc = lane & 7;
        k_dma[i] = (uint32_t)(row * ROW8 + ((pc ^ k_swz(row)) << 4));
        v_dma[i] = (uint32_t)(row * ROW8 + ((pc ^ v_swz(row)) << 4));
    }
    // One descriptor per panel for every copy, the block's offset in soffset;
    // its range ends at the workgroup's last needed key.  The buffer unit
    // range-checks voffset + soffset, and a lane past the range reads nothing
    // and writes zeros to LDS: rows past N of a ragged last block arrive as
    // zeros, and copies of blocks past the workgroup's last one, issued
    // without a guard, only clear their slot.
    const int lim = min(N, n_blk_wg * KB);
    const uint32_t lds_wave = lds_base + 8 * DPW * wave * ROW8;
    const u32x4 k_desc = sgpr_rsrc(kbase, (uint32_t)lim * ROW8);
    const u32x4 v_desc = sgpr_rsrc(vbase, (uint32_t)lim * ROW8);
    auto dma_block = [&](auto ring_t, auto slot_t, const u32x4& desc, const uint32_t* voff, int g) {
        constexpr uint32_t DST = decltype(ring_t)::value + decltype(slot_t)::value * BLK_BYTES;
        const uint32_t soff = (uint32_t)g * BLK_BYTES;
        lds_dma16_at<DST>(desc, lds_wave, voff[0], soff);
        if constexpr (DPW > 1) lds_dma16_at<DST + 8 * ROW8>(desc, lds_wave, voff[1], soff);
    };
    using R_K = std::integral_constant<uint32_t, K_RING>;
    using R_V = std::integral_constant<uint32_t, V_RING>;
    using S0 = std::integral_constant<uint32_t, 0>;
    using S1 = std::integral_constant<uint32_t, 1>;
    using S2 = std::integral_constant<uint32_t, 2>;
    using S3 = std::integral_constant<uint32_t, 3>;

    // ---- per-lane LDS read offsets (relative to a block slot)
    // K: rows 32*sb + l32, chunks 4*ks + 2*hh + u (u = 0, 1) -> bytes 64ks+32hh.. of d
    uint32_t k_rd[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int u = 0; u < 2; ++u)
            k_rd[ks][u] = (uint32_t)(l32 * ROW8 + (((4 * ks + 2 * hh + u) ^ k_swz(l32)) << 4));
    // V: transposing reads t = 0..3 of d block db.  In each 16-lane group lane
    // lam names row piece jj = lam/2 (8 bytes at column d0 + 8*(lam&1)); the
    // piece's row is the key that byte jj of P's read t stands for:
    // key(t, jj) = 16t + 8*(jj/4) + 4*hh + jj%4.  t only adds 16 rows (2 KiB).
    uint32_t v_rd[4];
    {
        const int lam = lane & 15;
        const int jj = lam >> 1;
        const int row = 8 * (jj >> 2) + 4 * hh + (jj & 3);
        const int gh = (lane >> 4) & 1;   // which 16 columns of the 32-column d block
#pragma unroll
        for (int db = 0; db < 4; ++db)
            v_rd[db] = (uint32_t)(row * ROW8 + (((2 * db + gh) ^ v_swz(row)) << 4) + 8 * (lam & 1));
    }

    // ---- prologue
    if constexpr (SAFE) {
        // the zero block masked products run against (first read after a barrier)
#pragma unroll
        for (int i = 0; i < BLK_BYTES / (16 * NTH); ++i)
            *(u32x4*)(lds + ZERO_OFF + 16 * (tid + NTH * i)) = u32x4{0u, 0u, 0u, 0u};
    }
    dma_block(R_K{}, S0{}, k_desc, k_dma, 0);
    dma_block(R_V{}, S0{}, v_desc, v_dma, 0);
    dma_block(R_K{}, S1{}, k_desc, k_dma, 1);
    dma_block(R_K{}, S2{}, k_desc, k_dma, 2);

    i32x8 qf[2];   // B operand of S^T: head dims 64ks + 32hh + 0..31 of this lane's row
    {
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.q + q_panel, (uint32_t)N * ROW8);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4 lo = buf_load16(qr, (uint32_t)myq * ROW8 + 64 * ks + 32 * hh);
            const u32x4 hi = buf_load16(qr, (uint32_t)myq * ROW8 + 64 * ks + 32 * hh + 16);
            qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }
    // a negative score scale is applied as |scale| on -Q (sign bits flipped,
    // exact) and a zero one as zero scores
    if (p.q_mode != 0) {
        const int flip = p.q_mode == 1 ? (int)0x80808080u : 0;
        const int keep = p.q_mode == 1 ? -1 : 0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) qf[ks][i] = (qf[ks][i] & keep) ^ flip;
    }
    const float c = p.c;
    i32x8 ones = {ONE4, ONE4, ONE4, ONE4, ONE4, ONE4, ONE4, ONE4};
    asm volatile("" : "+v"(ones));   // keep it in registers: not rebuilt every block

    // S^T of one 64-key block (two 32-key halves), from a K ring slot
    auto scores = [&](f32x16 (&s)[2], uint32_t kslot) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            s[sb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint32_t base = kslot + sb * 32 * ROW8;
                const u32x4 lo = *(const u32x4*)(lds + base + k_rd[ks][0]);
                const u32x4 hi = *(const u32x4*)(lds + base + k_rd[ks][1]);
                const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[sb] = mfma8(a, qf[ks], s[sb]);
            }
        }
    };
    auto needs_mask = [&](int g) {
        return (CAUSAL && g * KB + KB - 1 > wq0) || (g * KB + KB > N);
    };
    bool seen_g = false;   // exact kernel: some key of the masked block is visible to this lane's row
    auto apply_mask = [&](f32x16 (&s)[2], int g) {
        bool any = false;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = g * KB + 32 * sb + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool bad = (key >= N) || (CAUSAL && key > myq);
                if constexpr (SAFE) any = any || !bad;
                s[sb][r] = bad ? -INFINITY : s[sb][r];
            }
        if constexpr (SAFE) seen_g = any;
    };

    f32x16 o[4];          // O^T: 4 blocks of 32 head dims x 32 query columns
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    f32x16 ol = {};       // every row: sum of the e4m3 weights applied (O's divisor)
    const bool live = myq < N;   // a row that is written (padding rows past N are not)
    float m = -INFINITY;  // reference: raw score q8.k8 of this lane's row
    float mb = 0.f;       // m * c (-inf while the row has seen no finite score)
    float l = 0.f;        // this lane's partial sum of the fp32 weights (the LSE)

    // O^T += V^T P^T for one block: A = V^T bytes in the key order of P's
    // bytes; sb is the E8M0 byte of the row's weight scale 2^-k
    auto pv = [&](const i32x8& pw, int sb, uint32_t vslot) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const i32x2 r0 = lds_read_tr8(lds, vslot + v_rd[db]);
            const i32x2 r1 = lds_read_tr8(lds, vslot + v_rd[db] + 16 * ROW8);
            const i32x2 r2 = lds_read_tr8(lds, vslot + v_rd[db] + 32 * ROW8);
            const i32x2 r3 = lds_read_tr8(lds, vslot + v_rd[db] + 48 * ROW8);
            const i32x8 a = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
            o[db] = mfma8_sb(a, pw, o[db], sb);
        }
        ol = mfma8_sb(ones, pw, ol, sb);
    };
    auto lane_max = [&](const f32x16 (&s)[2]) {
        // NaN-propagating maximum: three inputs per v_maximum3_f32 and no
        // canonicalising moves (fmaxf has to quiet each operand first).  A
        // NaN score yields NaN here; its row's weights, O and LSE are NaN
        // whatever the block's scale.
        float m0 = __builtin_elementwise_maximum(s[0][0], s[1][0]);
        float m1 = __builtin_elementwise_maximum(s[0][1], s[1][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) {
            m0 = __builtin_elementwise_maximum(m0, __builtin_elementwise_maximum(s[0][r], s[1][r]));
            m1 = __builtin_elementwise_maximum(m1, __builtin_elementwise_maximum(s[0][r + 1], s[1][r + 1]));
        }
        return __builtin_elementwise_maximum(m0, m1);
    };
    // weights e = 2^(s*c - mb) times 2^k, as e4m3: byte 16*sb + r = key
    // 32sb + 8(r/4) + 4hh + r%4, and k = floor(log2(448) - the row's largest
    // exponent in the block) puts the row's largest weight of the block in
    // (224, 448] (k clamped to +-100 for blocks far below the reference, and
    // for -inf or NaN scores).  ls = the fp32 weights' sum without the 2^k;
    // sk = the E8M0 byte 127 - k (both halves of the block, both lanes);
    // mx = the row's largest score in the block.
    auto probs = [&](const f32x16 (&s)[2], i32x8& pw, float& ls, int& sk, float& mx) {
        mx = wave_swap_max(lane_max(s));   // both lanes of the row
        const float kf = fminf(fmaxf(__builtin_floorf(LOG2_448 - fmaf(mx, c, -mb)), -K_CLAMP), K_CLAMP);
        const float mbk = mb - kf;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s[sb][4 * w + 0], c, -mbk));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s[sb][4 * w + 1], c, -mbk));
                const float e2 = __builtin_amdgcn_exp2f(fmaf(s[sb][4 * w + 2], c, -mbk));
                const float e3 = __builtin_amdgcn_exp2f(fmaf(s[sb][4 * w + 3], c, -mbk));
                a0 += e0 + e2;
                a1 += e1 + e3;
                // both halves of the dword are written: the old value needs no clearing
                int pk = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, pw[4 * sb + w], false);
                pk = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, pk, true);
                pw[4 * sb + w] = pk;
            }
        const int k = (int)kf;
        ls = ldexpf(a0 + a1, -k);
        sk = 127 - k;
    };
    // A masked block multiplies the V rows of keys some rows may not see by
    // zero weights, and 0 * NaN is NaN in the matrix core.  Before its main
    // loop each wave of the fast kernel scans the V rows of its masked blocks
    // in global memory; a workgroup that finds a NaN code there is redone by
    // the exact kernel.  The exact kernel runs a masked block's product
    // against a block of zeros instead of its V (O's divisor still counts its
    // weights) and saves the weights (e4m3 times 2^-k, exact in bf16); after
    // the loop it adds each saved block's terms p * v for the keys each row
    // sees (V from global memory), times the factor its weights have been
    // rescaled by since.
    int n_saved = 0;
    auto save_block = [&](const i32x8& pw, int sk, int gb) {
        char* base = lds + SAVE_OFF + wave * SAVE_WAVE_BYTES;
        char* wp = base + n_saved * SAVE_P + l32 * (KB * 2);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float unscale = ldexpf(1.0f, sk - 127);
                const int d = pw[4 * sb + w];   // keys 32sb + 8w + 4hh + 0..3
                const bf16x2 lo = {(__bf16)(__builtin_amdgcn_cvt_f32_fp8(d, 0) * unscale),
                                   (__bf16)(__builtin_amdgcn_cvt_f32_fp8(d, 1) * unscale)};
                const bf16x2 hi = {(__bf16)(__builtin_amdgcn_cvt_f32_fp8(d, 2) * unscale),
                                   (__bf16)(__builtin_amdgcn_cvt_f32_fp8(d, 3) * unscale)};
                *(uint2*)(wp + 2 * (32 * sb + 8 * w + 4 * hh)) =
                    uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            }
        ((float*)(base + MAX_SAVED * SAVE_P))[n_saved * 64 + lane] = 1.0f;
        if (lane == 0) ((int*)(base + MAX_SAVED * (SAVE_P + 256)))[n_saved] = gb;
        ++n_saved;
    };
    bool mask_prev = false;   // exact kernel: the previous step's block was masked
    bool keep_prev = false;   // ... and some row of the wave sees one of its keys
    auto step = [&](auto first_t, auto ks_t, auto vs_t, int g, f32x16 (&s)[2], f32x16 (&sn)[2],
                    const i32x8& pp, int sp, i32x8& pc, int& sc) {
        constexpr bool FIRST = decltype(first_t)::value;
        constexpr uint32_t KS = K_RING + decltype(ks_t)::value * BLK_BYTES;
        constexpr uint32_t VS = V_RING + decltype(vs_t)::value * BLK_BYTES;
        const bool valid = g < n_blk;
        const bool mask_g = needs_mask(g);
        if (!FIRST && valid && mask_g) apply_mask(s, g);
        if constexpr (SAFE) {
            // exact kernel: a masked block's product runs against the zero
            // block, and its weights are saved when some row sees one of its keys
            if constexpr (!FIRST) {
                pv(pp, sp, mask_prev ? (uint32_t)ZERO_OFF : VS);
                if (mask_prev && keep_prev && n_saved < MAX_SAVED) save_block(pp, sp, g - 1);
            }
            mask_prev = valid && mask_g;
            keep_prev = mask_prev && __builtin_amdgcn_ballot_w64(seen_g) != 0;
            scores(sn, KS);
        } else {
            scores(sn, KS);
            if constexpr (!FIRST) pv(pp, sp, VS);
        }
        float ls, mx;
        probs(s, pc, ls, sc, mx);
        asm volatile("" : "+v"(pc), "+v"(ls), "+v"(sc), "+v"(mx));
        // While a row has seen no finite score, mb is -inf, so any score makes
        // its sum inf or NaN and takes this branch, which moves m to the first
        // finite score and weighs the rest of the block against it.
        if (valid && __builtin_amdgcn_ballot_w64(!(ls <= MOVE_SUM)) != 0) {
            const float m_new = fmaxf(m, wave_swap_max(mx));
            const float alpha = m_new > m ? __builtin_amdgcn_exp2f((m - m_new) * c) : 1.0f;
            m = m_new;
            mb = (m == -INFINITY) ? 0.f : m * c;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
            for (int r = 0; r < 16; ++r) ol[r] *= alpha;
            if constexpr (SAFE) {
                float* fac = (float*)(lds + SAVE_OFF + wave * SAVE_WAVE_BYTES + MAX_SAVED * SAVE_P);
                for (int i = 0; i < n_saved; ++i) fac[i * 64 + lane] *= alpha;
            }
            probs(s, pc, ls, sc, mx);
            if (m == -INFINITY && live) mb = -INFINITY;
        }
        if (valid) l += ls;
    };

    f32x16 sa[2], sb2[2];   // scores of even / odd key blocks
    i32x8 pa = {}, pb = {};  // e4m3 weights of even / odd key blocks
    int ka = 127, kb = 127;  // their rows' E8M0 scale bytes (2^0 until set)
    // fast kernel: the V rows of the wave's masked blocks (a prefix and a
    // suffix of its blocks: causal diagonal, panel end), in range, checked in
    // global memory for a NaN code (e4m3 has no infinity)
    uint32_t nf_bits = 0u;
    if (!SAFE && n_blk > 0) {
        // one descriptor for the panel, the block in the offset: rows past N read as zeros
        const __amdgpu_buffer_rsrc_t vpanel = make_rsrc(vbase, (uint32_t)N * ROW8);
        auto vcheck = [&](int g) {
#pragma unroll
            for (int i = 0; i < BLK_BYTES / 1024; ++i) {
                const u32x4 x = buf_load16(vpanel, (uint32_t)(g * BLK_BYTES + 16 * lane + 1024 * i));
                // a byte with all seven low bits set (0x7F, 0xFF) carries into its top bit
#pragma unroll
                for (int e = 0; e < 4; ++e) nf_bits |= (x[e] & 0x7F7F7F7Fu) + 0x01010101u;
            }
        };
        int g = 0;
        for (; g < n_blk && needs_mask(g); ++g) vcheck(g);
        for (int h2 = n_blk - 1; h2 >= g && needs_mask(h2); --h2) vcheck(h2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): Q loads, the first DMA and the check done
    // the waves' answers meet in V slot 3 (not refilled before tile 1); a
    // workgroup with a NaN code in a masked block's V marks its first output
    // row and leaves the rows to the exact kernel
    uint32_t* const nf_wave = (uint32_t*)(lds + V_RING + 3 * BLK_BYTES);
    if constexpr (!SAFE) {
        const bool nf = __builtin_amdgcn_ballot_w64((nf_bits & 0x80808080u) != 0u) != 0;
        if (lane == 0) nf_wave[wave] = nf ? 1u : 0u;
    }
    __syncthreads();
    if constexpr (!SAFE) {
        uint32_t any = 0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) any |= nf_wave[w];
        if (any != 0u) {
            if (tid == 0) *(u32x4*)mark = u32x4{NF_MARK[0], NF_MARK[1], NF_MARK[2], NF_MARK[3]};
            return;
        }
    }
    if (n_blk > 0) {
        scores(sa, K_RING);
        if (needs_mask(0)) apply_mask(sa, 0);
        m = wave_swap_max(lane_max(sa));
        mb = (m == -INFINITY) ? (live ? -INFINITY : 0.f) : m * c;
    }
    __syncthreads();   // K slot 0 is refilled in the first tile

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using F = std::false_type;

    // Tile j = steps 2j and 2j+1.  Step g reads K block g+1 (slot (g+1)%4) and
    // V block g-1 (slot (g-1)%4), so during tile j the workgroup refills K
    // blocks 2j+3, 2j+4 and V blocks 2j+1, 2j+2 into slots freed by tile j-1.
    const int n_tiles = n_blk_wg / 2 + 1;
    // even j: K blocks 2j+3, 2j+4 in slots 3, 0 and V blocks 2j+1, 2j+2 in
    // slots 1, 2; odd j: K in slots 1, 2 and V in slots 3, 0
    auto refill_even = [&](int j) {
        dma_block(R_K{}, S3{}, k_desc, k_dma, 2 * j + 3);
        dma_block(R_K{}, S0{}, k_desc, k_dma, 2 * j + 4);
        dma_block(R_V{}, S1{}, v_desc, v_dma, 2 * j + 1);
        dma_block(R_V{}, S2{}, v_desc, v_dma, 2 * j + 2);
    };
    auto refill_odd = [&](int j) {
        dma_block(R_K{}, S1{}, k_desc, k_dma, 2 * j + 3);
        dma_block(R_K{}, S2{}, k_desc, k_dma, 2 * j + 4);
        dma_block(R_V{}, S3{}, v_desc, v_dma, 2 * j + 1);
        dma_block(R_V{}, S0{}, v_desc, v_dma, 2 * j + 2);
    };
    refill_even(0);
    if (0 <= n_blk) step(std::true_type{}, I1{}, I3{}, 0, sa, sb2, pb, kb, pa, ka);
    if (1 <= n_blk) step(F{}, I2{}, I0{}, 1, sb2, sa, pa, ka, pb, kb);
    wait_dma();
    __syncthreads();
    for (int j = 1; j < n_tiles; j += 2) {
        refill_odd(j);
        if (2 * j <= n_blk) step(F{}, I3{}, I1{}, 2 * j, sa, sb2, pb, kb, pa, ka);
        if (2 * j + 1 <= n_blk) step(F{}, I0{}, I2{}, 2 * j + 1, sb2, sa, pa, ka, pb, kb);
        wait_dma();
        __syncthreads();
        if (j + 1 >= n_tiles) break;
        refill_even(j + 1);
        if (2 * j + 2 <= n_blk) step(F{}, I1{}, I3{}, 2 * j + 2, sa, sb2, pb, kb, pa, ka);
        if (2 * j + 3 <= n_blk) step(F{}, I2{}, I0{}, 2 * j + 3, sb2, sa, pa, ka, pb, kb);
        wait_dma();
        __syncthreads();
    }

    // ---- exact kernel: the saved masked blocks' terms p * v, for the keys each
    // row sees, in fp32.  Output element (db, r) of a lane is head dim
    // 32 db + 8 (r / 4) + 4 hh + r % 4.
    if constexpr (SAFE) {
        const char* base = lds + SAVE_OFF + wave * SAVE_WAVE_BYTES;
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase, (uint32_t)N * ROW8);
        for (int i = 0; i < n_saved; ++i) {
            const int gb = __builtin_amdgcn_readfirstlane(((const int*)(base + MAX_SAVED * (SAVE_P + 256)))[i]);
            const float fac = ((const float*)(base + MAX_SAVED * SAVE_P))[i * 64 + lane];
            const char* wp = base + i * SAVE_P + l32 * (KB * 2);
#pragma unroll 1
            for (int j = 0; j < KB; ++j) {
                const int key = gb * KB + j;
                if ((key >= N) || (CAUSAL && key > myq)) continue;
                const float pj = (float)*(const __bf16*)(wp + 2 * j) * fac;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int v4 = (int)__builtin_amdgcn_raw_buffer_load_b32(
                            vr, (uint32_t)key * ROW8 + (uint32_t)(32 * db + 8 * q + 4 * hh), 0, 0);
                        o[db][4 * q + 0] = fmaf(pj, __builtin_amdgcn_cvt_f32_fp8(v4, 0), o[db][4 * q + 0]);
                        o[db][4 * q + 1] = fmaf(pj, __builtin_amdgcn_cvt_f32_fp8(v4, 1), o[db][4 * q + 1]);
                        o[db][4 * q + 2] = fmaf(pj, __builtin_amdgcn_cvt_f32_fp8(v4, 2), o[db][4 * q + 2]);
                        o[db][4 * q + 3] = fmaf(pj, __builtin_amdgcn_cvt_f32_fp8(v4, 3), o[db][4 * q + 3]);
                    }
            }
        }
    }

    // ---- epilogue: O = dv * O^T / sum(e4m3 weights) in bf16;
    // LSE = m*|scale dq dk| + ln(sum of fp32 weights); a row whose scores are
    // all -inf (or NaN) gets NaN, as the formula gives
    const float l_tot = wave_swap_sum(l);
    const float inv = p.dv / ol[0];
    // Fast kernel: O leaves through LDS as whole rows, as in the bf16 kernel:
    // staged row-major in the wave's 8 KiB of the K/V rings (bf16 rows of 256
    // bytes, 16-byte chunk c of row r at chunk c ^ (r mod 16)) once every
    // wave's copies have landed and no wave reads the rings, then stored 4
    // rows (1 KiB) per instruction.  The exact kernel, short of registers,
    // stores its rows directly.
    auto o_piece = [&](int db, int r4) {
        bf16x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(o[db][4 * r4 + i] * inv);
        return ov;
    };
    if constexpr (!SAFE) {
        wait_dma();
        __syncthreads();
        constexpr int OROW = HD * 2;   // bytes per bf16 O row
        char* const stage = lds + K_RING + wave * (32 * OROW);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int ch = 4 * db + r4;   // head dims 8*ch .. 8*ch+7; this lane's half at 4*hh
                *(bf16x4*)(stage + l32 * OROW + ((ch ^ (l32 & 15)) << 4) + 8 * hh) = o_piece(db, r4);
            }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int r = 4 * t + (lane >> 4), ch = lane & 15;
            const u32x4 x = *(const u32x4*)(stage + r * OROW + ((ch ^ (r & 15)) << 4));
            if (wq0 + r < N) *(u32x4*)(p.o + q_panel + (size_t)(wq0 + r) * HD + 8 * ch) = x;
        }
    } else if (myq < N) {
        uint16_t* orow = p.o + q_panel + (size_t)myq * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) *(bf16x4*)(orow + 32 * db + 8 * r4 + 4 * hh) = o_piece(db, r4);
    }
    if (myq < N) {
        if (p.lse != nullptr && hh == 0) {
            const size_t li = ((size_t)b * p.Hq + h) * (size_t)N + myq;
            p.lse[li] = m == -INFINITY ? __builtin_nanf("") : m * p.lse_scale + logf(l_tot);
        }
    }
}

// SAFE = false: the fast kernel, one workgroup per tile.  SAFE = true: the
// exact kernel on a small grid (at most EXACT_GRID workgroups): each thread
// checks one tile's mark, and each workgroup redoes its marked tiles one after
// another (most launches mark none, so most workgroups only read marks).
constexpr int EXACT_GRID = 256;
template <bool CAUSAL, int NW, bool SAFE>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd_fp8_kernel(Params p) {
    if constexpr (!SAFE) {
        fwd8_tile<CAUSAL, NW, false>(p, blockIdx.x);
    } else {
        constexpr int NTH = NW * 64;
        __shared__ int marked[NTH];
        __shared__ int n_marked;
        const int t = threadIdx.x;
        if (t == 0) n_marked = 0;
        __syncthreads();
        const int bid = blockIdx.x + t * gridDim.x;   // gridDim.x * NTH >= p.total
        int b, h, qt;
        if (bid < p.total && tile_of<CAUSAL, NW>(p, bid, b, h, qt)) {
            const size_t q_panel = ((size_t)b * p.Hq + h) * (size_t)p.N * HD;
            const u32x4 w = *(const u32x4*)(p.o + q_panel + (size_t)(qt * 32 * NW) * HD);
            if (w[0] == NF_MARK[0] && w[1] == NF_MARK[1] && w[2] == NF_MARK[2] && w[3] == NF_MARK[3])
                marked[atomicAdd(&n_marked, 1)] = bid;
        }
        __syncthreads();
        const int n = n_marked;
        for (int i = 0; i < n; ++i) {
            fwd8_tile<CAUSAL, NW, true>(p, __builtin_amdgcn_readfirstlane(marked[i]));
            // the next tile reuses the LDS: copies still in flight land first
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }
}

}  // namespace

extern "C" attn_status attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o,
                                    float* lse, int B, int H_q, int H_kv, int N, int D, int causal,
                                    float scale, float descale_q, float descale_k, float descale_v,
                                    void* stream) {
    if (!q8 || !k8 || !v8 || !o) return ATTN_ERR_NULL;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0) return ATTN_ERR_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_GQA;
    if (D != HD) return ATTN_ERR_HEAD_DIM;
    if (!std::isfinite(scale) || !std::isfinite(descale_q) || !std::isfinite(descale_k) ||
        !std::isfinite(descale_v))
        return ATTN_ERR_SCALE;
    const double prod = (double)scale * (double)descale_q * (double)descale_k;
    const float mag = (float)std::fabs(prod);
    if (!std::isfinite(mag)) return ATTN_ERR_SCALE;
    if ((int64_t)N * HD * 2 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    const int br = 32 * NW_LAUNCH;
    const int64_t n_qtiles = ((int64_t)N + br - 1) / br;
    const int64_t total = (int64_t)B * H_q * n_qtiles;
    if (total > INT32_MAX || (int64_t)B * H_q > INT32_MAX) return ATTN_ERR_SHAPE;
    const uintptr_t mis = ((uintptr_t)q8 | (uintptr_t)k8 | (uintptr_t)v8 | (uintptr_t)o) & 15;
    if (mis != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_ALIGN;
    const size_t q_bytes = (size_t)B * H_q * N * HD;
    const size_t kv_bytes = (size_t)B * H_kv * N * HD;
    const size_t o_bytes = 2 * q_bytes;
    const size_t lse_bytes = lse ? (size_t)B * H_q * N * 4 : 0;
    const void* ins[3] = {q8, k8, v8};
    const size_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
    for (int i = 0; i < 3; ++i)
        if (ranges_overlap(o, o_bytes, ins[i], in_bytes[i]) ||
            ranges_overlap(lse, lse_bytes, ins[i], in_bytes[i]))
            return ATTN_ERR_ALIAS;
    if (ranges_overlap(lse, lse_bytes, o, o_bytes)) return ATTN_ERR_ALIAS;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev)) return ATTN_ERR_DEVICE;

    Params p = {};
    p.q = (const uint8_t*)q8;
    p.k = (const uint8_t*)k8;
    p.v = (const uint8_t*)v8;
    p.o = (uint16_t*)o;
    p.lse = lse;
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.N = N;
    p.group = H_q / H_kv;
    p.n_qtiles = (int)n_qtiles;
    p.total = (int)total;
    p.q_mode = mag == 0.f ? 2 : (prod > 0 ? 0 : 1);
    // causal: interleave enough heads' tiles to fill one XCD's workgroup slots
    // (32 CUs x 2 four-wave workgroups)
    const int64_t slots = 32 * (8 / NW_LAUNCH);
    p.cgroup = (int)std::min<int64_t>((int64_t)B * H_q, (slots + n_qtiles - 1) / n_qtiles);
    int64_t dgrid = 0;
    int64_t dg = p.cgroup;
    if (causal && causal_deal((int64_t)B * H_q, dg, n_qtiles, slots, p.deal, dgrid) && dgrid <= INT32_MAX) {
        p.dealt = 1;
        p.cgroup = (int)dg;
        p.total = (int)dgrid;
    }
    p.c = (float)((double)(mag > 0.f ? mag : 1.0f) * 1.4426950408889634);
    p.lse_scale = mag;
    p.dv = descale_v;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)p.total);
    // the fast kernel, then the exact kernel on a small grid that redoes the
    // tiles the fast kernel marked
    const int nth = 64 * NW_LAUNCH;
    const dim3 egrid((unsigned)std::max(std::min(p.total, EXACT_GRID), (p.total + nth - 1) / nth));
    if (causal) {
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, NW_LAUNCH, false>), grid, dim3(nth), 0, s, p);
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<true, NW_LAUNCH, true>), egrid, dim3(nth), 0, s, p);
    } else {
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, NW_LAUNCH, false>), grid, dim3(nth), 0, s, p);
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<false, NW_LAUNCH, true>), egrid, dim3(nth), 0, s, p);
    }
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
