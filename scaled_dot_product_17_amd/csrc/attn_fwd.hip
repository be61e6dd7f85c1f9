// Fused scaled dot-product attention forward for MI355X (gfx950, CDNA4).
//
// O = softmax(scale * Q K^T [causal]) V and the per-row natural-log LSE, with
// K/V heads shared by contiguous groups of query heads (MHA/GQA/MQA).
//   * formula: page "GPU注意力算子性能优化" (QiMeng-Attention), section 1;
//   * tiles kept on chip, nothing intermediate written to global memory, and a
//     softmax merged online across key tiles: page "注意力机制的本质与计算挑战",
//     section 5.1, and page "从硬件视角看注意力机制优化", section 2.1;
//   * "local computation + global reduction" and the shared K/V of a GQA
//     group: the QiMeng page, sections 3.1.1 and 3.2;
//   * scale folded into the score stage, max-subtracted softmax, mask fused
//     into the softmax, double-buffered tile staging and look-ahead prefetch:
//     page "AVO算法优化Transformer注意力机制性能解析", sections 2.2, 3.1, 3.2, 5.1.
//
// Work decomposition (one workgroup = 8 waves = 256 query rows of one head):
//   * each wave owns 32 query rows; its Q rows live in VGPRs as the B operand
//     of v_mfma_f32_32x32x16_bf16 for the whole kernel;
//   * key blocks of 32 rows of K and V are copied HBM -> LDS by the buffer
//     unit's LDS DMA (no VGPR staging).  K runs one block ahead of V: while a
//     wave turns the scores of block j into probabilities, the MFMAs of the
//     scores of block j+1 and of O += V_{j-1}^T P_{j-1}^T are already in
//     flight, so the softmax VALU work overlaps matrix-core work in every wave;
//   * scores are computed transposed, S^T = K Q^T, so each lane owns one query
//     column: the row max and row sum are in-lane reductions plus one
//     permlane32 swap, and the output rescale is a per-lane scalar;
//   * the fp32 S^T accumulator, converted to bf16, is directly the B operand of
//     O^T += V^T P^T.  The MFMA's k index then visits keys in the order the
//     accumulator holds them; V^T fragments are read in the same key order with
//     the gfx950 transposing LDS read (ds_read_b64_tr_b16), so V never needs a
//     transposed copy;
//   * softmax in base 2 against a reference m: p = exp2(s*c - m*c) with
//     c = scale*log2(e), m starting at the row max of the first key block.
//     The reference only moves (rescaling O and the sums) when p could stop
//     being finite: the final O / sum(bf16 p) and LSE = m*scale + ln(sum p)
//     are the same quantities whichever reference was used.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "attn.h"
#include "cdna4.h"

namespace {

using namespace cdna4;

constexpr int HD = 128;                    // head dimension handled by this kernel
// A workgroup is NW waves = 32*NW query rows (NW = 8, or 4 for grids too small
// to fill the chip with 8-wave workgroups, short sequences and narrow windows,
// where twice as many workgroups balance the grid better and the two
// workgroups sharing a CU are not tied by one barrier).
constexpr int BR = 256;                    // query rows per 8-wave workgroup
constexpr int NWAVE = 8;
constexpr int N_CU = 256;                  // compute units of the chip (8 XCDs x 32)
constexpr int MIN_N_8W = 1024;             // shorter sequences use 4 waves
constexpr int ROW_BYTES = HD * 2;          // 256 B per K/V/Q/O row
constexpr int KB = 32;                     // keys per pipeline step (one MFMA M block)
constexpr int BLK_BYTES = KB * ROW_BYTES;  // 8 KiB per K or V block
constexpr int K_RING = 0;                  // LDS: a ring of 4 K blocks, then 4 V blocks
constexpr int V_RING = 4 * BLK_BYTES;
constexpr int LDS_BYTES = 8 * BLK_BYTES;   // 64 KiB
constexpr float MOVE_SUM = 18446744073709551616.0f;  // 2^64: a lane's block sum of p above
                                                      // this moves the softmax reference
// block-sparse masks: blocks of SP_BLOCK query rows x SP_BLOCK keys; a workgroup's
// 256 rows are two query blocks.  The union of their key-block lists is kept in
// LDS past the rings, one 16-bit entry per key block (index | 2 membership bits).
constexpr int SP_BLOCK = 128;
constexpr int SP_MAX = 2048;               // key blocks a mask may have (N <= 262144)
constexpr int SP_BYTES = 2 * SP_MAX + 64;  // union list + per-wave counts
// Exact kernel (non-finite V in a masked block): a zero block, and per wave up
// to MAX_SAVED masked blocks' bf16 weights (32 rows x 32 keys), the factor each
// block's weights have been rescaled by since (one per lane) and its index.
constexpr int MAX_SAVED = 4;
constexpr int SAVE_P = 32 * KB * 2;
constexpr int SAVE_WAVE_BYTES = MAX_SAVED * (SAVE_P + 64 * 4) + 16;
// Mark the fast kernel leaves in the first output row of a workgroup it hands
// to the exact kernel: eight signalling-NaN bf16 codes (0x7F81 .. 0x7F88).
// Arithmetic never produces them (every NaN it makes is quiet), so no output
// row can hold them.
__constant__ const uint32_t NF_MARK[4] = {0x7F827F81u, 0x7F847F83u, 0x7F867F85u, 0x7F887F87u};

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, Hq, Hkv, N;
    int group;        // Hq / Hkv
    int n_qtiles;     // ceil(N / BR)
    int total;        // B * Hq * n_qtiles workgroups
    int q_mode;       // 0: Q as given, 1: Q negated, 2: Q replaced by zeros
    int cgroup;       // dense causal: heads whose tiles are interleaved (<= 1: one head)
    float c;          // |scale| * log2(e), always > 0
    float lse_scale;  // |scale|
    // packed variable-length batch (VARLEN kernels only): B = 1 and N = tokens
    const int* cu;    // n_seq + 1 token offsets
    int n_seq;
    int dealt;        // the dealt grid order (dealt_tile) instead of the plain one
    Deal deal;        // its sizes
    int left, right;  // window: row i sees keys i-left .. i+right (< 0: unbounded)
    // block-sparse mask (SPARSE kernels only): lists of SP_BLOCK-key blocks per
    // (mask head, SP_BLOCK-row query block), block-compressed-row form
    const int* kb_ptr;  // mask_heads * n_sblk + 1 offsets into kb_idx
    const int* kb_idx;  // nnz key-block indices
    int nnz;
    int mask_heads;     // 1 (shared by all heads) or Hq
    int n_sblk;         // ceil(N / SP_BLOCK)
};

// LDS byte offset of the 16-byte chunk (row, chunk) of a K tile.  The chunk
// index is XOR-swizzled with the low 4 row bits so the 32 rows one MFMA A
// operand read touches (same logical chunk) fall in distinct banks.
__device__ __forceinline__ uint32_t k_lds_off(int row, int chunk) {
    return (uint32_t)(row * ROW_BYTES + ((chunk ^ (row & 15)) << 4));
}
// LDS byte offset of the 16-byte chunk (row, chunk) of a V tile.  The chunk
// index is XOR-swizzled with 4*(row mod 4): a transposing read touches 4
// consecutive rows x 64 contiguous bytes per half-wave, and this spreads the
// four rows over the four 64-byte bank groups.
__device__ __forceinline__ uint32_t v_lds_off(int row, int chunk) {
    return (uint32_t)(row * ROW_BYTES + ((chunk ^ ((row & 3) << 2)) << 4));
}

// Which (batch, head, query tile) workgroup id bid computes, and the token
// range [s0, s1) of its sequence (the whole panel when dense).  VARLEN: the
// batch index is the sequence of a packed batch (B = 1, N = all tokens).
// false: bid is padding of the grid or past its sequence's end.
template <bool CAUSAL, bool VARLEN, bool SPARSE, int NW>
__device__ __forceinline__ bool tile_of(const Params& p, int bid, int& b, int& h, int& qt, int& s0, int& s1) {
    constexpr int BRW = 32 * NW;
    const int logical = xcd_remap(bid, p.total);
    int bh;
    if ((VARLEN || (CAUSAL && !SPARSE)) && p.dealt) {
        // varlen batches of unequal lengths, and causal grids whose head groups
        // do not split evenly over the 8 XCDs: slices of groups dealt to the
        // XCDs in turn, each a strided share of its group's heaviest-first
        // list, so the XCDs receive equal work and finish together
        if (!dealt_tile(bid, p.B * p.Hq, p.cgroup > 1 ? p.cgroup : 1, p.n_qtiles, p.deal, bh, qt))
            return false;   // padding of the grid
    } else if (CAUSAL && !SPARSE) {
        // groups of cgroup (batch, head)s one after another, so the tiles of a
        // group share K/V in the L2 of one XCD; within a group tile-major,
        // heaviest tile first.  A group holds at least as many tiles as an XCD
        // has workgroup slots, so the light tiles of one group, not the heavy
        // tiles of the next, fill the end of each XCD's share of the grid.
        const int per = p.B * p.Hq;
        const int G = p.cgroup > 1 ? p.cgroup : 1;
        const int grp = logical / (G * p.n_qtiles);
        const int r = logical - grp * G * p.n_qtiles;
        const int gh = min(G, per - grp * G);   // heads in this group (the last may be short)
        qt = p.n_qtiles - 1 - r / gh;
        bh = grp * G + r % gh;
    } else {
        // one (batch, head) after another, so a head's tiles share K/V in the
        // L2 of one XCD
        bh = logical / p.n_qtiles;
        qt = logical % p.n_qtiles;
        if (CAUSAL) qt = p.n_qtiles - 1 - qt;   // heaviest tiles of a head first
    }
    b = bh / p.Hq;
    h = bh % p.Hq;
    // rows [s0, s1) of the panel form this tile's sequence (the whole panel when dense)
    s0 = 0;
    s1 = p.N;
    if constexpr (VARLEN) {
        s0 = min(max(p.cu[b], 0), p.N);
        s1 = min(max(p.cu[b + 1], s0), p.N);
        if (qt * BRW >= s1 - s0) return false;   // past this sequence's end
    }
    return true;
}

// One query tile (workgroup id bid).  SAFE = false: the fast kernel's body.
// SAFE = true: the exact form, for the tiles the fast kernel marked (see
// NF_MARK).
template <bool CAUSAL, bool VARLEN, bool SPARSE, int NW, bool SAFE>
__device__ __forceinline__ void fwd_tile(const Params& p, const int bid) {
    static_assert(NW == 8 || NW == 4, "workgroups of 4 or 8 waves");
    constexpr int BRW = 32 * NW;                 // query rows of this workgroup
    constexpr int NTH = NW * 64;
    constexpr int DMA_PER_WAVE = 32 / (4 * NW);  // 4-row DMA instructions per wave per key block
    constexpr int QB_WG = BRW / SP_BLOCK;        // SPARSE: query blocks per workgroup (1 or 2)
    constexpr int SP_PER_T = SP_MAX / NTH;       // SPARSE: key blocks each thread compacts
    constexpr int ZERO_OFF = LDS_BYTES + (SPARSE ? SP_BYTES : 0);   // exact kernel: a block of zeros
    constexpr int SAVE_OFF = ZERO_OFF + BLK_BYTES;                     // exact kernel: per-wave saved blocks
    // Fast dense and varlen kernels copy each wave's 32 Q rows into LDS: 8-wave
    // workgroups (one per CU) into 64 KiB past the rings, 4-wave ones into the
    // ring slots the prologue leaves free (K slot 3, V slots 1-3); their
    // waves' non-finite answers then move past the rings
    constexpr bool Q_STAGED = !SAFE && !SPARSE;
    constexpr int Q_EXTRA = !Q_STAGED ? 0 : NW == 8 ? NW * 32 * ROW_BYTES : 64;
    constexpr int NF_OFF = (Q_STAGED && NW == 4) ? LDS_BYTES : V_RING + 3 * BLK_BYTES;
    __shared__ __attribute__((aligned(1024))) char lds[ZERO_OFF + (SAFE ? BLK_BYTES + NW * SAVE_WAVE_BYTES : 0) + Q_EXTRA];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;   // query column owned by this lane
    const int hh = lane >> 5;    // which half of the wave

    // ---- which (batch, head, query tile) this workgroup computes
    int b, h, qt, s0, s1;
    if (!tile_of<CAUSAL, VARLEN, SPARSE, NW>(p, bid, b, h, qt, s0, s1)) return;   // whole workgroup, no barrier yet
    const int kvh = h / p.group;
    const int N = p.N;
    const int q0 = s0 + qt * BRW;
    const int wq0 = q0 + wave * 32;       // first query row of this wave
    const int myq = wq0 + l32;            // query row of this lane

    const int pbat = VARLEN ? 0 : b;      // batch index of the panels
    const size_t qo_panel = ((size_t)pbat * p.Hq + h) * (size_t)N * HD;
    const size_t kv_panel = ((size_t)pbat * p.Hkv + kvh) * (size_t)N * HD;
    uint16_t* const mark = p.o + qo_panel + (size_t)q0 * HD;   // the workgroup's first output row
    if constexpr (SAFE) {
        // only the workgroups the fast kernel marked (every thread reads the
        // same 16 bytes, so the exit is workgroup-uniform)
        const u32x4 w = *(const u32x4*)mark;
        if (w[0] != NF_MARK[0] || w[1] != NF_MARK[1] || w[2] != NF_MARK[2] || w[3] != NF_MARK[3]) return;
    }

    // ---- key blocks of 32 from key kb0: n_blk_wg streamed through LDS, n_blk used
    // by this wave.  Dense causal: a wave's 32 rows start on a block boundary, so
    // every block before its diagonal block is fully visible and only its last
    // block is masked.  VARLEN: each row i sees keys [lo_i, hi_i] of its sequence
    // (window and causal bounds); blocks before a wave's window are fully masked.
    int kb0 = 0, n_blk_wg, n_blk;
    int lo_i = 0, hi_i = N - 1;           // this lane's allowed keys (VARLEN)
    int lo_max = 0, hi_min = N - 1;       // keys every valid row of the wave allows (VARLEN)
    // SPARSE: the union of the workgroup's query blocks' lists (one or two),
    // built in LDS (the rings serve as scratch before the first copy); stream
    // block g is 32-key part g % 4 of union entry g / 4
    const uint16_t* sp = (const uint16_t*)(lds + LDS_BYTES);
    // Q rows into VGPRs, the B operand of S^T = K Q^T in k-steps of 16 head
    // dims.  SPARSE loads them first: they do not depend on the key-block
    // lists, so their latency hides behind the list reads below.
    bf16x8 qf[8];
    auto load_q = [&]() {
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.q + qo_panel, (uint32_t)N * ROW_BYTES);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(qr, (uint32_t)myq * ROW_BYTES + (16 * ks + 8 * hh) * 2));
    };
    if constexpr (SPARSE) {
        load_q();
        const int nsb = p.n_sblk;
        const size_t mh = p.mask_heads == 1 ? 0 : (size_t)h;
        // the lists' bounds, read before the flags are cleared (offsets
        // clamped to [0, nnz]: a malformed list cannot read out of range)
        int la[QB_WG], le[QB_WG];
#pragma unroll
        for (int half = 0; half < QB_WG; ++half) {
            const int qb = QB_WG * qt + half;
            la[half] = 0;
            le[half] = 0;
            if (qb < nsb) {
                la[half] = min(max(p.kb_ptr[mh * nsb + qb], 0), p.nnz);
                le[half] = min(max(p.kb_ptr[mh * nsb + qb + 1], la[half]), p.nnz);
            }
        }
        uint8_t* f0 = (uint8_t*)lds;             // key blocks listed by query block QB_WG*qt
        uint8_t* f1 = (uint8_t*)lds + SP_MAX;    // ... and by query block 2qt+1 (8 waves)
        int* wsum = (int*)(lds + LDS_BYTES + 2 * SP_MAX);
        for (int i = tid; i < 2 * SP_MAX / 4; i += NTH) ((uint32_t*)lds)[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int half = 0; half < QB_WG; ++half) {
            const int qb = QB_WG * qt + half;
            uint8_t* f = half ? f1 : f0;
            for (int x = la[half] + tid; x < le[half]; x += NTH) {
                const int kb = p.kb_idx[x];
                // causal: key blocks after the query block hold no visible key
                if (kb >= 0 && kb < nsb && (!CAUSAL || kb <= qb)) f[kb] = 1;
            }
        }
        __syncthreads();
        // compaction in key-block order: thread t owns SP_PER_T consecutive key
        // blocks, whose flags it reads as one word per query block
        static_assert(SP_PER_T == 8 || SP_PER_T == 4, "flag words of 8 or 4 bytes");
        using FlagWord = std::conditional_t<SP_PER_T == 8, uint64_t, uint32_t>;
        const FlagWord w0 = *(const FlagWord*)(f0 + SP_PER_T * tid);
        const FlagWord w1 = *(const FlagWord*)(f1 + SP_PER_T * tid);
        int bits[SP_PER_T], cnt = 0;
#pragma unroll
        for (int j = 0; j < SP_PER_T; ++j) {
            const int kb = SP_PER_T * tid + j;
            bits[j] = kb < nsb ? (int)(((w0 >> (8 * j)) & 1u) | (((w1 >> (8 * j)) & 1u) << 1)) : 0;
            cnt += bits[j] != 0;
        }
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int before = 0, n_u = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = wsum[w];
            before += w < wave ? c : 0;
            n_u += c;
        }
        int pos = before + incl - cnt;
        uint16_t* spw = (uint16_t*)(lds + LDS_BYTES);
#pragma unroll
        for (int j = 0; j < SP_PER_T; ++j)
            if (bits[j] != 0) spw[pos++] = (uint16_t)((SP_PER_T * tid + j) | (bits[j] << 14));
        __syncthreads();
        n_blk_wg = 4 * n_u;
        n_blk = wq0 < N ? n_blk_wg : 0;
    } else if constexpr (VARLEN) {
        const int r_end = min(q0 + BRW, s1);
        kb0 = p.left >= 0 ? max(s0, q0 - p.left) : s0;
        int khi = s1 - 1;
        if (CAUSAL) khi = min(khi, r_end - 1);
        if (p.right >= 0) khi = min(khi, r_end - 1 + p.right);
        n_blk_wg = (khi - kb0) / KB + 1;
        auto row_lo = [&](int i) { return p.left >= 0 ? max(s0, i - p.left) : s0; };
        auto row_hi = [&](int i) {
            int x = s1 - 1;
            if (CAUSAL) x = min(x, i);
            if (p.right >= 0) x = min(x, i + p.right);
            return x;
        };
        lo_i = row_lo(myq);
        hi_i = row_hi(myq);
        const int wlast = min(wq0 + 31, s1 - 1);
        lo_max = row_lo(wlast);
        hi_min = row_hi(wq0);
        n_blk = wq0 < s1 ? min(n_blk_wg, (row_hi(wlast) - kb0) / KB + 1) : 0;
    } else {
        const int n_blk_all = (N + KB - 1) / KB;
        n_blk_wg = n_blk_all;
        n_blk = n_blk_all;
        if (CAUSAL) {
            n_blk_wg = min(n_blk_all, (min(q0 + BRW, N) - 1) / KB + 1);
            n_blk = min(n_blk_all, wq0 / KB + 1);
        }
        if (wq0 >= N) n_blk = 0;   // a wave of padding rows past the end computes nothing
    }
    const uint16_t* kbase = p.k + kv_panel + (size_t)kb0 * HD;
    const uint16_t* vbase = p.v + kv_panel + (size_t)kb0 * HD;

    // ---- LDS rings: K block g lives in slot g % 4 of the K ring, V block g in
    // slot g % 4 of the V ring.  Each wave copies rows 8*wave .. 8*wave+7 of a
    // block with two DMA instructions of 4 rows (1 KiB, 16 bytes per lane in
    // lane order).  The bank swizzle is applied on the global side: lane L
    // fetches the logical chunk that belongs at its physical LDS position.
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    uint32_t k_dma[DMA_PER_WAVE], v_dma[DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int row = 4 * DMA_PER_WAVE * wave + 4 * i + (lane >> 4);
        const int pc = lane & 15;
        k_dma[i] = (uint32_t)(row * ROW_BYTES + ((pc ^ (row & 15)) << 4));
        v_dma[i] = (uint32_t)(row * ROW_BYTES + ((pc ^ ((row & 3) << 2)) << 4));
    }
    // first key of stream block g, and whether this wave's query block lists it (SPARSE)
    // SPARSE: the union list's first 64 entries are also held in one VGPR
    // (entry i in lane i) and read back with readlane, off the LDS latency;
    // later entries come from LDS
    int sp_reg = 0;
    if constexpr (SPARSE) sp_reg = lane < n_blk_wg / 4 ? (int)sp[lane] : 0;
    auto sp_ent = [&](int g) {
        const int e = g >> 2;
        return e < 64 ? __builtin_amdgcn_readlane(sp_reg, e) : __builtin_amdgcn_readfirstlane((int)sp[e]);
    };
    auto sp_key = [&](int g) { return (sp_ent(g) & 0x3FFF) * SP_BLOCK + (g & 3) * KB; };
    auto sp_member = [&](int g) { return ((sp_ent(g) >> (14 + (wave >> 2))) & 1) != 0; };
    // One descriptor per panel serves every copy, with the block's offset in
    // soffset.  Its range ends at the last key any block of this workgroup
    // needs (the sequence's or the panel's end, or the end of the workgroup's
    // last block).  The buffer unit range-checks voffset + soffset, and a lane
    // past the range reads nothing and writes zeros to LDS: rows past the end
    // of a ragged last block arrive as zeros (never as a stale row of an
    // earlier block), and copies of blocks past the workgroup's last one, which
    // the pipeline issues without a guard, only clear their slot.
    const int end = VARLEN ? s1 : N;
    const int lim = SPARSE ? end : min(end, kb0 + n_blk_wg * KB);
    const uint32_t lds_wave = lds_base + 4 * DMA_PER_WAVE * wave * ROW_BYTES;
    const u32x4 k_desc = sgpr_rsrc(kbase, (uint32_t)(lim - kb0) * ROW_BYTES);
    const u32x4 v_desc = sgpr_rsrc(vbase, (uint32_t)(lim - kb0) * ROW_BYTES);
    auto dma_block = [&](auto ring_t, auto slot_t, const u32x4& desc, const uint32_t* voff, int g) {
        constexpr uint32_t DST = decltype(ring_t)::value + decltype(slot_t)::value * BLK_BYTES;
        uint32_t soff = (uint32_t)g * BLK_BYTES;
        if constexpr (SPARSE) {
            if (g >= n_blk_wg) return;   // entries past the union list are not keys
            soff = (uint32_t)sp_key(g) * ROW_BYTES;
        }
        lds_dma16_at<DST>(desc, lds_wave, voff[0], soff);
        if constexpr (DMA_PER_WAVE > 1) lds_dma16_at<DST + 4 * ROW_BYTES>(desc, lds_wave, voff[1], soff);
    };

    // ---- per-lane LDS read offsets (relative to a block slot)
    uint32_t k_rd[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) k_rd[ks] = k_lds_off(l32, 2 * ks + hh);
    uint32_t v_rd[4];
    {
        const int g = lane >> 4;          // 16-lane group
        const int rs = (lane & 15) >> 2;  // source row within the 4-row block
        const int cs = lane & 3;          // source 4-element column block
        const int row = 4 * (g >> 1) + rs;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int col = 32 * db + 16 * (g & 1) + 4 * cs;  // element column
            v_rd[db] = v_lds_off(row, col >> 3) + ((col & 4) ? 8 : 0);
        }
    }

    // ---- prologue: K blocks 0-2 and V block 0 in flight, then Q into VGPRs
    if constexpr (SAFE) {
        // the zero block masked products run against (first read after the
        // barrier below)
#pragma unroll
        for (int i = 0; i < BLK_BYTES / (16 * NTH); ++i)
            *(u32x4*)(lds + ZERO_OFF + 16 * (tid + NTH * i)) = u32x4{0u, 0u, 0u, 0u};
    }
    using R_K = std::integral_constant<uint32_t, K_RING>;
    using R_V = std::integral_constant<uint32_t, V_RING>;
    using S0 = std::integral_constant<uint32_t, 0>;
    using S1 = std::integral_constant<uint32_t, 1>;
    using S2 = std::integral_constant<uint32_t, 2>;
    using S3 = std::integral_constant<uint32_t, 3>;
    dma_block(R_K{}, S0{}, k_desc, k_dma, 0);
    dma_block(R_V{}, S0{}, v_desc, v_dma, 0);
    dma_block(R_K{}, S1{}, k_desc, k_dma, 1);
    dma_block(R_K{}, S2{}, k_desc, k_dma, 2);

    // Staged Q: the wave's 32 rows copied by LDS DMA, 4 whole rows (1 KiB) per
    // instruction instead of 32 rows per load, with the K tiles' bank swizzle
    // applied on the global side (16-byte chunk c of row r at chunk
    // c ^ (r mod 16)); rows at or past N arrive as zeros (range-checked
    // voffset).  Each wave reads back only its own rows, after its own copies
    // have landed.
    const uint32_t q_lds = NW == 8 ? (uint32_t)(LDS_BYTES + wave * (32 * ROW_BYTES))
                                   : (uint32_t)(wave == 0 ? K_RING + 3 * BLK_BYTES : V_RING + wave * BLK_BYTES);
    auto stage_q = [&]() {
        const u32x4 qd = sgpr_rsrc(p.q + qo_panel, (uint32_t)N * ROW_BYTES);
        const uint32_t qbase = lds_base + q_lds;
        auto one = [&](auto i_t) {
            constexpr int i = decltype(i_t)::value;
            const int row = 4 * i + (lane >> 4);
            const uint32_t voff = (uint32_t)((wq0 + row) * ROW_BYTES + (((lane & 15) ^ (row & 15)) << 4));
            lds_dma16_at<(uint32_t)(i * 4 * ROW_BYTES)>(qd, qbase, voff, 0u);
        };
        one(std::integral_constant<int, 0>{});
        one(std::integral_constant<int, 1>{});
        one(std::integral_constant<int, 2>{});
        one(std::integral_constant<int, 3>{});
        one(std::integral_constant<int, 4>{});
        one(std::integral_constant<int, 5>{});
        one(std::integral_constant<int, 6>{});
        one(std::integral_constant<int, 7>{});
    };
    auto read_q = [&]() {
        const char* qs = lds + q_lds;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[ks] = *(const bf16x8*)(qs + l32 * ROW_BYTES + (((2 * ks + hh) ^ (l32 & 15)) << 4));
    };
    // A negative scale is applied as |scale| on -Q (a sign flip is exact in
    // bf16) and a zero scale as zero scores, so the exp2 argument below always
    // multiplies by a positive constant and masked -inf scores stay -inf.
    auto q_sign = [&]() {
        if (p.q_mode != 0) {
            const u32x4 flip = p.q_mode == 1 ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}
                                             : u32x4{0u, 0u, 0u, 0u};
            const u32x4 keep = p.q_mode == 1 ? u32x4{~0u, ~0u, ~0u, ~0u} : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                qf[ks] = __builtin_bit_cast(bf16x8, (__builtin_bit_cast(u32x4, qf[ks]) & keep) ^ flip);
        }
    };
    if constexpr (Q_STAGED) {
        stage_q();
    } else {
        if constexpr (!SPARSE) load_q();
        q_sign();
    }
    const float c = p.c;

    // S^T of one 32-key block, from a K ring slot
    auto scores = [&](f32x16& s, uint32_t kslot) {
        s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 a = *(const bf16x8*)(lds + kslot + k_rd[ks]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
        }
    };
    // Blocks a wave must mask are a prefix (g < g_lo: before the window of the
    // wave's last row) and a suffix (g >= g_hi: past the causal diagonal of its
    // first row, its window end, or the sequence's or panel's end).  Dense rows
    // of a wave start on a block boundary, so the causal suffix starts at the
    // wave's diagonal block wq0 / KB; a ragged panel's last block is N / KB.
    // Block n_blk (the drain step's) is always in the suffix.
    int g_lo = 0, g_hi = N / KB;
    if constexpr (VARLEN) {
        g_lo = lo_max > kb0 ? (lo_max - kb0 + KB - 1) / KB : 0;
        g_hi = hi_min >= kb0 ? (hi_min - kb0 + 1) / KB : 0;
    } else if constexpr (CAUSAL && !SPARSE) {
        g_hi = min(g_hi, wq0 / KB);
    }
    // SPARSE with one query block per workgroup (the 4-wave kernels): every
    // union entry is listed by that block, and only the last entry can hold a
    // masked key (the diagonal block when causal, since a causal list holds no
    // block past it; the panel's ragged last block), so the steps before it
    // read no list entry from LDS to decide
    constexpr bool SP_ONE = SPARSE && QB_WG == 1;
    const int g_tail = SPARSE ? n_blk_wg - 4 : 0;   // first stream block of the last union entry
    auto member = [&](int g) {
        if constexpr (SP_ONE) return true;
        else return sp_member(g);
    };
    // key >= N (ragged tail) or key > query (causal) -> -inf
    auto needs_mask = [&](int g) {
        if constexpr (SPARSE) {
            if (SP_ONE && g < g_tail) return false;
            const int kb = sp_key(g);
            return !member(g) || (CAUSAL && kb + KB - 1 > wq0) || (kb + KB > N);
        }
        if constexpr (VARLEN) return g < g_lo || g >= g_hi;
        return g >= g_hi;
    };
    // true when key `key` of a block (listed or not for this wave's query
    // block: SPARSE) is not visible to this lane's row
    auto key_bad = [&](int key, bool listed) {
        if constexpr (VARLEN) return key < lo_i || key > hi_i;
        else return !listed || (key >= N) || (CAUSAL && key > myq);
    };
    bool seen_g = false;      // exact kernel: some key of the masked block is visible to this lane's row
    auto apply_mask = [&](f32x16& s, int g) {
        const int kbase_g = SPARSE ? sp_key(g) : kb0 + g * KB;
        const bool listed = SPARSE ? sp_member(g) : true;
        bool any = false;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool bad = key_bad(kbase_g + 8 * (r >> 2) + 4 * hh + (r & 3), listed);
            if constexpr (SAFE) any = any || !bad;
            s[r] = bad ? -INFINITY : s[r];
        }
        if constexpr (SAFE) seen_g = any;
    };
    bool mask_prev = false;   // exact kernel: the previous step's block was masked
    bool keep_prev = false;   // ... and some row of the wave sees one of its keys
    int n_saved = 0;          // exact kernel: masked blocks saved for the exact phase

    f32x16 o[4];          // O^T: 4 blocks of 32 head dims x 32 query columns
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    const bool live = myq < s1;   // a row that is written (padding rows past the end are not)
    float m = -INFINITY;  // reference max of the raw scores q.k of this lane's row
    float mb = 0.f;       // m * c, or 0 while m is -inf
    float l = 0.f;        // this lane's partial sum of p (fp32): the LSE
    float lb = 0.f;       // partial sum of bf16(p), the weights the PV MFMA applies: O's divisor

    // O^T += V^T P^T for one block; the MFMA k index walks keys in the order
    // the score accumulator holds them (P was built from it lane by lane).
    auto pv = [&](const u32x4 (&pw)[2], uint32_t vslot) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const uint32_t off = vslot + v_rd[db] + (uint32_t)(16 * kk) * ROW_BYTES;
                const bf16x4 lo = lds_read_tr(lds, off);
                const bf16x4 hi = lds_read_tr(lds, off + 8 * ROW_BYTES);
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pw[kk]),
                                                                o[db], 0, 0, 0);
            }
    };
    // A masked block multiplies the V rows of keys some rows may not see by
    // zero weights, and 0 * NaN or 0 * inf is NaN in the matrix core.  Before
    // its main loop each wave of the fast kernel scans the V rows of its
    // masked blocks in global memory; a workgroup that finds a non-finite value
    // there is redone by the exact kernel.  The exact kernel runs a masked
    // block's product against a block of zeros instead of its V (same code
    // path, so the loop keeps its registers) and saves the block's weights;
    // after the loop it adds each saved block's terms p * v for the keys each
    // row sees (V read from global memory), times the factor its weights have
    // been rescaled by since.  So a NaN or an infinity reaches exactly the rows
    // that see its key.
    auto save_block = [&](const u32x4 (&pw)[2], int gb) {
        char* base = lds + SAVE_OFF + wave * SAVE_WAVE_BYTES;
        char* wp = base + n_saved * SAVE_P + l32 * (KB * 2);   // this row's 32 weights
        // keys 8a + 4hh + (0..3) of the row are accumulator registers 4a .. 4a+3
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const u32x4& w = pw[a >> 1];
            *(uint2*)(wp + 2 * (8 * a + 4 * hh)) = uint2{w[2 * (a & 1)], w[2 * (a & 1) + 1]};
        }
        ((float*)(base + MAX_SAVED * SAVE_P))[n_saved * 64 + lane] = 1.0f;
        if (lane == 0) ((int*)(base + MAX_SAVED * (SAVE_P + 256)))[n_saved] = gb;
        ++n_saved;
    };

    // P = exp2(s*c - mb) rounded to bf16 in pairs (the B operand of the PV
    // MFMA); ls sums the fp32 p, lbs the bf16 pairs (v_dot2 against (1, 1)).
    auto probs = [&](const f32x16& s, u32x4 (&pw)[2], float& ls, float& lbs) {
        const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
        float ls0 = 0.f, ls1 = 0.f, lb0 = 0.f, lb1 = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * i], c, -mb));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * i + 1], c, -mb));
                ls0 += e0;
                ls1 += e1;
                const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
                if (i & 1) lb1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, lb1, false);
                else lb0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, lb0, false);
                pw[kk][i] = __builtin_bit_cast(uint32_t, pr);
            }
        ls = ls0 + ls1;
        lbs = lb0 + lb1;
    };

    auto row_max = [&](const f32x16& s) {
        float mx = fmaxf(s[0], s[1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
        return wave_swap_max(mx);
    };

    // Key block g (valid while g < n_blk; g == n_blk drains the last PV: its
    // block is masked whole, so its weights and sums are exact zeros).
    // Issued together, with no dependence on this block's softmax:
    //   * the scores sn of block g+1 (K ring slot KS),
    //   * O += V_{g-1}^T P_{g-1}^T for the previous block (V ring slot VS),
    // while the VALU turns the scores s of block g into P_g against the current
    // reference m.  p only has to stay finite: bf16 and fp32 keep their
    // relative precision at any magnitude, and O / sum(bf16 p) and
    // m*scale + ln(sum p) do not depend on which reference was used.  So the
    // reference only moves when a lane's block sum exceeds 2^64 (or is not
    // finite): then (rare, wave-uniform branch) every row moves to its true
    // running max, O and the sums are rescaled once the previous PV has
    // landed, and P_g is recomputed.
    auto step = [&](auto first_t, auto ks_t, auto vs_t, int g, f32x16& s, f32x16& sn,
                    const u32x4 (&pp)[2], u32x4 (&pc)[2]) {
        constexpr bool FIRST = decltype(first_t)::value;
        constexpr uint32_t KS = K_RING + decltype(ks_t)::value * BLK_BYTES;
        constexpr uint32_t VS = V_RING + decltype(vs_t)::value * BLK_BYTES;
        const bool valid = g < n_blk;
        // SPARSE: a wave skips the work of blocks its own query block does not
        // list (wave-uniform): the scores of g+1, the softmax of g, the PV of g-1
        const bool use_n = !SPARSE || (g + 1 < n_blk_wg && member(g + 1));
        const bool use_g = !SPARSE || (valid && member(g));
        const bool use_p = !SPARSE || (g >= 1 && member(g - 1));
        const bool mask_g = needs_mask(g);
        if (!FIRST && use_g && mask_g) apply_mask(s, g);
        if constexpr (SAFE) {
            // exact kernel: a masked block's product runs against the zero
            // block, and its weights are saved when some row sees one of its keys
            if constexpr (!FIRST)
                if (use_p) {
                    pv(pp, mask_prev ? (uint32_t)ZERO_OFF : VS);
                    if (mask_prev && keep_prev && n_saved < MAX_SAVED) save_block(pp, g - 1);
                }
            mask_prev = valid && use_g && mask_g;
            keep_prev = mask_prev && __builtin_amdgcn_ballot_w64(seen_g) != 0;
            if (use_n) scores(sn, KS);
        } else {
            if (use_n) scores(sn, KS);
            if constexpr (!FIRST)
                if (use_p) pv(pp, VS);
        }
        if (!use_g) return;
        float ls, lbs;
        probs(s, pc, ls, lbs);
        // Issue order of the step's 16 MFMAs, 24 LDS operand reads, 16 exp2
        // and the rest of the softmax VALU: three reads ahead, then per MFMA
        // one or two reads, three VALU and one exp2, so every MFMA has vector
        // work beside it and its operand was requested a slot earlier (same-box
        // A/B of the orders tried: this one 3-5% faster than the compiler's own).
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU (not MFMA, not transcendental)
            __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);   // transcendental (exp2)
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        // keep P_g ahead of the branch below (not sunk into its fall-through
        // path), so its VALU work interleaves with the MFMAs issued above
        asm volatile("" : "+v"(pc[0]), "+v"(pc[1]), "+v"(ls), "+v"(lbs));
        // While a row has seen no finite score (m = -inf: a window or block list
        // that has not started, or -inf scores), mb is -inf, so any score makes
        // its sum inf or NaN and takes the branch below, which moves m to the
        // first finite score and weighs the rest of the block against it.
        const uint64_t over = __builtin_amdgcn_ballot_w64(!(ls <= MOVE_SUM));
        if (over != 0) {
            const float m_new = fmaxf(m, row_max(s));
            const bool move = m_new > m;
            const float alpha = move ? __builtin_amdgcn_exp2f((m - m_new) * c) : 1.0f;
            m = m_new;
            mb = (m == -INFINITY) ? 0.f : m * c;
            l *= alpha;
            lb *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            if constexpr (SAFE) {
                float* fac = (float*)(lds + SAVE_OFF + wave * SAVE_WAVE_BYTES + MAX_SAVED * SAVE_P);
                for (int i = 0; i < n_saved; ++i) fac[i * 64 + lane] *= alpha;
            }
            probs(s, pc, ls, lbs);
            if (m == -INFINITY && live) mb = -INFINITY;
        }
        l += ls;
        lb += lbs;
    };

    f32x16 sa, sb;    // scores of even / odd key blocks
    u32x4 pa[2], pb[2];  // bf16 P of even / odd key blocks
    // Masked blocks are a prefix and a suffix of the wave's blocks (window
    // start; causal diagonal, window end, sequence or panel end).  Their V rows
    // in range are read from global memory and checked for a non-finite value.
    uint32_t nf_bits = 0u;
    if (!SAFE && n_blk > 0) {
        const int end = VARLEN ? s1 : N;
        auto vcheck = [&](int g) {
            const int key = SPARSE ? sp_key(g) : kb0 + g * KB;
            if (key >= end) return;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(vbase + (size_t)(key - kb0) * HD,
                                                       (uint32_t)(end - key) * ROW_BYTES);
#pragma unroll
            for (int i = 0; i < BLK_BYTES / 1024; ++i) {
                const u32x4 x = buf_load16(r, (uint32_t)(16 * lane + 1024 * i));
                // a bf16 half with an all-ones exponent carries into its top bit
#pragma unroll
                for (int e = 0; e < 4; ++e) nf_bits |= (x[e] & 0x7F807F80u) + 0x00800080u;
            }
        };
        int g = 0;
        for (; g < n_blk && needs_mask(g); ++g) vcheck(g);
        for (int h = n_blk - 1; h >= g && needs_mask(h); --h) vcheck(h);
    }
    // vmcnt(0) through the builtin, so the compiler also knows the Q loads are
    // complete and never waits on vmcnt (which counts the DMA) inside the loop
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if constexpr (Q_STAGED) {
        read_q();
        q_sign();
    }
    // fast kernel: the waves' answers meet in V slot 3 (not refilled before
    // tile 1), or past the rings where staged Q uses that slot; a workgroup
    // with a non-finite V value in a masked block marks its first output row
    // and leaves the rows to the exact kernel
    uint32_t* const nf_wave = (uint32_t*)(lds + NF_OFF);
    if constexpr (!SAFE) {
        const bool nf = __builtin_amdgcn_ballot_w64((nf_bits & 0x80008000u) != 0u) != 0;
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
        // block 0's scores and the first reference (its row max)
        scores(sa, K_RING);
        if (needs_mask(0)) apply_mask(sa, 0);
        m = row_max(sa);
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
    // The loop runs one step past the last block so every wave drains its PV.
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
    // tile 0: step 0 has no previous block
    refill_even(0);
    if (0 <= n_blk) step(std::true_type{}, I1{}, I3{}, 0, sa, sb, pb, pa);
    if (1 <= n_blk) step(F{}, I2{}, I0{}, 1, sb, sa, pa, pb);
    wait_dma();
    __syncthreads();
    for (int j = 1; j < n_tiles; j += 2) {
        // odd tile: blocks 2j = 2 (mod 4), 2j+1 = 3 (mod 4)
        refill_odd(j);
        if (2 * j <= n_blk) step(F{}, I3{}, I1{}, 2 * j, sa, sb, pb, pa);
        if (2 * j + 1 <= n_blk) step(F{}, I0{}, I2{}, 2 * j + 1, sb, sa, pa, pb);
        wait_dma();
        __syncthreads();
        if (j + 1 >= n_tiles) break;
        // even tile: blocks 2j+2 = 0 (mod 4), 2j+3 = 1 (mod 4)
        refill_even(j + 1);
        if (2 * j + 2 <= n_blk) step(F{}, I1{}, I3{}, 2 * j + 2, sa, sb, pb, pa);
        if (2 * j + 3 <= n_blk) step(F{}, I2{}, I0{}, 2 * j + 3, sb, sa, pa, pb);
        wait_dma();
        __syncthreads();
    }

    // ---- exact kernel: the saved masked blocks' terms p * v, for the keys each
    // row sees, in fp32 (V from global memory; the wave's own LDS area holds
    // the weights and the factors they have been rescaled by since).  Output
    // element (db, r) of a lane is head dim 32 db + 8 (r / 4) + 4 hh + r % 4.
    if constexpr (SAFE) {
        const char* base = lds + SAVE_OFF + wave * SAVE_WAVE_BYTES;
        const int end = VARLEN ? s1 : N;
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase, (uint32_t)(end - kb0) * ROW_BYTES);
        for (int i = 0; i < n_saved; ++i) {
            const int gb = __builtin_amdgcn_readfirstlane(((const int*)(base + MAX_SAVED * (SAVE_P + 256)))[i]);
            const float fac = ((const float*)(base + MAX_SAVED * SAVE_P))[i * 64 + lane];
            const char* wp = base + i * SAVE_P + l32 * (KB * 2);
            const int kbase_g = SPARSE ? sp_key(gb) : kb0 + gb * KB;
            const bool listed = SPARSE ? sp_member(gb) : true;
#pragma unroll 1
            for (int j = 0; j < KB; ++j) {
                const int key = kbase_g + j;
                if (key_bad(key, listed)) continue;
                const float pj = (float)*(const __bf16*)(wp + 2 * j) * fac;
                const uint32_t row_off = (uint32_t)(key - kb0) * ROW_BYTES;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t off = row_off + 2u * (uint32_t)(32 * db + 8 * q + 4 * hh);
                        const bf16x4 v4 = __builtin_bit_cast(
                            bf16x4, __builtin_amdgcn_raw_buffer_load_b64(vr, off, 0, 0));
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            o[db][4 * q + rr] = fmaf(pj, (float)v4[rr], o[db][4 * q + rr]);
                    }
            }
        }
    }

    // ---- epilogue: O = O^T / sum bf16(p) (bf16, round to nearest even),
    // LSE = m*scale + ln(sum p).  Dividing by the sum of the weights the MFMA
    // actually applied makes the rounding of a dominant weight cancel.
    const float l_tot = wave_swap_sum(l);
    const float lb_tot = wave_swap_sum(lb);
    // SPARSE: a row that sees no key (its lists hold none of its keys) gets
    // O = 0 and LSE = -inf.  A row that sees keys whose scores are all -inf
    // gets NaN, as the formula gives (m = -inf, exp(-inf - m) = NaN).
    // The union list is in key order, so a row sees a key exactly when the
    // list is not empty and, causal, its first key block starts at or before
    // the row (every listed block holds a key below N).
    bool empty = false;
    if constexpr (SPARSE) empty = n_blk_wg == 0 || (CAUSAL && sp_key(0) > myq);
    const float inv = empty ? 0.f : 1.0f / lb_tot;
    // O leaves through LDS.  A lane holds its row's values in 8-byte pieces of
    // 4 head dims, so direct stores would touch 32 rows per instruction; staged
    // row-major in the wave's 8 KiB of the K/V rings (16-byte chunk c of row r
    // at chunk c ^ (r mod 16), so the 16 rows a write phase touches fall in
    // distinct banks), they leave as 4 whole rows (1 KiB) per store.  The
    // rings are free once every wave's copies, including the drain step's
    // past-the-end ones, have landed and no wave reads them.
    wait_dma();
    __syncthreads();
    char* const stage = lds + K_RING + wave * (32 * ROW_BYTES);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(o[db][4 * r4 + i] * inv);
            const int ch = 4 * db + r4;   // head dims 8*ch .. 8*ch+7; this lane's half at 4*hh
            *(bf16x4*)(stage + l32 * ROW_BYTES + ((ch ^ (l32 & 15)) << 4) + 8 * hh) = ov;
        }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int r = 4 * t + (lane >> 4), ch = lane & 15;
        const u32x4 x = *(const u32x4*)(stage + r * ROW_BYTES + ((ch ^ (r & 15)) << 4));
        if (wq0 + r < s1) *(u32x4*)(p.o + qo_panel + (size_t)(wq0 + r) * HD + 8 * ch) = x;
    }
    if (myq < s1) {
        if (p.lse != nullptr && hh == 0) {
            const size_t li = ((size_t)pbat * p.Hq + h) * (size_t)N + myq;
            p.lse[li] = empty ? -INFINITY : m == -INFINITY ? __builtin_nanf("") : m * p.lse_scale + logf(l_tot);
        }
    }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
void set_scale(Params& p, float scale) {
    const float mag = std::fabs(scale);
    p.q_mode = scale > 0.f ? 0 : (scale < 0.f ? 1 : 2);
    p.c = (float)((double)(mag > 0.f ? mag : 1.0f) * 1.4426950408889634);
    p.lse_scale = mag;
}

// SAFE = false: the fast kernel, one workgroup per tile.  SAFE = true: the
// exact kernel on a small grid (at most EXACT_GRID workgroups): each thread
// checks one tile's mark, and each workgroup redoes its marked tiles one after
// another (most launches mark none, so most workgroups only read marks).
constexpr int EXACT_GRID = 256;
template <bool CAUSAL, bool VARLEN, bool SPARSE, int NW, bool SAFE>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(Params p) {
    if constexpr (!SAFE) {
        fwd_tile<CAUSAL, VARLEN, SPARSE, NW, false>(p, blockIdx.x);
    } else {
        constexpr int NTH = NW * 64;
        __shared__ int marked[NTH];
        __shared__ int n_marked;
        const int t = threadIdx.x;
        if (t == 0) n_marked = 0;
        __syncthreads();
        const int bid = blockIdx.x + t * gridDim.x;   // gridDim.x * NTH >= p.total
        int b, h, qt, s0, s1;
        if (bid < p.total && tile_of<CAUSAL, VARLEN, SPARSE, NW>(p, bid, b, h, qt, s0, s1)) {
            const size_t qo_panel = ((size_t)(VARLEN ? 0 : b) * p.Hq + h) * (size_t)p.N * HD;
            const u32x4 w = *(const u32x4*)(p.o + qo_panel + (size_t)(s0 + qt * 32 * NW) * HD);
            if (w[0] == NF_MARK[0] && w[1] == NF_MARK[1] && w[2] == NF_MARK[2] && w[3] == NF_MARK[3])
                marked[atomicAdd(&n_marked, 1)] = bid;
        }
        __syncthreads();
        const int n = n_marked;
        for (int i = 0; i < n; ++i) {
            fwd_tile<CAUSAL, VARLEN, SPARSE, NW, true>(p, __builtin_amdgcn_readfirstlane(marked[i]));
            // the next tile reuses the LDS: copies still in flight (the pipeline
            // issues some past a tile's last block) land first
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }
}

template <bool VARLEN, bool SPARSE, int NW = NWAVE>
attn_status launch_fwd(const Params& p, bool causal, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    // the fast kernel, then the exact kernel over the same grid: it redoes the
    // workgroups the fast kernel marked (a NaN or infinity in the V rows of a
    // masked block) and every other workgroup of it exits at once
    const dim3 grid((unsigned)p.total), block(NW * 64);
    const dim3 egrid((unsigned)std::max(std::min(p.total, EXACT_GRID), (p.total + NW * 64 - 1) / (NW * 64)));
    if (causal) {
        hipLaunchKernelGGL((attn_fwd_kernel<true, VARLEN, SPARSE, NW, false>), grid, block, 0, s, p);
        hipLaunchKernelGGL((attn_fwd_kernel<true, VARLEN, SPARSE, NW, true>), egrid, block, 0, s, p);
    } else {
        hipLaunchKernelGGL((attn_fwd_kernel<false, VARLEN, SPARSE, NW, false>), grid, block, 0, s, p);
        hipLaunchKernelGGL((attn_fwd_kernel<false, VARLEN, SPARSE, NW, true>), egrid, block, 0, s, p);
    }
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H_q, int H_kv, int N, int D, int causal, float scale,
                                void* stream) {
    if (!q || !k || !v || !o) return ATTN_ERR_NULL;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0) return ATTN_ERR_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_GQA;
    if (D != HD) return ATTN_ERR_HEAD_DIM;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    // one head panel is addressed with 32-bit byte offsets
    if ((int64_t)N * ROW_BYTES >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    // measured (same-process sweeps, 256-20480 tokens, 1-128 heads): 8-wave
    // workgroups win once their grid fills the chip, a causal tile counting as
    // half a tile (it sees half the keys on average), for sequences of at
    // least 1024 tokens; 4-wave workgroups (two per CU) win on smaller grids
    // and shorter sequences
    const int64_t tiles8 = (int64_t)B * H_q * (((int64_t)N + BR - 1) / BR);
    const bool short_n = N < MIN_N_8W || tiles8 < (causal ? 2 : 1) * (int64_t)N_CU;
    const int br = short_n ? BR / 2 : BR;
    const int64_t n_qtiles = ((int64_t)N + br - 1) / br;
    const int64_t total = (int64_t)B * H_q * n_qtiles;
    if (total > INT32_MAX || (int64_t)B * H_q > INT32_MAX) return ATTN_ERR_SHAPE;
    const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15;
    if (mis != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_ALIGN;
    const size_t qo_bytes = (size_t)B * H_q * N * HD * 2;
    const size_t kv_bytes = (size_t)B * H_kv * N * HD * 2;
    const size_t lse_bytes = (size_t)B * H_q * N * 4;
    if (ranges_overlap(o, qo_bytes, q, qo_bytes) || ranges_overlap(o, qo_bytes, k, kv_bytes) ||
        ranges_overlap(o, qo_bytes, v, kv_bytes))
        return ATTN_ERR_ALIAS;
    if (lse && (ranges_overlap(lse, lse_bytes, q, qo_bytes) || ranges_overlap(lse, lse_bytes, k, kv_bytes) ||
                ranges_overlap(lse, lse_bytes, v, kv_bytes) || ranges_overlap(lse, lse_bytes, o, qo_bytes)))
        return ATTN_ERR_ALIAS;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev)) return ATTN_ERR_DEVICE;

    Params p = {};
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (uint16_t*)o;
    p.lse = lse;
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.N = N;
    p.group = H_q / H_kv;
    p.n_qtiles = (int)n_qtiles;
    p.total = (int)total;
    // causal: interleave the tiles of enough heads to fill one XCD's workgroup
    // slots (32 CUs x 2 four-wave or 1 eight-wave workgroups)
    const int64_t slots = short_n ? 64 : 32;
    p.cgroup = (int)std::min<int64_t>((int64_t)B * H_q, (slots + n_qtiles - 1) / n_qtiles);
    int64_t grid = 0;
    int64_t dg = p.cgroup;
    if (causal && causal_deal((int64_t)B * H_q, dg, n_qtiles, slots, p.deal, grid) && grid <= INT32_MAX) {
        p.dealt = 1;
        p.cgroup = (int)dg;
        p.total = (int)grid;
    }
    set_scale(p, scale);
    return short_n ? launch_fwd<false, false, NWAVE / 2>(p, causal != 0, stream)
                   : launch_fwd<false, false, NWAVE>(p, causal != 0, stream);
}

extern "C" attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const int* cu_seqlens, int n_seq,
                                       int max_seqlen, int total, int H_q, int H_kv, int D,
                                       int causal, int window_left, int window_right, float scale,
                                       void* stream) {
    if (!q || !k || !v || !o || !cu_seqlens) return ATTN_ERR_NULL;
    if (n_seq <= 0 || max_seqlen <= 0 || total <= 0 || H_q <= 0 || H_kv <= 0 || D <= 0)
        return ATTN_ERR_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_GQA;
    if (D != HD) return ATTN_ERR_HEAD_DIM;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if ((int64_t)total * ROW_BYTES >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    // 8-wave workgroups (256-row tiles) by the dense rule: when the mean
    // sequence holds at least MIN_N_8W tokens and the batch's 256-row tiles
    // fill the chip (a causal tile counting as half), unless a window
    // narrower than 8192 keys bounds the rows (a windowed tile's masked edge
    // blocks grow with its rows).  4-wave ones otherwise: twice the
    // workgroups balance short and windowed tiles better.  Measured (same
    // process, bitwise equal): causal mix of 8 sequences +3.1%, 8 equal causal
    // sequences +2.9%, 4096-key causal window +0.1%, 2049-key window -9%.
    const bool windowed = window_left >= 0 || (!causal && window_right >= 0);
    const int64_t width = (window_left < 0 ? (int64_t)max_seqlen : window_left) +
                          (causal ? 0 : (window_right < 0 ? (int64_t)max_seqlen : window_right)) + 1;
    const int64_t tiles8 = (int64_t)H_q * (((int64_t)total + BR - 1) / BR);
    const bool eight = !(windowed && width < 8192) && (int64_t)total >= (int64_t)MIN_N_8W * n_seq &&
                       tiles8 >= (causal ? 2 : 1) * (int64_t)N_CU;
    const int br = eight ? BR : BR / 2;
    const int64_t slots = eight ? 32 : 64;   // an XCD's workgroup slots: 32 CUs x 1 or 2
    const int64_t n_qtiles = ((int64_t)max_seqlen + br - 1) / br;
    // Sequences of nearly equal length (the longest within 1.25x the mean)
    // take the dense order: a few heads at a time, whose K/V stays in one
    // XCD's L2 (grouped as for dense causal grids).  Unequal lengths are dealt
    // to the XCDs in turn (dealt_tile): with 32 groups of (sequence, head)
    // pairs or more, whole groups, one after another on each XCD, which
    // balances them on average; with fewer, 8 slices of every group, one per
    // XCD and run row by row, so each XCD gets an eighth of every group's work
    // whatever the lengths (whole groups would leave XCDs idle, or give one XCD
    // a long sequence's every tile).
    const bool unequal = n_seq > 1 && (int64_t)max_seqlen * n_seq * 4 > (int64_t)total * 5;
    const int64_t pairs = (int64_t)n_seq * H_q;
    const int64_t cgroup = std::min<int64_t>(pairs, (slots + n_qtiles - 1) / n_qtiles);
    const int64_t n_groups = (pairs + cgroup - 1) / cgroup;
    int64_t grid = pairs * n_qtiles;
    Deal deal{};
    int64_t dg = cgroup;
    bool dealt = unequal;
    if (unequal) {
        deal = n_groups < 32 ? make_deal(pairs, cgroup, n_qtiles, 8, true, grid)
                             : make_deal(pairs, cgroup, n_qtiles, 1, false, grid);
    } else if (causal) {
        // nearly equal lengths, causal: the dense causal rule
        int64_t g = 0;
        if (causal_deal(pairs, dg, n_qtiles, slots, deal, g) && g <= INT32_MAX) {
            dealt = true;
            grid = g;
        }
    }
    if (grid > INT32_MAX || n_seq == INT32_MAX) return ATTN_ERR_SHAPE;
    const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15;
    if (mis != 0 || (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) != 0) return ATTN_ERR_ALIGN;
    const size_t qo_bytes = (size_t)H_q * total * HD * 2;
    const size_t kv_bytes = (size_t)H_kv * total * HD * 2;
    const size_t lse_bytes = lse ? (size_t)H_q * total * 4 : 0;
    const size_t cu_bytes = (size_t)(n_seq + 1) * 4;
    const void* ins[4] = {q, k, v, cu_seqlens};
    const size_t in_bytes[4] = {qo_bytes, kv_bytes, kv_bytes, cu_bytes};
    for (int i = 0; i < 4; ++i)
        if (ranges_overlap(o, qo_bytes, ins[i], in_bytes[i]) || (lse && ranges_overlap(lse, lse_bytes, ins[i], in_bytes[i])))
            return ATTN_ERR_ALIAS;
    if (lse && ranges_overlap(lse, lse_bytes, o, qo_bytes)) return ATTN_ERR_ALIAS;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev)) return ATTN_ERR_DEVICE;

    Params p = {};
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (uint16_t*)o;
    p.lse = lse;
    p.B = n_seq;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.N = total;
    p.group = H_q / H_kv;
    p.n_qtiles = (int)n_qtiles;
    p.total = (int)grid;
    p.cu = cu_seqlens;
    p.n_seq = n_seq;
    p.dealt = dealt;
    p.deal = deal;
    p.cgroup = (int)dg;
    p.left = window_left < 0 ? -1 : window_left;
    p.right = window_right < 0 ? -1 : window_right;
    set_scale(p, scale);
    return eight ? launch_fwd<true, false, NWAVE>(p, causal != 0, stream)
                 : launch_fwd<true, false, NWAVE / 2>(p, causal != 0, stream);
}

extern "C" attn_status attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o,
                                            float* lse, const int* kb_ptr, const int* kb_idx,
                                            int nnz, int mask_heads, int B, int H_q, int H_kv,
                                            int N, int D, int causal, float scale, void* stream) {
    if (!q || !k || !v || !o || !kb_ptr || (nnz > 0 && !kb_idx)) return ATTN_ERR_NULL;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || N <= 0 || D <= 0 || nnz < 0) return ATTN_ERR_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_GQA;
    if (mask_heads != 1 && mask_heads != H_q) return ATTN_ERR_SHAPE;
    if (D != HD) return ATTN_ERR_HEAD_DIM;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if ((int64_t)N * ROW_BYTES >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    const int64_t n_sblk = ((int64_t)N + SP_BLOCK - 1) / SP_BLOCK;
    if (n_sblk > SP_MAX) return ATTN_ERR_SHAPE;
    // 4-wave workgroups of 128 rows: each is one query block with one list, so
    // no workgroup streams key blocks that only some of its waves need
    const int br = BR / 2;
    const int64_t n_qtiles = ((int64_t)N + br - 1) / br;
    const int64_t total = (int64_t)B * H_q * n_qtiles;
    if (total > INT32_MAX || (int64_t)B * H_q > INT32_MAX) return ATTN_ERR_SHAPE;
    const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15;
    if (mis != 0 || (((uintptr_t)lse | (uintptr_t)kb_ptr | (uintptr_t)kb_idx) & 3) != 0)
        return ATTN_ERR_ALIGN;
    const size_t qo_bytes = (size_t)B * H_q * N * HD * 2;
    const size_t kv_bytes = (size_t)B * H_kv * N * HD * 2;
    const size_t lse_bytes = lse ? (size_t)B * H_q * N * 4 : 0;
    const size_t ptr_bytes = (size_t)(mask_heads * n_sblk + 1) * 4;
    const size_t idx_bytes = (size_t)nnz * 4;
    const void* ins[5] = {q, k, v, kb_ptr, kb_idx};
    const size_t in_bytes[5] = {qo_bytes, kv_bytes, kv_bytes, ptr_bytes, idx_bytes};
    for (int i = 0; i < 5; ++i)
        if (ins[i] && in_bytes[i] &&
            (ranges_overlap(o, qo_bytes, ins[i], in_bytes[i]) ||
             (lse && ranges_overlap(lse, lse_bytes, ins[i], in_bytes[i]))))
            return ATTN_ERR_ALIAS;
    if (lse && ranges_overlap(lse, lse_bytes, o, qo_bytes)) return ATTN_ERR_ALIAS;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev)) return ATTN_ERR_DEVICE;

    Params p = {};
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (uint16_t*)o;
    p.lse = lse;
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.N = N;
    p.group = H_q / H_kv;
    p.n_qtiles = (int)n_qtiles;
    p.total = (int)total;
    p.kb_ptr = kb_ptr;
    p.kb_idx = kb_idx;
    p.nnz = nnz;
    p.mask_heads = mask_heads;
    p.n_sblk = (int)n_sblk;
    set_scale(p, scale);
    return launch_fwd<false, true, NWAVE / 2>(p, causal != 0, stream);
}

extern "C" double attn_fwd_flops(int B, int H_q, int N, int D, int causal) {
    const double f = 4.0 * B * H_q * (double)N * (double)N * D;
    return causal ? 0.5 * f : f;
}
