// Small gfx950 (CDNA4) device and host helpers shared by the kernels:
// vector types, buffer descriptors, LDS DMA, the transposing LDS read, cross-
// half wave reductions, the XCD-aware workgroup order and argument checks.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <numeric>

namespace cdna4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t RSRC_DWORD3 = 0x00020000u;  // raw buffer, 32-bit dwords (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)RSRC_DWORD3);
}

// 16-byte buffer load into VGPRs; offsets at or beyond the range return zeros.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Raw buffer descriptor in SGPRs for inline assembly.
__device__ __forceinline__ u32x4 sgpr_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), RSRC_DWORD3};
}

// LDS DMA: the buffer unit copies rsrc[voff .. voff+15] (or +3) of every lane
// to LDS byte lds_addr + 16*lane (or 4*lane) without passing through VGPRs.
// Lanes whose offset is out of range copy nothing.  Inline assembly, so the
// compiler does not order later LDS reads behind it; the caller waits for
// completion (vmcnt) before the workgroup barrier that publishes the data.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(u32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
}
// LDS DMA of 16 bytes per lane from a fixed descriptor: the buffer unit copies
// rsrc[soff + voff .. +15] of every lane to LDS byte lds_sbase + IMM + 16*lane.
// soff (an SGPR) carries the block offset, so one descriptor serves every
// block of a panel; IMM is a compile-time LDS offset, so m0 is one scalar add.
template <uint32_t IMM>
__device__ __forceinline__ void lds_dma16_at(u32x4 rsrc, uint32_t lds_sbase, uint32_t voff,
                                             uint32_t soff) {
    asm volatile("s_add_u32 m0, %2, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_sbase), "s"(soff), "i"(IMM)
                 : "memory", "m0", "scc");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ds_read_b64_tr_b16: each 16-lane group reads a 4 x 16 block of bf16 and
// every lane receives one column of it (4 values), so a row-major tile is
// read as the column-major MFMA operand.
__device__ __forceinline__ bf16x4 lds_read_tr(const char* lds, uint32_t off) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + off));
    return __builtin_bit_cast(bf16x4, r);
}

// Row max and row sum of an S^T accumulator: lane L and lane L ^ 32 hold the
// two halves of one query column's values; permlane32 swaps the halves.
__device__ __forceinline__ float wave_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                              false, false);
    return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float wave_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                              false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Maps the hardware workgroup id to a logical id so that consecutive logical
// ids land on the same XCD (the dispatcher deals workgroups to the 8 XCDs
// round-robin): tiles of one head then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int nx = 8;
    const int q = total / nx, r = total % nx;
    const int x = bid % nx, s = bid / nx;
    const int start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    return start + s;
}

// Dealt grid order.  The query tiles of `per` heads (or (sequence, head)
// pairs) form groups of G heads, each group's G * n tiles listed heaviest
// first (tile-major: every head's last tile, then every head's second-to-last,
// ...).  Each group is cut into S slices: slice s takes the list positions
// S*j + s for even j and S*j + S-1-s for odd j, so the slices of a group carry
// equal work.  Slices (group-major) are dealt to the 8 XCDs in turn (the
// dispatcher sends workgroup i to XCD i mod 8), U slices to each XCD, len
// positions per slice.  An XCD runs its slices one after another (inter = 0),
// or row by row, the heaviest positions of all its slices first (inter = 1).
struct Deal {
    int S, U, len, inter;
};
// false: bid is padding of the grid.  (Host-callable too, for checks of the
// order on the CPU.)
__host__ __device__ __forceinline__ bool dealt_tile(int bid, int per, int G, int n, const Deal& d, int& bh,
                                                    int& qt) {
    const int x = bid & 7, sx = bid >> 3;
    int k, j;
    if (d.inter) {
        k = sx % d.U;
        j = sx / d.U;
    } else {
        k = sx / d.len;
        j = sx - k * d.len;
    }
    const int u = x + 8 * k;
    const int grp = u / d.S, s = u - grp * d.S;
    const int gh = G < per - grp * G ? G : per - grp * G;   // heads in this group (the last may be short)
    const int r = d.S * j + ((j & 1) ? d.S - 1 - s : s);
    if (gh <= 0 || r >= gh * n) return false;
    qt = n - 1 - r / gh;
    bh = grp * G + r % gh;
    return true;
}

// ---- host side
// The dealt order's sizes for per heads in groups of G with n tiles each, S
// slices per group; the grid is 8 * U * len workgroups.
inline Deal make_deal(int64_t per, int64_t G, int64_t n, int S, bool inter, int64_t& grid) {
    const int64_t n_groups = (per + G - 1) / G;
    const int64_t U = (n_groups * S + 7) / 8;
    const int64_t len = (G * n + S - 1) / S;
    grid = 8 * U * len;
    return Deal{S, (int)std::min<int64_t>(U, INT32_MAX), (int)std::min<int64_t>(len, INT32_MAX), inter ? 1 : 0};
}

// Causal dense grids.  The plain order hands each XCD a contiguous eighth of
// the groups' heaviest-first lists, which balances the XCDs only when whole,
// equal groups split evenly over them: with 1, 2 or 4 groups the first XCDs get
// the heavy tiles of a group and the others its light ones (a simulated
// makespan of 1.5-1.9x the ideal for one to four long heads), and a short last
// group shifts every boundary.  So unless the groups are full and a multiple
// of 8, or at least 32 (then the plain order is balanced to a few percent),
// the grid is dealt instead, in groups of G' heads, G' the largest divisor of
// per not above G (so every group is full): S = 8 / gcd(groups, 8) slices per
// group make the slice count a multiple of 8, and an XCD with at most 16
// slices runs them row by row (at most 16 heads in flight on it, so K/V is
// still shared in its L2); with more, one after another when a slice holds at
// least an XCD's workgroup slots.  false: keep the plain order.  true: G is
// set to G'.
inline bool causal_deal(int64_t per, int64_t& G, int64_t n, int64_t slots, Deal& d, int64_t& grid) {
    const int64_t ng = (per + G - 1) / G;
    if ((per % G == 0 && ng % 8 == 0) || ng >= 32) return false;
    int64_t g = G;
    while (per % g != 0) --g;
    const int64_t ngd = per / g;
    const int S = 8 / (int)std::gcd(ngd, (int64_t)8);
    const int64_t U = ngd * S / 8;
    if (U <= 16) {
        d = make_deal(per, g, n, S, true, grid);
    } else if (g * n / S >= slots) {
        d = make_deal(per, g, n, S, false, grid);
    } else {
        return false;
    }
    G = g;
    return true;
}

inline bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na != 0 && nb != 0 && x < y + nb && y < x + na;
}

// Per-process cache of "is device d a gfx950".
inline bool device_is_gfx950(int dev) {
    constexpr int MAX_DEVICES = 64;
    static std::atomic<int> cache[MAX_DEVICES];   // 0 unknown, 1 gfx950, 2 other
    if (dev < 0 || dev >= MAX_DEVICES) return false;
    int s = cache[dev].load(std::memory_order_relaxed);
    if (s == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        s = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        cache[dev].store(s, std::memory_order_relaxed);
    }
    return s == 1;
}

}  // namespace cdna4
