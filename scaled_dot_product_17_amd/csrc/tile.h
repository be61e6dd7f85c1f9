// LDS layout and MFMA operand reads of 32-row bf16 tiles (rows of 128 head
// dims, 256 bytes) on gfx950, shared by kernels that stage K, V, Q or dO rows
// through LDS and feed v_mfma_f32_32x32x16_bf16.
#pragma once

#include "cdna4.h"

namespace tile {

using cdna4::bf16x2;
using cdna4::bf16x4;
using cdna4::bf16x8;

constexpr int HD = 128;                    // head dimension
constexpr int ROW_BYTES = HD * 2;          // 256 B per bf16 row
constexpr int KB = 32;                     // rows per MFMA block
constexpr int BLK_BYTES = KB * ROW_BYTES;  // 8 KiB

// 16-byte chunk c of row r sits at chunk position c ^ swz(r).  A row-wise MFMA
// operand read (16 rows, one chunk) hits 16 distinct positions; a transposing
// read (4 rows x 4 chunks) puts each row in its own 64-byte bank group.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ uint32_t off(int row, int chunk) {
    return (uint32_t)(row * ROW_BYTES + ((chunk ^ swz(row)) << 4));
}
// Global byte offset (within a 4-row group starting at row0) that lane must
// fetch so that an LDS DMA of 16 bytes per lane, in lane order, lands in the
// swizzled layout.
__device__ __forceinline__ uint32_t dma_src(int row0, int lane) {
    const int row = row0 + (lane >> 4);
    return (uint32_t)(row * ROW_BYTES + (((lane & 15) ^ swz(row)) << 4));
}

// Per-lane offsets of the two operand read patterns of a 32-row block.
//   row(ks): A operand with rows = MFMA m, 8 consecutive head dims of k step ks.
//   tr(db, kk): A operand with head dims 32db.. = MFMA m and rows 16kk.. = MFMA k
//   in the order an fp32 accumulator holds them (rows 8(r/4) + 4(lane/32) + r%4
//   of register r), so an accumulator turned into bf16 pairs is the matching B
//   operand.  Rows 16..31 add 16 * ROW_BYTES (the swizzle repeats every 16 rows).
struct Reads {
    uint32_t rd_row[8];
    uint32_t tr_lo[4], tr_hi[4];
    __device__ __forceinline__ void init(int lane) {
        const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) rd_row[ks] = off(l32, 2 * ks + hh);
        const int g = lane >> 4;          // 16-lane group
        const int rs = (lane & 15) >> 2;  // row within the 4-row group
        const int cs = lane & 3;          // 4-element column group
        const int row = 4 * (g >> 1) + rs;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int col = 32 * db + 16 * (g & 1) + 4 * cs;
            const uint32_t half = (col & 4) ? 8u : 0u;
            tr_lo[db] = off(row, col >> 3) + half;
            tr_hi[db] = off(row + 8, col >> 3) + half;
        }
    }
    __device__ __forceinline__ bf16x8 tr(const char* lds, uint32_t base, int db, int kk) const {
        const bf16x4 lo = cdna4::lds_read_tr(lds, base + tr_lo[db] + (uint32_t)(16 * kk * ROW_BYTES));
        const bf16x4 hi = cdna4::lds_read_tr(lds, base + tr_hi[db] + (uint32_t)(16 * kk * ROW_BYTES));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ __forceinline__ bf16x8 row(const char* lds, uint32_t base, int ks) const {
        return *(const bf16x8*)(lds + base + rd_row[ks]);
    }
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace tile
