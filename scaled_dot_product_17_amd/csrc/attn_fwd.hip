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
//     into the softmax, double-buffered tile staging: page
//     "AVO算法优化Transformer注意力机制性能解析", sections 2.2, 3.1, 3.2, 5.1.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head):
//   * each wave owns 32 query rows; its Q rows live in VGPRs as the B operand
//     of v_mfma_f32_32x32x16_bf16 for the whole kernel;
//   * key tiles of 64 rows of K and V are staged HBM -> VGPR -> LDS, double
//     buffered, one barrier per tile;
//   * scores are computed transposed, S^T = K Q^T, so each lane owns one query
//     column: the row max and row sum are in-lane reductions plus one
//     permlane32 swap, and the output rescale is a per-lane scalar;
//   * the fp32 S^T accumulator, converted to bf16, is directly the B operand of
//     O^T += V^T P^T.  The MFMA's k index then visits keys in the order the
//     accumulator holds them; V^T fragments are read in the same key order with
//     the gfx950 transposing LDS read (ds_read_b64_tr_b16), so V never needs a
//     transposed copy;
//   * softmax in base 2: p = exp2(s * scale*log2(e) - m * scale*log2(e)).  The
//     running max is exact (O and l are rescaled whenever any row's max grows);
//     a wave skips the rescale when no row's max grew.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;                    // head dimension handled by this kernel
constexpr int BR = 128;                    // query rows per workgroup
constexpr int BC = 64;                     // keys per tile
constexpr int NWAVE = 4;                   // waves per workgroup
constexpr int NTHREAD = NWAVE * 64;
constexpr int ROW_BYTES = HD * 2;          // 256 B per K/V/Q/O row
constexpr int TILE_BYTES = BC * ROW_BYTES; // 16 KiB per K or V tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES; // two stages of K and V: 64 KiB
constexpr uint32_t RSRC_DWORD3 = 0x00020000u;  // raw buffer, 32-bit dwords (gfx9 family)

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
    float c;          // |scale| * log2(e), always > 0
    float lse_scale;  // |scale|
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)RSRC_DWORD3);
}

// 16-byte buffer load; offsets at or beyond the range return zeros.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS byte address of the 16-byte chunk (row, chunk) of a K tile.  The chunk
// index is XOR-swizzled with the low 4 row bits so the 32 rows one MFMA A
// operand touches (same logical chunk) fall in distinct banks.
__device__ __forceinline__ uint32_t k_lds_off(int row, int chunk) {
    return (uint32_t)(row * ROW_BYTES + ((chunk ^ (row & 15)) << 4));
}
// LDS byte address of the 16-byte chunk (row, chunk) of a V tile.  The chunk
// index is XOR-swizzled with 4*(row mod 4): a transposing read touches 4
// consecutive rows x 64 contiguous bytes per half-wave, and this spreads the
// four rows over the four 64-byte bank groups.
__device__ __forceinline__ uint32_t v_lds_off(int row, int chunk) {
    return (uint32_t)(row * ROW_BYTES + ((chunk ^ ((row & 3) << 2)) << 4));
}

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

__device__ __forceinline__ bf16x4 lds_read_tr(const char* lds, uint32_t off) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + off));
    return __builtin_bit_cast(bf16x4, r);
}

// Maps the hardware workgroup id to a logical id so that consecutive logical
// ids land on the same XCD (the dispatcher deals workgroups to the 8 XCDs
// round-robin).  Tiles of one head then share that XCD's L2 for K/V.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int nx = 8;
    const int q = total / nx, r = total % nx;
    const int x = bid % nx, s = bid / nx;
    const int start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    return start + s;
}

template <bool CAUSAL>
__global__ __launch_bounds__(NTHREAD, 2) void attn_fwd_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;   // query column owned by this lane
    const int hh = lane >> 5;    // which half of the wave

    // ---- which (batch, head, query tile) this workgroup computes
    const int logical = xcd_remap(blockIdx.x, p.total);
    const int bh = logical / p.n_qtiles;
    int qt = logical % p.n_qtiles;
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;   // heaviest tiles of a head first
    const int b = bh / p.Hq;
    const int h = bh % p.Hq;
    const int kvh = h / p.group;
    const int N = p.N;
    const int q0 = qt * BR;
    const int wq0 = q0 + wave * 32;       // first query row of this wave
    const int myq = wq0 + l32;            // query row of this lane

    const uint32_t panel_bytes = (uint32_t)N * ROW_BYTES;
    const size_t qo_panel = ((size_t)b * p.Hq + h) * (size_t)N * HD;
    const size_t kv_panel = ((size_t)b * p.Hkv + kvh) * (size_t)N * HD;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.q + qo_panel, panel_bytes);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(p.k + kv_panel, panel_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(p.v + kv_panel, panel_bytes);

    // ---- Q fragments: B operand of S^T = K Q^T, k-steps of 16 head dims
    bf16x8 qf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(qr, (uint32_t)myq * ROW_BYTES + (16 * ks + 8 * hh) * 2));
    // A negative scale is applied as |scale| on -Q (a sign flip is exact in
    // bf16) and a zero scale as zero scores, so the exp2 argument below always
    // multiplies by a positive constant and masked -inf scores stay -inf.
    if (p.q_mode != 0) {
        const u32x4 flip = p.q_mode == 1 ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}
                                         : u32x4{0u, 0u, 0u, 0u};
        const u32x4 keep = p.q_mode == 1 ? u32x4{~0u, ~0u, ~0u, ~0u} : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, (__builtin_bit_cast(u32x4, qf[ks]) & keep) ^ flip);
    }

    // ---- number of key tiles this workgroup visits
    const int n_ktiles_all = (N + BC - 1) / BC;
    int n_kt = n_ktiles_all;
    if (CAUSAL) {
        const int last_q = min(q0 + BR, N) - 1;
        n_kt = min(n_ktiles_all, last_q / BC + 1);
    }

    // ---- per-thread staging coordinates: 4 rows x one 16-byte chunk of each tile
    const int st_row = tid >> 4;   // 0..15, plus 16*it
    const int st_chunk = tid & 15;
    uint32_t k_st_off[4], v_st_off[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        k_st_off[it] = k_lds_off(st_row + 16 * it, st_chunk);
        v_st_off[it] = TILE_BYTES + v_lds_off(st_row + 16 * it, st_chunk);
    }

    // ---- per-lane LDS read addresses (stage 0; stage 1 adds STAGE_BYTES)
    uint32_t k_rd[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) k_rd[ks] = k_lds_off(l32, 2 * ks + hh);
    uint32_t v_rd[4];
    {
        const int g = lane >> 4;        // 16-lane group
        const int rs = (lane & 15) >> 2;  // source row within the 4-row block
        const int cs = lane & 3;          // source 4-element column block
        const int row = 4 * (g >> 1) + rs;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int col = 32 * db + 16 * (g & 1) + 4 * cs;  // element column
            v_rd[db] = TILE_BYTES + v_lds_off(row, col >> 3) + ((col & 4) ? 8 : 0);
        }
    }

    u32x4 kst[4], vst[4];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const uint32_t goff = (uint32_t)(j * BC + st_row + 16 * it) * ROW_BYTES + st_chunk * 16;
            kst[it] = buf_load16(kr, goff);
            vst[it] = buf_load16(vr, goff);
        }
    };
    auto store_tile = [&](int stage) {
        char* base = lds + stage * STAGE_BYTES;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            *(u32x4*)(base + k_st_off[it]) = kst[it];
            *(u32x4*)(base + v_st_off[it]) = vst[it];
        }
    };

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;   // running max of raw scores (exact)
    float l_run = 0.f;         // this lane's partial row sum
    const float c = p.c;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < n_kt; ++j) {
        const int stage = j & 1;
        if (j + 1 < n_kt) load_tile(j + 1);
        const char* sb = lds + stage * STAGE_BYTES;
        const int key0 = j * BC;
        // causal: a tile whose first key is past this wave's last query is skipped
        const bool active = !CAUSAL || key0 <= wq0 + 31;
        if (active) {
            // ---- S^T = K Q^T for keys key0..key0+63 (two 32-key blocks)
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const bf16x8 a = *(const bf16x8*)(sb + k_rd[ks] + kb * 32 * ROW_BYTES);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kb], 0, 0, 0);
                }
            }
            // ---- mask: key > query (causal) or key >= N (ragged tail)
            const bool need_mask = (CAUSAL && key0 + BC - 1 > wq0) || (key0 + BC > N);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                        const bool bad = (key >= N) || (CAUSAL && key > myq);
                        sacc[kb][r] = bad ? -INFINITY : sacc[kb][r];
                    }
            }
            // ---- online softmax
            float mx = sacc[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
            mx = wave_swap_max(mx);
            const float m_new = fmaxf(m_run, mx);
            const bool grew = m_new > m_run;
            if (__builtin_amdgcn_ballot_w64(grew)) {
                const float alpha = grew ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                m_run = m_new;
            }
            const float mb = (m_run == -INFINITY) ? 0.f : m_run * c;
            bf16x8 pf[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * kk + i], c, -mb));
                        l_run += e;
                        pf[kb][kk][i] = (__bf16)e;
                    }
            // ---- O^T += V^T P^T; the MFMA k index walks keys in accumulator order
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const uint32_t rowoff = (uint32_t)(32 * kb + 16 * kk) * ROW_BYTES;
                        const bf16x4 lo = lds_read_tr(sb, v_rd[db] + rowoff);
                        const bf16x4 hi = lds_read_tr(sb, v_rd[db] + rowoff + 8 * ROW_BYTES);
                        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][kk], oacc[db], 0, 0, 0);
                    }
        }
        if (j + 1 < n_kt) store_tile(stage ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l (bf16, round to nearest even), LSE = m*scale + ln l
    const float l_tot = wave_swap_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (myq < N) {
        uint16_t* orow = p.o + qo_panel + (size_t)myq * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[db][4 * r4 + i] * inv);
                *(bf16x4*)(orow + 32 * db + 8 * r4 + 4 * hh) = ov;
            }
        if (p.lse != nullptr && hh == 0) {
            const size_t li = ((size_t)b * p.Hq + h) * (size_t)N + myq;
            p.lse[li] = m_run * p.lse_scale + logf(l_tot);
        }
    }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
constexpr int MAX_DEVICES = 64;
std::atomic<int> g_arch_ok[MAX_DEVICES];   // 0 unknown, 1 gfx950, 2 other

bool device_is_gfx950(int dev) {
    if (dev < 0 || dev >= MAX_DEVICES) return false;
    int s = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (s == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        s = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_ok[dev].store(s, std::memory_order_relaxed);
    }
    return s == 1;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
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
    const int64_t n_qtiles = ((int64_t)N + BR - 1) / BR;
    const int64_t total = (int64_t)B * H_q * n_qtiles;
    if (total > INT32_MAX || (int64_t)B * H_q > INT32_MAX) return ATTN_ERR_SHAPE;
    const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15;
    if (mis != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_ALIGN;
    const size_t qo_bytes = (size_t)B * H_q * N * HD * 2;
    const size_t kv_bytes = (size_t)B * H_kv * N * HD * 2;
    const size_t lse_bytes = (size_t)B * H_q * N * 4;
    if (overlaps(o, qo_bytes, q, qo_bytes) || overlaps(o, qo_bytes, k, kv_bytes) ||
        overlaps(o, qo_bytes, v, kv_bytes))
        return ATTN_ERR_ALIAS;
    if (lse && (overlaps(lse, lse_bytes, q, qo_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
                overlaps(lse, lse_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, o, qo_bytes)))
        return ATTN_ERR_ALIAS;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev)) return ATTN_ERR_DEVICE;

    Params p;
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
    const float mag = std::fabs(scale);
    p.q_mode = scale > 0.f ? 0 : (scale < 0.f ? 1 : 2);
    p.c = (float)((double)(mag > 0.f ? mag : 1.0f) * 1.4426950408889634);
    p.lse_scale = mag;

    hipStream_t s = (hipStream_t)stream;
    if (causal)
        hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3((unsigned)total), dim3(NTHREAD), 0, s, p);
    else
        hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3((unsigned)total), dim3(NTHREAD), 0, s, p);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_LAUNCH;
    return ATTN_OK;
}

extern "C" const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "B, H_q, H_kv, N and D must be positive and the sizes must fit";
        case ATTN_ERR_GQA: return "H_q must be a multiple of H_kv";
        case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (this build supports D = 128)";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
        case ATTN_ERR_ALIAS: return "an output overlaps an input or the other output";
        case ATTN_ERR_LAUNCH: return "kernel launch failed";
        case ATTN_ERR_DEVICE: return "the current device is not a gfx950 GPU";
        default: return "unknown status";
    }
}

extern "C" double attn_fwd_flops(int B, int H_q, int N, int D, int causal) {
    const double f = 4.0 * B * H_q * (double)N * (double)N * D;
    return causal ? 0.5 * f : f;
}
