// LDS tile layout and streaming shared by the forward and backward kernels.
#pragma once

#include "fa_params.hpp"

namespace fa355 {

// Direct HBM->LDS loads issued as inline assembly, so that the compiler does not
// see them.  The compiler cannot tell which LDS bytes a direct-to-LDS load
// writes, so for the ones it sees it makes LDS reads wait for all of them
// (s_waitcnt vmcnt(0)): in the forward's key loop that put a wait for the next
// tiles' loads, issued at the top of the iteration, in front of the current V
// tile's reads, in the middle of the iteration.  Every caller here waits for its
// loads explicitly (s_waitcnt vmcnt(0) and a barrier) before reading what they
// load, and issues them only after a barrier that ends all reads of the bytes
// they overwrite.  Lane l's `size` bytes at base + voff + soff land at
// lds + size * l, through a raw buffer resource (gfx9-family word 3) whose range
// ends at `bytes`: reads past it return zeros and touch no memory.  M0 carries
// the LDS address and is restored afterwards; the load writes no VGPR.
// (base and bytes are wave-uniform; the SGPR operand needs them in scalar registers)
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return (u32x4){(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu),
                   (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

__device__ __forceinline__ void dma_lds16(const u32x4& rsrc, FA_LDS void* lds, int voff, int soff) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(l), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
}

__device__ __forceinline__ void dma_lds4(const u32x4& rsrc, FA_LDS void* lds, int voff, int soff) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(l), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
}


// LDS tiles are row-major [row][D] bf16 with the 16-byte chunks of each row
// permuted: logical chunk c of row r sits at physical chunk c ^ tile_swz(r).
// Measured on gfx950 (bank-conflict counter), the LDS serves a ds_read_b128 in
// groups of 16 lanes and a ds_read_b64_tr_b16 in groups of 32 lanes, each group
// conflict-free when it touches 256 distinct bytes modulo 256.  The kernels read
// (a) 16 consecutive rows at one logical chunk (row-wise operands) and (b) 4
// consecutive rows (from a multiple of 4) at 4 adjacent chunks, 64 bytes each
// (transposed operands).  The XOR below makes (a) a permutation of the 16 chunk
// slots and sends the 4 rows of (b) to 4 different 64-byte bank groups.
template <int D>
__device__ __forceinline__ int tile_swz(int row) {
    if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
    else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);   // 128-byte rows: 2 per 256 bytes
}

// Byte offset of the 16-byte chunk holding logical chunk `chunk` of `row`.
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
    return row * D * 2 + 16 * (chunk ^ tile_swz<D>(row));
}

// Byte offset a lane passes to ds_read_b64_tr_b16 for a 4 x 16 block whose rows
// start at `row0` (multiple of 4) and whose columns start at `col0` (multiple of
// 16): lane s of the 16-lane group names row row0 + s/4, columns col0 + 4*(s%4).
template <int D>
__device__ __forceinline__ int tr_off(int row0, int col0, int sl) {
    const int row = row0 + (sl >> 2);
    const int col = col0 + 4 * (sl & 3);
    return tile_off<D>(row, col >> 3) + 2 * (col & 7);
}

// Stream rows [r0, r0 + ROWS) of a [rows x D] bf16 tile into LDS (wave-cooperative:
// every wave covers a disjoint 1 KB slice per instruction).  Rows past `nrows`
// are clamped to the last valid row (finite data; the consumer masks them).
template <int D, int ROWS, int NW>
__device__ __forceinline__ void load_tile_lds(char* lds_tile, const bf16* base, int64_t row_stride,
                                              int r0, int nrows, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int ROWS_PER_INST = 1024 / (D * 2);
    constexpr int INSTS = ROWS * D * 2 / 1024 / NW;
    static_assert(ROWS * D * 2 % (1024 * NW) == 0, "tile must split evenly over waves");
#pragma unroll
    for (int i = 0; i < INSTS; ++i) {
        const int inst = wave * INSTS + i;
        const int r = inst * ROWS_PER_INST + lane / CPR;
        const int lc = (lane % CPR) ^ tile_swz<D>(r);   // logical chunk stored in this slot
        const int row = min(r0 + r, nrows - 1);
        global_to_lds16(base + (int64_t)row * row_stride + lc * 8,
                        (FA_LDS void*)(lds_tile + inst * 1024));
    }
}

__device__ __forceinline__ bool wave_any(bool pred) {
    return __builtin_amdgcn_ballot_w64(pred) != 0;
}

// Per-lane byte offsets for streaming a [ROWS x D] bf16 tile (rows `row_bytes`
// apart in memory) into LDS with 16-byte buffer loads: instruction i of wave w
// writes the 1 KB LDS slice (w * INSTS + i) of the swizzled tile, lane l's 16
// bytes landing at slice + 16 l.
template <int D, int ROWS, int NW>
struct TileLoader {
    static constexpr int CPR = D / 8;
    static constexpr int ROWS_PER_INST = 1024 / (D * 2);
    static constexpr int INSTS = ROWS * D * 2 / 1024 / NW;
    static_assert(ROWS * D * 2 % (1024 * NW) == 0, "tile must split evenly over waves");
    int voff[INSTS];

    __device__ __forceinline__ TileLoader(int row_bytes, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < INSTS; ++i) {
            const int r = (wave * INSTS + i) * ROWS_PER_INST + lane / CPR;
            const int lc = (lane % CPR) ^ tile_swz<D>(r);   // logical chunk stored in this slot
            voff[i] = r * row_bytes + 16 * lc;
        }
    }

    // Rows [first, first + ROWS) of the tensor starting at `base`, whose valid
    // rows span `bytes` bytes; `first_bytes` = first * row_bytes (wave-uniform).
    // Rows past `bytes` read as zeros and touch no memory (dma_lds16).
    __device__ __forceinline__ void load(FA_LDS char* lds_tile, const void* base, uint32_t bytes,
                                         int first_bytes, int wave) const {
        const u32x4 rsrc = raw_rsrc(base, bytes);
#pragma unroll
        for (int i = 0; i < INSTS; ++i)
            dma_lds16(rsrc, (FA_LDS void*)(lds_tile + (wave * INSTS + i) * 1024), voff[i], first_bytes);
    }
};

// Epilogue store of a wave's 32 output rows of D values from transposed
// accumulators (acc[cb] register r of lane l holds row l % 32, column
// cb*32 + 8 (r / 4) + 4 (l / 32) + r % 4), each multiplied by `mul`: the wave
// writes its rows into its own LDS slice (`slice`, 32 * (2 D + 16) bytes, rows
// padded by 16 bytes against bank conflicts) and stores them back as whole
// 16-byte chunks, 64 / (D / 8) rows per instruction, instead of 8-byte pieces of
// 32 rows.  Row i goes to `base + (row0 + i) * stride` if row0 + i < nrows.  The
// caller makes sure no other wave reads `slice` meanwhile.
template <int D>
__device__ __forceinline__ void store_rows_via_lds(FA_LDS char* slice, const f32x16 (&acc)[D / 32], float mul,
                                                   bf16* base, int64_t stride, int row0, int nrows, int lane) {
    constexpr int RS = D * 2 + 16;
    constexpr int CPRW = D / 8;
    constexpr int RPI = 64 / CPRW;
    const int col = lane & 31;
    const int h2 = lane >> 5;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int d0 = cb * 32 + 8 * rg + 4 * h2;
            const u32x2 u = (u32x2){pack_bf16x2(acc[cb][4 * rg] * mul, acc[cb][4 * rg + 1] * mul),
                                    pack_bf16x2(acc[cb][4 * rg + 2] * mul, acc[cb][4 * rg + 3] * mul)};
            *reinterpret_cast<FA_LDS u32x2*>(slice + col * RS + 2 * d0) = u;
        }
    const int rr = lane / CPRW;
    const int ch = lane % CPRW;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int row = i * RPI + rr;
        const u32x4 v4 = *reinterpret_cast<const FA_LDS u32x4*>(slice + row * RS + 16 * ch);
        if (row0 + row < nrows) *reinterpret_cast<u32x4*>(base + (int64_t)(row0 + row) * stride + 8 * ch) = v4;
    }
}

template <int D>
constexpr int kRowSliceBytes = 32 * (D * 2 + 16);   // one wave's slice for store_rows_via_lds

// store_rows_via_lds with a fixed number of store instructions: the rows sit
// unpadded in the slice (32 * 2D bytes) with their 16-byte chunks XOR-permuted
// by the row (as conflict-free as the padding), and every store is issued, as a
// buffer store through `rsrc`, whose range ends at the last valid row's D values
// so that the hardware drops the rows past it.  Each wave issues exactly
// 32 / (64 / (D / 8)) store instructions, so that a later s_waitcnt can leave
// them outstanding and wait only for loads issued before them.  Row i goes to
// byte offset (row0 + i) * row_bytes of the resource.
// `between()` runs after the slice has been read back (the reads may still be
// in flight) and before the stores.
template <int D, typename F>
__device__ __forceinline__ void store_rows_fixed(FA_LDS char* slice, const f32x16 (&acc)[D / 32], float mul,
                                                 const void* base, uint32_t bytes, int row_bytes, int row0,
                                                 int lane, F&& between) {
    constexpr int RS = D * 2;
    constexpr int CPRW = D / 8;
    constexpr int RPI = 64 / CPRW;
    const int col = lane & 31;
    const int h2 = lane >> 5;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const u32x2 u = (u32x2){pack_bf16x2(acc[cb][4 * rg] * mul, acc[cb][4 * rg + 1] * mul),
                                    pack_bf16x2(acc[cb][4 * rg + 2] * mul, acc[cb][4 * rg + 3] * mul)};
            const int chunk = (cb * 4 + rg) ^ (col & (CPRW - 1));
            *reinterpret_cast<FA_LDS u32x2*>(slice + col * RS + 16 * chunk + 8 * h2) = u;
        }
    const int rr = lane / CPRW;
    const int ch = lane % CPRW;
    u32x4 v4[32 / RPI];
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int row = i * RPI + rr;
        v4[i] = *reinterpret_cast<const FA_LDS u32x4*>(slice + row * RS + 16 * (ch ^ (row & (CPRW - 1))));
    }
    between();
#if defined(__HIP_DEVICE_COMPILE__)
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                                        0x00020000);
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(v4[i], rsrc, (row0 + i * RPI + rr) * row_bytes + 16 * ch, 0, 0);
#endif
}

// One fp32 per lane at byte offset `off` of a resource of `bytes` bytes from
// `base` (dropped by the hardware when off >= bytes): one store instruction.
__device__ __forceinline__ void store_f32_fixed(const float* base, uint32_t bytes, int off, float v) {
#if defined(__HIP_DEVICE_COMPILE__)
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes,
                                                        0x00020000);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsrc, off, 0, 0);
#endif
}

// s_waitcnt lgkmcnt(0), the other counters at their maxima (gfx9 encoding).
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N), the other counters at their maxima (gfx9 encoding),
// through the builtin so that the compiler's bookkeeping of loads sees it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// 64 consecutive fp32 values base[first..first+63] into LDS (one per lane, in
// lane order), through a buffer resource whose range ends at `bytes`: values
// past it read as zeros.  `first_bytes` = 4 * first (wave-uniform).
__device__ __forceinline__ void load_f32x64_lds(FA_LDS char* lds, const float* base, uint32_t bytes,
                                                int first_bytes) {
    dma_lds4(raw_rsrc(base, bytes), (FA_LDS void*)lds, lane_x4_here(), first_bytes);
}

}  // namespace fa355
