// Device primitives for gfx950 (CDNA4): MFMA tiles, wave64 cross-half exchange,
// direct global->LDS loads, transposed LDS reads and bf16 packing.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (C[32x32] += A[32x16] * B[16x32]),
// for lane l of a 64-wide wave, half h = l / 32:
//   A: lane l holds A[l % 32][8h .. 8h+7]
//   B: lane l holds B[8h .. 8h+7][l % 32]
//   C: lane l, register r holds C[8*(r/4) + 4h + (r%4)][l % 32]
// The sum index k may be permuted freely as long as A and B agree on it; the
// kernels use that to feed an accumulator tile straight back in as an operand.
//
// ds_read_b64_tr_b16: within each group of 16 lanes, lane s names 8 bytes (4 bf16)
// of a 4 x 16 block (row s/4, columns 4*(s%4)..+3); lane i receives column i of
// that block (its 4 rows).  Reading a row-major [key][dim] tile this way yields
// four consecutive keys of one dimension per lane, i.e. the operand a product over
// keys needs.
//
// global_load_lds_dwordx4: each lane fetches 16 bytes from its own global
// address; lane l's bytes land at (LDS base + 16*l), base uniform over the wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa355 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane (l ^ 32) of the same register, via v_permlane32_swap.
// Only the lane-dependent select of one result is used: combining both results
// of the swap directly in one arithmetic operation (max(r0, r1), r0 + r1) is
// miscompiled by the ROCm 7.2 compiler for gfx950 (it reuses r0 for r1).
__device__ __forceinline__ float other_half(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // lanes 0-31 receive the upper half in r[1]; lanes 32-63 the lower half in r[0]
    return __builtin_bit_cast(float, (__lane_id() < 32) ? r[1] : r[0]);
}

__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, other_half(x)); }

__device__ __forceinline__ float sum_halves(float x) { return x + other_half(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even pack of two floats (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 p = (bf16x2){(bf16)a, (bf16)b};
    return __builtin_bit_cast(uint32_t, p);
}

// 8 consecutive accumulator floats -> one bf16x8 operand.
__device__ __forceinline__ bf16x8 pack8(const float* f) {
    u32x4 u = (u32x4){pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
    return __builtin_bit_cast(bf16x8, u);
}

// acc + the two bf16 values packed in `pair` (v_dot2_f32_bf16 against (1, 1): the
// products are exact, so this adds two bf16 values in fp32).  Written as inline
// assembly: the ROCm 7.2 compiler lowers __builtin_amdgcn_fdot2_f32_bf16 on the
// dwords of a 4-dword vector to v_dot2c_f32_bf16 instructions that all read the
// vector's first dword (seen in the generated code).  The VOP3P form names its
// source register explicitly.
__device__ __forceinline__ float add2_bf16(uint32_t pair, float acc) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(r) : "v"(pair), "s"(0x3f803f80u), "v"(acc));
    return r;
}

// acc + the sum of the 8 bf16 values of p.
__device__ __forceinline__ float sum8_bf16(bf16x8 p, float acc) {
    const u32x4 u = __builtin_bit_cast(u32x4, p);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = add2_bf16(u[j], acc);
    return acc;
}

__device__ __forceinline__ bf16x8 load16(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ void store8(bf16* p, float a, float b, float c, float d) {
    u32x2 u = (u32x2){pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2*>(p) = u;
}

__device__ __forceinline__ void global_to_lds16(const void* g, FA_LDS void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima: gfx9 encoding),
// through the builtin so that the compiler's own bookkeeping of outstanding
// loads sees it, then a compiler barrier for the LDS accesses that follow.
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 lds_read16(const FA_LDS char* p) {
    return *reinterpret_cast<const FA_LDS bf16x8*>(p);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const FA_LDS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        reinterpret_cast<FA_LDS bf16x4*>(const_cast<FA_LDS char*>(p)));
}

__device__ __forceinline__ bf16x8 join(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 4 * (lane index), recomputed where it is used (volatile: never hoisted into a
// register that would stay live across a loop).
__device__ __forceinline__ int lane_x4_here() {
    int v;
    asm volatile(
        "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
        "v_mbcnt_hi_u32_b32 %0, -1, %0\n\t"
        "v_lshlrev_b32 %0, 2, %0"
        : "=v"(v));
    return v;
}

// Work item of work-group `id` in a 1-D grid of n_tiles * bh_count work-groups:
// the (batch or sequence, head) pair `bh` and the tile rank within that pair.
// The hardware deals consecutive work-group ids round-robin to the 8 XCDs, each
// with its own L2.  When bh_count is a multiple of 8, XCD x gets the pairs
// bh = x, x + 8, x + 16, ... -- every XCD a share of every sequence, so unequal
// sequence lengths do not unbalance the XCDs -- and each pair's tiles run
// consecutively there, sharing that pair's K/V in the XCD's L2.  Otherwise
// XCD x gets a contiguous range of the logical order (or, if the grid is not a
// multiple of 8, the plain order).
__device__ __forceinline__ void xcd_work_item(int id, int n_tiles, int bh_count, int& bh, int& rank) {
    const int total = n_tiles * bh_count;
    if ((bh_count & 7) == 0) {
        const int j = id >> 3;
        bh = (j / n_tiles) * 8 + (id & 7);
        rank = j % n_tiles;
        return;
    }
    const int L = (total & 7) == 0 ? (id & 7) * (total >> 3) + (id >> 3) : id;
    bh = L / n_tiles;
    rank = L % n_tiles;
}

// Item `id` of the longest-first order: rank-major (rank 0 = each pair's
// longest tile), pairs dealt over the 8 XCDs as in xcd_work_item when bh_count
// is a multiple of 8 (item id runs on XCD id % 8 when the grid is a multiple of 8).
__device__ __forceinline__ void lpt_work_item(int id, int n_tiles, int bh_count, int& bh, int& rank) {
    if ((bh_count & 7) == 0) {
        const int per = bh_count >> 3;   // pairs per XCD
        const int j = id >> 3;
        bh = (j % per) * 8 + (id & 7);
        rank = j / per;
        return;
    }
    bh = id % bh_count;
    rank = id / bh_count;
}

// Items 0 .. total-1 of a persistent grid (a multiple of 8 work-groups): rounds
// of one item per work-group, even rounds in work-group order and odd rounds
// with each XCD's work-groups reversed, so that a work-group's items in
// longest-first order sum to about the same on every work-group.  Calls
// run(item) with a wave-uniform item, separated by a barrier because the next
// item reuses the LDS.
template <typename F>
__device__ __forceinline__ void persistent_items(int total, F&& run) {
    const int grid = gridDim.x;
    const int g = blockIdx.x;
    const int g_rev = 8 * ((grid >> 3) - 1 - (g >> 3)) + (g & 7);   // same XCD, reversed
#pragma unroll 1
    for (int base = 0, r = 0; base < total; base += grid, ++r) {
        const int it = __builtin_amdgcn_readfirstlane(base + ((r & 1) ? g_rev : g));
        if (it >= total) continue;
        run(it);
        if (base + grid < total) __syncthreads();
    }
}

}  // namespace fa355
