// FP8 (OCP e4m3) forward with a random Hadamard rotation of Q and K.
//
// Method ("LLM Systems 22: Flash Attention", §4.1.3 Low-precision - FP8): the
// low-precision products double the matrix-unit rate, and multiplying Q and K
// by a random orthogonal J (J J^T = I) keeps S = Q K^T = (QJ)(KJ)^T while
// spreading outlier dimensions, so that quantisation loses less.  Here
// J = diag(sigma) H / sqrt(d) with H the Sylvester Hadamard matrix and sigma
// random signs supplied by the caller.  The rotation is applied unnormalised
// (x diag(sigma) H, a fast Walsh-Hadamard transform per row) and the 1/d that
// restores J's normalisation is folded into the score scale.
//
// Quantisation (fp8_quant_kernel, one pass; grid over (tensor, batch*head,
// 64-row block)): rotates Q and K (V is left as it is), reduces the block's
// largest magnitude to one power-of-two scale s = 2^ceil(log2(amax / 448)) --
// the smallest with amax / s <= 448, decided exactly from the binary exponent --
// and writes the e4m3 codes of x / s (exact division) with round-to-nearest-even
// v_cvt_pk_fp8_f32.  No value can exceed 448, so the conversion's out-of-range
// behaviour is never reached.
//
// Attention over the codes (fa_fwd_fp8_kernel): the bf16 forward's structure
// with v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3; its e8m0 block-scale
// operands are 2^0 except for the V tile's scale in O^T += V^T P^T):
//   S^T = K Q^T: 64-deep k-steps over the head dim (2 per 32x32 block, d = 128);
//   raw scores q8.k8 times c = scale*log2(e)/d * s_q(wave's block) * s_k(tile)
//   give the base-2 exponent; the reference maximum m is kept in those units;
//   P~ * 16 = exp2(S c - m + 4) is converted to e4m3 in registers and is the
//   B operand of O^T += V^T P^T, one 64-deep step per 64-key tile, with the
//   tile's V scale applied by the MFMA's own power-of-two scale operand; the row
//   sum l keeps the unrounded values; O = acc / l, LSE = (m + log2 l - 4) ln 2.
//   The reference moves only when a tile's row maximum exceeds it by more than
//   2^4 ("LLM Systems 22: Flash Attention", §4.2.1: the online-softmax variant
//   that skips most rescaling; the threshold is this design's): otherwise P~
//   stays <= 16 (so P~ * 16 <= 256, inside e4m3's range) and the rescale of
//   O, 64 multiplies per lane that would otherwise run on most tiles, is
//   skipped.  Here, where the products take fewer cycles than the softmax's
//   vector work, that is about 9% of the kernel.
//
// gfx950 layouts (measured): the 32x32x64 f8 operands give lane l (half
// h = l / 32) row or column l % 32 and the 32 bytes k = 32h .. 32h + 31; the
// accumulator is the bf16 MFMA's.  ds_read_b64_tr_b8: in each group of 16 lanes
// lane s names 8 bytes; lane i receives byte i % 8 of the chunks named by lanes
// 2t + i / 8, t = 0..7 (8 rows of one column).
#pragma once

#include <type_traits>

#include "fa_tiles.hpp"

namespace fa355 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kFp8D = 128;          // head dim of the FP8 path
constexpr int kFp8QuantRows = 64;   // rows per quantisation block (= the key tile)
constexpr float kFp8RescaleLog2 = 4.f;   // the reference maximum moves on a rise above 2^this

struct Fp8QuantParams {
    const bf16* x[3];      // q, k, v [B, N_t, H, 128] bf16
    uint8_t* codes[3];     // same layout, e4m3
    float* scales;         // [3][B*H][nblk] powers of two, one per 64-row block
    const float* signs;    // [128] +1 / -1
    int n[3];              // rows per batch entry of each tensor
    int B, H, nblk;        // nblk = blocks of the longest tensor (the scales' row stride)
    int rotate;            // rotate q and k (tensors 0 and 1)
};

struct Fp8AttnParams {
    const uint8_t* q8;
    const uint8_t* k8;
    const uint8_t* v8;
    const float* sq;       // [B*H][sq_stride], one per 64-row block of q
    const float* sk;       // [B*H][sk_stride], one per 64-row block (= key tile) of k
    const float* sv;       // same layout as sk
    bf16* o;               // [B, Nq, H, 128]
    float* lse;            // [B, H, Nq]
    int batch, H, nq, nk, n_tiles, sq_stride, sk_stride;
    float qk_scale_log2;   // scale * log2(e) (/ d when Q and K were rotated)
};

// ------------------------------------------------------------------ quantisation

// Value of lane (lane ^ M) within each row of 16 lanes, through DPP (no LDS):
// quad permutations for M = 1, 2; "rotate right" by 8 for M = 8; for M = 4 the
// rotations by 12 (lane + 4) and by 4 (lane - 4), chosen by lane bit 2.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int M>
__device__ __forceinline__ float xor_lane16(float x, int lane) {
    if constexpr (M == 1) return dpp_f32<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    if constexpr (M == 2) return dpp_f32<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    if constexpr (M == 8) return dpp_f32<0x128>(x);   // row_ror:8
    if constexpr (M == 4) {
        const float up = dpp_f32<0x12C>(x);           // row_ror:12 -> lane + 4
        const float dn = dpp_f32<0x124>(x);           // row_ror:4  -> lane - 4
        return (lane & 4) ? dn : up;
    }
    return x;
}

// Butterfly across lanes: the lane with bit M clear holds a and gets a + b; its
// partner holds b and gets a - b, i.e. o + sgn * own with sgn = -1 there.
template <int M>
__device__ __forceinline__ void fwht_lane_stage(float* v, int chunk) {
    const float sgn = (chunk & M) ? -1.f : 1.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_fmaf(sgn, v[e], xor_lane16<M>(v[e], chunk));
}

// 16 threads per 128-element row, 8 consecutive elements each (elements
// 8 chunk .. 8 chunk + 7, their signs sg[0..7]; chunk = lane % 16).  Rotates v[8]
// in place: y = x diag(sigma) H over the row (fp32 butterflies a + b, a - b).
__device__ __forceinline__ void fwht_row8(float* v, const float* sg, int chunk) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= sg[e];
#pragma unroll
    for (int s = 1; s < 8; s <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((e & s) == 0) {
                const float a = v[e], b = v[e + s];
                v[e] = a + b;
                v[e + s] = a - b;
            }
    fwht_lane_stage<1>(v, chunk);
    fwht_lane_stage<2>(v, chunk);
    fwht_lane_stage<4>(v, chunk);
    fwht_lane_stage<8>(v, chunk);
}

// The R rows row0 + r0 + 16 i (i < R) of tensor t at chunk `chunk`, loaded
// together (R loads in flight per thread), converted to fp32 and rotated if asked;
// rows past n read as zeros.
template <int R>
__device__ __forceinline__ void fp8_load_rows(const Fp8QuantParams& p, int t, int b, int h, int row0,
                                              int r0, int chunk, const float* sg, float (*v)[8]) {
    bf16x8 x[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int row = row0 + r0 + 16 * i;
        const int rr = row < p.n[t] ? row : 0;
        x[i] = load16(p.x[t] + (((int64_t)b * p.n[t] + rr) * p.H + h) * kFp8D + 8 * chunk);
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const bool live = row0 + r0 + 16 * i < p.n[t];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = live ? (float)x[i][e] : 0.f;
        if (p.rotate && t < 2) fwht_row8(v[i], sg, chunk);
    }
}

__device__ __forceinline__ void fp8_signs8(const Fp8QuantParams& p, int t, int chunk, float* sg) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = (p.rotate && t < 2) ? p.signs[8 * chunk + e] : 1.f;
}

__device__ __forceinline__ float block_max256(float x, float* red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    x = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return x;
}

// Exponent k of the smallest power of two with amax / 2^k <= 448 (amax > 0):
// amax = f 2^E with f in [0.5, 1) and 448 = 0.875 * 2^9.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
    int E;
    const float f = frexpf(amax, &E);
    return f <= 0.875f ? E - 9 : E - 8;
}

// grid (B*H*nblk, 3), 256 threads: 64 rows x 16 chunks, 4 rows per thread
__global__ __launch_bounds__(256) void fp8_quant_kernel(Fp8QuantParams p) {
    constexpr int R = kFp8QuantRows / 16;
    __shared__ float red[4];
    const int t = blockIdx.y;
    const int blk = blockIdx.x % p.nblk;
    const int bh = blockIdx.x / p.nblk;
    const int b = bh / p.H, h = bh % p.H;
    const int row0 = blk * kFp8QuantRows;
    if (row0 >= p.n[t]) return;   // uniform over the block
    const int chunk = threadIdx.x & 15;
    float sg[8];
    fp8_signs8(p, t, chunk, sg);
    float v[R][8];
    fp8_load_rows<R>(p, t, b, h, row0, threadIdx.x >> 4, chunk, sg, v);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[i][e]));
    mx = block_max256(mx, red);
    const int k = mx > 0.f ? fp8_scale_exp(mx) : 0;
    if (threadIdx.x == 0) p.scales[((int64_t)t * p.B * p.H + bh) * p.nblk + blk] = ldexpf(1.f, k);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int row = row0 + (threadIdx.x >> 4) + 16 * i;
        int w0 = 0, w1 = 0;
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[i][0], -k), ldexpf(v[i][1], -k), w0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[i][2], -k), ldexpf(v[i][3], -k), w0, true);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[i][4], -k), ldexpf(v[i][5], -k), w1, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[i][6], -k), ldexpf(v[i][7], -k), w1, true);
        if (row < p.n[t]) {
            uint8_t* dst = p.codes[t] + (((int64_t)b * p.n[t] + row) * p.H + h) * kFp8D + 8 * chunk;
            *reinterpret_cast<i32x2*>(dst) = (i32x2){w0, w1};
        }
    }
}

// ------------------------------------------------------------------- attention

// LDS tiles of e4m3 rows (128 B): the 16-byte chunks of row r are permuted by
// XOR with bits (2, 1, 3) of r.  Row-wise operand reads (16 consecutive rows at
// one chunk, two rows per 256 bytes) and the transposed V reads (8 rows
// {0..3, 8..11} + 4h + 16j at two adjacent chunks) both cover 256 distinct bytes
// modulo 256 per 16 / 32 lanes served together.
__device__ __forceinline__ int fp8_swz(int row) {
    return ((row >> 2) & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
}
__device__ __forceinline__ int fp8_off(int row, int chunk) { return row * 128 + 16 * (chunk ^ fp8_swz(row)); }

struct Fp8Cfg {
    static constexpr int NW = 4;
    static constexpr int BM = 32 * NW;
    static constexpr int BN = 64;
    static constexpr int ROW = 128;                      // bytes per row
    static constexpr int TILE_BYTES = BN * ROW;          // 8 KB
    static constexpr int INSTS = TILE_BYTES / 1024 / NW; // loads per wave per tile
    static constexpr int LDS_BYTES = 2 * 2 * TILE_BYTES;
};

// Per-lane offsets for a 64 x 128 B tile: instruction i of wave w fills the 1 KB
// slice w*INSTS + i (8 rows), lane l's 16 bytes at slice + 16 l.
struct Fp8TileLoader {
    int voff[Fp8Cfg::INSTS];
    __device__ __forceinline__ Fp8TileLoader(int row_bytes, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < Fp8Cfg::INSTS; ++i) {
            const int r = (wave * Fp8Cfg::INSTS + i) * 8 + (lane >> 3);
            const int lc = (lane & 7) ^ fp8_swz(r);
            voff[i] = r * row_bytes + 16 * lc;
        }
    }
    // (compiler-invisible direct-to-LDS loads, as TileLoader's: the kernel waits
    // for them explicitly before reading the tile)
    __device__ __forceinline__ void load(FA_LDS char* lds_tile, const void* base, uint32_t bytes,
                                         int first_bytes, int wave) const {
        const u32x4 rsrc = raw_rsrc(base, bytes);
#pragma unroll
        for (int i = 0; i < Fp8Cfg::INSTS; ++i)
            dma_lds16(rsrc, (FA_LDS void*)(lds_tile + (wave * Fp8Cfg::INSTS + i) * 1024), voff[i], first_bytes);
    }
};

__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
    // operand formats 0 = e4m3; scale exponents 127 = 2^0 for both operands
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The same with A's products scaled by 2^(ea - 127) in the matrix unit (e8m0
// block-scale operand; measured: exact powers of two).
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64_scale_a(i32x8 a, i32x8 b, f32x16 c, int ea) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, 127);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const FA_LDS char* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        reinterpret_cast<FA_LDS i32x2*>(const_cast<FA_LDS char*>(p)));
}

// 3 work-groups per CU (12 waves): at most 168 VGPRs and 3 x 32 KB of LDS
// (measured 14% faster than 2 per CU)
template <bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void fa_fwd_fp8_kernel(Fp8AttnParams p) {
    using C = Fp8Cfg;
    // the K/V buffers, or at the end the 4 waves' row slices of the O epilogue
    constexpr int LDS = C::LDS_BYTES > C::NW * kRowSliceBytes<kFp8D> ? C::LDS_BYTES
                                                                      : C::NW * kRowSliceBytes<kFp8D>;
    __shared__ __attribute__((aligned(1024))) char smem[LDS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int h2 = lane >> 5;
    const int col = lane & 31;

    int bh, rank;
    xcd_work_item(blockIdx.x, p.n_tiles, p.H * p.batch, bh, rank);
    const int tile = p.n_tiles - 1 - rank;   // longest causal rows first
    const int h = bh % p.H;
    const int b = bh / p.H;
    const int nq = p.nq, nk = p.nk;
    const int q_start = tile * C::BM;
    if (q_start >= nq) return;
    const int kv_end = CAUSAL ? min(nk, q_start + C::BM) : nk;
    const int n_kv = (kv_end + C::BN - 1) / C::BN;
    const int64_t tok = (int64_t)p.H * kFp8D;
    const uint8_t* kbase = p.k8 + (int64_t)b * nk * tok + h * kFp8D;
    const uint8_t* vbase = p.v8 + (int64_t)b * nk * tok + h * kFp8D;
    const int row_bytes = p.H * kFp8D;
    const uint32_t kv_bytes = (uint32_t)nk * row_bytes;
    const Fp8TileLoader loader(row_bytes, wave, lane);
    FA_LDS char* ldsb = (FA_LDS char*)smem;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);

    const int qw0 = q_start + wave * 32;
    const int qi = qw0 + col;
    // B operand of S^T = K Q^T: lane (query, h2) holds dims 64 ks + 32 h2 .. +31
    const uint8_t* qptr = p.q8 + ((int64_t)b * nq + min(qi, nq - 1)) * tok + h * kFp8D + 32 * h2;
    i32x8 qf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(qptr + 64 * ks);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(qptr + 64 * ks + 16);
        qf[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }

    f32x16 acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
    float m = kNegInf;   // reference maximum of the base-2 exponents S c
    float l = 0.f;       // running sum of 16 P~ over the keys this lane holds
    const int nbq = (nq + kFp8QuantRows - 1) / kFp8QuantRows;
    const float c0 = p.qk_scale_log2 * p.sq[(int64_t)bh * p.sq_stride + min(qw0 / kFp8QuantRows, nbq - 1)];
    const float* skh = p.sk + (int64_t)bh * p.sk_stride;
    const float* svh = p.sv + (int64_t)bh * p.sk_stride;

    // transposed V reads: lane (h2, group half gh, i = lane % 16) names key row
    // 16 rho + 4 h2 + 8 ((i/2) >> 2) + ((i/2) & 3) and byte 8 (i & 1) of chunk 2 cb + gh
    const int gi = lane & 15;
    const int gh = (lane >> 4) & 1;
    const int trow = 4 * h2 + 8 * ((gi >> 1) >> 2) + ((gi >> 1) & 3);

    i32x8 pk = {};   // P^T operand of the current tile
    if (n_kv > 0) {
        loader.load(ldsb, kbase, kv_bytes, 0, wave_s);
        loader.load(ldsb + C::TILE_BYTES, vbase, kv_bytes, 0, wave_s);
    }
    // the key and value scales of tile t (= scale block t) are fetched one tile
    // ahead, before that tile's loads, so that waiting for them never waits for
    // the next tile's K/V loads
    float sk_next = n_kv > 0 ? skh[0] : 1.f;
    float sv_next = n_kv > 0 ? svh[0] : 1.f;
    // One key tile in LDS buffer `buf` (0 or 1).  The causal kernel runs two tiles
    // per trip with `buf` a compile-time constant, carried in the LDS reads'
    // immediate offsets instead of vector adds (5% faster); the non-causal kernel,
    // which would spill at three waves per SIMD that way, passes it at run time.
    auto step = [&](int t, auto buf) __attribute__((always_inline)) {
        const int B0 = int(buf) * 2 * C::TILE_BYTES;         // this tile's buffer
        const int B1 = (1 - int(buf)) * 2 * C::TILE_BYTES;   // the next tile's
        const FA_LDS char* kt = ldsb + B0;
        const FA_LDS char* vt = kt + C::TILE_BYTES;
        wait_vmem();
        __syncthreads();
        const float sk_t = sk_next, sv_t = sv_next;
        if (t + 1 < n_kv) {
            sk_next = skh[t + 1];
            sv_next = svh[t + 1];
            loader.load(ldsb + B1, kbase, kv_bytes, (t + 1) * C::BN * row_bytes, wave_s);
            loader.load(ldsb + B1 + C::TILE_BYTES, vbase, kv_bytes, (t + 1) * C::BN * row_bytes, wave_s);
        }
        const int kv0 = t * C::BN;
        if (CAUSAL && kv0 > qw0 + 31) return;
        const float c = c0 * sk_t;
        const int ev = 127 + __builtin_amdgcn_frexp_expf(sv_t) - 1;   // s_v = 2^(ev - 127)

        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
            const int row = kb * 32 + col;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const i32x4 lo = *reinterpret_cast<const FA_LDS i32x4*>(kt + fp8_off(row, 4 * ks + 2 * h2));
                const i32x4 hi = *reinterpret_cast<const FA_LDS i32x4*>(kt + fp8_off(row, 4 * ks + 2 * h2 + 1));
                s[kb] = mfma_fp8_32x32x64(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qf[ks], s[kb]);
            }
        }

        const bool need_mask = (CAUSAL && kv0 + C::BN - 1 > qw0) || (kv0 + C::BN > nk);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                    if ((CAUSAL && key > qi) || key >= nk) s[kb][r] = kNegInf;
                }
        }

        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_halves(mx) * c;
        const bool grow = mx > m + kFp8RescaleLog2;   // (m = -inf: any finite maximum)
        const float m_new = grow ? mx : m;
        const float m_ref = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_ref);      // 1 unless the reference moved
        const float off = (8.f - kFp8RescaleLog2) - m_ref;   // P~ * 16 <= 256
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = fast_exp2(__builtin_fmaf(s[kb][r], c, off));
                s[kb][r] = pr;
                rs += pr;
            }
        l = l * alpha + rs;
        m = m_new;
        if (wave_any(grow)) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        }

        // P^T operand: byte 16 kb + r = register r of key block kb.  The two
        // conversions overwrite both halves of the word, so the previous tile's
        // word serves as the "old" input (no zeroing move).
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int kb = w >> 2, r0 = 4 * (w & 3);
            int x = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][r0], s[kb][r0 + 1], pk[w], false);
            x = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][r0 + 2], s[kb][r0 + 3], x, true);
            pk[w] = x;
        }

        // O^T[dim][query] += V^T P^T: V^T byte 8 rho + t' of lane (d, h2) is key
        // 16 rho + 4 h2 + 8 (t' >> 2) + (t' & 3), the key of P's byte 8 rho + t'
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            i32x2 part[4];
#pragma unroll
            for (int rho = 0; rho < 4; ++rho) {
                const int row = 16 * rho + trow;
                part[rho] = lds_read_tr8(vt + fp8_off(row, 2 * cb + gh) + 8 * (gi & 1));
            }
            const i32x4 a01 = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3);
            const i32x4 a23 = __builtin_shufflevector(part[2], part[3], 0, 1, 2, 3);
            acc[cb] = mfma_fp8_32x32x64_scale_a(__builtin_shufflevector(a01, a23, 0, 1, 2, 3, 4, 5, 6, 7), pk,
                                                acc[cb], ev);
        }
    };
    if constexpr (CAUSAL) {
        for (int t = 0; t < n_kv; t += 2) {
            step(t, std::integral_constant<int, 0>{});
            if (t + 1 < n_kv) step(t + 1, std::integral_constant<int, 1>{});
        }
    } else {
        for (int t = 0; t < n_kv; ++t) step(t, t & 1);
    }

    const float lt = sum_halves(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // O through this wave's LDS slice, out as whole 16-byte chunks (as the bf16 forward)
    __syncthreads();   // every wave is done with the K/V buffers
    store_rows_via_lds<kFp8D>((FA_LDS char*)smem + wave * kRowSliceBytes<kFp8D>, acc, inv,
                              p.o + (int64_t)b * nq * tok + h * kFp8D, tok, qw0, nq, lane);
    if (qi < nq) {
        if (h2 == 0) {
            p.lse[((int64_t)b * p.H + h) * nq + qi] =
                lt > 0.f ? (m + __builtin_amdgcn_logf(lt) - (8.f - kFp8RescaleLog2)) * kLn2 : kNegInf;
        }
    }
}

}  // namespace fa355
