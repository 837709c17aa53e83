// Decoding kernels: a few new query tokens against a long key/value cache,
// grouped-query heads, split along the keys.
//
// Method ("LLM Systems 22: Flash Attention", §5.1 Motivation, §5.2 Solution):
// with Nq = 1..4 query tokens a query-tile grid has far too few work-groups to
// keep the machine busy, and the work is dominated by reading the cache.  So
//   * split-KV: the keys of every (sequence, key/value head) are cut into
//     chunks processed independently; each chunk produces its own normalised
//     partial output O_s and statistic LSE_s (= m_s + ln l_s), and a second,
//     light kernel merges them: LSE = ln sum_s e^(LSE_s),
//     O = sum_s e^(LSE_s - LSE) O_s (the online-softmax merge of the (m, l)
//     statistics, "08 · FlashAttention", §二);
//   * GQA packing: the G = Hq / Hkv query heads that read one key/value head,
//     times the Nq tokens, are packed into the 32 rows of one MFMA tile, so a
//     32-row tile is full for G * Nq = 32 (e.g. 8 heads x 4 tokens).
//
// gfx950 mapping: one work-group = one wave = one (sequence, key/value head,
// 32-row tile, key chunk).  The packed Q rows stay in registers; the chunk's
// K and V stream through the wave's own LDS in 32-key tiles, double-buffered
// with buffer loads (rows past the cache read as zeros).  S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with the forward kernel's layouts
// and LDS swizzle; the online softmax is the forward's.  The work is bound by
// HBM: per 32-key tile a wave reads 2 x 32 x d x 2 bytes and issues 16 MFMAs.
//
// Causal alignment (a reading; the pages do not fix it): the Nq tokens are the
// newest positions, so token i sees keys j <= i + Nk - Nq.
#pragma once

#include "fa_tiles.hpp"

namespace fa355 {

struct DecodeParams {
    const bf16* q;     // [B, Nq, Hq, d]
    const bf16* k;     // [B, Nk, Hkv, d]
    const bf16* v;     // [B, Nk, Hkv, d]
    bf16* o;           // [B, Nq, Hq, d]
    float* lse;        // [B, Hq, Nq], natural log
    float* opart;      // [B, Hkv, row_tiles*32, splits, d]  chunk outputs O_s (normalised)
    float* lpart;      // [B, Hkv, row_tiles*32, splits]     chunk LSE_s (natural log)
    int B, Nq, Nk, Hq, Hkv, G;
    int rows;          // G * Nq packed rows per key/value head
    int row_tiles;     // ceil(rows / 32)
    int splits;        // key chunks per (sequence, key/value head)
    int split_len;     // keys per chunk, a multiple of 32
    float scale;
    float scale_log2;  // scale * log2(e)
};

template <int D>
struct DecCfg {
    static constexpr int BN = 32;                 // keys per tile
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int TILE_BYTES = BN * ROW_BYTES;
    static constexpr int KSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    static constexpr int LDS_BYTES = 4 * TILE_BYTES;   // [buffer][K | V]
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fa_decode_split_kernel(DecodeParams p) {
    using C = DecCfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    FA_LDS char* lds = (FA_LDS char*)smem;

    const int lane = threadIdx.x & 63;
    const int h2 = lane >> 5;
    const int col = lane & 31;
    const int sl = lane & 15;
    const int g = (lane >> 4) & 1;

    int idx = blockIdx.x;
    const int split = idx % p.splits;
    idx /= p.splits;
    const int rt = idx % p.row_tiles;
    idx /= p.row_tiles;
    const int hkv = idx % p.Hkv;
    const int b = idx / p.Hkv;

    // this lane's packed row: query head hkv*G + pr/Nq, token pr%Nq (padding rows
    // repeat the last real row and are not stored)
    const int pr = rt * 32 + col;
    const int prc = min(pr, p.rows - 1);
    const int tq = prc % p.Nq;
    const int hq = hkv * p.G + prc / p.Nq;
    const int last_key = CAUSAL ? tq + p.Nk - p.Nq : p.Nk - 1;   // last key this row sees

    const int k0 = split * p.split_len;
    const int k1 = min(p.Nk, k0 + p.split_len);
    const int n_t = k1 > k0 ? (k1 - k0 + C::BN - 1) / C::BN : 0;

    const bf16* qptr = p.q + ((int64_t)(b * p.Nq + tq) * p.Hq + hq) * D + 8 * h2;
    bf16x8 qf[C::KSTEPS];
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) qf[s] = load16(qptr + 16 * s);

    const int row_bytes = p.Hkv * D * 2;
    const int64_t kv_off = ((int64_t)b * p.Nk * p.Hkv + hkv) * D;
    const bf16* kbase = p.k + kv_off;
    const bf16* vbase = p.v + kv_off;
    const uint32_t kv_bytes = (uint32_t)p.Nk * row_bytes;
    const TileLoader<D, C::BN, 1> loader(row_bytes, 0, lane);
    auto issue = [&](int t) {
        FA_LDS char* kt = lds + (t & 1) * 2 * C::TILE_BYTES;
        loader.load(kt, kbase, kv_bytes, (k0 + t * C::BN) * row_bytes, 0);
        loader.load(kt + C::TILE_BYTES, vbase, kv_bytes, (k0 + t * C::BN) * row_bytes, 0);
    };

    f32x16 acc[C::DBLK];
#pragma unroll
    for (int cb = 0; cb < C::DBLK; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
    float m = kNegInf;
    float l = 0.f;
    const float c = p.scale_log2;

    if (n_t > 0) issue(0);
    for (int t = 0; t < n_t; ++t) {
        wait_vmem();                  // tile t is in LDS (one wave: no barrier needed)
        if (t + 1 < n_t) issue(t + 1);
        const FA_LDS char* kt = lds + (t & 1) * 2 * C::TILE_BYTES;
        const FA_LDS char* vt = kt + C::TILE_BYTES;
        const int kv0 = k0 + t * C::BN;

        // S^T[key][row] = K Q^T for the tile's 32 keys
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st)
            s = mfma_32x32x16(lds_read16(kt + tile_off<D>(col, 2 * st + h2)), qf[st], s);

        // keys past the cache, past this chunk, or after the row's token
        if ((CAUSAL && kv0 + C::BN - 1 > p.Nk - p.Nq) || kv0 + C::BN > k1) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
                if (key > last_key || key >= k1) s[r] = kNegInf;
            }
        }

        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = max_halves(mx);
        const float m_new = fmaxf(m, mx);
        const float m_ref = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2((m - m_ref) * c);
        const float mc = m_ref * c;
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(__builtin_fmaf(s[r], c, -mc));
            s[r] = pv;
            rs += pv;
        }
        l = l * alpha + rs;
        m = m_new;
        if (wave_any(alpha != 1.f)) {
#pragma unroll
            for (int cb = 0; cb < C::DBLK; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        }
        // P^T operand for keys {16*ks + 4*h2 + 0..3, 16*ks + 8 + 4*h2 + 0..3}
        bf16x8 pk[2];
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            float tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = s[8 * ks2 + e];
            pk[ks2] = pack8(tmp);
        }
        // O^T[dim][row] += V^T P^T, V^T through transposed LDS reads in the same key order
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
            for (int cb = 0; cb < C::DBLK; ++cb) {
                const int c0 = cb * 32 + 16 * g;
                const int rk = ks2 * 16 * C::ROW_BYTES;   // 16 more rows keep the swizzle
                const bf16x8 a = join(lds_read_tr(vt + tr_off<D>(4 * h2, c0, sl) + rk),
                                      lds_read_tr(vt + tr_off<D>(4 * h2 + 8, c0, sl) + rk));
                acc[cb] = mfma_32x32x16(a, pk[ks2], acc[cb]);
            }
        }
    }

    // chunk result: O_s = acc / l_s, LSE_s = m_s + ln l_s (-inf and 0 when the row
    // saw no key of the chunk)
    const float lt = sum_halves(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (pr < p.rows) {
        const int64_t slot = ((int64_t)(b * p.Hkv + hkv) * p.row_tiles * 32 + pr) * p.splits + split;
        float* optr = p.opart + slot * D;
#pragma unroll
        for (int cb = 0; cb < C::DBLK; ++cb)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = cb * 32 + 8 * rg + 4 * h2;
                f32x4 w;
                w[0] = acc[cb][4 * rg] * inv;
                w[1] = acc[cb][4 * rg + 1] * inv;
                w[2] = acc[cb][4 * rg + 2] * inv;
                w[3] = acc[cb][4 * rg + 3] * inv;
                *reinterpret_cast<f32x4*>(optr + d0) = w;
            }
        if (h2 == 0) p.lpart[slot] = lt > 0.f ? (m * c + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
    }
}

// Merge of the chunk results of one packed row.  One thread per output element;
// the chunk LSEs are first staged in LDS and reduced by the whole work-group
// (max, then the sum of e^(LSE_s - max)), so that the per-element pass only
// streams the chunk outputs, several loads in flight per thread.
constexpr int kDecodeMaxSplits = 1024;

template <int D>
__global__ __launch_bounds__(D) void fa_decode_combine_kernel(DecodeParams p) {
    __shared__ float wgt[kDecodeMaxSplits];
    __shared__ float red[D / 64];
    int idx = blockIdx.x;
    const int pr = idx % p.rows;
    idx /= p.rows;
    const int hkv = idx % p.Hkv;
    const int b = idx / p.Hkv;
    const int dim = threadIdx.x;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int tq = pr % p.Nq;
    const int hq = hkv * p.G + pr / p.Nq;
    const int64_t slot0 = ((int64_t)(b * p.Hkv + hkv) * p.row_tiles * 32 + pr) * p.splits;
    const float* lp = p.lpart + slot0;

    float top = kNegInf;
    for (int s = dim; s < p.splits; s += D) {
        const float x = lp[s];
        wgt[s] = x;
        top = fmaxf(top, x);
    }
#pragma unroll
    for (int w = 32; w > 0; w >>= 1) top = fmaxf(top, __shfl_xor(top, w));
    if (lane == 0) red[wv] = top;
    __syncthreads();
    top = red[0];
#pragma unroll
    for (int i = 1; i < D / 64; ++i) top = fmaxf(top, red[i]);
    const float base = top == kNegInf ? 0.f : top;
    __syncthreads();   // everyone has read red[] before it is reused
    float part = 0.f;
    for (int s = dim; s < p.splits; s += D) {
        const float e = fast_exp2((wgt[s] - base) * kLog2e);   // -inf chunks -> 0
        wgt[s] = e;
        part += e;
    }
#pragma unroll
    for (int w = 32; w > 0; w >>= 1) part += __shfl_xor(part, w);
    if (lane == 0) red[wv] = part;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) tot += red[i];
    const float inv = tot > 0.f ? 1.f / tot : 0.f;

    const float* op = p.opart + slot0 * D + dim;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 4 <= p.splits; s += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = __builtin_fmaf(wgt[s + u], op[(int64_t)(s + u) * D], acc[u]);
    }
    for (; s < p.splits; ++s) acc[0] = __builtin_fmaf(wgt[s], op[(int64_t)s * D], acc[0]);
    const float o = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * inv;
    p.o[((int64_t)(b * p.Nq + tq) * p.Hq + hq) * D + dim] = (bf16)o;
    if (dim == 0)
        p.lse[((int64_t)b * p.Hq + hq) * p.Nq + tq] = tot > 0.f ? base + __builtin_amdgcn_logf(tot) * kLn2 : kNegInf;
}

}  // namespace fa355
