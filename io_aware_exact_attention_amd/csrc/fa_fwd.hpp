// Forward kernel: O = softmax(scale * Q K^T) V and LSE, without writing S or P.
//
// Method ("08 · FlashAttention", §二; "LLM Systems 22: Flash Attention", §3.1):
// each work-group owns a tile of BM query rows and streams the key/value rows in
// tiles of BN.  Per query row it keeps a reference maximum m, a running sum l and an
// unnormalised accumulator O; a new tile with scores S' updates them as
//     m_new = rowmax S' if that exceeds m by more than 2 ln 2, else m,
//     P~ = exp(S' - m_new),
//     l <- e^(m - m_new) l + rowsum P~,   O <- e^(m - m_new) O + P~ V',
// and O / l is written once at the end with LSE = m + ln l.  Any m at or below
// the true maximum gives the same result; keeping m unless the maximum rises
// by a factor above 4 ("LLM Systems 22: Flash Attention", §4.2.1: the online
// softmax that skips most rescaling) leaves P~ <= 4 and lets a wave skip O's
// rescale on most tiles.  (P~ is rounded to bf16 for the P V product; O is
// divided by the sum of those rounded values, LSE uses the unrounded l.)  Work is done in the
// base-2 domain: exp(x*scale) = exp2(x * scale*log2 e), the scale folded into
// one FMA per score.  With the causal mask only key tiles at or below the
// diagonal are visited, and only tiles that straddle it are masked.
//
// gfx950 mapping (one work-group = 4 waves = BM 128 query rows, 32 per wave):
//   * Q rows stay in registers for the whole kernel as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//   * K and V tiles (BN = 64 rows at d = 128, 128 at d = 64) stream from HBM into LDS with direct
//     global->LDS 16-byte loads, double-buffered so the next tile's load
//     overlaps this tile's math; one barrier per tile.
//   * Because S^T's accumulator gives each lane one query and 16 keys per
//     32-key block, the row max/sum are in-lane reductions plus one
//     permlane32 swap, the rescale factor is lane-local, and the probabilities
//     feed the P V product (computed as O^T = V^T P^T) directly as the B
//     operand, with no LDS round trip.  V^T's operand comes from LDS through
//     the transposing ds_read_b64_tr_b16.
//   * LDS tiles are XOR-swizzled at 16-byte granularity so that both the
//     row-wise K reads and the transposed V reads are free of bank conflicts.
#pragma once

#include <type_traits>

#include "fa_tiles.hpp"

namespace fa355 {

// Key tiles of 64 rows at d = 128 and 128 rows at d = 64: a tile's barrier, row
// maximum exchange and rescale test then cover as many bytes of K and V either
// way (measured at d = 64 against 64-row tiles: B4 H16 N1024 non-causal 6%
// faster, B8 H16 N4096 2-2.5%, B4 H16 N1024 causal the same).  The key-split
// kernel keeps 64-row tiles at d = 64 (at 128 it needs 8 bytes of scratch).
template <int D, int BN_ = (D == 64 ? 128 : 64)>
struct FwdCfg {
    static constexpr int NW = 4;                 // waves per work-group
    static constexpr int BM = 32 * NW;           // query rows per work-group
    static constexpr int BN = BN_;               // key rows per tile
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int TILE_BYTES = BN * ROW_BYTES;
    static constexpr int KSTEPS = D / 16;        // MFMA k-steps over the head dim
    static constexpr int DBLK = D / 32;          // 32-wide blocks of the head dim
    static constexpr int KB = BN / 32;           // 32-key blocks per tile
    static constexpr int LDS_BYTES = 2 * 2 * TILE_BYTES;   // [buffer][K | V]
    // the online softmax's reference maximum moves only on a rise above 2^2 (exp2 units)
    static constexpr float RESCALE_LOG2 = 2.f;
};

// One work item: query tile `tile` of (batch or sequence, head) pair `bh`, with
// the work-group's LDS at `smem`.
//
// Software-pipelined over key tiles: the scores of tile t+1 are formed while tile
// t's probabilities are exponentiated, and tile t's P V product runs while tile
// t+1's row maximum is reduced, so each wave keeps the matrix unit and the
// vector unit busy at once instead of alternating between them.  K tiles and V
// tiles therefore live one tile apart in two double buffers: when iteration t
// starts, K(t+1) and V(t) are in LDS and the loads of K(t+2) and V(t+1) go out.
//
// SPLIT = 2 (key-split form, 8 waves): waves 0-3 take the first ceil(n/2) of the
// work-group's n key tiles and waves 4-7 the rest, each half with its own LDS
// buffers; both halves run the same number of barriers.  At the end the second
// half's (m, l, lr, O) go through LDS to the wave of the first half that holds the
// same query rows, which combines the two online-softmax states exactly as a new
// tile would (scale each by e^(m_half - m_max), add) and writes the output.
//
// CARRY = true (dense, one key range; the persistent kernel's multi-round
// form): consecutive items of a work-group overlap.  After its key loop an item
// issues the next item's first K, V and second K tiles (into the first three
// 16 KB tiles of the LDS) before its own epilogue, which goes through row
// slices above them (3 * 16 KB on, within the 16 KB the kernel adds to the K/V
// buffers); once a wave has read its slice back it loads the next item's Q rows
// for that wave into the same slice, then issues a fixed number of buffer
// stores.  The next item (nx.pre) waits only for those loads, leaving the stores
// outstanding, and reads its Q fragments from the slice.  All these loads go
// straight to LDS, so the compiler's bookkeeping of register loads never spans
// two items.
struct FwdNext {
    bool pre;    // this item's Q and first tiles were issued by the previous item
    bool has;    // there is a next item: (bh, tile)
    int bh, tile;
};

template <int D>
constexpr int kCarrySliceOff = 3 * FwdCfg<D>::TILE_BYTES;
template <int D>
constexpr int kCarryLdsBytes = FwdCfg<D>::LDS_BYTES + 16384;
template <int D>
constexpr int kCarryStores = 32 / (64 / (D / 8)) + 1;   // O row stores + the LSE store, per wave

template <int D, bool CAUSAL, bool VARLEN, int SPLIT, bool CARRY>
__device__ __forceinline__ void fwd_tile(const AttnParams& p, char* smem, int bh, int tile, const FwdNext& nx) {
    using C = FwdCfg<D, SPLIT == 2 ? 64 : FwdCfg<D>::BN>;
    static_assert(SPLIT == 1 || SPLIT == 2, "one or two key halves");
    static_assert(!CARRY || (SPLIT == 1 && !VARLEN), "carried items: dense, one key range");
    static_assert(!CARRY || kCarrySliceOff<D> + C::NW * 32 * 2 * D <= kCarryLdsBytes<D>, "slices fit");
    // (wave-uniform, so that its branches are scalar ones)
    const bool pre = CARRY && __builtin_amdgcn_readfirstlane((int)nx.pre) != 0;
    // (carried items run in a loop: opaque to the optimiser, so that offsets
    // derived from the lane are recomputed per item instead of held across items)
    int tid = threadIdx.x;
    if constexpr (CARRY) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = (tid >> 6) & (C::NW - 1);   // row block of this wave
    const int half = SPLIT == 2 ? (tid >> 6) / C::NW : 0;
    const int h2 = lane >> 5;
    const int col = lane & 31;
    const int sl = lane & 15;
    const int g = (lane >> 4) & 1;

    const int h = bh % p.H;
    const int b = bh / p.H;
    int qs, nq, ks, nk;
    seq_range<VARLEN>(p, b, qs, nq, ks, nk);
    const int q_start = tile * C::BM;
    if (q_start >= nq) return;
    const int kv_end = CAUSAL ? min(nk, q_start + C::BM) : nk;
    const int n_all = (kv_end + C::BN - 1) / C::BN;   // the work-group's key tiles
    // this half's key tiles [kt0, kt0 + n_kv), and the loop's trip count (the same
    // for every wave of the work-group: each trip has one barrier)
    const int n_first = SPLIT == 2 ? (n_all + 1) / 2 : n_all;
    const int kt0 = half ? n_first : 0;
    const int n_kv = half ? n_all - n_first : n_first;
    const int n_iter = n_first;
    const int64_t tok = (int64_t)p.H * D;
    const int row_bytes = p.H * D * 2;
    // this half's keys start at row kt0 * BN (at most nk: an empty second half
    // issues no loads)
    const int k_first = min(kt0 * C::BN, nk);
    const bf16* kbase = p.k + (int64_t)(ks + k_first) * tok + h * D;
    const bf16* vbase = p.v + (int64_t)(ks + k_first) * tok + h * D;
    const uint32_t kv_bytes = (uint32_t)(nk - k_first) * row_bytes;
    const TileLoader<D, C::BN, C::NW> loader(row_bytes, wave, lane);
    FA_LDS char* ldsb = (FA_LDS char*)smem + half * C::LDS_BYTES;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // LDS destinations are wave-uniform

    const int qw0 = q_start + wave * 32;   // first query row of this wave
    const int qi = qw0 + col;              // this lane's query row
    // this wave's key tiles: under the causal mask the ones that start at or
    // before its last row.  Only the last of them can need a mask (the diagonal
    // tile, or the ragged tail of the keys).
    // (In the key-split form, the last tile of the first half is masked too when
    // the wave's range continues in the second half; such a tile lies wholly
    // below the wave's first row and within the keys, so the mask leaves it as is.)
    int n_w = CAUSAL ? min(n_all, (qw0 + 31) / C::BN + 1) : n_all;
    n_w = min(max(n_w - kt0, 0), n_kv);
    // An empty asm hides the count from the optimiser, as the causal count
    // already is (it depends on the wave).  When it can prove the loop's tile
    // cases uniform (the non-causal n_w is the work-group's n_kv), the ROCm 7.2
    // compiler schedules across their branches and runs out of registers: the
    // d = 128 non-causal kernel spilled 232 bytes per lane to scratch and took
    // 1.90 ms on B8 H16 N4096 instead of 1.10 ms.  Behind the asm every forward
    // variant fits in 223 registers with no scratch.
    asm volatile("" : "+v"(n_w));
    bf16x8 qf[C::KSTEPS];
    if constexpr (CARRY) {
        // (carried items take Q through this wave's slice of the LDS, rows past
        // nq as zeros: below; the first item of a work-group loads it there too,
        // so that no Q fragment register is ever the target of a memory load
        // whose wait the compiler would place inside the key loop)
        if (!pre) {
            const TileLoader<D, C::BM, C::NW> qload(row_bytes, wave, lane);
            qload.load((FA_LDS char*)smem + kCarrySliceOff<D>, p.q + (int64_t)qs * tok + h * D,
                       (uint32_t)nq * row_bytes, q_start * row_bytes, wave_s);
        }
    } else {
        const bf16* qptr = p.q + (int64_t)(qs + min(qi, nq - 1)) * tok + h * D + 8 * h2;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) qf[s] = load16(qptr + 16 * s);
    }

    f32x16 acc[C::DBLK];
#pragma unroll
    for (int cb = 0; cb < C::DBLK; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
    float m = kNegInf;   // reference maximum of raw scores q.k (this row)
    float l = 0.f;       // running sum, over the keys this lane holds (gives LSE)
    float lr = 0.f;      // the same sum of the bf16-rounded P~ that the P V product uses
    float alpha = 0.f;   // e^(m_old - m) of the tile whose scores are held
    float mc = 0.f;      // reference maximum * scale * log2(e) of that tile
    const float c = p.scale_log2;

    // LDS: buffer j (j = 0, 1) holds a K tile at 2 j TILE_BYTES and a V tile
    // TILE_BYTES after it.  K(t) sits in buffer t % 2, V(t) in buffer t % 2.
    if (!pre) {
        if (n_kv > 0) {
            loader.load(ldsb, kbase, kv_bytes, 0, wave_s);
            loader.load(ldsb + C::TILE_BYTES, vbase, kv_bytes, 0, wave_s);
        }
        if (n_kv > 1) loader.load(ldsb + 2 * C::TILE_BYTES, kbase, kv_bytes, C::BN * row_bytes, wave_s);
        if constexpr (CARRY) wait_vmem();   // (before this wave reads its Q rows)
    } else {
        // (a carried item: its loads were issued before the previous item's
        // kCarryStores<D> stores, which may stay in flight)
        wait_vmcnt<kCarryStores<D>>();
    }
    if constexpr (CARRY) {   // this wave's Q rows, from its own slice
        const FA_LDS char* qt = (const FA_LDS char*)smem + kCarrySliceOff<D>;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) qf[s] = lds_read16(qt + tile_off<D>(wave * 32 + col, 2 * s + h2));
    }

    // per-lane byte offsets of the K operand reads (one per k-step) within a tile
    int koff[C::KSTEPS];
#pragma unroll
    for (int st = 0; st < C::KSTEPS; ++st) koff[st] = tile_off<D>(col, 2 * st + h2);

    // S^T[key][query] = K Q^T for the 64 keys of the K tile at `kt`
    auto scores = [&](const FA_LDS char* kt, f32x16 (&sc)[C::KB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st)
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)   // row kb*32 + col: 32 more rows keep the swizzle
                sc[kb] = mfma_32x32x16(lds_read16(kt + koff[st] + kb * 32 * C::ROW_BYTES), qf[st], sc[kb]);
    };
    // causal diagonal / ragged tail of key tile t
    // (a key is masked iff it exceeds the last key the row may see, min(qi, nk - 1)
    // causal, nk - 1 otherwise; relative to the lane's first key of the tile that is
    // one compare of each register's constant key offset)
    auto mask = [&](f32x16 (&sc)[C::KB], int t) __attribute__((always_inline)) {
        const int kv0 = (kt0 + t) * C::BN;
        const int lim = (CAUSAL ? min(qi, nk - 1) : nk - 1) - kv0 - 4 * h2;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sc[kb][r] = kNegInf;
    };
    // new running maximum from the held scores: sets m, alpha, mc
    auto row_max = [&](const f32x16 (&sc)[C::KB]) __attribute__((always_inline)) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        mx = max_halves(mx);
        // the reference moves only when the tile's maximum exceeds it by more than
        // RESCALE_LOG2 in exp2 units, so P~ <= 2^RESCALE_LOG2; otherwise it stays and
        // alpha = 1 (a first finite maximum always moves it from -inf)
        const float m_new = (mx * c > m * c + C::RESCALE_LOG2) ? mx : m;
        const float m_ref = (m_new == kNegInf) ? 0.f : m_new;
        alpha = fast_exp2((m - m_ref) * c);
        mc = m_ref * c;
        m = m_new;
    };
    // P~ = exp2(S c - m c) of the held scores, packed to bf16 as the P^T operand
    // (registers 8*(ks&1)..+7 of key block ks/2 hold keys 16*ks + {4*h2 + 0..3,
    // 8 + 4*h2 + 0..3} of this lane's query); updates l and lr.  O is
    // normalised by the sum of the rounded values it was formed from, so that
    // O = sum_j bf16(P~_j) v_j / sum_j bf16(P~_j) is a convex combination of the
    // v_j, whose error from P's rounding scales with v_j - O rather than v_j.
    auto probs = [&](f32x16 (&sc)[C::KB], bf16x8 (&pk)[C::BN / 16]) __attribute__((always_inline)) {
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = fast_exp2(__builtin_fmaf(sc[kb][r], c, -mc));
                sc[kb][r] = pr;
                rs += pr;
            }
        l = l * alpha + rs;
        float rr = lr * alpha;
#pragma unroll
        for (int ks2 = 0; ks2 < C::BN / 16; ++ks2) {
            float tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = sc[ks2 >> 1][8 * (ks2 & 1) + e];
            pk[ks2] = pack8(tmp);
            rr = sum8_bf16(pk[ks2], rr);
        }
        lr = rr;
    };
    // O^T[dim][query] += V^T P^T; V^T operand via transposed LDS reads
    // of the same key order: rows 16*ks + 4*h2 + 0..3 and +8
    auto pv = [&](const FA_LDS char* vt, const bf16x8 (&pk)[C::BN / 16]) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < C::DBLK; ++cb) {
#pragma unroll
            for (int ks2 = 0; ks2 < C::BN / 16; ++ks2) {
                const int c0 = cb * 32 + 16 * g;
                const int rk = ks2 * 16 * C::ROW_BYTES;   // 16 more rows keep the swizzle
                bf16x8 a = join(lds_read_tr(vt + tr_off<D>(4 * h2, c0, sl) + rk),
                                lds_read_tr(vt + tr_off<D>(4 * h2 + 8, c0, sl) + rk));
                acc[cb] = mfma_32x32x16(a, pk[ks2], acc[cb]);
            }
        }
    };

    f32x16 s[C::KB];   // scores of the tile the loop is at
    if constexpr (!CARRY) wait_vmem();
    __syncthreads();
    if (n_w > 0) {
        scores(ldsb, s);
        if (n_w == 1) mask(s, 0);
        row_max(s);
    }
    // Iteration t: exponentiate the held S(t), form S(t+1), then O += P(t) V(t)
    // and the maximum of S(t+1).  Two per trip of the loop below, so that every
    // LDS buffer offset is a compile-time constant.
    auto iter = [&](int t, auto par) __attribute__((always_inline)) {
        constexpr int PB = decltype(par)::value;   // t % 2
        const FA_LDS char* k_next = ldsb + (1 - PB) * 2 * C::TILE_BYTES;   // K(t+1)
        const FA_LDS char* v_cur = ldsb + PB * 2 * C::TILE_BYTES + C::TILE_BYTES;   // V(t)
        // (iteration 0 of a carried item: only the previous item's stores can
        // be in flight)
        if (CARRY && pre && t == 0)
            wait_vmcnt<kCarryStores<D>>();
        else
            wait_vmem();
        __syncthreads();
        if (t + 2 < n_kv)   // K(t+2) replaces K(t), whose scores every wave has formed
            loader.load(ldsb + PB * 2 * C::TILE_BYTES, kbase, kv_bytes, (t + 2) * C::BN * row_bytes, wave_s);
        if (t + 1 < n_kv)   // V(t+1) replaces V(t-1), whose product every wave has formed
            loader.load(ldsb + (1 - PB) * 2 * C::TILE_BYTES + C::TILE_BYTES, vbase, kv_bytes,
                        (t + 1) * C::BN * row_bytes, wave_s);
        if (t >= n_w) return;
        // O's rescale for tile t, only when some row of the wave moved its reference
        // (26% of the wave-tiles of B8 H16 N4096 causal, against 78% with a
        // reference that follows every new maximum)
        if (wave_any(alpha != 1.f)) {
#pragma unroll
            for (int cb = 0; cb < C::DBLK; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        }
        // one basic block per case: the compiler interleaves its products with its
        // vector work only within a block
        auto full = [&](auto masked) __attribute__((always_inline)) {
            bf16x8 pk[C::BN / 16];
            f32x16 sn[C::KB];
            probs(s, pk);
            scores(k_next, sn);
            pv(v_cur, pk);
            if constexpr (decltype(masked)::value) mask(sn, t + 1);
            row_max(sn);
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) s[kb] = sn[kb];
        };
        if (t + 2 < n_w) {
            full(std::false_type{});
        } else if (t + 2 == n_w) {   // S(t+1) is the wave's last tile: masked
            full(std::true_type{});
        } else {                     // the wave's last tile
            bf16x8 pk[C::BN / 16];
            probs(s, pk);
            pv(v_cur, pk);
        }
    };
    for (int t = 0; t < n_iter; t += 2) {
        iter(t, std::integral_constant<int, 0>{});
        if (t + 1 < n_iter) iter(t + 1, std::integral_constant<int, 1>{});
    }

    if constexpr (SPLIT == 2) {
        // merge area [row block][value][lane] (fp32): O's 16 * DBLK accumulators,
        // then m, l, lr -- written by the second half, read by the first
        constexpr int NV = 16 * C::DBLK + 3;
        static_assert(C::NW * NV * 64 * 4 <= 2 * C::LDS_BYTES, "merge area fits the K/V buffers");
        FA_LDS float* mx = (FA_LDS float*)smem + wave * NV * 64 + lane;
        __syncthreads();   // every wave is done with its K/V buffers
        if (half == 1) {
#pragma unroll
            for (int cb = 0; cb < C::DBLK; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx[(cb * 16 + r) * 64] = acc[cb][r];
            mx[(NV - 3) * 64] = m;
            mx[(NV - 2) * 64] = l;
            mx[(NV - 1) * 64] = lr;
        }
        __syncthreads();
        if (half == 1) return;
        const float m1 = mx[(NV - 3) * 64];
        const float mm = fmaxf(m, m1);
        const float m_ref = (mm == kNegInf) ? 0.f : mm;
        const float a0 = fast_exp2((m - m_ref) * c);
        const float a1 = fast_exp2((m1 - m_ref) * c);
        l = l * a0 + mx[(NV - 2) * 64] * a1;
        lr = lr * a0 + mx[(NV - 1) * 64] * a1;
#pragma unroll
        for (int cb = 0; cb < C::DBLK; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][r] = acc[cb][r] * a0 + mx[(cb * 16 + r) * 64] * a1;
        m = mm;
    }

    const float lt = sum_halves(l);
    const float lrt = sum_halves(lr);
    const float inv = lrt > 0.f ? 1.f / lrt : 0.f;
    if constexpr (CARRY) {
        __syncthreads();   // every wave is done with the K/V buffers
        const bool has = __builtin_amdgcn_readfirstlane((int)nx.has) != 0;
        const bf16* qb_n = p.q;
        uint32_t qbytes_n = 0;
        int qfirst_n = 0;
        if (has) {   // the next item's first three K/V tiles
            const int hn = nx.bh % p.H;
            const int bn = nx.bh / p.H;
            int qs_n, nq_n, ks_n, nk_n;
            seq_range<false>(p, bn, qs_n, nq_n, ks_n, nk_n);
            const int q_start_n = nx.tile * C::BM;
            const int kv_end_n = CAUSAL ? min(nk_n, q_start_n + C::BM) : nk_n;
            const bf16* kb_n = p.k + (int64_t)ks_n * tok + hn * D;
            const bf16* vb_n = p.v + (int64_t)ks_n * tok + hn * D;
            const uint32_t kvb_n = (uint32_t)nk_n * row_bytes;
            loader.load(ldsb, kb_n, kvb_n, 0, wave_s);
            loader.load(ldsb + C::TILE_BYTES, vb_n, kvb_n, 0, wave_s);
            if (kv_end_n > C::BN) loader.load(ldsb + 2 * C::TILE_BYTES, kb_n, kvb_n, C::BN * row_bytes, wave_s);
            qb_n = p.q + (int64_t)qs_n * tok + hn * D;
            qbytes_n = (uint32_t)nq_n * row_bytes;
            qfirst_n = q_start_n * row_bytes;
        }
        // O (through this wave's slice), then LSE: kCarryStores<D> store
        // instructions per wave; between reading the slice back and the stores,
        // the next item's Q rows of this wave go into the slice
        FA_LDS char* slice = (FA_LDS char*)smem + kCarrySliceOff<D> + wave * 32 * 2 * D;
        store_rows_fixed<D>(slice, acc, inv, p.o + (int64_t)qs * tok + h * D,
                            (uint32_t)(nq - 1) * row_bytes + 2 * D, row_bytes, qw0, lane, [&]() {
            if (has) {
                wait_lgkmcnt0();   // this wave's slice reads are done
                const TileLoader<D, C::BM, C::NW> qload(row_bytes, wave, lane);
                qload.load((FA_LDS char*)smem + kCarrySliceOff<D>, qb_n, qbytes_n, qfirst_n, wave_s);
            }
        });
        store_f32_fixed(p.lse + ((int64_t)b * p.H + h) * p.nq, (uint32_t)nq * 4, h2 ? 0x7ffffff0 : 4 * qi,
                        lt > 0.f ? (m * c + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf);
        return;
    }
    if constexpr (SPLIT == 1) {
        // O through LDS, stored back as whole 16-byte chunks (bitwise the same
        // output; 0.3-3% faster than 8-byte stores of 32 rows each)
        static_assert(C::NW * kRowSliceBytes<D> <= C::LDS_BYTES, "row slices fit the K/V buffers");
        __syncthreads();   // every wave is done with the K/V buffers
        store_rows_via_lds<D>((FA_LDS char*)smem + wave * kRowSliceBytes<D>, acc, inv,
                              p.o + (int64_t)qs * tok + h * D, tok, qw0, nq, lane);
    }
    if (qi < nq) {
        if constexpr (SPLIT == 2) {
            bf16* optr = p.o + (int64_t)(qs + qi) * tok + h * D;
#pragma unroll
            for (int cb = 0; cb < C::DBLK; ++cb)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int d0 = cb * 32 + 8 * rg + 4 * h2;
                    store8(optr + d0, acc[cb][4 * rg] * inv, acc[cb][4 * rg + 1] * inv,
                           acc[cb][4 * rg + 2] * inv, acc[cb][4 * rg + 3] * inv);
                }
        }
        if (h2 == 0) {
            p.lse[((int64_t)b * p.H + h) * p.nq + qi] =
                lt > 0.f ? (m * c + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
        }
    }
}

template <int D, bool CAUSAL, bool VARLEN, int SPLIT = 1>
__device__ __forceinline__ void fwd_tile(const AttnParams& p, char* smem, int bh, int tile) {
    fwd_tile<D, CAUSAL, VARLEN, SPLIT, false>(p, smem, bh, tile, FwdNext{false, false, 0, 0});
}

// One work-group per query tile, in the order xcd_work_item gives.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[FwdCfg<D>::LDS_BYTES];
    int bh, rank;
    xcd_work_item(blockIdx.x, p.n_tiles, p.H * p.batch, bh, rank);
    fwd_tile<D, CAUSAL, VARLEN>(p, smem, bh, p.n_tiles - 1 - rank);   // longest causal rows first
}

// Key-split form for grids that fill at most one round of the CUs' work-group
// slots (short causal sequences, few heads): one 8-wave work-group per query
// tile, each half of its waves taking half of the tile's key tiles, so the
// longest tile's chain of key tiles is halved.  Tiles are numbered longest
// first (lpt_work_item); with one such work-group per CU, the hardware hands
// the shorter tiles of the second round to the CUs that finish first.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_split_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * FwdCfg<D, 64>::LDS_BYTES];
    int bh, rank;
    lpt_work_item(blockIdx.x, p.n_tiles, p.H * p.batch, bh, rank);
    fwd_tile<D, CAUSAL, false, 2>(p, smem, bh, p.n_tiles - 1 - rank);
}

// Persistent form ("LLM Systems 22: Flash Attention", §4.1.4 persistent kernels,
// §4.1.5 longest-processing-time-first): a fixed grid (a multiple of 8, about
// the number of work-groups the CUs hold at once) loops over the work items,
// dealt in rounds of one item per work-group, alternating direction ("snake"):
// in even rounds work-group g takes item round * grid + g, in odd rounds the
// work-groups of each XCD take theirs in reverse order.  A plain round-robin
// deal gives work-group 0 the longest item of every round (9% above the mean on
// B8 H16 N4096, 12% on N32768, which is the kernel's tail); the snake deal keeps
// every work-group within one item unit of the greedy longest-first schedule.
// Item i runs on XCD i % 8, and the items are numbered in one of two orders:
//   * XCD_ORDER = false (lpt_work_item), longest first over all pairs: all
//     pairs' last query tile (the one with the most causal keys), then all
//     second-to-last ones, ...  For grids of one round, where it pairs long and
//     short tiles on a CU.
//   * XCD_ORDER = true (xcd_work_item, the per-tile kernel's order): each XCD
//     takes its pairs one after another, each pair's tiles longest first, so the
//     work-groups resident on an XCD work on about two pairs at a time and share
//     their K/V in its L2 (longest first over all pairs keeps 16 pairs in flight
//     per XCD on B8 H16 N4096, whose 2 MB of K/V each do not fit the 4 MB L2:
//     0.636 against 0.611 ms).  For causal grids of several rounds.
// No atomics, no workspace.
template <int D, bool CAUSAL, bool XCD_ORDER>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_persistent_kernel(AttnParams p) {
    // The multi-round form at d = 128 carries each item's successor (16 KB more
    // LDS).  Measured on MI355X, alternating, bitwise the same output: B16 H16
    // N1024 5% faster, B8 H16 N2048 2%, B4 H16 N4096 and B2 H32 N8192 0.6%, the
    // headline B8 H16 N4096 and the long context within 0.7% either way; at
    // d = 64 (B8 H16 N4096) 1.6% slower, so not there.
    constexpr bool CARRY = XCD_ORDER && D == 128;
    __shared__ __attribute__((aligned(1024))) char smem[CARRY ? kCarryLdsBytes<D> : FwdCfg<D>::LDS_BYTES];
    const int bh_count = p.H * p.batch;
    const int total = p.n_tiles * bh_count;
    const int grid = gridDim.x;   // a multiple of 8
    const int g = blockIdx.x;
    const int g_rev = 8 * ((grid >> 3) - 1 - (g >> 3)) + (g & 7);   // same XCD, reversed
    auto item = [&](int it, int& bh, int& tile) {
        int rank;
        if constexpr (XCD_ORDER)
            xcd_work_item(it, p.n_tiles, bh_count, bh, rank);
        else
            lpt_work_item(it, p.n_tiles, bh_count, bh, rank);
        tile = p.n_tiles - 1 - rank;
    };
    FwdNext nx{false, false, 0, 0};
    for (int base = 0, r = 0; base < total; base += grid, ++r) {
        const int it = base + ((r & 1) ? g_rev : g);
        if (it >= total) continue;   // (only in the last round)
        int bh, tile;
        item(it, bh, tile);
        // this work-group's next item: the next round's (rounds alternate direction)
        const int it_next = base + grid + ((r & 1) ? g : g_rev);
        nx.has = CARRY && it_next < total;
        if (nx.has) item(it_next, nx.bh, nx.tile);
        fwd_tile<D, CAUSAL, false, 1, CARRY>(p, smem, bh, tile, nx);
        nx.pre = nx.has;
        __syncthreads();   // the next item's loads reuse the LDS buffers
    }
}

}  // namespace fa355
