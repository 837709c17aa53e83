// libfa355: C ABI (include/fa355.h) — host-side validation and kernel launch.
//
// Validation mirrors the eligibility limits of the method's kernels listed in
// "08 · FlashAttention", §四 (bf16 only, head dim limited, contiguous tensors,
// causal or no mask) and, as that section asks, refuses unsupported calls with an
// explicit error instead of falling back silently.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/fa355.h"
#include "fa_bwd.hpp"
#include "fa_decode.hpp"
#include "fa_fp8.hpp"
#include "fa_fwd.hpp"

using namespace fa355;

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_common(int H, int d, float scale, int causal) {
    if (H <= 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// tokens * H * d elements must be addressable; grid sizes must fit an int.
// seq_q / seq_k: rows of one sequence.  The kernels address one sequence's
// rows of one tensor through a buffer resource with a 32-bit signed range, so
// seq * H * d * 2 bytes must stay below 2 GiB.
int check_sizes(int64_t tokens_q, int64_t tokens_k, int64_t seq_q, int64_t seq_k, int H, int d,
                int64_t grid) {
    const int64_t lim = (int64_t)1 << 40;
    const int64_t span = (int64_t)1 << 31;
    if (tokens_q <= 0 || tokens_k <= 0) return FA_ERR_SHAPE;
    if (seq_q * H * d * 2 >= span || seq_k * H * d * 2 >= span) return FA_ERR_UNSUPPORTED;
    if (tokens_q > INT_MAX || tokens_k > INT_MAX) return FA_ERR_SHAPE;
    if (tokens_q * H * d > lim || tokens_k * H * d > lim) return FA_ERR_SHAPE;
    if (grid <= 0 || grid > INT_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

bool env_validate_cu() {
    const char* e = std::getenv("FA355_VALIDATE_CU_SEQLENS");
    return e && e[0] == '1';
}

// Debug-only check of cu_seqlens contents (copies to the host; synchronises).
int validate_cu(const int* cu_q, const int* cu_k, int nseq, int max_q, int max_k, int causal,
                hipStream_t s, int64_t* total_q, int64_t* total_k) {
    std::vector<int> hq(nseq + 1), hk(nseq + 1);
    if (hipMemcpyAsync(hq.data(), cu_q, sizeof(int) * (nseq + 1), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(hk.data(), cu_k, sizeof(int) * (nseq + 1), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return FA_ERR_LAUNCH;
    if (hq[0] != 0 || hk[0] != 0) return FA_ERR_SHAPE;
    for (int i = 0; i < nseq; ++i) {
        const int lq = hq[i + 1] - hq[i], lk = hk[i + 1] - hk[i];
        if (lq < 0 || lk < 0 || lq > max_q || lk > max_k) return FA_ERR_SHAPE;
        if (causal && lq != lk) return FA_ERR_UNSUPPORTED;
    }
    *total_q = hq[nseq];
    *total_k = hk[nseq];
    return FA_OK;
}

template <typename K>
int launch(K kernel, int grid, int block, hipStream_t s, const AttnParams& p) {
    void* args[] = {const_cast<AttnParams*>(&p)};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block),
                                   args, 0, s);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int D, bool VARLEN>
int launch_fwd_d(const AttnParams& p, int causal, hipStream_t s) {
    const int grid = p.n_tiles * p.H * p.batch;
    const int block = FwdCfg<D>::NW * 64;
    return causal ? launch(fa_fwd_kernel<D, true, VARLEN>, grid, block, s, p)
                  : launch(fa_fwd_kernel<D, false, VARLEN>, grid, block, s, p);
}

template <bool VARLEN>
int launch_fwd(const AttnParams& p, int d, int causal, hipStream_t s) {
    return d == 64 ? launch_fwd_d<64, VARLEN>(p, causal, s) : launch_fwd_d<128, VARLEN>(p, causal, s);
}

// Work-group slots of the current device: every kernel here runs 2 work-groups
// per CU.
int fwd_slots(int* slots) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return FA_ERR_LAUNCH;
    *slots = 2 * cus;
    return FA_OK;
}

// Grid of a backward pass with `items` work items (`n_tiles` per sequence): one
// work-group per item, or, for dense causal passes of more than one round of the
// work-group slots, a persistent grid of one work-group per slot (rounded down
// to a multiple of 8) that deals the items itself in the same order, when the
// pass has at most four rounds, or at most 32 tiles per sequence with rounds
// times tiles per sequence at most 256 (eight rounds of 32 tiles, sixteen of
// 16).  Measured on MI355X (fa_bwd, alternating, bitwise the same gradients):
// faster at B8 H16 N2048 d128 (506 against 522-550 us), B4 H16 N4096 (3%), B8
// H16 N4096 (the headline, 0.5-2% on two boxes), B8 H16 N4096 d64 (2-2.5%), B32
// H16 N2048 (2%), B64 H16 N1024 d64 (6.5%); slower at B16 H16 N4096 (0.5%, 16
// rounds of 32 tiles), B2 H32 N8192 (0.7%, 64 tiles), B1 H16 N32768 (3.3%, 256
// tiles) and non-causal (3-4%), which keep one work-group per item.
template <bool VARLEN>
int bwd_grid(int64_t items, int n_tiles, int causal, int* grid) {
    int slots = 0;
    const int st = fwd_slots(&slots);
    if (st) return st;
    if (items > INT_MAX) return FA_ERR_SHAPE;
    *grid = (int)items;
    if (!VARLEN && causal && items > slots &&
        (items <= 4 * (int64_t)slots || (n_tiles <= 32 && items * n_tiles <= 256 * (int64_t)slots)))
        *grid = slots / 8 * 8;
    return FA_OK;
}

// Backward stages.  `p.n_tiles` is set per stage from the stage's own tiling.
template <int D, bool VARLEN>
int launch_bwd_dot_d(AttnParams p, hipStream_t s) {
    using Pre = BwdPreCfg<D>;
    p.n_tiles = (p.nq + Pre::ROWS - 1) / Pre::ROWS;
    return launch(fa_bwd_dot_kernel<D, VARLEN>, p.n_tiles * p.H * p.batch, Pre::THREADS, s, p);
}

template <int D, bool VARLEN>
int launch_bwd_dkdv_d(AttnParams p, int causal, hipStream_t s) {
    using KV = BwdKVCfg<D>;
    p.n_tiles = (p.nk + KV::BN - 1) / KV::BN;
    int grid = 0;
    const int st = bwd_grid<VARLEN>((int64_t)p.n_tiles * p.H * p.batch, p.n_tiles, causal, &grid);
    if (st) return st;
    if (!VARLEN && grid < p.n_tiles * p.H * p.batch) return launch(fa_bwd_dkdv_persistent_kernel<D>, grid, KV::NW * 64, s, p);
    return causal ? launch(fa_bwd_dkdv_kernel<D, true, VARLEN>, grid, KV::NW * 64, s, p)
                  : launch(fa_bwd_dkdv_kernel<D, false, VARLEN>, grid, KV::NW * 64, s, p);
}

template <int D, bool VARLEN, bool DOT>
int launch_bwd_dq_d(AttnParams p, int causal, hipStream_t s) {
    using Q = BwdQCfg<D>;
    p.n_tiles = (p.nq + Q::BM - 1) / Q::BM;
    int grid = 0;
    const int st = bwd_grid<VARLEN>((int64_t)p.n_tiles * p.H * p.batch, p.n_tiles, causal, &grid);
    if (st) return st;
    if (!VARLEN && grid < p.n_tiles * p.H * p.batch) return launch(fa_bwd_dq_persistent_kernel<D, DOT>, grid, Q::NW * 64, s, p);
    return causal ? launch(fa_bwd_dq_kernel<D, true, VARLEN, DOT>, grid, Q::NW * 64, s, p)
                  : launch(fa_bwd_dq_kernel<D, false, VARLEN, DOT>, grid, Q::NW * 64, s, p);
}

template <int D>
int launch_bwd_fused_d(AttnParams p, int causal, hipStream_t s) {
    using KV = BwdKVCfg<D>;
    using Q = BwdQCfg<D>;
    p.n_tiles = (p.nk + KV::BN - 1) / KV::BN;
    const int64_t grid = ((int64_t)p.n_tiles + (p.nq + Q::BM - 1) / Q::BM) * p.H * p.batch;
    if (grid > INT_MAX) return FA_ERR_SHAPE;
    return causal ? launch(fa_bwd_fused_kernel<D, true>, (int)grid, KV::NW * 64, s, p)
                  : launch(fa_bwd_fused_kernel<D, false>, (int)grid, KV::NW * 64, s, p);
}

// Dense backwards whose dK/dV and dQ work items (128-row tiles) together number
// at most this many per CU run both passes in one launch (fa_bwd_fused_kernel,
// after the row-dot kernel).  Measured on MI355X (fa_bwd, both forms bitwise
// equal): causal, against two per-tile kernels 12-27% faster from 1 to 4 items
// per CU, and against the two persistent kernels (which take the passes of more
// than one round of slots) 18% faster at 5 items per CU (B5 H16 N1024 d128) and
// 5-6% at 6, but equal to 6% slower at 7 and 8-12% slower at 8 (B8 H16 N1024 d64
// and d128); non-causal (every tile equally long), 8% faster at 2 items per CU
// but 12% slower at 4, where the separate kernels' single rounds are already
// balanced and the separate row-dot kernel costs more than the merged tails save.
#ifndef FA355_FUSED_BWD_CAUSAL_ITEMS_PER_CU
#define FA355_FUSED_BWD_CAUSAL_ITEMS_PER_CU 6
#endif
#ifndef FA355_FUSED_BWD_FULL_ITEMS_PER_CU
#define FA355_FUSED_BWD_FULL_ITEMS_PER_CU 2
#endif

int use_fused_bwd(const AttnParams& p, int causal, bool* fused) {
    int slots = 0;
    const int st = fwd_slots(&slots);   // two work-groups per CU
    if (st) return st;
    const int64_t items = ((int64_t)(p.nk + 127) / 128 + (p.nq + 127) / 128) * p.H * p.batch;
    const int64_t per_cu = causal ? FA355_FUSED_BWD_CAUSAL_ITEMS_PER_CU : FA355_FUSED_BWD_FULL_ITEMS_PER_CU;
    *fused = items <= per_cu * (slots / 2);
    return FA_OK;
}

// The whole backward is kStageDqDot (the dQ kernel with the row-dot folded in:
// it writes -D and LSE * log2(e) as well as dQ), then dK/dV; for small dense
// grids it is the row-dot kernel, then both passes in one launch.  The row-dot
// kernel alone (kStageDot) fills the same workspace for the stand-alone dK/dV
// and dQ stages.  Stages run in this order: dQ + row-dot, row-dot, dK/dV, dQ.
enum BwdStage { kStageDot = 1, kStageDkdv = 2, kStageDq = 4, kStageDqDot = 8,
                kStageAll = kStageDqDot | kStageDkdv };

template <bool VARLEN>
int launch_bwd(const AttnParams& p, int d, int causal, hipStream_t s, int stages = kStageAll) {
    int st = FA_OK;
    if (!VARLEN && stages == kStageAll) {
        bool fused = false;
        st = use_fused_bwd(p, causal, &fused);
        if (st) return st;
        if (fused) {
            st = d == 64 ? launch_bwd_dot_d<64, VARLEN>(p, s) : launch_bwd_dot_d<128, VARLEN>(p, s);
            if (!st)
                st = d == 64 ? launch_bwd_fused_d<64>(p, causal, s) : launch_bwd_fused_d<128>(p, causal, s);
            return st;
        }
    }
    if (stages & kStageDqDot)
        st = d == 64 ? launch_bwd_dq_d<64, VARLEN, true>(p, causal, s)
                     : launch_bwd_dq_d<128, VARLEN, true>(p, causal, s);
    if (!st && (stages & kStageDot))
        st = d == 64 ? launch_bwd_dot_d<64, VARLEN>(p, s) : launch_bwd_dot_d<128, VARLEN>(p, s);
    if (!st && (stages & kStageDkdv))
        st = d == 64 ? launch_bwd_dkdv_d<64, VARLEN>(p, causal, s)
                     : launch_bwd_dkdv_d<128, VARLEN>(p, causal, s);
    if (!st && (stages & kStageDq))
        st = d == 64 ? launch_bwd_dq_d<64, VARLEN, false>(p, causal, s)
                     : launch_bwd_dq_d<128, VARLEN, false>(p, causal, s);
    return st;
}

// The backward workspace holds two fp32 planes laid out like lse: -D, then LSE * log2(e).
void set_workspace(AttnParams& p, void* ws) {
    p.dvec = static_cast<float*>(ws);
    p.lse2 = p.dvec + (size_t)p.batch * p.H * p.nq;
}

// Decoding: split the keys so that about kDecodeWaves chunk waves run, each
// chunk a multiple of the 32-key tile.  Everything the workspace size depends on
// is derived here, from the shapes only.
constexpr int kDecodeWaves = kDecodeMaxSplits;

struct DecodePlan {
    int G, rows, row_tiles, splits, split_len;
    size_t opart_floats, lpart_floats;
};

DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    DecodePlan pl{};
    pl.G = Hq / Hkv;
    pl.rows = pl.G * Nq;
    pl.row_tiles = (pl.rows + 31) / 32;
    const int64_t units = (int64_t)B * Hkv * pl.row_tiles;
    const int64_t want = std::max<int64_t>(1, (kDecodeWaves + units - 1) / units);
    int64_t len = (Nk + want - 1) / want;
    len = std::max<int64_t>(32, (len + 31) / 32 * 32);
    pl.split_len = (int)len;
    pl.splits = (int)((Nk + len - 1) / len);   // <= kDecodeWaves = kDecodeMaxSplits
    const size_t slots = (size_t)B * Hkv * pl.row_tiles * 32 * pl.splits;
    pl.opart_floats = slots * d;
    pl.lpart_floats = slots;
    return pl;
}

AttnParams base_params(const void* q, const void* k, const void* v, int batch, int H, int nq,
                       int nk, float scale) {
    AttnParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = static_cast<const bf16*>(q);
    p.k = static_cast<const bf16*>(k);
    p.v = static_cast<const bf16*>(v);
    p.batch = batch;
    p.H = H;
    p.nq = nq;
    p.nk = nk;
    p.scale = scale;
    p.scale_log2 = scale * kLog2e;
    return p;
}

// Argument checks shared by the dense backward entry points (all but the workspace).
int check_bwd_dense(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, const void* dq, const void* dk, const void* dv, int B, int H,
                    int Nq, int Nk, int d, float scale, int causal) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
    if (B <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
    int st = check_common(H, d, scale, causal);
    if (st) return st;
    if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    return check_sizes((int64_t)B * Nq, (int64_t)B * Nk, Nq, Nk, H, d, (int64_t)((Nq + 15) / 16) * H * B);
}

int launch_bwd_dense(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace, int B, int H,
                     int Nq, int Nk, float scale, int d, int causal, void* stream) {
    AttnParams p = base_params(q, k, v, B, H, Nq, Nk, scale);
    p.o_in = static_cast<const bf16*>(o);
    p.dout = static_cast<const bf16*>(dout);
    p.lse_in = lse;
    p.dq = static_cast<bf16*>(dq);
    p.dk = static_cast<bf16*>(dk);
    p.dv = static_cast<bf16*>(dv);
    set_workspace(p, workspace);
    return launch_bwd<false>(p, d, causal, static_cast<hipStream_t>(stream));
}

// ---- no-allocation backward: the workspace lives in a static device array.
// Each device that runs the library holds its own copy of `scratch` until the
// process ends.  On the host the array's name only stands for the symbol; its
// device address comes from hipGetSymbolAddress, taken once per device (with that
// device current) and kept below.  Every call on one device uses the same
// memory, so calls that overlap on a device (different streams, no ordering)
// race on it.  The dQ kernel writes every row of both planes before the dK/dV
// kernel reads them, so the array needs no clearing between calls.
constexpr size_t kNoAllocScratchBytes = FA_BWD_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_LAUNCH;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

// Dense forward arguments -> kernel parameters (shared by fa_fwd and fa_fwd_persistent).
int prepare_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                int Nk, int d, float scale, int causal, AttnParams* out) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
    int st = check_common(H, d, scale, causal);
    if (st) return st;
    if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    const int ntq = (Nq + FwdCfg<128>::BM - 1) / FwdCfg<128>::BM;
    st = check_sizes((int64_t)B * Nq, (int64_t)B * Nk, Nq, Nk, H, d, (int64_t)ntq * H * B);
    if (st) return st;
    *out = base_params(q, k, v, B, H, Nq, Nk, scale);
    out->o = static_cast<bf16*>(o);
    out->lse = lse;
    out->n_tiles = ntq;
    return FA_OK;
}


// The persistent forward on a grid of about as many work-groups as the CUs hold
// at once (a multiple of the 8 XCDs).
// Items are numbered longest first over all pairs when they fit in one round,
// and pair by pair per XCD (the per-tile kernel's order) otherwise.
template <int D, bool CAUSAL>
int launch_fwd_persistent_d(const AttnParams& p, int grid, bool one_round, hipStream_t s) {
    return one_round ? launch(fa_fwd_persistent_kernel<D, CAUSAL, false>, grid, FwdCfg<D>::NW * 64, s, p)
                     : launch(fa_fwd_persistent_kernel<D, CAUSAL, true>, grid, FwdCfg<D>::NW * 64, s, p);
}

int launch_fwd_persistent(const AttnParams& p, int d, int causal, int slots, hipStream_t s) {
    const int64_t items = (int64_t)p.n_tiles * p.H * p.batch;
    const int grid = (int)std::max<int64_t>(8, std::min<int64_t>((int64_t)slots / 8 * 8, (items + 7) / 8 * 8));
    const bool one_round = items <= grid;
    if (d == 64)
        return causal ? launch_fwd_persistent_d<64, true>(p, grid, one_round, s)
                      : launch_fwd_persistent_d<64, false>(p, grid, one_round, s);
    return causal ? launch_fwd_persistent_d<128, true>(p, grid, one_round, s)
                  : launch_fwd_persistent_d<128, false>(p, grid, one_round, s);
}

// The key-split forward (causal grids only): one 8-wave work-group per query tile.
int launch_fwd_split(const AttnParams& p, int d, hipStream_t s) {
    const int grid = p.n_tiles * p.H * p.batch;
    return d == 64 ? launch(fa_fwd_split_kernel<64, true>, grid, 2 * FwdCfg<64>::NW * 64, s, p)
                   : launch(fa_fwd_split_kernel<128, true>, grid, 2 * FwdCfg<128>::NW * 64, s, p);
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is non-positive, inconsistent or too large";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim must be 64 or 128, causal needs Nq == Nk, scale must be finite and positive";
        case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointers must be 16-byte aligned (fp32 buffers 4-byte)";
        case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
        default: return "FA_ERR_UNKNOWN";
    }
}

int fa_version(void) { return kVersion; }

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
           int Nk, int d, float scale, int causal, void* stream) {
    AttnParams p;
    int st = prepare_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, &p);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // A grid that fits in one round of work-group slots leaves its time to the
    // longest query tile's chain of key tiles.  Causal, with at most one tile per
    // CU, or with tiles of at least 16 (128-row) query blocks per sequence, it
    // runs the key-split kernel, which halves that chain (its outputs differ from
    // the per-tile kernel's only in the order the two halves' sums are added).
    // Otherwise it runs the persistent kernel, whose deal pairs long and short
    // tiles on a CU: measured on MI355X, the key-split kernel was 17-28% faster
    // at 256 or 512 tiles of N = 4096 and 17% faster at 256 tiles of N = 1024,
    // but 8-10% slower at 512 tiles of N = 1024, where its second round of
    // work-groups costs more than the halved chain saves.  Larger causal grids of
    // sequences up to 32 query tiles (N <= 4096) also run the persistent kernel,
    // in the per-tile kernel's order (2.3% faster on B8 H16 N4096, 9-17% on
    // B4 H16 N4096, B8 H16 N2048, B16 H16 N1024; equal at N = 8192, 1% slower at
    // N = 32768, 2-8% slower non-causal); the rest run one work-group per tile.
    int slots = 0;
    st = fwd_slots(&slots);
    if (st) return st;
    const int64_t items = (int64_t)p.n_tiles * H * B;
    if (causal && (items <= slots / 2 || (items <= slots && p.n_tiles >= 16)))
        return launch_fwd_split(p, d, s);
    if (items <= slots || (causal && p.n_tiles <= 32)) return launch_fwd_persistent(p, d, causal, slots, s);
    return launch_fwd<false>(p, d, causal, s);
}

int fa_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int Nq, int Nk, int d, float scale, int causal, void* stream) {
    AttnParams p;
    int st = prepare_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, &p);
    if (st) return st;
    int slots = 0;
    st = fwd_slots(&slots);
    if (st) return st;
    return launch_fwd_persistent(p, d, causal, slots, static_cast<hipStream_t>(stream));
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq, int max_seqlen_q,
                  int max_seqlen_k, int H, int d, float scale, int causal, void* stream) {
    if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
    if (nseq <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0) return FA_ERR_SHAPE;
    int st = check_common(H, d, scale, causal);
    if (st) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
        return FA_ERR_ALIGN;
    const int ntq = (max_seqlen_q + FwdCfg<128>::BM - 1) / FwdCfg<128>::BM;
    st = check_sizes((int64_t)nseq * max_seqlen_q, (int64_t)nseq * max_seqlen_k, max_seqlen_q,
                     max_seqlen_k, H, d,
                     (int64_t)ntq * H * nseq);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (env_validate_cu()) {
        int64_t tq, tk;
        st = validate_cu(cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q, max_seqlen_k, causal, s, &tq, &tk);
        if (st) return st;
    }
    AttnParams p = base_params(q, k, v, nseq, H, max_seqlen_q, max_seqlen_k, scale);
    p.o = static_cast<bf16*>(o);
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.n_tiles = ntq;
    return launch_fwd<true>(p, d, causal, s);
}

size_t fa_bwd_workspace_bytes(int batch_or_nseq, int H, int nq, int d) {
    (void)d;
    if (batch_or_nseq <= 0 || H <= 0 || nq <= 0) return 0;
    return 2 * sizeof(float) * (size_t)batch_or_nseq * (size_t)H * (size_t)nq;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
           int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream) {
    int st = check_bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, scale, causal);
    if (st) return st;
    if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq, d)) return FA_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return FA_ERR_ALIGN;
    return launch_bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, scale, d,
                            causal, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, void* stream) {
    int st = check_bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, scale, causal);
    if (st) return st;
    if (fa_bwd_workspace_bytes(B, H, Nq, d) > kNoAllocScratchBytes) return FA_ERR_WORKSPACE;
    void* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st) return st;
    return launch_bwd_dense(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, Nq, Nk, scale, d, causal,
                            stream);
}

int fa_bwd_dq_dot(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* workspace, size_t workspace_bytes, void* dq, int B, int H,
                  int Nq, int Nk, int d, float scale, int causal, void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq) return FA_ERR_NULL;
    if (B <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
    int st = check_common(H, d, scale, causal);
    if (st) return st;
    if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq, d)) return FA_ERR_WORKSPACE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(lse, 4) || !aligned(workspace, 4))
        return FA_ERR_ALIGN;
    st = check_sizes((int64_t)B * Nq, (int64_t)B * Nk, Nq, Nk, H, d, (int64_t)((Nq + 15) / 16) * H * B);
    if (st) return st;
    AttnParams p = base_params(q, k, v, B, H, Nq, Nk, scale);
    p.o_in = static_cast<const bf16*>(o);
    p.dout = static_cast<const bf16*>(dout);
    p.lse_in = lse;
    p.dq = static_cast<bf16*>(dq);
    set_workspace(p, workspace);
    return launch_bwd<false>(p, d, causal, static_cast<hipStream_t>(stream), kStageDqDot);
}

int fa_bwd_dot(const void* o, const void* dout, const float* lse, void* workspace,
               size_t workspace_bytes, int B, int H, int Nq, int d, void* stream) {
    if (!o || !dout || !lse) return FA_ERR_NULL;
    if (B <= 0 || Nq <= 0) return FA_ERR_SHAPE;
    int st = check_common(H, d, 1.f, 0);
    if (st) return st;
    if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq, d)) return FA_ERR_WORKSPACE;
    if (!aligned(o, 16) || !aligned(dout, 16) || !aligned(lse, 4) || !aligned(workspace, 4))
        return FA_ERR_ALIGN;
    st = check_sizes((int64_t)B * Nq, (int64_t)B * Nq, Nq, Nq, H, d, (int64_t)((Nq + 15) / 16) * H * B);
    if (st) return st;
    AttnParams p = base_params(nullptr, nullptr, nullptr, B, H, Nq, Nq, 1.f);
    p.o_in = static_cast<const bf16*>(o);
    p.dout = static_cast<const bf16*>(dout);
    p.lse_in = lse;
    set_workspace(p, workspace);
    return launch_bwd<false>(p, d, 0, static_cast<hipStream_t>(stream), kStageDot);
}

static int bwd_stage(int stage, const void* q, const void* k, const void* v, const void* dout,
                     const void* workspace, size_t workspace_bytes, void* dq, void* dk, void* dv,
                     int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream) {
    if (!q || !k || !v || !dout) return FA_ERR_NULL;
    if (stage == kStageDkdv && (!dk || !dv)) return FA_ERR_NULL;
    if (stage == kStageDq && !dq) return FA_ERR_NULL;
    if (B <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
    int st = check_common(H, d, scale, causal);
    if (st) return st;
    if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq, d)) return FA_ERR_WORKSPACE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
        !aligned(workspace, 4) || (dq && !aligned(dq, 16)) || (dk && !aligned(dk, 16)) ||
        (dv && !aligned(dv, 16)))
        return FA_ERR_ALIGN;
    st = check_sizes((int64_t)B * Nq, (int64_t)B * Nk, Nq, Nk, H, d, (int64_t)((Nq + 15) / 16) * H * B);
    if (st) return st;
    AttnParams p = base_params(q, k, v, B, H, Nq, Nk, scale);
    p.dout = static_cast<const bf16*>(dout);
    set_workspace(p, const_cast<void*>(workspace));
    p.dq = static_cast<bf16*>(dq);
    p.dk = static_cast<bf16*>(dk);
    p.dv = static_cast<bf16*>(dv);
    return launch_bwd<false>(p, d, causal, static_cast<hipStream_t>(stream), stage);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const void* workspace,
                size_t workspace_bytes, void* dk, void* dv, int B, int H, int Nq, int Nk, int d,
                float scale, int causal, void* stream) {
    return bwd_stage(kStageDkdv, q, k, v, dout, workspace, workspace_bytes, nullptr, dk, dv, B, H, Nq,
                     Nk, d, scale, causal, stream);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const void* workspace,
              size_t workspace_bytes, void* dq, int B, int H, int Nq, int Nk, int d, float scale,
              int causal, void* stream) {
    return bwd_stage(kStageDq, q, k, v, dout, workspace, workspace_bytes, dq, nullptr, nullptr, B, H,
                     Nq, Nk, d, scale, causal, stream);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                  int max_seqlen_q, int max_seqlen_k, int H, int d, float scale, int causal,
                  void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k)
        return FA_ERR_NULL;
    if (nseq <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0) return FA_ERR_SHAPE;
    int st = check_common(H, d, scale, causal);
    if (st) return st;
    if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(nseq, H, max_seqlen_q, d))
        return FA_ERR_WORKSPACE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) ||
        !aligned(workspace, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
        return FA_ERR_ALIGN;
    st = check_sizes((int64_t)nseq * max_seqlen_q, (int64_t)nseq * max_seqlen_k, max_seqlen_q,
                     max_seqlen_k, H, d,
                     (int64_t)((max_seqlen_q + 15) / 16) * H * nseq);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (env_validate_cu()) {
        int64_t tq, tk;
        st = validate_cu(cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q, max_seqlen_k, causal, s, &tq, &tk);
        if (st) return st;
    }
    AttnParams p = base_params(q, k, v, nseq, H, max_seqlen_q, max_seqlen_k, scale);
    p.o_in = static_cast<const bf16*>(o);
    p.dout = static_cast<const bf16*>(dout);
    p.lse_in = lse;
    p.dq = static_cast<bf16*>(dq);
    p.dk = static_cast<bf16*>(dk);
    p.dv = static_cast<bf16*>(dv);
    set_workspace(p, workspace);
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    return launch_bwd<true>(p, d, causal, s);
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || Hq % Hkv != 0 || (d != 64 && d != 128))
        return 0;
    const DecodePlan pl = decode_plan(B, Hq, Hkv, Nq, Nk, d);
    return sizeof(float) * (pl.opart_floats + pl.lpart_floats);
}

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                  size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                  int causal, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B <= 0 || Nq <= 0 || Nk <= 0 || Hkv <= 0) return FA_ERR_SHAPE;
    int st = check_common(Hq, d, scale, causal);
    if (st) return st;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (causal && Nq > Nk) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(workspace, 16))
        return FA_ERR_ALIGN;
    const size_t need = fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    // one sequence's cache rows of one tensor go through a buffer resource (< 2 GiB)
    if ((int64_t)Nk * Hkv * d * 2 >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 40;
    if ((int64_t)B * Nq * Hq * d > lim || (int64_t)B * Nk * Hkv * d > lim) return FA_ERR_SHAPE;
    const DecodePlan pl = decode_plan(B, Hq, Hkv, Nq, Nk, d);
    const int64_t grid1 = (int64_t)B * Hkv * pl.row_tiles * pl.splits;
    const int64_t grid2 = (int64_t)B * Hkv * pl.rows;
    if (grid1 > INT_MAX || grid2 > INT_MAX) return FA_ERR_SHAPE;
    DecodeParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = static_cast<const bf16*>(q);
    p.k = static_cast<const bf16*>(k);
    p.v = static_cast<const bf16*>(v);
    p.o = static_cast<bf16*>(o);
    p.lse = lse;
    p.opart = static_cast<float*>(workspace);
    p.lpart = p.opart + pl.opart_floats;
    p.B = B;
    p.Nq = Nq;
    p.Nk = Nk;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = pl.G;
    p.rows = pl.rows;
    p.row_tiles = pl.row_tiles;
    p.splits = pl.splits;
    p.split_len = pl.split_len;
    p.scale = scale;
    p.scale_log2 = scale * kLog2e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* args[] = {&p};
    const void* k1;
    const void* k2;
    if (d == 64) {
        k1 = causal ? reinterpret_cast<const void*>(fa_decode_split_kernel<64, true>)
                    : reinterpret_cast<const void*>(fa_decode_split_kernel<64, false>);
        k2 = reinterpret_cast<const void*>(fa_decode_combine_kernel<64>);
    } else {
        k1 = causal ? reinterpret_cast<const void*>(fa_decode_split_kernel<128, true>)
                    : reinterpret_cast<const void*>(fa_decode_split_kernel<128, false>);
        k2 = reinterpret_cast<const void*>(fa_decode_combine_kernel<128>);
    }
    if (hipLaunchKernel(k1, dim3((unsigned)grid1), dim3(64), args, 0, s) != hipSuccess) return FA_ERR_LAUNCH;
    if (hipLaunchKernel(k2, dim3((unsigned)grid2), dim3(d), args, 0, s) != hipSuccess) return FA_ERR_LAUNCH;
    return FA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- FP8 forward

namespace {

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Fp8Layout {
    size_t q8, k8, v8, scales, total;
    int nblk;   // 64-row blocks of the longer of q and k: the scales' row stride
};

Fp8Layout fp8_layout(int B, int Nq, int Nk, int H) {
    Fp8Layout L;
    const size_t bh = (size_t)B * H;
    L.nblk = (std::max(Nq, Nk) + kFp8QuantRows - 1) / kFp8QuantRows;
    L.q8 = 0;
    L.k8 = L.q8 + round256(bh * Nq * kFp8D);
    L.v8 = L.k8 + round256(bh * Nk * kFp8D);
    L.scales = L.v8 + round256(bh * Nk * kFp8D);
    L.total = L.scales + round256(3 * bh * L.nblk * sizeof(float));
    return L;
}

int check_fp8_shape(int B, int Nq, int Nk, int H, int d, float scale, int causal) {
    if (B <= 0 || Nq <= 0 || Nk <= 0 || H <= 0) return FA_ERR_SHAPE;
    if (d != kFp8D) return FA_ERR_UNSUPPORTED;
    if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
    // one sequence's K/V code rows go through a buffer resource (< 2 GiB)
    if ((int64_t)Nk * H * d >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 40;
    if ((int64_t)B * Nq * H * d > lim || (int64_t)B * Nk * H * d > lim) return FA_ERR_SHAPE;
    const int64_t n_tiles = (Nq + Fp8Cfg::BM - 1) / Fp8Cfg::BM;
    if (n_tiles * B * H > INT_MAX) return FA_ERR_SHAPE;
    const int64_t nblk = (std::max(Nq, Nk) + kFp8QuantRows - 1) / kFp8QuantRows;
    if (nblk * B * H > INT_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

int launch_fp8_attn(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                    const float* sv, int sq_stride, int sk_stride, void* o, float* lse, int B, int Nq,
                    int Nk, int H, float qk_scale, int causal, hipStream_t s) {
    Fp8AttnParams p;
    std::memset(&p, 0, sizeof(p));
    p.q8 = static_cast<const uint8_t*>(q8);
    p.k8 = static_cast<const uint8_t*>(k8);
    p.v8 = static_cast<const uint8_t*>(v8);
    p.sq = sq;
    p.sk = sk;
    p.sv = sv;
    p.o = static_cast<bf16*>(o);
    p.lse = lse;
    p.batch = B;
    p.H = H;
    p.nq = Nq;
    p.nk = Nk;
    p.n_tiles = (Nq + Fp8Cfg::BM - 1) / Fp8Cfg::BM;
    p.sq_stride = sq_stride;
    p.sk_stride = sk_stride;
    p.qk_scale_log2 = qk_scale * kLog2e;
    const int grid = p.n_tiles * H * B;
    void* args[] = {&p};
    const void* k = causal ? reinterpret_cast<const void*>(fa_fwd_fp8_kernel<true>)
                           : reinterpret_cast<const void*>(fa_fwd_fp8_kernel<false>);
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3(Fp8Cfg::NW * 64), args, 0, s) == hipSuccess
               ? FA_OK
               : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t fa_fp8_workspace_bytes(int B, int Nq, int Nk, int H, int d) {
    if (B <= 0 || Nq <= 0 || Nk <= 0 || H <= 0 || d != kFp8D) return 0;
    return fp8_layout(B, Nq, Nk, H).total;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* signs, void* o, float* lse,
               void* workspace, size_t workspace_bytes, int B, int Nq, int Nk, int H, int d,
               float scale, int causal, int rotate, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (rotate != 0 && rotate != 1) return FA_ERR_UNSUPPORTED;
    if (rotate && !signs) return FA_ERR_NULL;
    int st = check_fp8_shape(B, Nq, Nk, H, d, scale, causal);
    if (st) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        (rotate && !aligned(signs, 4)) || !aligned(workspace, 256))
        return FA_ERR_ALIGN;
    const Fp8Layout L = fp8_layout(B, Nq, Nk, H);
    if (!workspace || workspace_bytes < L.total) return FA_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    Fp8QuantParams qp;
    std::memset(&qp, 0, sizeof(qp));
    qp.x[0] = static_cast<const bf16*>(q);
    qp.x[1] = static_cast<const bf16*>(k);
    qp.x[2] = static_cast<const bf16*>(v);
    qp.codes[0] = reinterpret_cast<uint8_t*>(ws + L.q8);
    qp.codes[1] = reinterpret_cast<uint8_t*>(ws + L.k8);
    qp.codes[2] = reinterpret_cast<uint8_t*>(ws + L.v8);
    qp.scales = reinterpret_cast<float*>(ws + L.scales);
    qp.signs = signs;
    qp.n[0] = Nq;
    qp.n[1] = Nk;
    qp.n[2] = Nk;
    qp.B = B;
    qp.H = H;
    qp.nblk = L.nblk;
    qp.rotate = rotate;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* args[] = {&qp};
    const dim3 qgrid((unsigned)(B * H * L.nblk), 3);
    if (hipLaunchKernel(reinterpret_cast<const void*>(fp8_quant_kernel), qgrid, dim3(256), args, 0, s) != hipSuccess)
        return FA_ERR_LAUNCH;
    const size_t plane = (size_t)B * H * L.nblk;
    const float qk_scale = rotate ? scale / (float)d : scale;
    return launch_fp8_attn(qp.codes[0], qp.codes[1], qp.codes[2], qp.scales, qp.scales + plane,
                           qp.scales + 2 * plane, L.nblk, L.nblk, o, lse, B, Nq, Nk, H, qk_scale, causal, s);
}

int fa_fwd_fp8_codes(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                     const float* sv, void* o, float* lse, int B, int Nq, int Nk, int H, int d,
                     float qk_scale, int causal, void* stream) {
    if (!q8 || !k8 || !v8 || !sq || !sk || !sv || !o || !lse) return FA_ERR_NULL;
    int st = check_fp8_shape(B, Nq, Nk, H, d, qk_scale, causal);
    if (st) return st;
    if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(sq, 4) || !aligned(sk, 4) || !aligned(sv, 4))
        return FA_ERR_ALIGN;
    return launch_fp8_attn(q8, k8, v8, sq, sk, sv, (Nq + kFp8QuantRows - 1) / kFp8QuantRows,
                           (Nk + kFp8QuantRows - 1) / kFp8QuantRows, o, lse, B, Nq, Nk, H, qk_scale,
                           causal, static_cast<hipStream_t>(stream));
}

}  // extern "C"
