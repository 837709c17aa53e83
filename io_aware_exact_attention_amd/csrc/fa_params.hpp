// Kernel argument bundle and per-sequence addressing shared by all kernels.
#pragma once

#include "fa_device.hpp"

namespace fa355 {

struct AttnParams {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const bf16* o_in;    // backward: forward output O
    const bf16* dout;    // backward: dO
    const float* lse_in; // backward: forward LSE
    bf16* o;             // forward output
    float* lse;          // forward LSE
    bf16* dq;
    bf16* dk;
    bf16* dv;
    float* dvec;         // backward workspace plane 0: -D_i = -rowsum(dO * O), laid out like lse
    float* lse2;         // backward workspace plane 1: LSE_i * log2(e), laid out like lse
    const int* cu_q;     // varlen prefix offsets (nseq+1), else null
    const int* cu_k;
    int batch;           // B, or nseq for varlen
    int H;
    int nq;              // Nq, or max_seqlen_q for varlen (also the lse row stride)
    int nk;              // Nk, or max_seqlen_k for varlen
    int n_tiles;         // tiles of the kernel's own outer axis per (batch, head)
    float scale;         // multiplies Q K^T
    float scale_log2;    // scale * log2(e)
};

// Token range of batch entry / sequence b: rows [q0, q0+nq) of q, [k0, k0+nk) of k.
// A packed sequence's lengths are clamped to [0, max_seqlen]: offsets that break
// the documented precondition (a sequence longer than max_seqlen, decreasing
// offsets) then leave rows uncomputed instead of indexing past the
// [nseq, H, max_seqlen_q] planes of lse and the backward workspace.
template <bool VARLEN>
__device__ __forceinline__ void seq_range(const AttnParams& p, int b, int& q0, int& nq,
                                          int& k0, int& nk) {
    if constexpr (VARLEN) {
        q0 = p.cu_q[b];
        nq = min(max(p.cu_q[b + 1] - q0, 0), p.nq);
        k0 = p.cu_k[b];
        nk = min(max(p.cu_k[b + 1] - k0, 0), p.nk);
    } else {
        q0 = b * p.nq;
        nq = p.nq;
        k0 = b * p.nk;
        nk = p.nk;
    }
}

}  // namespace fa355
