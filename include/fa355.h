/*
 * fa355.h — C ABI of libfa355: exact, IO-aware softmax attention on MI355X (gfx950).
 *
 * What is computed (per batch entry b and head h):
 *     S = scale * Q K^T            (Nq x Nk scores)
 *     P = softmax(S) row by row    (causal: key j is visible to query i iff j <= i)
 *     O = P V
 *     LSE_i = m_i + ln(l_i)        (row maximum m_i of S and denominator l_i)
 * The definition is "08 · FlashAttention", §一; the per-row log-sum-exp kept for
 * the backward is "LLM Systems 22: Flash Attention", §3.2 (Backward:
 * Recomputation).  The forward never writes S or P to device memory: it runs the
 * online-softmax update of "08 · FlashAttention", §二 over key tiles held on chip.
 * The backward recomputes P tile by tile from LSE (same §3.2) and returns
 * dQ, dK, dV of L = sum(O * dO).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *     The library allocates nothing, keeps no mutable global state (apart from
 *     fa_bwd_noalloc's static device array, described there) and never
 *     synchronises the device; all work is enqueued on `stream` (a hipStream_t,
 *     NULL for the default stream) in stream order and returns immediately.
 *   - q, k, v, o, dout, dq, dk, dv are bf16 (IEEE bfloat16), contiguous, with the
 *     head dimension fastest:
 *         dense   [B, N, H, d]   element (b, n, h, c) at ((b*N + n)*H + h)*d + c
 *         packed  [total, H, d]  (varlen) row t = token t of the packed batch
 *     These are the [total, num_heads, head_size] tensors of the mha_fwd entry
 *     point in "Flash Attention 实现深度解析", §3.1.  Pointers must be 16-byte
 *     aligned.
 *   - lse is fp32: dense [B, H, Nq]; varlen [nseq, H, max_seqlen_q] (rows at or
 *     past a sequence's length are not written).  Natural-log units of the
 *     scaled scores.  4-byte aligned.
 *   - d must be 64 or 128.  Causal dense calls need Nq == Nk.  Only the causal
 *     mask is supported; no arbitrary masks ("08 · FlashAttention", §四 lists
 *     these limits of the method's kernels and asks for an error, never a silent
 *     fallback).
 *   - Every call validates its arguments on the host before launching anything.
 *     On a validation error nothing is enqueued or written and a negative
 *     fa_status is returned.  A failed launch returns FA_ERR_LAUNCH.  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Calls are reentrant and thread-safe (no shared mutable state; fa_bwd_noalloc
 *     calls that overlap on one GPU share its device array, see there).
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = -1,        /* a required pointer is NULL                         */
    FA_ERR_SHAPE = -2,       /* a size is <= 0, or sizes are inconsistent/too big   */
    FA_ERR_UNSUPPORTED = -3, /* d not in {64,128}, causal with Nq != Nk, bad scale,
                                one sequence's rows of a tensor >= 2 GiB */
    FA_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte (fp32: 4-byte) aligned */
    FA_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch            */
    FA_ERR_WORKSPACE = -6    /* workspace missing or smaller than required          */
} fa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int fa_version(void);

/*
 * Forward, dense batch.
 *   q [B,Nq,H,d], k,v [B,Nk,H,d]  (read)      o [B,Nq,H,d] (written)
 *   lse [B,H,Nq] fp32 (written)
 *   scale: multiplies Q K^T (1/sqrt(d) for standard attention); must be finite and > 0.
 *   causal: 0 or 1.
 * Kernel choice (every choice computes the same O and LSE within rounding):
 *   - causal, with at most one query tile (128 rows) of all (batch, head) pairs
 *     per CU, or at most two per CU and at least 16 tiles per sequence: the
 *     key-split kernel, one 8-wave work-group per query tile whose two halves
 *     of waves take half of the tile's key tiles each and merge their running
 *     (max, sum, O) through LDS ("LLM Systems 22: Flash Attention", §4.1.5
 *     load balancing: the longest tile's chain of key tiles is halved);
 *   - otherwise, when the tiles fit on the GPU at once (two work-groups per
 *     CU), or causal with at most 32 query tiles per sequence (N <= 4096):
 *     fa_fwd_persistent's kernel (bitwise the per-tile kernel's results);
 *   - otherwise one work-group per query tile.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream);

/*
 * Forward, dense batch, as a persistent kernel ("LLM Systems 22: Flash
 * Attention", §4.1.4 Persistent Kernels, §4.1.5 Load Balancing: longest-
 * processing-time first): a fixed grid of about as many work-groups as the CUs
 * hold at once loops over the query tiles, each XCD working on its own (batch,
 * head) pairs.  When the tiles fit in one round they are taken longest first
 * over all pairs (every pair's tile with the most causal keys, then the next,
 * ...); otherwise each XCD takes its pairs one after another, each pair's tiles
 * longest first, so that its resident work-groups share a few pairs' K/V in L2.  Arguments, results and errors as fa_fwd; the
 * outputs are bitwise those of fa_fwd wherever fa_fwd does not take the
 * key-split kernel (the same tile computation).
 */
int fa_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream);

/*
 * Forward, packed variable-length batch ("08 · FlashAttention", §四: packing
 * with cu_seqlens instead of a padding mask).
 *   cu_seqlens_q, cu_seqlens_k: int32 device arrays of nseq+1 prefix offsets,
 *   starting at 0 and non-decreasing; sequence s owns rows [cu[s], cu[s+1]).
 *   max_seqlen_q / max_seqlen_k bound every sequence length (precondition; with
 *   the environment variable FA355_VALIDATE_CU_SEQLENS=1 the offsets are copied to
 *   the host and checked, which synchronises the stream).
 *   Causal varlen needs equal query and key lengths per sequence.
 *   q [total_q,H,d], k,v [total_k,H,d], o [total_q,H,d], lse [nseq,H,max_seqlen_q].
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                  int max_seqlen_q, int max_seqlen_k, int H, int d, float scale,
                  int causal, void* stream);

/*
 * Bytes of device workspace fa_bwd / fa_bwd_varlen need: two fp32 planes, each
 * with one value per query row and head laid out like lse: -D_i, where
 * D_i = sum_c dO_ic * O_ic, then LSE_i * log2(e).
 * batch_or_nseq = B (dense) or nseq (varlen); nq = Nq (dense) or max_seqlen_q.
 * Returns 0 for non-positive arguments.
 */
size_t fa_bwd_workspace_bytes(int batch_or_nseq, int H, int nq, int d);

/*
 * Backward, dense batch.  Inputs q, k, v, o, dout [B,N,H,d] and lse from the
 * forward with the same arguments; outputs dq [B,Nq,H,d], dk, dv [B,Nk,H,d]
 * (fully overwritten).  workspace: device buffer of at least
 * fa_bwd_workspace_bytes(B,H,Nq,d) bytes, 4-byte aligned; its contents on entry
 * do not matter and on return are unspecified.
 * Kernels: fa_bwd_dq_dot's then fa_bwd_dkdv's; for small grids (at most 6
 * causal or 2 non-causal dK/dV plus dQ tiles of 128 rows per CU) fa_bwd_dot's
 * kernel, then one launch holding both passes' tiles, so that each pass's causal
 * tail overlaps the other's work ("LLM Systems 22: Flash Attention", §4.1.5
 * load balancing).  Causal passes of more than 2 tiles per CU and either at
 * most 8 per CU, or at most 32 tiles per sequence with rounds of the CUs' work-
 * group slots times tiles per sequence at most 256, run on a persistent grid of
 * two work-groups per CU that deals the tiles in the same order.  Every form
 * gives the same gradients bit for bit.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int H, int Nq, int Nk, int d, float scale,
           int causal, void* stream);

/*
 * Backward, dense batch, that allocates nothing: for callers that cannot call
 * hipMalloc or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments, results and errors as
 * fa_bwd without the workspace.  The backward's two fp32 planes (8*B*H*Nq bytes)
 * live instead in a static device array of FA_BWD_NOALLOC_MAX_BYTES bytes that
 * each GPU the library runs on holds until the process ends; larger calls fail
 * with FA_ERR_WORKSPACE.  The array's device address is looked up once per
 * device, on the first call with that device current (FA_ERR_LAUNCH if that
 * fails).  Every call on one GPU uses the same array: calls that may overlap on
 * one GPU (different streams without ordering between them) race on it and
 * give undefined gradients; stream-ordered calls are safe.  Nothing in the array
 * needs clearing: each call writes every value it later reads.
 */
#define FA_BWD_NOALLOC_MAX_BYTES ((size_t)16 << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, void* stream);

/*
 * The backward's stages, exposed separately (dense batch only) for callers that
 * time them or need only some gradients.  Arguments mean what they mean in
 * fa_bwd; `workspace` is fa_bwd's workspace (fa_bwd_workspace_bytes(B,H,Nq,d)
 * bytes, 4-byte aligned).
 *   fa_bwd_dq_dot: dQ, and fills the workspace as fa_bwd_dot does, from q, k,
 *                  v, o, dout and lse                          (writes dq)
 *   fa_bwd_dot:    fills the workspace: -D_i (D_i = sum_c dO_ic * O_ic) and
 *                  LSE_i * log2(e), from o, dout and lse
 *   fa_bwd_dkdv:   dK, dV from q, k, v, dout and the workspace (writes dk, dv)
 *   fa_bwd_dq:     dQ from q, k, v, dout and the workspace     (writes dq)
 * fa_bwd is fa_bwd_dq_dot then fa_bwd_dkdv.  fa_bwd_dkdv and fa_bwd_dq need a
 * workspace that fa_bwd_dq_dot or fa_bwd_dot filled on the same stream; both fill
 * it with the same values bit for bit.  Errors as fa_bwd.
 */
int fa_bwd_dq_dot(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* workspace, size_t workspace_bytes, void* dq, int B,
                  int H, int Nq, int Nk, int d, float scale, int causal, void* stream);
int fa_bwd_dot(const void* o, const void* dout, const float* lse, void* workspace,
               size_t workspace_bytes, int B, int H, int Nq, int d, void* stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                const void* workspace, size_t workspace_bytes, void* dk, void* dv, int B, int H,
                int Nq, int Nk, int d, float scale, int causal, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
              const void* workspace, size_t workspace_bytes, void* dq, int B, int H, int Nq,
              int Nk, int d, float scale, int causal, void* stream);

/* Backward, packed variable-length batch; arguments as fa_fwd_varlen and fa_bwd. */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  void* workspace, size_t workspace_bytes, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int nseq, int max_seqlen_q, int max_seqlen_k,
                  int H, int d, float scale, int causal, void* stream);

/*
 * Decoding ("LLM Systems 22: Flash Attention", §5.1 Motivation, §5.2 Solution):
 * Nq new query tokens per sequence (typically 1..4) against an Nk-token
 * key/value cache, Hq query heads grouped onto Hkv key/value heads (query head
 * h reads key/value head h / (Hq/Hkv)).  The keys are split into chunks
 * processed in parallel (split-KV); each chunk's normalised output and
 * log-sum-exp go to the workspace and a second kernel merges them.  The query
 * heads of one group and the Nq tokens are packed into the rows of one matrix
 * tile (GQA packing).
 *   q [B,Nq,Hq,d], k, v [B,Nk,Hkv,d], o [B,Nq,Hq,d] bf16; lse [B,Hq,Nq] fp32,
 *   natural log of the scaled scores.  d in {64,128}; Hkv must divide Hq.
 *   causal: the Nq tokens are the newest positions, token i sees keys
 *   j <= i + Nk - Nq (needs Nq <= Nk); otherwise every key.
 *   workspace: at least fa_decode_workspace_bytes(...) bytes, 16-byte aligned,
 *   contents irrelevant on entry and unspecified on return.
 * Errors as fa_fwd; FA_ERR_WORKSPACE for a missing or small workspace,
 * FA_ERR_UNSUPPORTED also when Nk * Hkv * d * 2 bytes reach 2 GiB.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d);
int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                  size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                  int causal, void* stream);

/*
 * FP8 forward ("LLM Systems 22: Flash Attention", §4.1.3 Low-precision - FP8):
 * the forward with both products on e4m3 operands.  Q and K are first
 * multiplied by the random orthogonal J = diag(signs) H_d / sqrt(d) (H_d the
 * Sylvester Hadamard matrix), which leaves Q K^T unchanged and spreads outlier
 * dimensions before quantisation; V is quantised as it is.  Each block of 64
 * rows of each (batch, head) of each tensor gets one power-of-two scale
 * s = 2^ceil(log2(amax / 448)) and codes e4m3(x / s) (OCP E4M3, round to
 * nearest even).  The probabilities are quantised as e4m3(16 * exp(S - m))
 * for the P V product, m a per-row reference maximum that moves, over 64-key
 * tiles, only when a tile's maximum exceeds it by more than ln 16 (the
 * conditional rescale of "LLM Systems 22: Flash Attention", §4.2.1; so
 * exp(S - m) <= 16); the row sums use the unrounded values.
 *   q [B,Nq,H,d], k, v [B,Nk,H,d], o [B,Nq,H,d] bf16; lse [B,H,Nq] fp32.
 *   d must be 128.  causal needs Nq == Nk.  Inputs must be finite.
 *   signs: device fp32 [d], each +1 or -1 (required when rotate = 1; ignored
 *   when rotate = 0, which quantises Q and K unrotated).
 *   workspace: at least fa_fp8_workspace_bytes(...) bytes, 256-byte aligned;
 *   on return it holds, at offsets rounded up to 256 bytes, the codes of q
 *   [B,Nq,H,d], k and v [B,Nk,H,d] (uint8), then the scales [3][B*H][nblk]
 *   fp32 (q, k, v; nblk = ceil(max(Nq, Nk) / 64); entries past a tensor's own
 *   blocks are unused).
 * Errors as fa_fwd; FA_ERR_UNSUPPORTED for d != 128 or when Nk*H*d bytes reach
 * 2 GiB; FA_ERR_WORKSPACE for a missing or small workspace.
 */
size_t fa_fp8_workspace_bytes(int B, int Nq, int Nk, int H, int d);
int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* signs, void* o, float* lse,
               void* workspace, size_t workspace_bytes, int B, int Nq, int Nk, int H, int d,
               float scale, int causal, int rotate, void* stream);

/*
 * The attention stage of fa_fwd_fp8 alone, over caller-supplied e4m3 codes
 * q8 [B,Nq,H,d], k8, v8 [B,Nk,H,d] (uint8, 16-byte aligned) and power-of-two
 * scales per 64-row block, sq [B*H][ceil(Nq/64)], sk, sv [B*H][ceil(Nk/64)]
 * fp32: S_ij = qk_scale * sq(i) * sk(j) * (q8_i . k8_j),
 * O_i = sum_j e4m3(16 P~_ij) sv(j) v8_j / (16 l_i), P~ and l as above.  d must be 128; scales
 * that are not powers of two give unspecified results.
 */
int fa_fwd_fp8_codes(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                     const float* sv, void* o, float* lse, int B, int Nq, int Nk, int H, int d,
                     float qk_scale, int causal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
