/*
 * fa.h — C ABI of an MI355X (gfx950) exact-attention forward library.
 *
 * What is computed.  For each (batch b, head h), with per-head matrices
 * Q [Nq x d], K [Nk x d], V [Nk x d]:
 *
 *     S = scale * Q K^T,   P = softmax(S) row-wise,   O = P V,
 *     LSE_i = ln sum_j exp(S_ij)
 *
 * exactly (not an approximation), but without ever writing S or P to device
 * memory: keys are streamed tile by tile and each query row carries a running
 * state (m = largest score so far, l = sum of exp(s - m), u = sum of
 * exp(s - m) v), rescaled whenever m grows, with O = u / l formed once at the
 * end.  Sources: FlashAttention explainer (cztcode.com/2026/5368) §1 for the
 * definition and the N x N intermediates, §2 for the (m, l, u) recurrence,
 * §3 for merging the states of two key blocks and for the saved normalisation
 * statistics, §6 for causal block skipping and the prefill/decode split;
 * Flash Attention wiki note (astro-wiki) "Online Softmax", "Tiling" and the
 * FlashAttention-2 notes (query-tile-outer loop order, division deferred to
 * the end); AI圣经13 FlashAttention review (chengyansuo.com) §03 (one fused
 * kernel; statistics kept for recomputation; head dimension 64 to 128).
 *
 * Conventions (where the pages are silent):
 *   - causal masking is bottom-right aligned: query i sees key j iff
 *     j <= i + (Nk - Nq);
 *   - a query row that sees no key gets O = 0 and LSE = -inf;
 *   - LSE is float32, natural log, of the scaled scores;
 *   - O has the dtype of the inputs.
 *
 * Ownership and threading.  The caller allocates and owns every buffer
 * (inputs, outputs, workspace) and picks the stream.  The library allocates
 * no device memory, keeps no pointer after a call returns and holds no
 * mutable global state beyond a cache of each device's compute-unit count
 * (read on first use, never changed after); calls are thread-safe.
 *
 * Alignment.  q, k, v, o, kcache, vcache and the workspace must be 16-byte
 * aligned; lse, seqlens, offsets and the decode output 4-byte aligned
 * (FA_ERR_INVALID_ARG / FA_ERR_WORKSPACE otherwise).
 *
 * Errors.  Every entry point returns an fa_status and never throws.  All
 * argument checks run before any HIP call, so an invalid call has no side
 * effect.  FA_OK means the work was enqueued on `stream` (results are valid
 * once the stream has reached that point).  A failed launch returns
 * FA_ERR_HIP.  Device-side contract violations (seqlens[b] > max_seqlen,
 * cache ranges out of bounds, overlapping input/output buffers) are undefined
 * behaviour.  There is no fallback path: an unsupported request fails.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, non-finite scale, size too large */
  FA_ERR_UNSUPPORTED = -2, /* head dimension other than 64 or 128 */
  FA_ERR_WORKSPACE = -3,   /* decode workspace missing or smaller than required */
  FA_ERR_HIP = -4,         /* the HIP runtime refused the launch */
  FA_ERR_SCRATCH = -5      /* more chunk state than fa_decode_varlen_noalloc's fixed scratch */
} fa_status;

/*
 * Prefill / general forward pass, bf16 inputs and output.
 *
 *   q   bf16 [B, H, Nq, d]  contiguous, row-major (device)
 *   k   bf16 [B, H, Nk, d]  contiguous (device)
 *   v   bf16 [B, H, Nk, d]  contiguous (device)
 *   o   bf16 [B, H, Nq, d]  contiguous, written (device)
 *   lse fp32 [B, H, Nq]     written (device)
 *   d in {64, 128}; B, H, Nq, Nk >= 1; Nq, Nk <= 2^30 (longer sequences
 *   return FA_ERR_INVALID_ARG); scale finite (usually 1/sqrt(d));
 *   causal != 0 applies the bottom-right causal mask and skips key tiles that
 *   lie wholly above the diagonal (explainer §6).
 *
 * Products of bf16 inputs accumulate in fp32; the softmax runs in fp32; P is
 * rounded to bf16 (nearest-even) before the P V product.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           hipStream_t stream);

/*
 * Same contract with fp32 q, k, v, o: the explainer's §1 definition and §2
 * running-state recurrence evaluated in plain fp32 throughout (no
 * reduced-precision products), so the result differs from the exact one only
 * by fp32 rounding.  A parity kernel, not a fast path.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int Nq, int Nk, int d, float scale, int causal,
               hipStream_t stream);

/*
 * Block-sparse forward (review §05: long sequences by skipping whole tiles
 * through a sparsity pattern; the pages give no pattern, so it is an input).
 * Key j is visible to query i only if block_mask admits the pair of 64-row /
 * 64-key blocks, and with causal != 0 also j <= i + Nk - Nq.  Tiles the mask
 * excludes for a whole workgroup of 256 queries are neither loaded nor
 * computed.
 *
 *   block_mask  uint8 [H, ceil(Nq / 64), ceil(Nk / 64)] (device), nonzero =
 *               admitted; shared by the batch
 *   the rest    as for fa_fwd; d must be 128 (else FA_ERR_UNSUPPORTED) and
 *               ceil(Nk / 64) <= 1024
 *
 * A row with no visible key gets O = 0 and LSE = -inf.
 */
int fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                        const uint8_t* block_mask, int B, int H, int Nq, int Nk, int d,
                        float scale, int causal, hipStream_t stream);

/*
 * Backward pass by recomputation (review §03: the forward keeps only O and the
 * row statistics; the backward rebuilds the score and probability blocks on
 * chip).  Gradients of L with respect to q, k, v for a given dL/dO, for the
 * same attention fa_fwd computes (same scale, same causal alignment).
 *
 *   q, k, v, o, dout  bf16 [B, H, N, d]   (device); o and lse from fa_fwd
 *   lse               fp32 [B, H, Nq]     (device)
 *   dq                fp32 [B, H, Nq, d]  written (device)
 *   dk, dv            fp32 [B, H, Nk, d]  written (device)
 *   workspace         device scratch of at least fa_bwd_workspace_bytes(B, H,
 *                     Nq) bytes (the row terms of the pass), owned by the
 *                     caller, no initialisation needed; calls that run at the
 *                     same time must not share it
 *   d                 64 or 128
 *
 * Alignment as for fa_fwd (dq, dk, dv 16-byte aligned); errors as for fa_fwd,
 * plus FA_ERR_WORKSPACE.  Three kernels are enqueued on `stream`.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Nq);
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, float* dq, float* dk, float* dv,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Forward over a packed batch of sequences of different lengths (variable
 * length / padding-free prefill; the pages list padding masks among the
 * semantics to get right).  Every sequence attends only within itself; with
 * causal != 0 query i of a sequence with Lq queries and Lk keys sees key j iff
 * j <= i + Lk - Lq (bottom-right: its queries are the last of its keys, as in
 * a chunked prefill that appends Lq tokens to Lk - Lq cached ones).
 *
 *   q             bf16 [total_q, H, d]     token-major, contiguous (device)
 *   k, v          bf16 [total_k, H, d]     (device)
 *   o             bf16 [total_q, H, d]     written (device)
 *   lse           fp32 [H, total_q]        written (device)
 *   cu_seqlens_q  int32 [B + 1]            cu[0] = 0, non-decreasing,
 *   cu_seqlens_k  int32 [B + 1]            cu[B] = total rows (device);
 *                 sequence b owns rows cu[b] .. cu[b+1]-1
 *   total_q       query rows (host); max_seqlen_q an upper bound of every
 *                 sequence's query count (host; sizes the grid, no device
 *                 read on the host), 1 <= max_seqlen_q <= min(total_q, 2^30)
 *   d             64 or 128
 *
 * A query row that sees no key gets O = 0 and LSE = -inf.  Errors as for
 * fa_fwd; the cu_seqlens contract is on the caller (device data).
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int B, int H, int d, int total_q, int max_seqlen_q, float scale, int causal,
                  hipStream_t stream);

/*
 * Decode: one new query per sequence over a packed, variable-length KV cache
 * (explainer §6: a single query sees its whole history; batched decode mixes
 * history lengths).  Each sequence's keys are cut into chunks that are
 * processed in parallel; each chunk leaves a partial state (m, l, u) in the
 * workspace, and the states of a sequence are merged with the block-merge
 * rule of explainer §3/§7 (a sequence that fits in one chunk is finished on
 * the spot).  Calls of at most 4096 chunk workgroups in all (B x H x chunks),
 * at most 1024 chunks per sequence, are merged by the chunk of each sequence
 * that finishes last, in the same launch; larger calls get a second, merging
 * kernel, which costs them less than the last arriver's coherent writes.
 *
 *   q        bf16 [B, H, d]        (device)
 *   kcache   bf16 [T, H, d]        token-major (device)
 *   vcache   bf16 [T, H, d]        token-major (device)
 *   seqlens  int32 [B]             history length of each sequence (device)
 *   offsets  int32 [B]             first cache row of each sequence (device);
 *                                  sequence b owns rows offsets[b] ..
 *                                  offsets[b] + seqlens[b] - 1
 *   o        bf16 [B, H, d]        written (device)
 *   lse      fp32 [B, H]           written (device)
 *   max_seqlen  an upper bound of seqlens[] (host; sizes the grid, so no
 *               device-to-host copy is needed); 0 <= seqlens[b] <= max_seqlen
 *               <= 2^30; B and H at most 65535
 *   workspace   device scratch of at least fa_decode_workspace_bytes(B, H, d,
 *               max_seqlen) bytes, owned by the caller.  Its first 65536 bytes
 *               are arrival counters: they must be ZERO before the first call
 *               that uses the workspace (zero-fill it once after allocating
 *               it: hipMemset, torch.zeros), and every call leaves them zero
 *               again when it completes, so a workspace can serve any number
 *               of later calls, of any shape, without clearing.  The rest
 *               needs no initialisation.  Calls that run at the same time must
 *               not share a workspace.
 *
 * A sequence with seqlens[b] == 0 gets O = 0 and LSE = -inf.  Cache row
 * addresses are computed in 64-bit, so T * H * d may exceed 2^31.
 * fa_decode_workspace_bytes returns 0 for invalid arguments.
 */
size_t fa_decode_workspace_bytes(int B, int H, int d, int max_seqlen);
int fa_decode_varlen(const void* q, const void* kcache, const void* vcache,
                     const int32_t* seqlens, const int32_t* offsets,
                     void* o, float* lse,
                     int B, int H, int d, int max_seqlen, float scale,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * The chunk size fa_decode_varlen picks (keys per chunk): 256, doubled while
 * the grid would exceed 16384 workgroups or a sequence 256 chunks.  0 for
 * invalid arguments.
 */
int fa_decode_split_keys(int B, int H, int d, int max_seqlen);

/*
 * fa_decode_varlen with the chunk size given (for tuning and tests): the same
 * contract, plus
 *   split_keys  keys per chunk, a positive multiple of 64 giving at most 4096
 *               chunks for max_seqlen (FA_ERR_INVALID_ARG otherwise)
 *   workspace   at least fa_decode_split_workspace_bytes(B, H, d, max_seqlen,
 *               split_keys) bytes, with the same counter rule
 * fa_decode_split_workspace_bytes(..., 0) equals fa_decode_workspace_bytes;
 * it returns 0 for invalid arguments.
 */
size_t fa_decode_split_workspace_bytes(int B, int H, int d, int max_seqlen, int split_keys);
int fa_decode_varlen_split(const void* q, const void* kcache, const void* vcache,
                           const int32_t* seqlens, const int32_t* offsets,
                           void* o, float* lse,
                           int B, int H, int d, int max_seqlen, float scale, int split_keys,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Decode over a paged KV cache (explainer §6 names paging as the concern of
 * batched decode): the same computation as fa_decode_varlen, but the cache is
 * a pool of fixed-size pages and each sequence lists its pages in a block
 * table.  Key t of sequence b is in page block_table[b * max_blocks + t /
 * page_size], slot t % page_size.
 *
 *   q            bf16 [B, H, d]                         (device)
 *   kpages       bf16 [num_pages, page_size, H, d]      (device)
 *   vpages       bf16 [num_pages, page_size, H, d]      (device)
 *   block_table  int32 [B, max_blocks]                  (device); entries
 *                j < ceil(seqlens[b] / page_size) must lie in [0, num_pages)
 *                (an entry outside reads page num_pages - 1 instead of
 *                faulting; later entries are never read)
 *   seqlens      int32 [B]                              (device)
 *   o, lse, max_seqlen, scale: as for fa_decode_varlen
 *   workspace    at least fa_decode_split_workspace_bytes(B, H, d, max_seqlen,
 *                split_keys or, for 0, fa_decode_paged_split_keys(...)) bytes,
 *                with the counter rule of fa_decode_varlen
 *   page_size    tokens per page, a power of two, 1 .. 65536
 *   max_blocks   entries per block-table row; max_blocks * page_size >=
 *                max_seqlen, else FA_ERR_INVALID_ARG
 *   split_keys   as for fa_decode_varlen_split, and a chunk may span at most
 *                1024 pages (ceil(split_keys / page_size) + 1 <= 1024); 0 lets
 *                the library choose, as fa_decode_paged_split_keys reports
 *
 * fa_decode_paged_split_keys: the chunk size the library picks for split_keys
 * = 0 (the packed plan, halved while a chunk would span more than 1024
 * pages); 0 for invalid arguments or when no chunk size meets both the page
 * limit and the 4096-chunk limit (fa_decode_paged then rejects split_keys =
 * 0).  Every nonzero value it returns is accepted by fa_decode_paged.
 */
int fa_decode_paged_split_keys(int B, int H, int d, int max_seqlen, int page_size);
int fa_decode_paged(const void* q, const void* kpages, const void* vpages,
                    const int32_t* block_table, const int32_t* seqlens,
                    void* o, float* lse,
                    int B, int H, int d, int page_size, int num_pages, int max_blocks,
                    int max_seqlen, float scale, int split_keys,
                    void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * fa_decode_varlen without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same computation, arguments and results as
 * fa_decode_varlen with the automatic chunk size, minus the workspace: the
 * chunk states go to a fixed scratch array of FA_DECODE_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library holds on each device it runs on until the
 * process ends, and a second kernel merges them.  The call allocates and
 * frees nothing.
 *
 * Limit: B * H * ceil(max_seqlen / fa_decode_split_keys(B, H, d, max_seqlen))
 * * (d + 2) * 4 bytes must not exceed the scratch (e.g. 64 sequences x 32
 * heads of up to 16384 keys at d = 128 use 8.5 MB); larger calls return
 * FA_ERR_SCRATCH before any HIP call.  Nothing in the scratch needs to start
 * at zero.  All calls on one device share its scratch: calls that overlap in
 * time on one device (other streams, other threads) race and give wrong
 * results; calls ordered on one stream are safe.  The first call on a device
 * looks up that device's scratch address (a runtime query, no allocation).
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_decode_varlen_noalloc(const void* q, const void* kcache, const void* vcache,
                             const int32_t* seqlens, const int32_t* offsets,
                             void* o, float* lse,
                             int B, int H, int d, int max_seqlen, float scale,
                             hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
