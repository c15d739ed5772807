/*
 * libfa355 — exact tiled attention (FlashAttention forward) for AMD MI355X (gfx950).
 *
 * The operation (all entry points): for every query row i of a (batch, head)
 * or packed sequence,
 *     O_i = sum_j P_ij V_j,   P_ij = exp(S_ij - m_i) / l_i,   S_ij = scale * <Q_i, K_j>,
 *     m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i),  lse_i = m_i + ln l_i,
 * over the keys j visible to row i.  This is standard attention as the Ascend
 * CANN ops-transformer FlashAttention explainer states it (section 背景: S = QKᵀ,
 * a row softmax, then times V) computed the way its section 原理 describes:
 * query-row blocks against streamed key/value blocks with a running maximum m
 * and running sum l (steps 1-4), so that S and P never reach device memory.
 * The result is exact attention; only floating-point rounding order differs
 * (Was FlashAttention bei Transformer-Inference verändert, opening section).
 *
 * Visibility: key j < Lk of the same sequence; with causal != 0 also
 * j <= i + Lk - Lq (lower-triangular mask, bottom-right aligned when Lq != Lk;
 * the Hugging Face Flash-Attention-2 integration guide, parameter table,
 * is_causal row).  A row with no visible key gets O = 0 and lse = -inf.
 *
 * Precision: Q, K, V and O share one element type.  Scores, the running
 * statistics and the output accumulator are float32.  For fp16/bf16 inputs
 * the probabilities are rounded to the input type (round-to-nearest-even)
 * before the P·V product; for fp32 inputs they stay fp32.  lse is float32,
 * natural log, of the scaled scores.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *    aligned, densely packed in the stated layout; the library never
 *    allocates, frees or retains them and keeps no state between calls.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; results are valid once the stream reaches them.
 *  - Validation happens before any HIP call.  Errors are returned as
 *    fa_status_t; nothing is printed, thrown or aborted.  FA_ERR_HIP reports a
 *    failed launch or a missing / non-gfx950 device.
 *  - `scale` must be finite and >= 0 (FA_ERR_INVALID_ARG otherwise).
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    on every run (fixed reduction order, no floating-point atomics).
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define FA355_API __attribute__((visibility("default")))
#else
#define FA355_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype_t;

/*
 * Status codes.  They map the error catalog of the Hugging Face
 * Flash-Attention-2 integration guide (section 常见错误排查: an unsupported
 * dtype, an unsupported head_dim, a GPU the kernels do not run on): dtype and
 * head_dim -> FA_ERR_UNSUPPORTED, device -> FA_ERR_HIP.  Arguments the guide's
 * calls would reject as malformed -> FA_ERR_INVALID_ARG; a caller workspace
 * that is too small -> FA_ERR_WORKSPACE.
 */
typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, size out of range, misaligned pointer, non-finite scale */
  FA_ERR_UNSUPPORTED = 2, /* head_dim not 64/128, unknown dtype, unsupported chunk size */
  FA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_bytes figure */
  FA_ERR_HIP = 4,         /* no usable gfx950 device, or a kernel launch failed */
  FA_ERR_TOO_LARGE = 5    /* fa_fwd_varlen_noalloc: the schedule exceeds the static scratch */
} fa_status_t;

/*
 * Fixed-length attention (prefill).
 *   q   : [B, Nq, H, D]   element type `dtype`
 *   k, v: [B, Nk, H, D]
 *   o   : [B, Nq, H, D]   written
 *   lse : [B, H, Nq] float32, written; may be NULL (not written)
 *   seqlens_k: device int32[B] or NULL.  If given, batch entry b has
 *       Lk = min(max(seqlens_k[b], 0), Nk) real keys and rows Lk..Nk-1 of k
 *       and v are padding that is never read into the result (key-padding mask;
 *       the slavadubrov.com page's question of whether the mask and cache
 *       layout are supported).  If NULL, Lk = Nk.  Lq = Nq always.
 *   D in {64, 128}; B, H >= 1; Nq, Nk >= 0 (Nq == 0 is a no-op; Nk == 0 gives
 *   empty rows).  scale is used as given (the Python binding defaults it to
 *   1/sqrt(D), the guide's softmax_scale default).
 */
FA355_API fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int D, float scale, int causal,
                   const int32_t* seqlens_k, fa_dtype_t dtype, void* stream);

/*
 * Fixed-length attention with the other mask families the Hugging Face
 * Flash-Attention-2 integration guide names (原因分析, item 1: prefix mask,
 * ALiBi).  Arguments as fa_fwd, plus:
 *   prefix: >= 0; only with causal = 1 (else FA_ERR_INVALID_ARG).  Keys
 *       0 .. prefix-1 are seen by every query as well (bidirectional over the
 *       prefix, causal after it): query i sees key j iff
 *       j <= i + Lk - Lq or j < prefix.  0 = plain causal.
 *   alibi_slopes: device float[H] or NULL (4-byte aligned).  If given, the
 *       score of query i and key j is scale * q.k - slope_h * |j - (i + Lk - Lq)|
 *       (for causal rows the usual slope_h * (j - i) form, up to a per-row
 *       constant that softmax ignores); lse includes the bias.
 * fp16 and bf16 only: fp32 with a prefix or slopes is FA_ERR_UNSUPPORTED.
 * fa_fwd(...) is fa_fwd_masked(..., 0, NULL, ...).
 */
FA355_API fa_status_t fa_fwd_masked(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int H, int Nq, int Nk, int D,
                                    float scale, int causal, const int32_t* seqlens_k,
                                    int prefix, const float* alibi_slopes,
                                    fa_dtype_t dtype, void* stream);

/*
 * Packed variable-length attention (the guide's flash_attn_varlen, FAQ 4).
 *   q   : [total_q, H, D];  k, v: [total_k, H, D];  o: like q
 *   lse : [H, total_q] float32 or NULL
 *   cu_seqlens_q, cu_seqlens_k: device int32[nseq + 1], non-decreasing,
 *       starting at 0; sequence s owns q rows cu_seqlens_q[s]..cu_seqlens_q[s+1]-1
 *       and k/v rows cu_seqlens_k[s]..cu_seqlens_k[s+1]-1, and attends only to
 *       its own keys.  cu_seqlens_q[nseq] must equal total_q.
 *   workspace: device buffer of at least fa_fwd_varlen_workspace_bytes(nseq,
 *       total_q) bytes, 16-byte aligned, used for the tile schedule; its
 *       contents on entry do not matter.  Two calls in flight on different
 *       streams need different workspaces.
 */
FA355_API size_t fa_fwd_varlen_workspace_bytes(int nseq, int total_q);
FA355_API fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int nseq, int total_q, int total_k, int H, int D, float scale,
                          int causal, void* workspace, size_t workspace_bytes,
                          fa_dtype_t dtype, void* stream);

/*
 * fa_fwd_varlen for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results, minus the workspace: the tile schedule goes to
 * a static device array of FA_NOALLOC_SCRATCH_BYTES per GPU, which the
 * library holds until the process ends.  The call allocates nothing.
 *   Limit: the schedule, 4 * (2 + 4 * nseq + 2 * tiles) bytes rounded up to
 *   256, with tiles = ceil(total_q / rows) + nseq and rows the query rows per
 *   workgroup of the instance (fa_fwd_varlen_workspace_bytes(nseq, total_q)
 *   is an upper bound), must fit: with 1 MiB that is, e.g., 1,000 sequences
 *   of 16 million packed query rows.  Larger calls return FA_ERR_TOO_LARGE
 *   before any HIP call.
 *   The array keeps the last call's contents; the schedule kernel rewrites
 *   every entry the forward reads, so nothing is cleared.  All calls on one
 *   GPU share its array: calls that overlap on one GPU (other streams, other
 *   threads) race and may compute wrong results.
 */
#define FA_NOALLOC_SCRATCH_BYTES (1u << 20)
FA355_API fa_status_t fa_fwd_varlen_noalloc(const void* q, const void* k, const void* v, void* o,
                                            float* lse, const int32_t* cu_seqlens_q,
                                            const int32_t* cu_seqlens_k, int nseq, int total_q,
                                            int total_k, int H, int D, float scale, int causal,
                                            fa_dtype_t dtype, void* stream);

/*
 * Single-token decode with the key/value cache split into chunks (split-KV).
 * One query row per batch entry attends to all of its Lk = min(max(seqlens_k[b],0),
 * Nk_max) cached keys (no causal mask: the query is the newest position).
 * Each chunk of `chunk` keys is summarised by (m_c, l_c, unnormalised O_c) and
 * the chunks are merged in a fixed order, the block merge of the CSDN primer
 * 轻松读懂FlashAttention 上, section Softmax求解重构.
 *   q       : [B, H, D]
 *   k_cache, v_cache: [B, Nk_max, H, D]; rows >= Lk are never read
 *   o       : [B, H, D] written;  lse: [B, H] float32 or NULL
 *   seqlens_k: device int32[B]
 *   chunk   : keys per split, one of 64, 128, 256, 512
 *   workspace: device buffer of at least fa_decode_workspace_bytes(...) bytes
 *       holding the per-chunk partials; contents on entry do not matter.
 * Two kernel launches on `stream`; stream order is the only synchronisation.
 */
FA355_API size_t fa_decode_workspace_bytes(int B, int H, int Nk_max, int D, int chunk);
FA355_API fa_status_t fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                              void* o, float* lse, const int32_t* seqlens_k,
                              int B, int H, int Nk_max, int D, float scale, int chunk,
                              void* workspace, size_t workspace_bytes,
                              fa_dtype_t dtype, void* stream);

/*
 * The same split-KV decode over a paged cache: the keys and values of all
 * batch entries live in one pool of fixed-size pages and a page table names
 * each entry's pages in key order (the cache-layout question of the
 * slavadubrov.com page's checklist, row on head dimension, mask and cache
 * layout; the computation is the decode above on the gathered cache).
 *   k_pages, v_pages: [num_pages, page_size, H, D]; key t of batch entry b is
 *       row t % page_size of page block_table[b * max_pages + t / page_size]
 *   block_table: device int32 [B, max_pages], 4-byte aligned; only the first
 *       ceil(Lk / page_size) entries of a row are read; an entry outside
 *       [0, num_pages) is a caller error: it is clamped into the pool (no read
 *       leaves the cache) and that entry's output is unspecified
 *   page_size: power of two, 16 .. 1024 (else FA_ERR_UNSUPPORTED)
 *   Lk = min(max(seqlens_k[b], 0), max_pages * page_size)
 *   workspace: at least fa_decode_workspace_bytes(B, H, max_pages * page_size,
 *       D, chunk) bytes
 * Other arguments, errors and ordering as fa_decode_splitkv; the caller owns
 * every buffer.  Bit-identical to fa_decode_splitkv on the gathered cache.
 */
FA355_API fa_status_t fa_decode_splitkv_paged(const void* q, const void* k_pages,
                              const void* v_pages, void* o, float* lse,
                              const int32_t* seqlens_k, const int32_t* block_table,
                              int B, int H, int num_pages, int page_size, int max_pages,
                              int D, float scale, int chunk,
                              void* workspace, size_t workspace_bytes,
                              fa_dtype_t dtype, void* stream);

/*
 * Backward pass of fixed-length attention: the gradients dQ, dK, dV of a
 * loss L given dO = dL/dO, for the forward pass fa_fwd computed (same q, k,
 * v, scale, causal, seqlens_k; its o and lse).  The probabilities are
 * recomputed from q, k and lse rather than stored (the recompute of the CSDN
 * primer 轻松读懂FlashAttention 上, section Softmax求解重构):
 *   dV = P^T dO,  dS = P o (dO V^T - rowsum(dO o O)),  dQ = scale dS K,
 *   dK = scale dS^T Q.
 *   q, o, dout, dq: [B, Nq, H, D];  k, v, dk, dv: [B, Nk, H, D];  dtype fp16 or
 *       bf16 (fp32: FA_ERR_UNSUPPORTED); dq, dk, dv written in that dtype
 *   lse: [B, H, Nq] float32 from fa_fwd (rows with no visible key: -inf)
 *   seqlens_k: as fa_fwd; padding keys (rows Lk .. Nk-1) get dk = dv = 0
 *   workspace: device buffer of at least fa_bwd_workspace_bytes(B, H, Nq)
 *       bytes (per query row rowsum(dO o O) and lse in base-2 units, float32);
 *       contents on entry do not matter
 * Three kernel launches on `stream` (row sums, then dK/dV, then dQ); no
 * atomics, so the result is bit-reproducible.  The caller owns every buffer.
 */
FA355_API size_t fa_bwd_workspace_bytes(int B, int H, int Nq);
FA355_API fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             int B, int H, int Nq, int Nk, int D, float scale, int causal,
                             const int32_t* seqlens_k, void* workspace, size_t workspace_bytes,
                             fa_dtype_t dtype, void* stream);

/*
 * Backward pass of fa_fwd_varlen (packed variable-length batches): the
 * gradients of each sequence's own attention, for the o and lse that
 * fa_fwd_varlen wrote with the same cu_seqlens, scale and causal.
 *   q, o, dout, dq: [total_q, H, D];  k, v, dk, dv: [total_k, H, D]; fp16 or
 *       bf16 (fp32: FA_ERR_UNSUPPORTED)
 *   lse: [H, total_q] float32 from fa_fwd_varlen
 *   cu_seqlens_q, cu_seqlens_k: device int32 [nseq + 1], as fa_fwd_varlen
 *       (each range clamped to [0, total])
 *   max_seqlen_q, max_seqlen_k: at least the longest query / key range (they
 *       size the grid; rows past them are not computed)
 *   workspace: at least fa_bwd_workspace_bytes(1, H, total_q) bytes
 * dq rows and dk / dv rows that belong to a sequence are written; rows
 * outside every range are left untouched.  Ordering, reproducibility and
 * errors as fa_bwd.
 */
FA355_API fa_status_t fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout, void* dq, void* dk,
                                    void* dv, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, int nseq, int total_q,
                                    int total_k, int max_seqlen_q, int max_seqlen_k, int H, int D,
                                    float scale, int causal, void* workspace,
                                    size_t workspace_bytes, fa_dtype_t dtype, void* stream);

/*
 * Backward pass of fa_fwd_masked: as fa_bwd, for the o and lse that
 * fa_fwd_masked wrote with the same prefix and alibi_slopes (prefix mask:
 * with causal only, keys [0, prefix) are seen by every query; ALiBi: score
 * += -slope_h * |j - (i + Lk - Lq)|).  The bias does not depend on q or k,
 * so it changes the recomputed probabilities only.
 *   prefix: >= 0, and 0 unless causal (else FA_ERR_INVALID_ARG)
 *   alibi_slopes: NULL or a 4-byte aligned device array of H floats
 * Other arguments, layouts, errors and ordering as fa_bwd.
 */
FA355_API fa_status_t fa_bwd_masked(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout, void* dq, void* dk,
                                    void* dv, int B, int H, int Nq, int Nk, int D, float scale,
                                    int causal, const int32_t* seqlens_k, int prefix,
                                    const float* alibi_slopes, void* workspace,
                                    size_t workspace_bytes, fa_dtype_t dtype, void* stream);

/*
 * Attention dropout (training), forward and backward.  The Hugging Face
 * Flash-Attention-2 integration guide's parameter table lists dropout_p: the
 * probability of dropping an attention weight, 0 outside training, applied
 * inside the fused kernel.  Here it acts on the normalised probabilities,
 * O = (P o Z) V with Z = keep / (1 - p_eff); lse stays that of the undropped
 * softmax.  Keep decisions: pair (query i, key j) of batch entry b and head
 * h takes byte (j mod 4), least significant first, of word ((j / 4) mod 4)
 * of Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) with counter
 * (j / 16, i, h, b) and key (seed mod 2^32, seed / 2^32); the pair is kept
 * iff that byte is >= t = round(256 * dropout_p), at most 255, so
 * p_eff = t / 256.  The decisions depend only on (seed, b, h, i, j), so the
 * backward redraws exactly the forward's.
 *   dropout_p: in [0, 1) (else FA_ERR_INVALID_ARG); t = 0 is no dropout
 *   seed: any 64-bit value; use a new one for every forward pass
 * fa_fwd_dropout: arguments, layout and errors as fa_fwd; fp16/bf16 only
 * (fp32: FA_ERR_UNSUPPORTED).  fa_bwd_dropout: as fa_bwd, for the o and lse
 * that fa_fwd_dropout wrote with the same dropout_p and seed.
 */
FA355_API fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int H, int Nq, int Nk, int D, float scale,
                                     int causal, const int32_t* seqlens_k, float dropout_p,
                                     uint64_t seed, fa_dtype_t dtype, void* stream);
FA355_API fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk,
                                     void* dv, int B, int H, int Nq, int Nk, int D, float scale,
                                     int causal, const int32_t* seqlens_k, float dropout_p,
                                     uint64_t seed, void* workspace, size_t workspace_bytes,
                                     fa_dtype_t dtype, void* stream);

/*
 * Packed variable-length batches with the mask families or dropout: the
 * options of fa_fwd_masked / fa_fwd_dropout (the guide's flash_attn_varlen
 * parameter table names causal, alibi_slopes and dropout_p for the packed
 * call too) on the batches of fa_fwd_varlen, and their gradients on those of
 * fa_bwd_varlen.  Positions count within each sequence: query row i of
 * sequence s sits at key position i + Lk(s) - Lq(s), the prefix covers
 * that sequence's keys [0, prefix), ALiBi distances are within the
 * sequence, and the dropout counters take the sequence index s in the
 * place of the batch index b.  fp16/bf16 only (fp32: FA_ERR_UNSUPPORTED);
 * fa_fwd_varlen_ex / fa_bwd_varlen_ex below take all options together.
 * Arguments, layouts, workspaces, errors and ordering as fa_fwd_varlen /
 * fa_bwd_varlen plus, for the options, as fa_fwd_masked / fa_fwd_dropout;
 * a backward call must repeat the forward call's options.
 */
FA355_API fa_status_t fa_fwd_varlen_masked(const void* q, const void* k, const void* v, void* o,
                                           float* lse, const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, int nseq, int total_q,
                                           int total_k, int H, int D, float scale, int causal,
                                           int prefix, const float* alibi_slopes,
                                           void* workspace, size_t workspace_bytes,
                                           fa_dtype_t dtype, void* stream);
FA355_API fa_status_t fa_fwd_varlen_dropout(const void* q, const void* k, const void* v, void* o,
                                            float* lse, const int32_t* cu_seqlens_q,
                                            const int32_t* cu_seqlens_k, int nseq, int total_q,
                                            int total_k, int H, int D, float scale, int causal,
                                            float dropout_p, uint64_t seed, void* workspace,
                                            size_t workspace_bytes, fa_dtype_t dtype,
                                            void* stream);
FA355_API fa_status_t fa_bwd_varlen_masked(const void* q, const void* k, const void* v,
                                           const void* o, const float* lse, const void* dout,
                                           void* dq, void* dk, void* dv,
                                           const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, int nseq, int total_q,
                                           int total_k, int max_seqlen_q, int max_seqlen_k,
                                           int H, int D, float scale, int causal, int prefix,
                                           const float* alibi_slopes, void* workspace,
                                           size_t workspace_bytes, fa_dtype_t dtype,
                                           void* stream);
FA355_API fa_status_t fa_bwd_varlen_dropout(const void* q, const void* k, const void* v,
                                            const void* o, const float* lse, const void* dout,
                                            void* dq, void* dk, void* dv,
                                            const int32_t* cu_seqlens_q,
                                            const int32_t* cu_seqlens_k, int nseq, int total_q,
                                            int total_k, int max_seqlen_q, int max_seqlen_k,
                                            int H, int D, float scale, int causal,
                                            float dropout_p, uint64_t seed, void* workspace,
                                            size_t workspace_bytes, fa_dtype_t dtype,
                                            void* stream);

/*
 * Every option at once: the prefix mask, ALiBi and dropout together (the
 * guide's flash_attn and flash_attn_varlen calls take them together).  The
 * entry points above are these with the other options off; the rules of
 * each option, and the arguments, layouts, workspaces and errors, are those
 * given there.  dropout_p = 0 is no dropout.  A backward call repeats the
 * forward call's options.  fp16/bf16 for any option (fp32 with none only).
 */
FA355_API fa_status_t fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Nq, int Nk, int D, float scale, int causal,
                                const int32_t* seqlens_k, int prefix, const float* alibi_slopes,
                                float dropout_p, uint64_t seed, fa_dtype_t dtype, void* stream);
FA355_API fa_status_t fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                int B, int H, int Nq, int Nk, int D, float scale, int causal,
                                const int32_t* seqlens_k, int prefix, const float* alibi_slopes,
                                float dropout_p, uint64_t seed, void* workspace,
                                size_t workspace_bytes, fa_dtype_t dtype, void* stream);
FA355_API fa_status_t fa_fwd_varlen_ex(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k, int nseq, int total_q,
                                       int total_k, int H, int D, float scale, int causal,
                                       int prefix, const float* alibi_slopes, float dropout_p,
                                       uint64_t seed, void* workspace, size_t workspace_bytes,
                                       fa_dtype_t dtype, void* stream);
FA355_API fa_status_t fa_bwd_varlen_ex(const void* q, const void* k, const void* v,
                                       const void* o, const float* lse, const void* dout,
                                       void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k, int nseq, int total_q,
                                       int total_k, int max_seqlen_q, int max_seqlen_k, int H,
                                       int D, float scale, int causal, int prefix,
                                       const float* alibi_slopes, float dropout_p, uint64_t seed,
                                       void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                                       void* stream);

/* Static strings; never NULL. */
FA355_API const char* fa_status_string(fa_status_t status);
FA355_API const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
