/*
 * attn.h -- C ABI of the exact tiled attention library for AMD Instinct
 * MI355X (gfx950).  Library file: libeta_attn.so.
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T + mask) V
 * tile by tile with the online-softmax recurrence (running max, running sum,
 * unnormalised accumulator, one division at the end), so the score and
 * probability matrices never reach device memory.  Sources, cited by page
 * title and section:
 *   "Modern attention kernels" (blog.ecitis.org): "Standard attention
 *     materializes quadratic state" (the formula, Nq and Nk), "Online softmax
 *     makes tiling exact", "Kernel structure" (tiles, causal skipping),
 *     "Backward pass recomputes scores", "Work partitioning in
 *     FlashAttention-2", "Prefill and decode need different kernels", "Paged
 *     attention changes addressing", "Failure modes" (page-table mismatch).
 *   "Attention kernels" (inference.tusharamrit.in): online-softmax
 *     derivation, FlashDecoding split-context merge, grouped-query sharing.
 *   "Flash attention and IO-aware attention" (aigrafen.se): backward saves
 *     only the row statistics.
 *
 * Common conventions
 *   - Every pointer argument except `buf`/`stream` is a DEVICE pointer to
 *     memory the caller owns; the library keeps no state between calls and
 *     never allocates device memory.  Scratch memory is passed in through
 *     `workspace`, sized by the matching *_workspace_size query.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; results are valid once the caller has
 *     synchronised the stream.  Calls are reentrant.
 *   - Tensors are contiguous and row-major with the head dimension fastest:
 *     Q, O, dQ, dO: [B, H, Nq, d]; K, V, dK, dV: [B, Hkv, Nk, d];
 *     LSE: [B, H, Nq] float32.  All tensor pointers must be 16-byte aligned.
 *   - dtype ATTN_DTYPE_BF16: Q/K/V/O/dQ/dK/dV/dO are bfloat16, accumulation
 *     is float32, outputs are rounded to nearest even.  ATTN_DTYPE_F32: all
 *     float32 (forward only).
 *   - Head dimension d must be 64 or 128.  H must be a multiple of Hkv; query
 *     head h reads KV head h / (H / Hkv) (contiguous groups).  One head's
 *     rows (N * d * element size) must stay below 2 GiB (32-bit offsets;
 *     else ATTN_ERR_UNSUPPORTED).
 *   - causal != 0 applies the causal mask aligned to the bottom-right corner:
 *     query row i may see key j iff j <= i + (Nk - Nq).  A row that sees no
 *     key gets O = 0 and LSE = -inf.
 *   - LSE is the natural-log log-sum-exp of the row's scaled, masked scores:
 *     LSE = m + ln(l).  It is the only statistic the backward needs.
 *   - Errors: arguments are validated on the host BEFORE anything is
 *     enqueued; a failed validation returns its status and launches nothing.
 *     ATTN_ERR_HIP reports a failed launch (hipGetLastError).  Data-dependent
 *     device errors cannot be reported.  attn_last_error() returns a
 *     human-readable detail of the last failure on the calling thread.
 */
#ifndef ETA_ATTN_H
#define ETA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, inconsistent strides */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request the library does not implement (e.g. d=96) */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query */
  ATTN_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} attn_status_t;

typedef enum { ATTN_DTYPE_F32 = 0, ATTN_DTYPE_BF16 = 1 } attn_dtype_t;

typedef enum { ATTN_PHASE_FWD = 0, ATTN_PHASE_DECODE = 1, ATTN_PHASE_BWD = 2 } attn_phase_t;

/*
 * Forward (prefill) attention.  "Modern attention kernels", "Standard
 * attention materializes quadratic state" defines S = Q K^T * scale,
 * P = softmax(S), O = P V for Nq queries and Nk keys; "Kernel structure"
 * gives the tiled loop and the causal tile skipping.
 *   Q [B,H,Nq,d], K and V [B,Hkv,Nk,d]  (inputs, device, dtype)
 *   O [B,H,Nq,d]                         (output, device, dtype)
 *   LSE [B,H,Nq]                         (output, device, float32; may not be NULL)
 *   B, H, Hkv, Nq, Nk >= 1; d in {64, 128}; scale > 0 and finite.
 * Returns ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED or ATTN_ERR_HIP.
 */
attn_status_t attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                       int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                       attn_dtype_t dtype, void* stream);

/*
 * Forward with a local (banded) mask.  "Modern attention kernels", "Kernel
 * structure": local attention changes the range of key tiles a query tile
 * visits; "Attention kernels", sparse-attention paragraph: a sliding window
 * lets each position see a fixed number of recent positions.
 *   Query row i sits at position p = i + (Nk - Nq) (bottom-right alignment, as
 *   for causal) and sees key j iff p - window_left <= j <= p + window_right.
 *   window_left, window_right >= 0, or -1 for no limit on that side:
 *     (-1, 0)  = the causal mask (same result as attn_fwd with causal = 1);
 *     (W-1, 0) = a causal sliding window of W keys;
 *     (-1, -1) = no mask.
 *   A row whose band holds no key gets O = 0, LSE = -inf.  Other arguments
 *   and errors as attn_fwd; with dtype F32 only (-1, 0) and (-1, -1) are
 *   supported (else ATTN_ERR_UNSUPPORTED); a side below -1 gives
 *   ATTN_ERR_INVALID_ARG.
 */
attn_status_t attn_fwd_local(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                             int window_left, int window_right, attn_dtype_t dtype,
                             void* stream);

/*
 * Bytes of workspace attn_fwd_splitkv needs (0 when it will not split the
 * key range for these sizes, or when the arguments are invalid).  Window
 * sides and chunk_keys as for attn_fwd_splitkv.  The workspace holds, per
 * query row and key part, the partial result: o / l (bf16, d values), then
 * its reference maximum and its sum l (fp32) ("Attention kernels",
 * FlashDecoding paragraph: partials of separate key ranges, combined by
 * rescaling with their maxima and sums), 2 d + 8 bytes per row.  Host
 * function; no device work.
 */
size_t attn_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d, int window_left,
                                       int window_right, int chunk_keys);

/*
 * attn_fwd_local for grids too small to fill the GPU: each 128-row query tile
 * may cut its key range into chunks computed by separate workgroups, whose
 * partials (o / l in bf16, max and sum in fp32) are merged by rescaling.  "Modern
 * attention kernels", "Work partitioning in FlashAttention-2" (a grid with
 * too few independent programs leaves hardware idle); "Attention kernels",
 * FlashDecoding paragraph (split the keys, merge the partials exactly).
 *   chunk_keys   0: the library splits only when B*H*ceil(Nq/128) < 512 and
 *                chooses the part size; > 0 (a multiple of 64): always split,
 *                each query tile's key range into equal parts of at most
 *                that many keys (rounded up to whole key tiles).
 *   workspace    device scratch of attn_fwd_splitkv_workspace_size(...) bytes
 *                (16-byte aligned; may be NULL when that size is 0).
 * The result equals attn_fwd_local's within rounding (the order of the
 * floating-point sums differs, and each partial is rounded to bf16 once).  dtype must be BF16 when a split happens.
 * Errors as attn_fwd_local, plus ATTN_ERR_INVALID_ARG for a bad chunk_keys
 * and ATTN_ERR_WORKSPACE for a missing or short workspace.
 */
attn_status_t attn_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                               int window_left, int window_right, attn_dtype_t dtype,
                               int chunk_keys, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Forward over a ragged (variable-length) batch in packed layout.  "Modern
 * attention kernels", "Numerical validation" (ragged sequence boundaries)
 * and "Paged attention changes addressing" (a serving engine runs tiled
 * prefill over many sequences at once).  Each sequence is its own attention
 * problem, with the causal/band alignment of attn_fwd_local inside it.
 *   Q, O         [total_q, H, d] bf16 (device): sequence s owns rows
 *                cu_seqlens_q[s] .. cu_seqlens_q[s+1] - 1.
 *   K, V         [total_k, Hkv, d] bf16 (device): sequence s owns rows
 *                cu_seqlens_k[s] .. cu_seqlens_k[s+1] - 1.
 *   LSE          [H, total_q] float32 output (device).
 *   cu_seqlens_q, cu_seqlens_k: int32 [num_seqs + 1] on the device,
 *                non-decreasing, starting at 0 and ending at total_q
 *                (total_k).  Offsets are clamped into the tensors, so bad
 *                offsets give wrong rows, never out-of-range accesses.
 *   max_seqlen_q bound on every sequence's query count (sizes the grid);
 *                rows past it are not computed.  1 <= max_seqlen_q <= total_q.
 *   window_left, window_right: as attn_fwd_local ((-1, 0) = causal,
 *                (-1, -1) = no mask).  A sequence with no keys gets O = 0,
 *                LSE = -inf on its rows.
 *   dtype must be BF16; d in {64, 128}; H % Hkv == 0; total_q*H*d*2 and
 *   total_k*Hkv*d*2 below 2 GiB (else ATTN_ERR_UNSUPPORTED).
 */
attn_status_t attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int num_seqs, int total_q, int total_k, int max_seqlen_q, int H,
                              int Hkv, int d, float scale, int window_left, int window_right,
                              attn_dtype_t dtype, void* stream);

/*
 * Prefill of a ragged batch against a paged KV cache (chunked prefill): the
 * combination "Modern attention kernels", "Paged attention changes
 * addressing" names for a serving engine.  Sequence s holds seqlens_k[s]
 * tokens in the cache (the new ones included, already written); its
 * cu_seqlens_q[s+1] - cu_seqlens_q[s] query rows are the LAST positions of
 * that context (bottom-right alignment).  One query row per sequence is
 * paged decode; as many rows as tokens is a full prefill.
 *   Q, O         [total_q, Hq, d] bf16; LSE [Hq, total_q] float32.
 *   K_cache, V_cache, block_table, num_blocks, max_blocks_per_seq and the
 *                strides: as attn_decode_paged; additionally block_size must
 *                be a multiple of 16 (else ATTN_ERR_UNSUPPORTED) and
 *                token_stride < 2^24.  As in attn_decode_paged, a live token
 *                whose block-table entry lies outside [0, num_blocks) is
 *                skipped (probability 0) and never read.
 *   seqlens_k    int32 [num_seqs] on the device; clamped to
 *                [0, max_blocks_per_seq * block_size].
 *   cu_seqlens_q, max_seqlen_q, window sides, errors: as attn_fwd_varlen.
 */
attn_status_t attn_prefill_paged(const void* Q, const void* K_cache, const void* V_cache,
                                 const int32_t* block_table, const int32_t* cu_seqlens_q,
                                 const int32_t* seqlens_k, void* O, float* LSE, int num_seqs,
                                 int total_q, int max_seqlen_q, int Hq, int Hkv, int d,
                                 int block_size, int num_blocks, int max_blocks_per_seq,
                                 int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                 float scale, int window_left, int window_right,
                                 attn_dtype_t dtype, void* stream);

/*
 * Forward restricted to listed score blocks of 128 queries x 128 keys.
 * "Modern attention kernels", "Kernel structure": arbitrary sparse masks need
 * an index structure telling the kernel which blocks exist; "Paged attention
 * changes addressing": sparse attention visits selected score blocks.
 *   row_ptr      int32 [num_layouts, ceil(Nq/128) + 1] (device): layout l
 *                lists for query block r the key blocks
 *                col_idx[row_ptr[l][r] .. row_ptr[l][r+1] - 1].
 *   col_idx      int32 [nnz] (device): key-block indices; each block at most
 *                once per row (order free).  Entries outside
 *                [0, ceil(Nk/128)) are ignored; offsets are clamped to nnz.
 *   num_layouts  >= 1; (batch b, head h) uses layout (b*H + h) % num_layouts
 *                (1: one pattern for all, H: per head, B*H: per batch and head).
 *   causal != 0 intersects the listed blocks with the bottom-right causal
 *   mask.  A row with no visible key gets O = 0, LSE = -inf.  Other
 *   arguments as attn_fwd; dtype must be BF16.
 */
attn_status_t attn_fwd_block_sparse(const void* Q, const void* K, const void* V, void* O,
                                    float* LSE, int B, int H, int Hkv, int Nq, int Nk, int d,
                                    float scale, int causal, const int32_t* row_ptr,
                                    const int32_t* col_idx, int num_layouts, int nnz,
                                    attn_dtype_t dtype, void* stream);

/*
 * Bytes of workspace attn_decode_paged needs for these sizes and any number
 * of KV heads (0 when the arguments are invalid).  chunk_tokens as for
 * attn_decode_paged.  The workspace holds the split-context partials of
 * "Attention kernels", FlashDecoding paragraph: per piece of a context, the
 * unnormalised o (fp32, per query head of the group), its maximum and sum,
 * plus each (sequence, KV head) pair's first and last piece index for the
 * merge.  Host function; no device work.
 */
size_t attn_decode_paged_workspace_size(int num_seqs, int Hq, int d, int max_context,
                                        int chunk_tokens);

/*
 * Single-query (decode) attention over a paged KV cache with grouped-query
 * heads and a split-context merge.  "Modern attention kernels", "Prefill and
 * decode need different kernels" and "Paged attention changes addressing":
 * token position pos of sequence s lives in physical block
 * block_table[s, pos / block_size] at slot pos % block_size; "Attention
 * kernels", FlashDecoding: the context is split into pieces whose partial
 * (o, m, l) are merged by max-rescaling.  The pieces are equal ranges of the
 * contexts of all (sequence, KV head) pairs laid end to end in 32-token
 * steps, one range per parallel work item, so a long context is split
 * across items and an item may cover the ends of several short ones.
 *   Q            [num_seqs, Hq, d]                 device, bf16
 *   K_cache, V_cache: element (blk, slot, kvh, c) at
 *                blk*block_stride + slot*token_stride + kvh*head_stride + c
 *                (strides in ELEMENTS; c contiguous), num_blocks blocks.
 *                The default layout [num_blocks, block_size, Hkv, d] has
 *                head_stride = d, token_stride = Hkv*d,
 *                block_stride = block_size*Hkv*d.
 *   block_table  [num_seqs, max_blocks_per_seq] int32, device.  Entries of
 *                live tokens must lie in [0, num_blocks); a live token whose
 *                entry does not is skipped (it gets probability 0) so a
 *                page-table mismatch cannot read outside the cache.
 *   context_lens [num_seqs] int32, device.  Tokens 0..ctx-1 are attended;
 *                ctx <= 0 gives O = 0, LSE = -inf; ctx > max_context is
 *                treated as max_context.  Cache slots past ctx (in the last
 *                page) are never read into the result, whatever they hold.
 *   O            [num_seqs, Hq, d] bf16 output; LSE [num_seqs, Hq] float32
 *                output or NULL.
 *   max_context  upper bound on context_lens (sizes the grid without reading
 *                device memory); must be <= max_blocks_per_seq*block_size.
 *   chunk_tokens tokens per parallel work item (its range of the steps laid
 *                end to end), a positive multiple of 32 up to 4064, or 0 to
 *                let the device choose from the actual context lengths.
 *   Hq % Hkv == 0 (a group of G = Hq / Hkv > 16 query heads is processed as
 *   subgroups of 16, each reading its KV head's cache rows once); d in
 *   {64, 128}; dtype must be BF16;
 *   block_size >= 1; the strides must describe non-overlapping rows, all
 *   multiples of 8, in one of two page layouts:
 *     token-major [block, slot, head, d]: head_stride >= d,
 *       token_stride >= Hkv*head_stride, block_stride >= block_size*token_stride;
 *     head-major [block, head, slot, d]: token_stride >= d,
 *       head_stride >= block_size*token_stride, block_stride >= Hkv*head_stride;
 *   and block_stride < 2^30 (else ATTN_ERR_UNSUPPORTED).
 *   workspace    device scratch of at least
 *                attn_decode_paged_workspace_size(...) bytes, 16-byte aligned.
 */
attn_status_t attn_decode_paged(const void* Q, const void* K_cache, const void* V_cache,
                                const int32_t* block_table, const int32_t* context_lens, void* O,
                                float* LSE, int num_seqs, int Hq, int Hkv, int d, int block_size,
                                int num_blocks, int max_blocks_per_seq, int max_context,
                                int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                float scale, attn_dtype_t dtype, int chunk_tokens,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the library's own scratch behind attn_decode_paged_noalloc (16 MiB):
 * calls whose attn_decode_paged workspace, computed for their Hkv, would
 * exceed it are rejected.  Host function; no device work.
 */
size_t attn_decode_paged_noalloc_max_bytes(void);

/*
 * attn_decode_paged for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as attn_decode_paged, minus
 * the workspace: the split partials go to a static device array of
 * attn_decode_paged_noalloc_max_bytes() bytes that each GPU holds from the
 * first call on it until the process ends.  Nothing is allocated or freed.
 *   Sizes whose partials do not fit give ATTN_ERR_WORKSPACE before any work.
 *   `stream` must belong to the current device (else ATTN_ERR_INVALID_ARG).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (on different streams, or from different threads without ordering)
 *   race and give undefined results; calls ordered on one stream are safe.
 *   The array keeps the last call's contents; each call writes every entry it
 *   reads before reading it, so nothing needs clearing between calls.
 */
attn_status_t attn_decode_paged_noalloc(const void* Q, const void* K_cache, const void* V_cache,
                                        const int32_t* block_table, const int32_t* context_lens,
                                        void* O, float* LSE, int num_seqs, int Hq, int Hkv, int d,
                                        int block_size, int num_blocks, int max_blocks_per_seq,
                                        int max_context, int64_t block_stride,
                                        int64_t token_stride, int64_t head_stride, float scale,
                                        attn_dtype_t dtype, int chunk_tokens, void* stream);

/*
 * Bytes of workspace attn_bwd needs: two fp32 values per query row, the row
 * term D = rowsum(dO * O) and the base-2 log-sum-exp.  These are the compact
 * per-row statistics the backward keeps instead of P ("Modern attention
 * kernels", "Backward pass recomputes scores"; "Flash attention and
 * IO-aware attention", backward paragraph).  Host function; no device work.
 */
size_t attn_bwd_workspace_size(int B, int H, int Nq, int d);

/*
 * Backward of attn_fwd by recomputation: "Modern attention kernels",
 * "Backward pass recomputes scores"; "Flash attention and IO-aware
 * attention", backward paragraph (only the row statistics are saved).
 *   Q, K, V, O, dO, LSE: as produced/consumed by attn_fwd (O and LSE must be
 *   the forward's outputs for these Q, K, V, scale and causal).
 *   dQ [B,H,Nq,d], dK and dV [B,Hkv,Nk,d]: outputs (bf16).  For Hkv < H the
 *   KV gradients are summed over the query heads of each group.
 *   dtype must be BF16; d in {64, 128}.
 *   workspace: at least attn_bwd_workspace_size(B, H, Nq, d) bytes,
 *   16-byte aligned.  No atomics are used: dQ, dK and dV are bitwise
 *   reproducible from run to run.
 */
attn_status_t attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                       const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int Hkv,
                       int Nq, int Nk, int d, float scale, int causal, attn_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of attn_fwd_local by recomputation, for the same band
 * (window_left, window_right as there; O and LSE must come from
 * attn_fwd_local with the same band).  Other arguments, workspace and errors
 * as attn_bwd.
 */
attn_status_t attn_bwd_local(const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B,
                             int H, int Hkv, int Nq, int Nk, int d, float scale, int window_left,
                             int window_right, attn_dtype_t dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Describe the kernel choice for a phase and shape ("Modern attention
 * kernels", "Prefill and decode need different kernels": record the kernel
 * choice separately per phase).  For ATTN_PHASE_DECODE, Nq is ignored, Nk is
 * max_context, B is num_seqs and H is Hq.  Writes a NUL-terminated string of
 * at most len bytes into buf (host memory) and returns the length it needed
 * (excluding the NUL), or -1 on invalid arguments.
 */
int attn_plan_describe(int phase, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                       attn_dtype_t dtype, char* buf, size_t len);

/*
 * Static string naming a status code (never NULL; a code outside the enum
 * gives "ATTN_ERR_UNKNOWN").  The codes report inputs the kernels would otherwise
 * mishandle, checked on the host before any launch: shapes a path does not
 * support, strides and block layouts that disagree with the cache
 * ("Modern attention kernels", "Failure modes": page-table mismatch between
 * allocator and kernel), workspaces that are too small.
 */
const char* attn_status_string(attn_status_t status);

/*
 * Detail of the last non-OK status returned on the calling thread ("" if
 * none): which argument failed which check (same passage as
 * attn_status_string).  The string is owned by the library and valid until
 * the thread's next call.
 */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ETA_ATTN_H */
