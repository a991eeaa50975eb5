/*
 * fp2.h - block-sparse causal GQA prefill attention with mean correction,
 *         for AMD Instinct MI355X (gfx950).
 *
 * Method: "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context
 * LLM Serving" (metallab.ai paper page).  Figure 3 gives the two stages:
 * Stage 1 packs the query heads that share a KV head (PackGQA), pools
 * block-mean statistics and emits a CSR index of the selected KV blocks per
 * KV head; Stage 2 runs attention over the selected blocks and folds every
 * unselected block in through the mean correction of Figure 4, both merged
 * in one online softmax.  Table 7 fixes the surrounding contract: a CSR
 * index per KV head, paged KV at any page size, BF16 and FP8.  The abstract
 * names the selection rule: instantaneous pattern discovery plus max-based
 * dynamic thresholding.
 *
 * Exact definition implemented (B = block size, c = 1/sqrt(d), G = Hq/Hkv):
 *   kbar_J, vbar_J  mean key / value over the tokens of KV block J
 *   qbar_I          mean query over the tokens of query block I and the G
 *                   query heads of one KV head
 *   s_IJ            float32 (qbar_I . kbar_J) * c, for J <= diag(I)
 *   keep            s_IJ >= max_J s_IJ - tau, or J == 0, or J == diag(I)
 *   out             softmax attention over the kept blocks' keys (causal,
 *                   bottom-right aligned when a prefix is cached), where
 *                   every skipped J in [1, diag(I)) adds B*exp(q.kbar_J*c - m)
 *                   to the denominator and the same weight times vbar_J to
 *                   the numerator.
 *   diag(I) = P/B + I for a sequence with a cached prefix of P tokens.
 *
 * Decoupled tiles (fp2_batch.kv_block = 64 with block = 128): query blocks
 * of 128 tokens are scored against KV blocks of 64 tokens, the pairing
 * Table 7 describes (its CSR index holds selected 64-token tiles).  kbar,
 * vbar and the CSR columns then count 64-token blocks, the diagonal of
 * query block I is the run of KV blocks holding one of its positions
 * (two, or one for a short last block), all of it forced, and the surrogate
 * covers the skipped J before that run with weight 64.
 *
 * Conventions for every entry point:
 *  - All device buffers are allocated and owned by the caller.  The library
 *    never allocates device memory, frees or synchronises; it enqueues
 *    kernels on the caller's stream (a hipStream_t passed as void*, NULL =
 *    default stream), and fp2_prefill_run also on a second stream of its own
 *    that it orders against the caller's (created with two events on the
 *    first call on a device; see there).  Buffers must stay valid until the
 *    stream has passed the work.  The stream must belong to the current
 *    device (FP2_ERR_INVALID otherwise; NULL is the current device's).
 *  - Arguments are checked on the host before anything is enqueued; on a
 *    failed check nothing is launched and the status says why
 *    (fp2_last_error() gives a message, per calling thread).
 *  - Page ids and device-side descriptor arrays are trusted: out-of-range
 *    page ids, or device arrays that disagree with their host mirrors, are
 *    undefined behaviour (a FP2_DEBUG_BOUNDS build checks page ids and the
 *    CSR on the device: fp2_debug_bounds_word()).
 *  - Layouts are row-major (C order).  "bf16" is bfloat16; "e4m3" is OCP
 *    FP8 E4M3 (bias 7, max 448, no infinities).
 */
#ifndef FP2_H
#define FP2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP2_OK = 0,
  FP2_ERR_INVALID = 1,     /* malformed argument (null pointer, bad size, ...)     */
  FP2_ERR_UNSUPPORTED = 2, /* well formed but outside what the kernels implement   */
  FP2_ERR_CAPACITY = 3,    /* an output or workspace buffer is too small           */
  FP2_ERR_HIP = 4          /* a HIP launch failed; the message holds HIP's text    */
} fp2_status;

typedef enum { FP2_BF16 = 0, FP2_FP8_E4M3 = 1 } fp2_dtype;

/* Output element type of fp2_prefill_run. */
typedef enum { FP2_OUT_BF16 = 0, FP2_OUT_F32 = 1 } fp2_out_dtype;

/* A variable-length batch of sequences (continuous batching).  Sequence s
 * holds seqlens_k[s] key tokens, of which the last n_s =
 * cu_seqlens_q[s+1]-cu_seqlens_q[s] are new queries; the first
 * P_s = seqlens_k[s]-n_s are a cached prefix (P_s must be a multiple of
 * block).  Query blocks and KV blocks are counted per sequence, with
 * KB = kv_block (or block when kv_block is 0):
 * cu_qblocks[s+1]-cu_qblocks[s] = ceil(n_s/block),
 * cu_kblocks[s+1]-cu_kblocks[s] = ceil(seqlens_k[s]/KB).
 * The device arrays and the host mirrors must hold the same values. */
typedef struct {
  int32_t num_seqs;              /* >= 0                                         */
  int32_t block;                 /* B: 64 or 128                                 */
  const int32_t *cu_seqlens_q;   /* device [num_seqs+1], cu_seqlens_q[0] == 0    */
  const int32_t *seqlens_k;      /* device [num_seqs]                            */
  const int32_t *cu_qblocks;     /* device [num_seqs+1]                          */
  const int32_t *cu_kblocks;     /* device [num_seqs+1]                          */
  const int32_t *h_cu_seqlens_q; /* host mirror of cu_seqlens_q                  */
  const int32_t *h_seqlens_k;    /* host mirror of seqlens_k                     */
  int32_t kv_block;              /* KV block size: 0 (= block), block, or 64 with
                                    block 128 (decoupled tiles, see above)       */
} fp2_batch;

/* Queries of the new tokens, packed over the batch: [total_q, Hq, d]. */
typedef struct {
  fp2_dtype dtype;
  int32_t num_q_heads;           /* Hq, a multiple of the KV head count          */
  int32_t head_dim;              /* d: 64 or 128                                 */
  const void *q;                 /* device, bf16 or e4m3 [total_q, Hq, d]        */
  const float *q_scale;          /* e4m3 only: device [total_qblocks, Hq], one
                                    scale per (query block, head); NULL for bf16 */
} fp2_q;

/* Paged KV cache.  Token t of sequence s lives in physical page
 * page_table[s*max_pages_per_seq + t/page_size], slot t%page_size. */
typedef struct {
  fp2_dtype dtype;               /* must equal the query dtype                   */
  int32_t num_kv_heads;          /* Hkv                                          */
  int32_t head_dim;              /* d, equal to the query head_dim               */
  int32_t page_size;             /* any size >= 1; e4m3 requires page_size == KB */
  int32_t num_pages;
  int32_t max_pages_per_seq;     /* >= ceil(seqlens_k[s]/page_size) for every s  */
  const void *k_pages;           /* device [num_pages, page_size, Hkv, d]        */
  const void *v_pages;           /* device [num_pages, page_size, Hkv, d]        */
  const float *k_scale;          /* e4m3 only: device [num_pages, Hkv]           */
  const float *v_scale;          /* e4m3 only: device [num_pages, Hkv]           */
  const int32_t *page_table;     /* device [num_seqs, max_pages_per_seq]         */
} fp2_kv;

/* Stage 1a - per-block key/value means (Figure 4's pooled statistics).
 * kbar, vbar: device float32 [Hkv, total_kblocks, d]; entry
 * [g, cu_kblocks[s]+J, :] is the mean of K (V) over the valid tokens of
 * KV block J (KB tokens) of sequence s, head g (e4m3 values times their
 * page scale). */
fp2_status fp2_block_stats(const fp2_batch *batch, const fp2_kv *kv,
                           float *kbar, float *vbar, void *stream);

/* Stage 1a for chunked prefill (Table 6 serves with chunked prefill; the
 * pooled statistics are Figure 3's), with the block means kept in a cache
 * beside the KV pages.  The pages do not say how the statistics of a cached
 * prefix are kept; this cache is the library's own design: the means of a
 * block whose tokens are all in the cached prefix do not change between
 * calls, so only the blocks holding new tokens are read again.  The cache has one row per KV block a page holds:
 * fp2_block_stats_cache_rows() = num_pages * max(1, page_size / KB) rows
 * (0 when page_size and the KV block KB do not divide one another:
 * unsupported).  Block J of sequence s lives in row
 * page_table[s][J*KB/page_size] * max(1, page_size/KB) + J % max(1,
 * page_size/KB).
 *   kbar_cache, vbar_cache  device float32 [cache_rows, Hkv, d], owned by the
 *                   caller alongside its KV pages
 *   refresh_prefix  1: compute every block of the batch; 0: only blocks
 *                   J >= prefix/KB (their rows are overwritten), the rows of
 *                   prefix blocks are used as an earlier call left them
 * The values are bit for bit those of fp2_block_stats. */
int64_t fp2_block_stats_cache_rows(const fp2_batch *batch, const fp2_kv *kv);
fp2_status fp2_block_stats_cached(const fp2_batch *batch, const fp2_kv *kv,
                                  float *kbar_cache, float *vbar_cache,
                                  int32_t refresh_prefix, void *stream);

/* Lays the cache rows of the batch's blocks out as the kbar, vbar arrays
 * [Hkv, total_kblocks, d] that fp2_plan_mask and fp2_prefill_run take. */
fp2_status fp2_gather_block_stats(const fp2_batch *batch, const fp2_kv *kv,
                                  const float *kbar_cache, const float *vbar_cache,
                                  float *kbar, float *vbar, void *stream);

/* Workspace bytes fp2_plan_mask needs for this batch (0 if empty). */
size_t fp2_plan_workspace_bytes(const fp2_batch *batch, int32_t num_kv_heads);

/* Largest possible number of kept entries: the causal (query block, KV
 * block, KV head) count.  col_capacity must be at least this.  row_ptr,
 * col_idx and nnz are int32: fp2_plan_mask and fp2_prefill_run return
 * FP2_ERR_UNSUPPORTED when this count, or the row count
 * num_kv_heads * total_qblocks + 1, exceeds 2^31 - 1. */
int64_t fp2_plan_max_nnz(const fp2_batch *batch, int32_t num_kv_heads);

/* Stage 1b - pattern discovery and max-based thresholding (Figure 3,
 * abstract), emitting a CSR index per KV head (Table 7).
 *   kbar       device float32 [Hkv, total_kblocks, d] from fp2_block_stats
 *   tau        threshold; +INFINITY keeps every causal block (dense), a
 *              negative value keeps only the forced blocks; NaN is invalid
 *   row_ptr    device int32 [Hkv*total_qblocks + 1]; row r = g*total_qblocks
 *              + global query block
 *   col_idx    device int32 [col_capacity]; KV-block indices within the
 *              sequence, ascending within each row
 *   nnz        device int32 [1]: number of entries written
 *   scores     optional device float32 [Hkv*total_qblocks, max_kblocks]
 *              (max_kblocks = largest ceil(seqlens_k/KB)): the float32 block
 *              scores, -INFINITY above the diagonal; NULL to skip
 *   workspace  device scratch of fp2_plan_workspace_bytes() bytes */
fp2_status fp2_plan_mask(const fp2_batch *batch, const fp2_q *q, int32_t num_kv_heads,
                         const float *kbar, float tau,
                         int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                         int32_t *nnz, float *scores,
                         void *workspace, size_t workspace_bytes, void *stream);

/* fp2_plan_mask for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and outputs, bit for bit, with the workspace taken
 * from a device array the library holds, FP2_PLAN_NOALLOC_MAX_BYTES on each
 * GPU it runs on, kept until the process ends.  The call itself allocates
 * nothing and records no memset.
 *   Returns FP2_ERR_CAPACITY when fp2_plan_workspace_bytes() of the batch
 *   exceeds FP2_PLAN_NOALLOC_MAX_BYTES (8 MiB: about 2 million bitmask words
 *   and counts, e.g. 128K tokens with 8 KV heads needs 1.1 MB).
 *   The array is shared by every call on one GPU and keeps the last call's
 *   contents (each call overwrites what it reads): calls that overlap on one
 *   GPU (two streams, or two threads) race and must be serialised by the
 *   caller.  Other arguments and errors as fp2_plan_mask. */
#define FP2_PLAN_NOALLOC_MAX_BYTES ((size_t)8 << 20)
fp2_status fp2_plan_mask_noalloc(const fp2_batch *batch, const fp2_q *q, int32_t num_kv_heads,
                                 const float *kbar, float tau,
                                 int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                                 int32_t *nnz, float *scores, void *stream);

/* Stage 1 in one fused pass (Figure 3: Stage 1 packs the query heads of a KV
 * head with PackGQA, pools block-mean statistics and emits the CSR index of
 * selected blocks in a single fused pass): the outputs of fp2_block_stats
 * (kbar, vbar) and of fp2_plan_mask (row_ptr, col_idx, nnz, scores), bit for
 * bit, from one launch that reads every K, V and Q byte once and writes the
 * block means and the pooled query means, then a selection pass that scores
 * the pooled means against kbar (both held in L2) and compacts the CSR.
 *   kbar, vbar   device float32 [Hkv, total_kblocks, d] (outputs)
 *   workspace    device scratch of fp2_stage1_workspace_bytes() bytes: the
 *                plan workspace, the pooled query means and 256 bytes for
 *                the selection pass's work counter (cleared by the call)
 * Other arguments, limits and errors as fp2_block_stats and fp2_plan_mask
 * (the query and KV dtypes and head sizes must agree). */
size_t fp2_stage1_workspace_bytes(const fp2_batch *batch, int32_t num_kv_heads, int32_t head_dim);
fp2_status fp2_stage1(const fp2_batch *batch, const fp2_q *q, const fp2_kv *kv, float tau,
                      float *kbar, float *vbar,
                      int32_t *row_ptr, int32_t *col_idx, int64_t col_capacity,
                      int32_t *nnz, float *scores,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes fp2_prefill_run needs for this batch, head size and KV
 * dtype (0 if the batch is empty or malformed).  For d = 128 with B = 128
 * over KB = 128 or KB = 64 (bf16 or e4m3), it holds V^T tiles of every KV block
 * (one bf16 128 x KB tile per block and KV head, e4m3 V dequantized: about
 * the size of bf16 V, i.e. of the e4m3 K and V together), bf16 kbar rows and
 * vbar^T tiles of the mean tokens, and the
 * work items in launch order (one per CSR row plus up to 256 chunks of
 * rows split for balance, heaviest first) with the float32 partial results
 * of split rows (about 132 KB per chunk and 256 packed query rows, so it
 * depends on num_q_heads); otherwise bf16 kbar and fp16 vbar copies.  0 also
 * when num_q_heads < num_kv_heads. */
size_t fp2_run_workspace_bytes(const fp2_batch *batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, fp2_dtype dtype);

/* Stage 2 - exact attention over the kept blocks plus the mean correction
 * of every skipped block (Figure 3 exact path, Figure 4 surrogate terms).
 *   row_ptr, col_idx  the CSR from fp2_plan_mask (any CSR whose rows are
 *                     ascending, lie in [0, diagonal] and hold block 0 and
 *                     the diagonal is valid)
 *   kbar, vbar        device float32 [Hkv, total_kblocks, d]
 *   mean_correction   0: skipped blocks are dropped; 1: corrected
 *   softmax_scale     logit scale, normally 1/sqrt(d)
 *   out_dtype         FP2_OUT_BF16 (rounded to nearest even) or FP2_OUT_F32
 *   out               device [total_q, Hq, d] of out_dtype
 *   workspace         device scratch of fp2_run_workspace_bytes() bytes;
 *                     required with d = 128 and B = 128 over KB = 128 or
 *                     KB = 64 (bf16 or e4m3), else only with
 *                     mean_correction (FP2_ERR_CAPACITY if
 *                     too small); its contents are overwritten
 * On that path (KB = 64: tiles of two kept 64-token blocks) the rows run as
 * work items launched heaviest
 * first; the exact tiles of a row heavier than a quarter of a CU's share
 * of the batch are cut into chunks whose float32 partials a second kernel
 * merges (at most 256 extra items).
 *   max_chunk_tiles   0: the library chooses the chunk size; > 0: a chunk
 *                     holds at most this many exact tiles (still within the
 *                     256 extra items); < 0: rows are never split.  The
 *                     result does not depend on it beyond float32 rounding
 *                     order; other paths ignore it.
 * On the work-item path the V^T and mean-token preparation runs on a second
 * stream the library keeps per device (created on the first call on that
 * device, default priority, never destroyed): it starts after the work
 * enqueued on `stream` before the call and `stream` waits for it before the
 * attention kernel, so the call keeps the usual stream order.  The fork and
 * join events are shared per device; a host lock serialises their use, so
 * concurrent calls from several threads are safe.  A device reset
 * (hipDeviceReset) invalidates that stream: the library is not meant to be
 * used across one. */
fp2_status fp2_prefill_run(const fp2_batch *batch, const fp2_q *q, const fp2_kv *kv,
                           const int32_t *row_ptr, const int32_t *col_idx,
                           const float *kbar, const float *vbar,
                           int32_t mean_correction, float softmax_scale,
                           fp2_out_dtype out_dtype, void *out, int32_t max_chunk_tiles,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Debug aid for the device data the host checks cannot see (page ids, the
 * CSR handed to fp2_prefill_run).  A library built with FP2_DEBUG_BOUNDS
 * (block_sparse_long_blocks_amd/build.py --debug-bounds) runs a check kernel
 * ahead of every call that reads them and keeps a device error word: bit 1, a
 * page id a sequence uses lies outside [0, num_pages) (fp2_block_stats,
 * fp2_block_stats_cached, fp2_gather_block_stats, fp2_stage1,
 * fp2_prefill_run); bit 2, a CSR row is not strictly ascending from block 0
 * through the row's last diagonal block; bit 4, the row pointers are out of
 * order or past the causal pair count (fp2_prefill_run).  While the word is
 * set, the kernels that read those data return at once, so later outputs of
 * that device are left unwritten instead of being read past buffers.
 *   word  host out: the error word (0 if every checked call was clean); the
 *         device word is cleared.
 * Reads the current device's word with a synchronous copy (it waits for the
 * device).  FP2_ERR_UNSUPPORTED from a release build, which trusts these data
 * (see the top of this file). */
fp2_status fp2_debug_bounds_word(uint32_t *word);

/* Message for the last non-OK status returned on the calling thread. */
const char *fp2_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FP2_H */
