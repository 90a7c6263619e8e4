/*
 * ts_mha.h -- C ABI of the MI355X (gfx950) attention library.
 *
 * The main operation: causal grouped-query attention over packed
 * variable-length sequences, with an optional sliding window and an optional
 * per-head attention sink (ts_mha_prefill).  Decode against a paged KV cache
 * (ts_mha_decode_with_kvcache) and prefill of new rows against such a cache
 * (ts_mha_prefill_with_kvcache) apply the same attention to query rows that
 * sit at the end of each sequence's cached keys; they are declared further
 * below.  ts_mha_prefill is the
 * `mha_prefill` public call listed in the
 * TokenSpeed-kernel README, section "Public API" (kept apart there from
 * `mha_prefill_with_kvcache`, so no cache is involved), for the GPT-OSS
 * attention of "TokenSpeed-kernel multi-silicon" (aixai.ru blog), section
 * "Числа: Gluon на AMD MI355X": attention sinks, sliding-window and full
 * layers, head_dim 64, 64 query heads over 8 KV heads, bf16 Q/K/V.
 *
 * Semantics (the pages give no formula; these are the readings this library
 * implements).  For sequence b with start s = cu_seqlens[b] and length
 * L = cu_seqlens[b+1] - s, query position i in [0, L), query head h, and
 * KV head g = h / (n_q_heads / n_kv_heads):
 *     visible keys  A_i = { j : 0 <= j <= i, and i - j < window if window > 0 }
 *     z_j           = softmax_scale * dot(q[s+i][h][:], k[s+j][g][:])
 *     sigma_h       = sinks[h] (a logit in the units of z; not multiplied by
 *                     softmax_scale), or -infinity when sinks == NULL
 *     out[s+i][h][:] = sum_{j in A_i} e^{z_j} v[s+j][g][:] / (e^{sigma_h} + sum_{j in A_i} e^{z_j})
 * The sink joins the softmax denominator and contributes no value.  Sequences
 * never attend to each other.  Results are computed with fp32 accumulation and
 * rounded to bf16 (round to nearest even).
 *
 * General rules for every entry point:
 *  - Every pointer named "device" must point to device memory of the current
 *    HIP device; the caller owns all buffers (a decode workspace included) and
 *    keeps them alive until the work on `stream` has finished.  No call
 *    allocates device memory or keeps per-call state; the one piece of device
 *    memory the library owns is the fixed scratch array of
 *    ts_mha_decode_with_kvcache_noalloc (below), one per GPU.
 *  - Arguments are validated on the host before any HIP call; a rejected call
 *    launches nothing and returns a negative TS_MHA_ERR_* code.  No C++
 *    exception crosses this interface.
 *  - Work is enqueued asynchronously on `stream`; device-side faults surface at
 *    the caller's next synchronisation, as with any HIP launch.
 *  - Calls are thread-safe.
 */
#ifndef TS_MHA_H
#define TS_MHA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TS_MHA_OK 0
#define TS_MHA_ERR_NULL_ARG (-1)     /* a required pointer is NULL */
#define TS_MHA_ERR_BAD_SHAPE (-2)    /* heads <= 0, n_q_heads % n_kv_heads != 0, n_seqs < 0,
                                        max_seqlen < 0, the launch grid would overflow, or one
                                        sequence's q rows ((max_seqlen + R) * n_q_heads * 2 *
                                        head_dim bytes, R = 256 at head_dim 64 and 128 at
                                        head_dim 128: the rows of one work-group) or k/v rows
                                        ((max_seqlen + 64) * n_kv_heads * 2 * head_dim bytes)
                                        would exceed 2^31 - 1 */
#define TS_MHA_ERR_UNSUPPORTED (-3)  /* head_dim not 64 or 128, or n_q_heads / n_kv_heads
                                        not in {1,2,4,8,16} */
#define TS_MHA_ERR_BAD_SCALE (-4)    /* softmax_scale not finite or <= 0 */
#define TS_MHA_ERR_ALIGN (-5)        /* q, k, v or out not 16-byte aligned; sinks or cu_seqlens not 4-byte aligned */
#define TS_MHA_ERR_NO_DEVICE (-6)    /* no HIP device is present */
#define TS_MHA_ERR_ARCH (-7)         /* the current device is not gfx950 */
#define TS_MHA_ERR_LAUNCH (-8)       /* the HIP launch failed; ts_mha_strerror adds the HIP error text */
#define TS_MHA_ERR_SEQLENS (-9)      /* only with TS_MHA_VALIDATE=1 in the environment: cu_seqlens[0] != 0,
                                        cu_seqlens decreasing, or a length above max_seqlen; for the
                                        cache calls a seqlens_k entry outside [0, max_seqlen_k] or
                                        below the sequence's new-row count */
#define TS_MHA_ERR_WORKSPACE (-10)   /* decode: workspace NULL or smaller than ts_mha_decode_workspace_size;
                                        noalloc decode: more than TS_MHA_NOALLOC_SCRATCH_BYTES needed */
#define TS_MHA_ERR_PAGES (-11)       /* only with TS_MHA_VALIDATE=1: a block-table entry that a sequence
                                        needs is outside [0, n_pages) */

/*
 * ts_mha_prefill -- enqueue one prefill attention pass (the operation above).
 *
 *  q            device, bf16 [T][n_q_heads][head_dim], contiguous, 16-byte aligned
 *  k, v         device, bf16 [T][n_kv_heads][head_dim], contiguous, 16-byte aligned
 *  sinks        device, fp32 [n_q_heads], or NULL for no sink
 *  cu_seqlens   device, int32 [n_seqs + 1]: cu_seqlens[0] = 0, non-decreasing,
 *               cu_seqlens[n_seqs] = T.  Empty sequences are allowed.
 *  n_q_heads, n_kv_heads   > 0, n_q_heads a multiple of n_kv_heads with
 *               group size n_q_heads / n_kv_heads in {1, 2, 4, 8, 16}
 *  head_dim     64 or 128 (the head widths of the kernel traits in the
 *               TokenSpeed-kernel README, "Public API"); q, k, v and out rows
 *               hold head_dim elements
 *  window       <= 0: full causal; > 0: key j visible to query i iff 0 <= i - j < window
 *  softmax_scale  finite, > 0; applied to q.k exactly as given
 *  out          device, bf16 [T][n_q_heads][head_dim], 16-byte aligned; every
 *               element is overwritten; must not overlap q, k, v, sinks or cu_seqlens
 *  n_seqs       >= 0; 0 is a no-op
 *  max_seqlen   >= every cu_seqlens[b+1] - cu_seqlens[b] (sizes the launch grid;
 *               positions beyond it are not computed)
 *  stream       hipStream_t to enqueue on; NULL = the default stream
 *
 *  At head_dim 64 the call picks between two kernels with bit-identical results
 *  (the exact fallback included: both decide it per 128 query rows):
 *  work-groups of 256 query rows, or of 128 when the former would give no
 *  compute unit more than two work-groups (short or few sequences).  The
 *  environment variable TS_MHA_PREFILL_KERNEL=wide|narrow forces one of them
 *  (for tests and measurement); head_dim 128 always uses 128-row work-groups.
 *
 *  Returns TS_MHA_OK or a TS_MHA_ERR_* code (see above).
 */
int ts_mha_prefill(const void* q, const void* k, const void* v, const float* sinks,
                   const int32_t* cu_seqlens, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, int32_t window, float softmax_scale, void* out,
                   int32_t n_seqs, int32_t max_seqlen, void* stream);

/*
 * ts_mha_strerror -- static, NUL-terminated description of a return code.
 * For TS_MHA_ERR_LAUNCH the text includes the HIP error of the most recent
 * failed launch on the calling thread.  Unknown codes give "unknown error".
 */
const char* ts_mha_strerror(int code);

/*
 * ts_mha_unmasked_pairs -- number of visible (query, key) pairs per head, the
 * unit of the throughput metric: sum over sequences of L(L+1)/2 for full
 * causal, or W(W+1)/2 + (L-W)W when 0 < W < L.  Each pair costs 2*head_dim
 * flops for q.k and 2*head_dim for the weighted sum of v.  The metric is the
 * prefill attention TFLOP/s of the chart in "TokenSpeed-kernel multi-silicon"
 * (aixai.ru blog), section "Числа: Gluon на AMD MI355X" (full causal,
 * head_dim 64, 64 query over 8 KV heads, sequence 1K-8K, batch 1-16); the
 * page does not say how it counts flops, so masked pairs are not counted here.
 *
 *  cu_seqlens_host  host, int32 [n_seqs + 1], non-decreasing
 *  Returns the count, or -1 if cu_seqlens_host is NULL, n_seqs < 0 or a
 *  length is negative.
 */
int64_t ts_mha_unmasked_pairs(const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t window);

/*
 * ts_mha_prefill_with_kvcache -- prefill of new query rows against a paged KV
 * cache (chunked prefill): each sequence's new rows attend to all its cached
 * keys, their own included.  The TokenSpeed-kernel README, section "Public
 * API", lists `mha_prefill_with_kvcache` beside `mha_prefill`; the pages give
 * no signature or layout.  Readings taken here (shared with
 * ts_mha_decode_with_kvcache below):
 *  - the cache already holds the new rows' own keys and values (the caller
 *    writes them first); seqlens_k[b] counts every cached key of sequence b;
 *  - the q_len = cu_seqlens_q[b+1] - cu_seqlens_q[b] new rows are the
 *    sequence's last q_len positions: row i sits at p = seqlens_k[b] - q_len + i
 *    (the causal diagonal aligned to the bottom right);
 *  - key position j lives in page block_table[b][j / page_size], slot
 *    j % page_size, of k_cache / v_cache [n_pages][page_size][n_kv_heads][head_dim];
 *  - visible keys, sink, scale and head mapping are those of ts_mha_prefill at
 *    position p.  With q_len == seqlens_k[b] the result is ts_mha_prefill's.
 *
 *  q, out        device, bf16 [Tq][n_q_heads][head_dim] packed by cu_seqlens_q,
 *                16-byte aligned; out fully overwritten, no overlap with any input
 *  head_dim      64 or 128 (128 runs the 128-row prefill kernel's paged form)
 *  k_cache, v_cache, sinks, block_table, n_pages, page_size, pages_per_seq
 *                as for ts_mha_decode_with_kvcache
 *  cu_seqlens_q  device, int32 [n_seqs + 1]: cu[0] = 0, non-decreasing, each
 *                length <= max_seqlen_q
 *  seqlens_k     device, int32 [n_seqs]: q_len_b <= seqlens_k[b] <= max_seqlen_k
 *  max_seqlen_q  >= every new-row count, <= max_seqlen_k (sizes the launch)
 *  max_seqlen_k  >= every seqlens_k[b], <= pages_per_seq * page_size and <= 2^30
 *
 *  Out-of-contract lengths or table entries never move a read outside the
 *  block table or the cache pool (page ids are clamped, keys at or past
 *  seqlens_k[b] read as zeros) but give meaningless rows; TS_MHA_VALIDATE=1
 *  checks them first.  Returns TS_MHA_OK or a TS_MHA_ERR_* code.
 */
int ts_mha_prefill_with_kvcache(const void* q, const void* k_cache, const void* v_cache,
                                const float* sinks, const int32_t* cu_seqlens_q,
                                const int32_t* seqlens_k, const int32_t* block_table,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                int32_t window, float softmax_scale, void* out, int32_t n_seqs,
                                int32_t n_pages, int32_t page_size, int32_t pages_per_seq,
                                int32_t max_seqlen_q, int32_t max_seqlen_k, void* stream);

/*
 * ts_mha_decode_with_kvcache -- decode attention against a paged KV cache:
 * one new query row per sequence, every query head.  The TokenSpeed-kernel
 * README, section "Public API", lists `mha_decode_with_kvcache` beside
 * `mha_prefill`, and "TokenSpeed-kernel multi-silicon" (aixai.ru blog),
 * section "Архитектура: три слоя вместо лабиринта", names it as one of the
 * runtime's attention calls; the pages give no signature or layout.  Readings
 * taken here:
 *  - the cache already holds the new token's own key and value (the caller
 *    writes them first); seqlens_k[b] counts every cached key of sequence b,
 *    that one included, so the query sits at position p = seqlens_k[b] - 1;
 *  - key position j of sequence b lives in page block_table[b][j / page_size],
 *    slot j % page_size, of k_cache / v_cache [n_pages][page_size][n_kv_heads][head_dim];
 *  - visible keys, sink, scale and the query-head to KV-head mapping are those
 *    of ts_mha_prefill at position p: keys j <= p with p - j < window when
 *    window > 0;
 *  - a sequence with seqlens_k[b] == 0 has no key and its output rows are zero.
 *
 *  q             device, bf16 [n_seqs][n_q_heads][head_dim], 16-byte aligned
 *  k_cache, v_cache  device, bf16 [n_pages][page_size][n_kv_heads][head_dim], 16-byte
 *                aligned.  Slots no sequence uses (and slots at or past
 *                seqlens_k[b] in a sequence's last page) may hold anything,
 *                NaN included: they are never read.
 *  sinks         device, fp32 [n_q_heads], or NULL for no sink
 *  seqlens_k     device, int32 [n_seqs], each in [0, max_seqlen_k]
 *  block_table   device, int32 [n_seqs][pages_per_seq]; the first
 *                ceil(seqlens_k[b] / page_size) entries of row b are page ids in
 *                [0, n_pages); the rest are ignored
 *  n_q_heads, n_kv_heads, head_dim, window, softmax_scale   as for ts_mha_prefill
 *                (head_dim 64 or 128)
 *  out           device, bf16 [n_seqs][n_q_heads][head_dim], 16-byte aligned, fully
 *                overwritten; must not overlap any input
 *  n_seqs        >= 0; 0 is a no-op
 *  n_pages       > 0, pages in the pool
 *  page_size     keys per page: a power of two >= 16
 *  pages_per_seq > 0, the row length of block_table
 *  max_seqlen_k  >= every seqlens_k[b], <= pages_per_seq * page_size and <= 2^30;
 *                sizes the launch (keys past it are not read)
 *  workspace     device scratch for partial results of long sequences, 256-byte
 *                aligned, at least ts_mha_decode_workspace_size(...) bytes (NULL
 *                allowed when that is 0); caller-owned, contents need no
 *                initialisation and are meaningless afterwards; calls that
 *                share a workspace must not run concurrently
 *  workspace_bytes  its size in bytes
 *  stream        hipStream_t to enqueue on; NULL = the default stream
 *
 *  Out-of-contract seqlens_k or block_table values never make the kernels
 *  read outside the block table or the cache pool (page ids are clamped into
 *  the pool), but the results are then meaningless; TS_MHA_VALIDATE=1 checks
 *  them on the host first (a synchronising read-back).
 *  How the keys are divided among work-groups (how many adjacent KV heads one
 *  work-group serves, and the split of long sequences into key chunks) follows
 *  from n_seqs, n_q_heads, n_kv_heads, head_dim, window and max_seqlen_k only:
 *  calls with equal values give identical bits, and a row's last bits may
 *  differ between calls with different ones (another summation order).
 *  Returns TS_MHA_OK or a TS_MHA_ERR_* code.
 */
int ts_mha_decode_with_kvcache(const void* q, const void* k_cache, const void* v_cache,
                               const float* sinks, const int32_t* seqlens_k,
                               const int32_t* block_table, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t window, float softmax_scale, void* out,
                               int32_t n_seqs, int32_t n_pages, int32_t page_size,
                               int32_t pages_per_seq, int32_t max_seqlen_k, void* workspace,
                               int64_t workspace_bytes, void* stream);

/*
 * ts_mha_decode_workspace_size -- bytes of workspace a ts_mha_decode_with_kvcache
 * call with these arguments needs (0: none).  The split of long sequences into
 * key chunks depends only on these arguments.  Returns a negative TS_MHA_ERR_*
 * code for shapes the decode call would reject.
 */
int64_t ts_mha_decode_workspace_size(int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t head_dim, int32_t window, int32_t max_seqlen_k);

/*
 * ts_mha_decode_with_kvcache_noalloc -- ts_mha_decode_with_kvcache for callers
 * that cannot allocate device memory (work captured into a HIP graph, serving
 * loops that may not call hipMalloc, harnesses that forbid it): the same
 * operation, kernels and results, with the partial results of split
 * sequences kept in a scratch array of the library instead of a caller's
 * workspace.  The call allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine.
 *
 *  Arguments as for ts_mha_decode_with_kvcache without workspace and
 *  workspace_bytes.
 *  Scratch: TS_MHA_NOALLOC_SCRATCH_BYTES (16 MiB) of device memory per GPU the
 *  library runs on, held from the first call on that GPU until the process
 *  ends, and shared by every call on that GPU.  A call whose split needs more
 *  (ts_mha_decode_workspace_size above that figure) returns
 *  TS_MHA_ERR_WORKSPACE and launches nothing.  Calls that overlap on one GPU
 *  (on different streams, or from different threads without ordering) race on
 *  the scratch and give undefined results; calls on one stream are ordered.
 *  The scratch needs no initialisation; its contents after a call are
 *  meaningless.  TS_MHA_VALIDATE is ignored here (its check reads the
 *  arguments back, which allocates host memory and synchronises).
 *  Returns TS_MHA_OK or a TS_MHA_ERR_* code.
 */
#define TS_MHA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int ts_mha_decode_with_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const float* sinks, const int32_t* seqlens_k,
                                       const int32_t* block_table, int32_t n_q_heads,
                                       int32_t n_kv_heads, int32_t head_dim, int32_t window,
                                       float softmax_scale, void* out, int32_t n_seqs,
                                       int32_t n_pages, int32_t page_size, int32_t pages_per_seq,
                                       int32_t max_seqlen_k, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TS_MHA_H */
