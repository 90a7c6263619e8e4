/*
 * ts_mha.h -- C ABI of the MI355X (gfx950) prefill attention library.
 *
 * One operation: causal grouped-query attention over packed variable-length
 * sequences, with an optional sliding window and an optional per-head
 * attention sink.  This is the `mha_prefill` public call listed in the
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
 *    HIP device; the caller owns all buffers and keeps them alive until the
 *    work on `stream` has finished.  The library allocates no device memory
 *    and keeps no per-call state.
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
                                        sequence's q rows ((max_seqlen + 256) * n_q_heads * 128
                                        bytes) or k/v rows ((max_seqlen + 64) * n_kv_heads * 128
                                        bytes) would exceed 2^31 - 1 bytes */
#define TS_MHA_ERR_UNSUPPORTED (-3)  /* head_dim != 64, or n_q_heads / n_kv_heads not in {1,2,4,8,16} */
#define TS_MHA_ERR_BAD_SCALE (-4)    /* softmax_scale not finite or <= 0 */
#define TS_MHA_ERR_ALIGN (-5)        /* q, k, v or out not 16-byte aligned; sinks or cu_seqlens not 4-byte aligned */
#define TS_MHA_ERR_NO_DEVICE (-6)    /* no HIP device is present */
#define TS_MHA_ERR_ARCH (-7)         /* the current device is not gfx950 */
#define TS_MHA_ERR_LAUNCH (-8)       /* the HIP launch failed; ts_mha_strerror adds the HIP error text */
#define TS_MHA_ERR_SEQLENS (-9)      /* only with TS_MHA_VALIDATE=1 in the environment: cu_seqlens[0] != 0,
                                        cu_seqlens decreasing, or a length above max_seqlen */

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
 *  head_dim     must be 64
 *  window       <= 0: full causal; > 0: key j visible to query i iff 0 <= i - j < window
 *  softmax_scale  finite, > 0; applied to q.k exactly as given
 *  out          device, bf16 [T][n_q_heads][head_dim], 16-byte aligned; every
 *               element is overwritten; must not overlap q, k, v, sinks or cu_seqlens
 *  n_seqs       >= 0; 0 is a no-op
 *  max_seqlen   >= every cu_seqlens[b+1] - cu_seqlens[b] (sizes the launch grid;
 *               positions beyond it are not computed)
 *  stream       hipStream_t to enqueue on; NULL = the default stream
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
 * flops for q.k and 2*head_dim for the weighted sum of v.
 *
 *  cu_seqlens_host  host, int32 [n_seqs + 1], non-decreasing
 *  Returns the count, or -1 if cu_seqlens_host is NULL, n_seqs < 0 or a
 *  length is negative.
 */
int64_t ts_mha_unmasked_pairs(const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t window);

#ifdef __cplusplus
}
#endif

#endif /* TS_MHA_H */
