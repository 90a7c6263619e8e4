// prefill_fwd.h -- internal interface between the C ABI layer and the gfx950
// prefill attention kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsmha {

struct PrefillArgs {
  const void* q;             // bf16 [T][n_q_heads][head_dim]
  const void* k;             // bf16 [T][n_kv_heads][head_dim], or the k cache (block_table set)
  const void* v;             // bf16 [T][n_kv_heads][head_dim], or the v cache
  const float* sinks;        // fp32 [n_q_heads] or nullptr
  const int32_t* cu_seqlens; // int32 [n_seqs + 1], the new query rows
  void* out;                 // bf16 [T][n_q_heads][head_dim]
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t window;            // <= 0: none
  float softmax_scale;
  int32_t n_seqs;
  int32_t max_seqlen;        // longest run of new query rows
  // paged K/V (prefill of new rows against a cache); block_table == nullptr
  // means k and v are packed like q
  const int32_t* seqlens_k = nullptr;    // int32 [n_seqs]
  const int32_t* block_table = nullptr;  // int32 [n_seqs][pages_per_seq]
  int32_t n_pages = 0;
  int32_t page_size = 0;                 // a power of two >= 16
  int32_t pages_per_seq = 0;
};

// Number of work-groups the launch will use (0 means nothing to launch), or
// -1 if the grid would not fit the launch limits.
int64_t prefill_grid_size(const PrefillArgs& a);

// Enqueue the kernel; returns the launch's hipError_t.
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Sequences per group of the kernels' direct order (cdna4.h, direct_block_item):
// as many as have their K and V (rows of row_bytes per KV head) within one
// XCD's L2, at least 1, at most n_seqs.
int32_t prefill_seq_group(const PrefillArgs& a, int row_bytes);

// The same two calls for the 128-row work-groups of prefill_fwd_narrow.hip, at
// head_dim 64 or 128 (a paged cache at head_dim 128 only: the grid size is -1
// for a paged cache at head_dim 64).
int64_t prefill_grid_size_narrow(const PrefillArgs& a, int head_dim);
hipError_t launch_prefill_narrow(const PrefillArgs& a, int head_dim, hipStream_t stream);

}  // namespace tsmha
