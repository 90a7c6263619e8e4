// decode_fwd.h -- internal interface between the C ABI layer and the gfx950
// decode attention kernels (one new query row per sequence against a paged
// KV cache).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsmha {

struct DecodeArgs {
  const void* q;              // bf16 [n_seqs][n_q_heads][head_dim]
  const void* k_cache;        // bf16 [n_pages][page_size][n_kv_heads][head_dim]
  const void* v_cache;        // bf16 [n_pages][page_size][n_kv_heads][head_dim]
  const float* sinks;         // fp32 [n_q_heads] or nullptr
  const int32_t* seqlens_k;   // int32 [n_seqs]
  const int32_t* block_table; // int32 [n_seqs][pages_per_seq]
  void* out;                  // bf16 [n_seqs][n_q_heads][head_dim]
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;           // 64 or 128
  int32_t window;             // <= 0: none
  float softmax_scale;
  int32_t n_seqs;
  int32_t n_pages;
  int32_t page_size;          // power of two, >= 16
  int32_t pages_per_seq;
  int32_t max_seqlen_k;
};

// How a decode call splits each sequence's keys: `chunk` keys per work-group
// (a multiple of 128), `n_splits` chunks per sequence, and the workspace bytes
// the partial results need (0 when n_splits == 1).
struct DecodePlan {
  int32_t chunk;
  int32_t n_splits;
  int64_t workspace_bytes;
  int32_t heads_per_group;    // KV heads per work-group (1, 2 or 4)
};

// The plan for these shapes, or n_splits = -1 if the launch would not fit.
DecodePlan decode_plan(const DecodeArgs& a);

// Enqueue the kernels (the split kernel, and the merge kernel when the plan
// has more than one split); `workspace` holds at least plan.workspace_bytes.
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, void* workspace,
                         hipStream_t stream);

}  // namespace tsmha
