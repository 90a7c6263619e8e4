// cdna4.h -- small gfx950 device helpers shared by the attention kernels:
// vector types, raw buffer descriptors, wave-wide buffer-to-LDS loads, vector
// memory waits and the LDS chunk swizzle of 128-byte rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsmha {
namespace cdna4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBufferConfig = 0x00020000;  // raw buffer descriptor word 3 (32-bit data)
// Cache policy of the output stores (nt | sc1): the rows are written once and
// not read again by the kernel, so they stream out instead of taking L2 lines
// that the K/V tiles other work-groups still read.
constexpr int kStreamStore = 0x12;
constexpr float kLog2e = 1.4426950408889634f;

// Raw buffer descriptor (base, stride 0, byte range n) in scalar registers.
// Loads at offsets past n return zeros and touch no memory.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int n) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(n);
  r[3] = kBufferConfig;
  return r;
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)p);
}

// One wave-wide 16-byte-per-lane load from a buffer straight into LDS: lane i's
// 16 bytes land at lds + 16 i (lds must be wave-uniform).  Inline assembly, so
// that the compiler does not make later LDS reads wait for it; the caller
// orders these loads itself with wait_vmem.  M0 carries the LDS address and
// is used by nothing else in these kernels.
__device__ __forceinline__ void lds_dma16(uint32_t lds, const i32x4& rsrc, int voffset) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rsrc)
      : "m0");
#pragma clang diagnostic pop
}

// The same load with the non-temporal hint (nt), for data that one work-group
// reads once per call (a decode step's cached keys and values): the lines
// stream through the caches instead of displacing what others re-read.
__device__ __forceinline__ void lds_dma16_nt(uint32_t lds, const i32x4& rsrc, int voffset) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rsrc)
      : "m0");
#pragma clang diagnostic pop
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Range tests on the bits of an fp32 value.  The kernels are compiled with
// -fno-honor-nans, under which the compiler may fold !(x <= c) into x > c,
// a test that a NaN passes; integer tests on the exponent field are exact.
// finite_bits: x is neither infinite nor NaN.
__device__ __forceinline__ bool finite_bits(float x) {
  return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u;
}
// positive_in_binade_range: x > 0 with 2^lo <= x < 2^(hi + 1) (false for NaN,
// infinities, zeros, denormals and negative values).
__device__ __forceinline__ bool positive_in_binade_range(float x, int lo, int hi) {
  const int e = (int)(__float_as_uint(x) >> 23) - 127;  // a set sign bit makes e >= 129
  return e >= lo && e <= hi;
}

// Sum of the 32 elements of two 16-wide vectors in a fixed pairwise order (a
// dependency chain of 5 additions instead of 31); the prefill kernels use it
// for the same 32 accumulator values of a row block, so both sum alike.
template <typename V16>
__device__ __forceinline__ float pairwise_sum32(const V16& a, const V16& b) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t[i] = a[2 * i] + a[2 * i + 1];
    t[8 + i] = b[2 * i] + b[2 * i + 1];
  }
#pragma unroll
  for (int n = 8; n >= 1; n >>= 1)
#pragma unroll
    for (int i = 0; i < n; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

// Work items of a grid of position blocks over packed sequences with the
// blocks that lie past their sequence's end left out.  A grid sized from the
// longest sequence holds a work-group for each such block, and under load each
// of them holds a compute unit's slot far longer than its few instructions, so
// when many blocks are empty the kernels compact the order instead (the grid
// keeps its size; its surplus ids come last and return at once).  Sequence b,
// rows cu[b] .. cu[b+1] - 1, has n_b = min(ceil(L_b / U), n_levels) blocks of
// U positions.  One lane per sequence (n_seqs <= 64): c0 = cu[lane] and
// c1 = cu[lane + 1] on lanes below n_seqs, 0 elsewhere.  All lanes of the wave
// call these, and get the same wave-uniform result: block `blk` of sequence
// `seq`, whose rows start at `start` and number `len`; false when item j is
// past the last one.
constexpr int kCompactMaxSeqs = 64;
struct BlockItem {
  int seq, blk, start, len;
};
extern "C" __device__ int __ockl_wfred_add_i32(int);

__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ void fill_block_item(int seq, int blk, int c0, int c1, BlockItem& it) {
  it.seq = seq;
  it.blk = blk;
  it.start = __builtin_amdgcn_readlane(c0, seq);
  it.len = __builtin_amdgcn_readlane(c1, seq) - it.start;
}

// Inclusive prefix sum over the 64 lanes: sums within rows of 16 lanes by
// shifts of 1, 2, 4 and 8, then row 0's total into row 1 and row 2's into
// row 3, then the total of rows 0-1 into rows 2-3 (DPP row broadcasts).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Sequence-major order: the blocks of sequence 0 first, then those of
// sequence 1, and so on, ascending within a sequence (one prefix sum).
__device__ __forceinline__ bool block_item_by_sequence(int n_seqs, int U, int n_levels, int j, int c0, int c1,
                                                       BlockItem& it) {
  const int nb = lane_id() < n_seqs ? min((c1 - c0 + U - 1) / U, n_levels) : 0;
  const int incl = wave_inclusive_sum(nb);
  if (j >= __builtin_amdgcn_readlane(incl, 63)) return false;
  // the sequences whose blocks all come before item j are the first lanes
  const int seq = __builtin_popcountll(__builtin_amdgcn_ballot_w64(incl <= j));
  fill_block_item(seq, j - (__builtin_amdgcn_readlane(incl, seq) - __builtin_amdgcn_readlane(nb, seq)), c0, c1, it);
  return true;
}

// Level-major order: block index from the last level down to 0 (under a
// causal mask the late blocks carry the most work, so it starts first), by
// sequence within a level; a binary search over levels, each step one wave sum.
__device__ __forceinline__ bool block_item_by_level(int n_seqs, int U, int n_levels, int j, int c0, int c1,
                                                    BlockItem& it) {
  const int nb = lane_id() < n_seqs ? min((c1 - c0 + U - 1) / U, n_levels) : 0;
  auto at_or_above = [&](int k) { return __ockl_wfred_add_i32(max(nb - k, 0)); };  // items at levels >= k
  if (j >= at_or_above(0)) return false;
  int lo = 0, hi = n_levels - 1;  // the item's level: the largest k with at_or_above(k) > j
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (at_or_above(mid) > j) lo = mid;
    else hi = mid - 1;
  }
  const int r = j - at_or_above(lo + 1);  // its rank among the sequences that reach level lo
  const bool active = nb > lo;
  const uint64_t act = __builtin_amdgcn_ballot_w64(active);
  const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(act >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0u));
  const uint64_t hit = __builtin_amdgcn_ballot_w64(active && below == r);
  if (hit == 0) return false;
  fill_block_item(__builtin_ctzll(hit), lo, c0, c1, it);
  return true;
}

// Whether a launch compacts its order: up to kCompactMaxSeqs sequences, and
// at least a fifth of the grid's blocks empty (total rows T against
// n_seqs * max_seqlen; a fuller grid loses less to its empty blocks than the
// search costs every work-group).
__device__ __forceinline__ bool compact_grid(int n_seqs, int total_rows, int max_seqlen) {
  return n_seqs <= kCompactMaxSeqs && 5LL * total_rows < 4LL * n_seqs * max_seqlen;
}

// Direct order of the position blocks of n_seqs sequences (n_levels blocks
// each): the sequences in groups of `group` (the last group may hold fewer),
// one group's blocks before the next group's, and within a group block level
// last-first, by sequence within a level.  Under a causal mask the late blocks
// carry the most key tiles, so the longest work of a group starts first; a
// group small enough that its K and V fit one XCD's L2 keeps the K/V tiles
// that the work-groups in flight read there, instead of sweeping every
// sequence's K/V of a large batch through it.
__device__ __forceinline__ void direct_block_item(int item, int n_seqs, int n_levels, int group, int& seq,
                                                  int& blk) {
  const int per_group = group * n_levels;
  const int grp = item / per_group;
  const int r = item - grp * per_group;
  const int gs = min(group, n_seqs - grp * group);
  seq = grp * group + r % gs;
  blk = n_levels - 1 - r / gs;
}

// Position of 16-byte chunk `ch` of row `row` (8 chunks of a 128-byte row) in
// an LDS tile.  The LDS serves 64 banks of 4 bytes per cycle, two 128-byte
// rows; the XOR key (row bit 1 as chunk bit 2, row bits 2..3 as chunk bits
// 0..1) spreads both 16 consecutive rows reading one chunk and 4 consecutive
// rows reading 4 adjacent chunks over 16 distinct bank groups.
__device__ __forceinline__ int swz_key(int row) { return ((row & 2) << 1) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ swz_key(row)); }

}  // namespace cdna4
}  // namespace tsmha
