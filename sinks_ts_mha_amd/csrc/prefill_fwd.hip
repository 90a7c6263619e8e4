// prefill_fwd.hip -- gfx950 (CDNA4) kernels for causal grouped-query prefill
// attention with an optional sliding window and per-head attention sinks.
//
// The operation is the `mha_prefill` call of the TokenSpeed-kernel README
// (section "Public API") for the GPT-OSS attention described in
// "TokenSpeed-kernel multi-silicon" (aixai.ru blog), section
// "Числа: Gluon на AMD MI355X": bf16 Q/K/V, head_dim 64, query heads grouped
// over KV heads, attention sinks, sliding-window and full layers.  That page
// lists the CDNA4 features its kernels rely on (matrix-core MFMA, explicit
// shared-memory layouts against bank conflicts, asynchronous loads into shared
// memory); this file is an independent HIP design for the same hardware.
//
// Work decomposition.  One work-group (4 waves, 256 threads) owns 256 query
// rows: all G query heads of one KV head g, for P = 256 / G consecutive
// positions of one sequence.  Every K/V tile it stages in LDS therefore serves
// the whole head group (the GQA reuse).  The work-group walks the 64-key tiles
// that intersect its causal (and window) range; tiles entirely visible to all
// of its rows skip the mask.  The grid runs the KV head fastest (consecutive
// work-group ids go to different XCDs, so each XCD's L2 serves fixed heads)
// and the position blocks last-first, the longest causal walks first, in
// groups of sequences whose K/V fit one XCD's L2; a ragged pack's blocks past
// their sequence's end are left out of the order (cdna4.h).
//
// Orientation.  Scores are formed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16.  In that instruction's accumulator layout lane l
// holds column l % 32 -- one query -- and 16 of the 32 keys of the block, the
// other 16 sitting in lane l ^ 32.  Row maxima and sums over keys are thus
// in-lane work plus one exchange with lane l ^ 32, and the per-query running
// state (max, sum, rescale factor) lives in the lane that owns the query.  The
// output is accumulated transposed too, O^T += V^T P^T: the probabilities P^T
// leave the score accumulators already in the B-operand layout of the second
// MFMA (its key order is a fixed permutation within each 16-key step, matched
// on the V side), and V^T is read from the row-major V tile with the gfx950
// LDS transpose read ds_read_b64_tr_b16.
//
// Staging.  K and V tiles move from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (no register round trip), double-buffered: the
// loads of tile t+1 are in flight while tile t is consumed, and one barrier per
// tile separates the two.  The buffer descriptor of each work-group spans only
// its own sequence, so rows past the sequence end read as zeros.  Each lane
// picks its source chunk so that the fixed lane-to-LDS order of these loads
// lands in the XOR-swizzled layout the readers expect.  The XOR pattern is laid
// out for an LDS that serves 256 bytes (64 banks) per cycle.
//
// Softmax.  Base 2 throughout: t = s * scale * log2(e), with s = q.k from
// the MFMA (bf16 products exact, fp32 sums) and the product by scale * log2 e
// taken in fp32, so no rounding beyond fp32's touches a logit.  A row's
// result does not depend on the reference m its probabilities exp2(t - m) are
// measured against, as long as nothing leaves fp32 range; the fast pass takes
// m = 0 for every row, so a probability is exp2 of its scaled score: no
// running maximum, no rescaling, and the per-element vector work is one
// multiply, one exp2 and half a bf16 pack.  Row sums
// accumulate on the matrix pipe (see row_sums).  If a row's sum leaves
// [2^-64, 2^65) or a value stops being finite (logits beyond about +-64 in
// base 2), the work-group redoes its rows with tile_exact, a streaming
// softmax with running maxima.  The sink's own term exp2(sigma - m) joins the
// denominator at the end.
//
// Scheduling.  Each tile runs in six steps over its four 32 x 32 score
// blocks; the softmax of one block is interleaved instruction by instruction
// with the MFMAs of its neighbours (sched_group_barrier), so a wave keeps the
// matrix pipe and the vector ALU busy at the same time.  Tiles that need the
// causal or window mask start their score accumulators from a 0 / -inf mask,
// and run in loops of their own, so that each loop body holds a single kind of
// tile.  A tile whose upper (or lower) 32 keys are hidden from every row of
// the work-group computes only its other half (tile_half): its skipped keys
// would add exact zeros.
//
// Output.  Each wave writes its normalised bf16 rows into its part of the
// query staging area and reads them back whole, so every store instruction
// writes complete 128-byte rows (1 KiB contiguous when the G heads of a
// position are) rather than 16-byte pieces of 32 rows.  The stores carry a
// streaming cache policy, so the output does not evict K/V lines from L2.
#include "prefill_fwd.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "cdna4.h"

namespace tsmha {

using namespace cdna4;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 64;                        // head_dim
constexpr int kBK = 64;                       // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 64 * kWaves;            // (query head, position) rows per work-group
constexpr int kRowBytes = kD * 2;             // one K or V row in bytes
constexpr int kChunks = kRowBytes / 16;       // 16-byte chunks per row
constexpr int kTileChunks = kBK * kChunks;    // 16-byte chunks per tile
constexpr int kTileBytes = kTileChunks * 16;
constexpr int kFastSumBinades = 64;  // the fast pass keeps row sums in [2^-64, 2^65)
constexpr int kSlots = 2;                     // LDS buffers for K and for V tiles
constexpr int64_t kSeqGroupBytes = 4 << 20;   // one XCD's L2
constexpr int kMaskCausal = 1;                // mask kinds: key past the row's position
constexpr int kMaskWindow = 2;                // ... key before the row's window


struct KParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* sinks;
  const int32_t* cu;
  uint16_t* out;
  int32_t n_kv_heads;
  int32_t n_seqs;
  int32_t n_pblocks;
  int32_t window;
  float c;  // softmax_scale * log2(e)
  // paged K/V only: k and v are the caches [n_pages][page_size][n_kv_heads][64]
  const int32_t* seqlens_k;    // cached keys per sequence, the new rows' own included
  const int32_t* block_table;  // [n_seqs][pages_per_seq] page ids
  int64_t page_elems;          // bf16 elements per page
  int32_t page_bytes;
  int32_t page_shift;
  int32_t pages_per_seq;
  int32_t n_pages;
  int32_t max_seqlen;
  int32_t seq_group;  // sequences per group of the direct order (>= 1)
};

namespace {

// max / sum of x over the lane pair (l, l ^ 32): v_permlane32_swap hands each
// lane both halves of the pair.
__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Maximum of the 16 values of one accumulator block: two chains of 3-input maxima.
__device__ __forceinline__ float max16(const f32x16& a) {
  float x = fmaxf(fmaxf(a[0], a[1]), a[2]);
  float y = fmaxf(fmaxf(a[3], a[4]), a[5]);
  x = fmaxf(fmaxf(x, a[6]), a[7]);
  y = fmaxf(fmaxf(y, a[8]), a[9]);
  x = fmaxf(fmaxf(x, a[10]), a[11]);
  y = fmaxf(fmaxf(y, a[12]), a[13]);
  return fmaxf(fmaxf(x, a[14]), fmaxf(y, a[15]));
}

}  // namespace

template <int G, bool WINDOWED, bool PAGED>
__global__ void __launch_bounds__(kThreads, 2) prefill_fwd_d64(KParams p) {
  constexpr int P = kRows / G;  // positions per work-group
  __shared__ u32x4 lds_k[kSlots * kTileChunks];
  __shared__ u32x4 lds_v[kSlots * kTileChunks];
  __shared__ u32x4 lds_q[kRows * kChunks];  // the work-group's query rows, staged once
  __shared__ int redo_vote[kWaves];

  const int Hkv = p.n_kv_heads;
  const int Hq = Hkv * G;
  const int id = blockIdx.x;
  // Consecutive work-group ids go to different XCDs; with the KV head as the
  // fastest index, each XCD's L2 sees the K/V of a fixed set of heads.
  const int g = id % Hkv;
  const int item = id / Hkv;
  // Position blocks are issued last-first: under a causal mask the late blocks
  // carry the most key tiles, so the longest work starts first (in groups of
  // sequences whose K/V fit one XCD's L2, cdna4.h's direct order).  When many
  // blocks lie past their sequence's end (the grid is sized for the longest
  // sequence) the order leaves them out, and its surplus ids come last and
  // return at once; a windowed layer's blocks all carry about the same work,
  // so its order only keeps a sequence's blocks together (their K/V tiles
  // overlap).
  int b, pblk;
  direct_block_item(item, p.n_seqs, p.n_pblocks, p.seq_group, b, pblk);
  int s, L;
  if (p.n_seqs <= kCompactMaxSeqs) {
    // the sequence bounds, one per lane, in one load for either order
    int c0 = 0, c1 = 0;
    if (lane_id() < p.n_seqs) {
      c0 = p.cu[lane_id()];
      c1 = p.cu[lane_id() + 1];
    }
    if (compact_grid(p.n_seqs, __builtin_amdgcn_readlane(c1, p.n_seqs - 1), p.max_seqlen)) {
      BlockItem bi;
      const bool found = WINDOWED ? block_item_by_sequence(p.n_seqs, P, p.n_pblocks, item, c0, c1, bi)
                                  : block_item_by_level(p.n_seqs, P, p.n_pblocks, item, c0, c1, bi);
      if (!found) return;
      b = bi.seq;
      pblk = bi.blk;
      s = bi.start;
      L = bi.len;
    } else {
      s = __builtin_amdgcn_readlane(c0, b);
      L = __builtin_amdgcn_readlane(c1, b) - s;
    }
  } else {
    s = p.cu[b];
    L = p.cu[b + 1] - s;
  }
  const int p0 = pblk * P;
  if (p0 >= L) return;
  // With a KV cache the L new rows are the last L of the sequence's Lk cached
  // positions: query row i sits at key position qoff + i.
  const int Lk = PAGED ? p.seqlens_k[b] : L;
  const int qoff = PAGED ? max(Lk - L, 0) : 0;

  // The prologue (address set-up and the first loads) runs at raised wave
  // priority: a work-group starting next to a busy one on its compute unit
  // would otherwise issue only in that one's gaps.  The tile walk runs at the
  // normal priority.
  __builtin_amdgcn_s_setprio(2);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int r16 = lane & 15;
  const int half16 = (lane >> 4) & 1;
  // scale * log2(e) in a VGPR, so that the per-score multiply takes the
  // VGPR-only encoding (which two waves of a SIMD can issue in alternate cycles)
  float cv = p.c;
  asm volatile("" : "+v"(cv));

  const int last = qoff + min(L, p0 + P) - 1;
  const int first = WINDOWED ? max(0, qoff + p0 - p.window + 1) : 0;
  const int kt0 = first / kBK;
  const int kt1 = last / kBK;

  // ---- K/V staging, double-buffered: tile t lives in slot (t - kt0) mod 2.
  // The loads of tile t + 1 are issued right after the barrier that opens tile
  // t and land while tile t is consumed.  Wave w fills LDS chunks
  // [128 w, 128 w + 128) of a tile with two wave-wide loads; the lane-to-LDS
  // order is fixed by the hardware, so each lane fetches the data chunk that
  // belongs at its swizzled position.  Rows past the sequence end fall outside
  // the descriptor's range and read as zeros.
  const int64_t seq_elems = (int64_t)s * Hkv * kD;
  const int nbytes = L * Hkv * kRowBytes;  // the sequence's K (or V) rows
  const int tile_stride = kBK * Hkv * kRowBytes;
  const i32x4 rk = buffer_rsrc(p.k + seq_elems, nbytes);
  const i32x4 rv = buffer_rsrc(p.v + seq_elems, nbytes);
  int voff[2], pvoff[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int row = (2 * w + it) * 8 + (lane >> 3);
    const int data_ch = (lane & 7) ^ swz_key(row);
    voff[it] = (row * Hkv + g) * kRowBytes + data_ch * 16;
    pvoff[it] = g * kRowBytes + data_ch * 16;
  }
  const uint32_t lds_k_base = lds_addr(lds_k) + w * 2048;  // this wave's part of slot 0
  const uint32_t lds_v_base = lds_addr(lds_v) + w * 2048;
  // Paged K/V: wave w loads rows 16 w .. 16 w + 15 of a tile, which lie in one
  // page (pages hold at least 16 keys).  Lane l of pgv holds that page for
  // tile pg_base - l; the walk only goes down, so the 64 ids are refilled when
  // it leaves them (and when the exact redo restarts from the top).  Page ids
  // are clamped into the table and the pool; keys at or past Lk read as zeros.
  const int32_t* brow = PAGED ? p.block_table + (int64_t)b * p.pages_per_seq : nullptr;
  const int pmask = PAGED ? (1 << p.page_shift) - 1 : 0;
  int pg_base = -(1 << 30);
  int pgv = 0;
  auto tile_page = [&](int t) -> int {
    if ((unsigned)(pg_base - t) >= 64u) {
      pg_base = t;
      const int tt = t - lane;
      const int pi = tt >= 0 ? min((tt * kBK + 16 * w) >> p.page_shift, p.pages_per_seq - 1) : 0;
      pgv = min(max(brow[pi], 0), p.n_pages - 1);
    }
    return __builtin_amdgcn_readlane(pgv, pg_base - t);
  };
  auto issue_tile = [&](int t, int buf) {
    if constexpr (PAGED) {
      const int64_t page_off = (int64_t)tile_page(t) * p.page_elems;
      const i32x4 rkp = buffer_rsrc(p.k + page_off, p.page_bytes);
      const i32x4 rvp = buffer_rsrc(p.v + page_off, p.page_bytes);
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int key = t * kBK + (2 * w + it) * 8 + (lane >> 3);
        const int vo = key < Lk ? (key & pmask) * Hkv * kRowBytes + pvoff[it] : p.page_bytes;
        lds_dma16(lds_k_base + buf * kTileBytes + it * 1024, rkp, vo);
        lds_dma16(lds_v_base + buf * kTileBytes + it * 1024, rvp, vo);
      }
    } else {
      const int off = t * tile_stride;  // carried in the VGPR offset, which the range check covers
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        lds_dma16(lds_k_base + buf * kTileBytes + it * 1024, rk, off + voff[it]);
        lds_dma16(lds_v_base + buf * kTileBytes + it * 1024, rv, off + voff[it]);
      }
    }
  };
  // ---- this lane's two query rows (one per 32-column block nb).  Lane l holds
  // head_dim elements 16 ks + 8 hi .. + 7 of its row for ks = 0..3.
  int pos[2], head[2];
  bf16x8 qf[2][4];
  float mref[2], lsum[2];
  f32x16 o[2][2];  // [d block][nb]: O^T, rows = head_dim, columns = queries
  // The sink logits are loaded here, without a branch (a descriptor of range
  // 0 when there are no sinks reads zeros), and first used in the epilogue:
  // the compiler does not see the inline-assembly loads below, so the wait it
  // places before a use of its own load also waits for them; a use in the
  // prologue would hold back the query loads until the first tile landed.
  const __amdgpu_buffer_rsrc_t rsink =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.sinks, 0, p.sinks ? Hq * 4 : 0, kBufferConfig);
  float sink_raw[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = 64 * w + 32 * nb + l32;
    head[nb] = g * G + r % G;
    pos[nb] = p0 + r / G;
    sink_raw[nb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsink, head[nb] * 4, 0, 0));
  }
  // the sink logit in base 2 (-inf without sinks)
  auto sink_t = [&](int nb) { return p.sinks ? sink_raw[nb] * kLog2e : -INFINITY; };

  // The first tile's page id is looked up before any inline-assembly load is
  // in flight (the compiler's wait for it would wait for those too).
  if constexpr (PAGED) {
    (void)tile_page(kt1);
    asm volatile("" : : "v"(pgv));  // the wait for the ids stays ahead of those loads
  }
  // The query rows go through LDS with the same wave-wide loads as K and V:
  // each 1 KiB load covers 8 whole rows (the G heads of a position are
  // contiguous), so it is fully coalesced, and rows past the sequence end
  // read as zeros.  Wave w loads its own 64 rows, in the layout of a K tile,
  // and reads them back as MFMA B operands.
  {
    const i32x4 rq = buffer_rsrc(p.q + (int64_t)s * Hq * kD, L * Hq * kRowBytes);
    const uint32_t lds_q_base = lds_addr(lds_q) + w * 64 * kRowBytes;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = 8 * it + (lane >> 3);  // within the wave's 64 rows
      const int r = 64 * w + row;
      const int data_ch = (lane & 7) ^ swz_key(row);
      lds_dma16(lds_q_base + it * 1024, rq, ((p0 + r / G) * Hq + g * G + r % G) * kRowBytes + data_ch * 16);
    }
  }
  // Tiles are walked from the last (the diagonal) back to the first.  The
  // first tile's loads follow the query loads, so the two latencies overlap
  // and the query rows, which land first, are converted while the tile is
  // still in flight.
  issue_tile(kt1, 0);
  wait_vmem<4>();  // the query rows have landed (loads complete in order; the tile's 4 may not)
  // The query operand is the bf16 query itself, so every score accumulator
  // holds q.k exactly up to fp32 summation; the scale (times log2 e) is
  // applied to it in fp32 before the exponential.
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[nb][ks] = __builtin_bit_cast(bf16x8, lds_q[w * 64 * kChunks + swz(32 * nb + l32, 2 * ks + hi)]);

  // K fragments (A operand) of key half mb for the four 16-wide steps of head_dim.
  // Per-lane byte offsets of the operand reads within a tile, fixed for the
  // whole walk: rows 32 mb + l32 share their swizzle key with row l32, and the
  // V rows of PV step s4 share theirs with step 0, so the key half, the PV
  // step and the LDS slot only add immediate offsets.
  uint32_t koff[4], vlo_off[2], vhi_off[2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = (uint32_t)(swz(l32, 2 * ks + hi) * 16) & 0xffffu;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int key_lo = 4 * hi + (r16 >> 2);
    const int key_hi = key_lo + 8;
    const int d = 32 * db + 16 * half16 + 4 * (r16 & 3);
    vlo_off[db] = (uint32_t)(key_lo * kRowBytes + (((d >> 3) ^ swz_key(key_lo)) << 4) + (d & 7) * 2) & 0xffffu;
    vhi_off[db] = (uint32_t)(key_hi * kRowBytes + (((d >> 3) ^ swz_key(key_hi)) << 4) + (d & 7) * 2) & 0xffffu;
  }
  auto read_k = [&](const u32x4* kl, int mb, bf16x8 (&ka)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      ka[ks] = *(const bf16x8*)((const lds_char*)kl + mb * 32 * kRowBytes + koff[ks]);
  };
  // V^T fragments (A operand of the PV MFMA) of PV step s4 (keys 16 s4 .. +15), both d blocks.
  auto read_v = [&](lds_char* vb, int s4, bf16x8 (&va)[2]) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + s4 * 16 * kRowBytes + vlo_off[db]));
      const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + s4 * 16 * kRowBytes + vhi_off[db]));
      const u32x2 u0 = __builtin_bit_cast(u32x2, t0);
      const u32x2 u1 = __builtin_bit_cast(u32x2, t1);
      va[db] = __builtin_bit_cast(bf16x8, u32x4{u0[0], u0[1], u1[0], u1[1]});
    }
  };
  // Scores of the 32 x 32 block (key half mb, query block nb).  On tiles that
  // are not fully visible the accumulator starts from the mask (0 for a
  // visible key, -inf for a hidden one), so the MFMA applies it.  Element e
  // holds key k0 + 4 hi + 32 mb + 8 (e / 4) + e % 4, compared against the
  // lane's diagonal offset so that the key offset stays an immediate.
  // Mask kinds: 0 none, 1 causal only, 2 window only, 3 both (kMaskCausal | kMaskWindow).
  auto qk = [&](auto mask_tag, const bf16x8 (&ka)[4], int mb, int nb, int k0) -> f32x16 {
    constexpr int M = decltype(mask_tag)::value;
    static_assert(WINDOWED || (M & kMaskWindow) == 0, "window mask without a window");
    f32x16 acc = {};
    if constexpr (M != 0) {
      const int di = qoff + pos[nb] - k0 - 4 * hi;
      // hidden <=> cc > di, or (with a window) cc <= di - window: the sign
      // bit of di - cc, or of cc - 1 - (di - window), selects the bits of
      // -inf, else 0.  Unsigned arithmetic: the second difference can pass
      // 2^31 only when cc > di, where the first is already negative.
      const uint32_t udw = (uint32_t)di - (uint32_t)p.window;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int cc = 32 * mb + 8 * (e / 4) + (e % 4);
        uint32_t t = 0;
        if constexpr (M & kMaskCausal) t |= (uint32_t)di - cc;
        if constexpr (M & kMaskWindow) t |= (uint32_t)cc - 1u - udw;
        acc[e] = __uint_as_float((uint32_t)((int32_t)t >> 31) & 0xff800000u);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[nb][ks], acc, 0, 0, 0);
    return acc;
  };
  // Probabilities of one score block against reference m, as bf16 P^T in the
  // PV B-operand order (plo: PV step 2 mb, phi: step 2 mb + 1).  Hidden keys
  // arrive as -inf and give 0.  The exact pass also returns the lane's sum of
  // the fp32 values.
  auto block_probs = [&](const f32x16& sc, float m, bf16x8& plo, bf16x8& phi) -> float {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = __builtin_amdgcn_exp2f(fmaf(sc[e], cv, -m));
      if (e < 8) plo[e] = (__bf16)pe; else phi[e - 8] = (__bf16)pe;
      if (e & 1) a1 += pe; else a0 += pe;
    }
    return a0 + a1;
  };
  // Probabilities of the fast pass: against reference 1, exp2 of the scaled score.
  auto block_probs_fast = [&](const f32x16& sc, bf16x8& plo, bf16x8& phi) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = __builtin_amdgcn_exp2f(sc[e] * cv);
      if (e < 8) plo[e] = (__bf16)pe; else phi[e - 8] = (__bf16)pe;
    }
  };
  // Row sums of the fast pass run on the matrix pipe: a 16 x 16 x 32 MFMA
  // whose A operand is a fixed 0/1 selector reads a P^T fragment as its
  // B operand.  Of the 64 lanes holding one 16-key step of 32 queries, lanes
  // n and n + 32 carry query n and lanes n + 16, n + 48 query n + 16; row 0
  // of the selector picks the first pair and row 1 the second, so output
  // rows 0 and 1 (lanes 0..15, elements 0 and 1) accumulate the sums of the
  // bf16 probabilities of queries n and n + 16.
  const int lsel = ((lane & 15) == 0 && ((lane >> 4) & 1) == 0) || ((lane & 15) == 1 && ((lane >> 4) & 1) == 1);
  const bf16x8 sel = __builtin_bit_cast(bf16x8, lsel ? u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}
                                                     : u32x4{0u, 0u, 0u, 0u});
  f32x4 lacc[2];
  auto row_sums = [&](const bf16x8 (&pf)[4][2], int mb, int nb) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      lacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pf[2 * mb + j][nb], lacc[nb], 0, 0, 0);
  };
  // O^T += V^T P^T over the 32 keys of half mb (PV steps 2 mb, 2 mb + 1) for query block nb.
  auto pv = [&](const bf16x8 (&va)[2][2], const bf16x8 (&pf)[4][2], int mb, int nb) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < 2; ++db)
        o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j][db], pf[2 * mb + j][nb], o[db][nb], 0, 0, 0);
  };
  // One MFMA, then n VALU instructions, k times (the order within a step).
  auto interleave = [](auto k_tag, auto n_tag) {
    constexpr int k = decltype(k_tag)::value;
    constexpr int n = decltype(n_tag)::value;
#pragma unroll
    for (int i = 0; i < k; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, n, 0);
    }
  };

  // ---- fast tile: every row keeps its reference fixed (no maxima, no
  // rescaling), and row sums accumulate on the matrix pipe.  The tile runs as
  // six steps over its four 32 x 32 blocks so that each block's softmax
  // overlaps the MFMAs of its neighbours:
  //   0: scores (0,0) (0,1)            1: scores (1,0) | probs (0,0)
  //   2: scores (1,1) | probs (0,1)    3: PV (0,0)     | probs (1,0)
  //   4: PV (0,1)     | probs (1,1)    5: PV (1,0) (1,1)
  using I4 = std::integral_constant<int, 4>;
  using I6 = std::integral_constant<int, 6>;
  auto tile_fast = [&](auto mask_tag, const u32x4* kl, lds_char* vb, int k0) {
    constexpr int nv = 6;  // vector instructions after each score MFMA
    constexpr int nw = 4;  // ... after each PV or row-sum MFMA
    bf16x8 ka[4], kb[4], pf[4][2], va[2][2], vc[2][2];
    read_k(kl, 0, ka);
    read_k(kl, 1, kb);
    const f32x16 s00 = qk(mask_tag, ka, 0, 0, k0);
    const f32x16 s01 = qk(mask_tag, ka, 0, 1, k0);
    __builtin_amdgcn_sched_barrier(0);
    read_v(vb, 0, va[0]);
    read_v(vb, 1, va[1]);
    const f32x16 s10 = qk(mask_tag, kb, 1, 0, k0);
    block_probs_fast(s00, pf[0][0], pf[1][0]);
    interleave(I4{}, std::integral_constant<int, nv>{});
    __builtin_amdgcn_sched_barrier(0);
    const f32x16 s11 = qk(mask_tag, kb, 1, 1, k0);
    block_probs_fast(s01, pf[0][1], pf[1][1]);
    interleave(I4{}, std::integral_constant<int, nv>{});
    __builtin_amdgcn_sched_barrier(0);
    read_v(vb, 2, vc[0]);
    read_v(vb, 3, vc[1]);
    pv(va, pf, 0, 0);
    row_sums(pf, 0, 0);
    block_probs_fast(s10, pf[2][0], pf[3][0]);
    interleave(I6{}, std::integral_constant<int, nw>{});
    __builtin_amdgcn_sched_barrier(0);
    pv(va, pf, 0, 1);
    row_sums(pf, 0, 1);
    block_probs_fast(s11, pf[2][1], pf[3][1]);
    interleave(I6{}, std::integral_constant<int, nw>{});
    __builtin_amdgcn_sched_barrier(0);
    pv(vc, pf, 1, 0);
    row_sums(pf, 1, 0);
    pv(vc, pf, 1, 1);
    row_sums(pf, 1, 1);
  };

  // ---- half tile: only key half mb of the tile, masked, for a tile whose
  // other 32 keys are hidden from every row (the upper half of a diagonal
  // tile whose rows all sit in its lower half, or the lower half of a tile
  // that has left every row's window).
  auto tile_half = [&](auto mb_tag, auto mask_tag, const u32x4* kl, lds_char* vb, int k0) {
    constexpr int mb = decltype(mb_tag)::value;
    bf16x8 ka[4], pf[4][2], va[2][2];
    read_k(kl, mb, ka);
    const f32x16 s0 = qk(mask_tag, ka, mb, 0, k0);
    const f32x16 s1 = qk(mask_tag, ka, mb, 1, k0);
    __builtin_amdgcn_sched_barrier(0);
    read_v(vb, 2 * mb, va[0]);
    read_v(vb, 2 * mb + 1, va[1]);
    block_probs_fast(s0, pf[2 * mb][0], pf[2 * mb + 1][0]);
    block_probs_fast(s1, pf[2 * mb][1], pf[2 * mb + 1][1]);
    __builtin_amdgcn_sched_barrier(0);
    pv(va, pf, mb, 0);
    row_sums(pf, mb, 0);
    pv(va, pf, mb, 1);
    row_sums(pf, mb, 1);
  };

  // ---- exact tile: streaming softmax with running maxima and fp32 row sums
  // on the vector ALU.  It runs every tile of a work-group whose fast pass
  // left range.  Each key half raises the row maxima, rescales the
  // accumulators, then adds its probabilities.
  auto tile_exact = [&](auto mask_tag, const u32x4* kl, lds_char* vb, int k0) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      bf16x8 ka[4], pf[4][2], va[2][2];
      read_k(kl, mb, ka);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const f32x16 sc = qk(mask_tag, ka, mb, nb, k0);
        // the largest scaled score (c > 0, and rounding is monotonic)
        const float mx = pair_max(max16(sc)) * cv;
        if (mx > mref[nb]) {
          const float alpha = __builtin_amdgcn_exp2f(mref[nb] - mx);
          lsum[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[db][nb][e] *= alpha;
          mref[nb] = mx;
        }
        const float m = (mref[nb] == -INFINITY) ? 0.f : mref[nb];
        lsum[nb] += block_probs(sc, m, pf[2 * mb][nb], pf[2 * mb + 1][nb]);
      }
      read_v(vb, 2 * mb, va[0]);
      read_v(vb, 2 * mb + 1, va[1]);
      pv(va, pf, mb, 0);
      pv(va, pf, mb, 1);
    }
  };

  // Walk the tiles of this work-group's key range from the last to the first.
  // Only tiles that are not fully visible to every row take the mask: tiles
  // [ktB, kt1] hold keys past some row's position (they also hold every row's
  // own key), tiles [kt0, ktA) may hold keys that left some row's window.
  //   unmasked <=> k0 + kBK - 1 <= p0  and (no window or (p0 + P - 1) - k0 < window)
  // The runs are separate loops so that each loop body holds one kind of
  // tile.
  const int ktB = max(kt0, min(kt1 + 1, (qoff + p0 + 1) / kBK));  // first tile with k0 + kBK - 1 > qoff + p0
  const int xa = qoff + p0 + P - p.window;  // first tile with k0 >= xa: all its keys inside every window
  const int ktA = (WINDOWED && xa > 0) ? min(ktB, max(kt0, (xa + kBK - 1) / kBK)) : kt0;
  auto walk = [&](auto tile_fn, int kt_hi, int kt_lo) {
    for (int kt = kt_hi; kt >= kt_lo; --kt) {
      const int buf = (kt1 - kt) & 1;
      wait_vmem<0>();   // this wave's loads of tile kt have landed
      __syncthreads();  // every wave's have; the previous tile is fully consumed
      if (kt > kt0) issue_tile(kt - 1, buf ^ 1);
      tile_fn(&lds_k[buf * kTileChunks], (lds_char*)&lds_v[buf * kTileChunks], kt * kBK);
    }
  };
  using MNone = std::integral_constant<int, 0>;
  using MCausal = std::integral_constant<int, kMaskCausal>;
  using MWindow = std::integral_constant<int, WINDOWED ? kMaskWindow : 0>;
  using MBoth = std::integral_constant<int, kMaskCausal | (WINDOWED ? kMaskWindow : 0)>;
  using Lo = std::integral_constant<int, 0>;
  using Hi = std::integral_constant<int, 1>;
  auto fast_both = [&](const u32x4* kl, lds_char* vb, int k0) { tile_fast(MBoth{}, kl, vb, k0); };
  auto fast_causal = [&](const u32x4* kl, lds_char* vb, int k0) { tile_fast(MCausal{}, kl, vb, k0); };
  auto fast_window = [&](const u32x4* kl, lds_char* vb, int k0) { tile_fast(MWindow{}, kl, vb, k0); };
  auto fast_open = [&](const u32x4* kl, lds_char* vb, int k0) { tile_fast(MNone{}, kl, vb, k0); };
  auto half_lo_both = [&](const u32x4* kl, lds_char* vb, int k0) { tile_half(Lo{}, MBoth{}, kl, vb, k0); };
  auto half_lo_causal = [&](const u32x4* kl, lds_char* vb, int k0) { tile_half(Lo{}, MCausal{}, kl, vb, k0); };
  auto half_hi_both = [&](const u32x4* kl, lds_char* vb, int k0) { tile_half(Hi{}, MBoth{}, kl, vb, k0); };
  auto half_hi_window = [&](const u32x4* kl, lds_char* vb, int k0) { tile_half(Hi{}, MWindow{}, kl, vb, k0); };
  auto reset = [&]() {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      mref[nb] = sink_t(nb);
      lsum[nb] = 0.f;
      lacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][nb][e] = 0.f;
    }
  };

  reset();
  mref[0] = mref[1] = 0.f;  // the fast pass measures every probability against 1
  __builtin_amdgcn_s_setprio(0);
  // Tile kt1 (always a masked one) skips its upper 32 keys when they lie past
  // every row's position; with a window, tile kt0 (then always masked too)
  // skips its lower 32 keys when they lie before every row's window.  The two
  // never fall on one tile (first <= last).
  const bool hi_half_hidden = (last & (kBK - 1)) < kBK / 2;
  const bool lo_half_hidden = WINDOWED && (first & (kBK - 1)) >= kBK / 2;
  const int top = hi_half_hidden ? kt1 - 1 : kt1;
  const int bot = lo_half_hidden ? kt0 + 1 : kt0;
  // Which tests a masked tile needs.  Tiles [ktB, kt1] need the causal one,
  // and the window one only if the window reaches them: it can hide a key of
  // tile kt from some row only if kt * kBK <= last - window.  Tiles below ktA
  // (below ktB) hold no key past any row's position: the window test alone.
  const bool diag_windowed = WINDOWED && last - p.window >= 0 && ktB <= (last - p.window) / kBK;
  if (!WINDOWED || !diag_windowed) {
    if (hi_half_hidden) walk(half_lo_causal, kt1, kt1);
    walk(fast_causal, top, max(ktB, bot));
  } else {
    if (hi_half_hidden) walk(half_lo_both, kt1, kt1);
    walk(fast_both, top, max(ktB, bot));
  }
  walk(fast_open, ktB - 1, ktA);
  if constexpr (WINDOWED) {
    walk(fast_window, ktA - 1, bot);
    if (lo_half_hidden) {
      if (kt0 < ktB) walk(half_hi_window, kt0, kt0);
      else walk(half_hi_both, kt0, kt0);
    }
  }
  // A row's sum from the row-sum accumulators: query q of block nb sits in
  // lane q % 16, element q / 16.
  float lrow[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float e0 = __shfl(lacc[nb][0], l32 & 15);
    const float e1 = __shfl(lacc[nb][1], l32 & 15);
    lrow[nb] = (l32 < 16) ? e0 : e1;
  }
  // The fast pass is kept unless a row's sum left [2^-64, 2^65) or a sum or
  // an output is not finite.  Then the rows are redone exactly.  The vote is
  // taken per half of the work-group (waves 0-1 and 2-3: 128 rows each, the
  // rows of one work-group of the 128-row kernel), so that a row's arithmetic
  // does not depend on which of the two kernels ran it.  All four waves walk
  // the redo, since each loads its part of every tile; a half whose fast
  // result stands stores it first and only loads.
  bool redo_mine = false, redo_any = false;
  {
    bool bad = false;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float osum = pairwise_sum32(o[0][nb], o[1][nb]);
      bad = bad || !positive_in_binade_range(lrow[nb], -kFastSumBinades, kFastSumBinades) ||
            !finite_bits(osum);
    }
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) redo_vote[w] = wave_bad ? 1 : 0;
    __syncthreads();
    const int hv = 2 * (w >> 1);
    redo_mine = (redo_vote[hv] | redo_vote[hv + 1]) != 0;
    redo_any = (redo_vote[0] | redo_vote[1] | redo_vote[2] | redo_vote[3]) != 0;
  }

  // ---- epilogue: add the sink's term to the row sum, normalise, store.
  // The rows go out through LDS: each wave writes its 64 normalised rows into
  // its own part of the query staging area (unused since the prologue), in
  // the staging layout, and reads them back one row per 8 lanes, so that each
  // store instruction writes 8 whole 128-byte rows (1 KiB contiguous when the
  // G heads of a position are) instead of 16-byte pieces of 32 rows.  Rows
  // past the sequence end fall outside the output descriptor's range and are
  // dropped.
  auto store_rows = [&]() {
    // The lane index is laundered so that no address term of the query loads,
    // which share these offsets, is kept live through the walk to be reused.
    int el = lane;
    asm volatile("" : "+v"(el));
    const int el32 = el & 31, ehi = el >> 5;
    u32x2* const lds_o = reinterpret_cast<u32x2*>(&lds_q[w * 64 * kChunks]);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float lt = lrow[nb];
      if (p.sinks) lt += __builtin_amdgcn_exp2f(sink_t(nb) - mref[nb]);
      const float inv = __builtin_amdgcn_rcpf(lt);  // v_rcp_f32: 1 ulp, far below the bf16 rounding
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          // head_dim elements 32 db + 8 vg + 4 hi .. + 3: half hi of chunk 4 db + vg
          bf16x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = (__bf16)(o[db][nb][4 * vg + e] * inv);
          lds_o[2 * swz(32 * nb + el32, 4 * db + vg) + ehi] = __builtin_bit_cast(u32x2, val);
        }
    }
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.out + (int64_t)s * Hq * kD), 0, L * Hq * kRowBytes, kBufferConfig);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = 8 * it + (el >> 3);  // within the wave's 64 rows
      const int r = 64 * w + row;
      const int ch = el & 7;
      const u32x4 x = lds_q[w * 64 * kChunks + swz(row, ch)];
      __builtin_amdgcn_raw_buffer_store_b128(x, ro, ((p0 + r / G) * Hq + g * G + r % G) * kRowBytes + ch * 16, 0, kStreamStore);
    }
  };

  if (redo_any) {
    if (redo_mine) reset();
    else store_rows();
    auto redo_tile = [&](const u32x4* kl, lds_char* vb, int k0) {
      if (redo_mine) tile_exact(MBoth{}, kl, vb, k0);
    };
    issue_tile(kt1, 0);
    walk(redo_tile, kt1, kt0);
    if (redo_mine) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) lrow[nb] = pair_sum(lsum[nb]);
    }
  }
  if (!redo_any || redo_mine) store_rows();
}

namespace {

template <int G>
hipError_t launch_group(const KParams& kp, int64_t grid, bool windowed, bool paged, hipStream_t stream) {
  const dim3 gd((unsigned)grid), bd(kThreads);
  if (paged) {
    if (windowed)
      hipLaunchKernelGGL((prefill_fwd_d64<G, true, true>), gd, bd, 0, stream, kp);
    else
      hipLaunchKernelGGL((prefill_fwd_d64<G, false, true>), gd, bd, 0, stream, kp);
  } else {
    if (windowed)
      hipLaunchKernelGGL((prefill_fwd_d64<G, true, false>), gd, bd, 0, stream, kp);
    else
      hipLaunchKernelGGL((prefill_fwd_d64<G, false, false>), gd, bd, 0, stream, kp);
  }
  return hipGetLastError();
}

int64_t pblocks(const PrefillArgs& a) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const int P = kRows / G;
  return ((int64_t)a.max_seqlen + P - 1) / P;
}

}  // namespace

int32_t prefill_seq_group(const PrefillArgs& a, int row_bytes) {
  // K and V of one sequence as one XCD's L2 sees them: consecutive work-group
  // ids go to different XCDs with the KV head fastest, so one XCD serves
  // n_kv_heads / 8 KV heads (one when there are 8 or fewer)
  const int64_t per_seq = std::max<int64_t>(1, (int64_t)a.max_seqlen * 2 * row_bytes * std::max(1, a.n_kv_heads / 8));
  return (int32_t)std::min<int64_t>(std::max<int64_t>(kSeqGroupBytes / per_seq, 1), std::max(1, a.n_seqs));
}

int64_t prefill_grid_size(const PrefillArgs& a) {
  // each sequence's K (or V) rows must be addressable by one buffer descriptor
  // (a cache is addressed page by page instead)
  if (!a.block_table && ((int64_t)a.max_seqlen + kBK) * a.n_kv_heads * kRowBytes > 0x7fffffffLL) return -1;
  // and its query rows, including a position block's rows past the end
  if (((int64_t)a.max_seqlen + kRows) * a.n_q_heads * kRowBytes > 0x7fffffffLL) return -1;
  const int64_t n = pblocks(a) * (int64_t)a.n_seqs * (int64_t)a.n_kv_heads;
  if (n > 0x7fffffffLL) return -1;
  return n;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int64_t grid = prefill_grid_size(a);
  if (grid <= 0) return hipSuccess;
  KParams kp;
  kp.q = static_cast<const uint16_t*>(a.q);
  kp.k = static_cast<const uint16_t*>(a.k);
  kp.v = static_cast<const uint16_t*>(a.v);
  kp.sinks = a.sinks;
  kp.cu = a.cu_seqlens;
  kp.out = static_cast<uint16_t*>(a.out);
  kp.n_kv_heads = a.n_kv_heads;
  kp.n_seqs = a.n_seqs;
  kp.n_pblocks = (int32_t)pblocks(a);
  kp.window = a.window > 0 ? a.window : 0;
  kp.c = (float)((double)a.softmax_scale * 1.4426950408889634);
  kp.seqlens_k = a.seqlens_k;
  kp.block_table = a.block_table;
  kp.page_elems = (int64_t)a.page_size * a.n_kv_heads * kD;
  kp.page_bytes = a.page_size * a.n_kv_heads * kRowBytes;
  kp.page_shift = a.page_size > 0 ? __builtin_ctz((unsigned)a.page_size) : 0;
  kp.pages_per_seq = a.pages_per_seq;
  kp.n_pages = a.n_pages;
  kp.max_seqlen = a.max_seqlen;
  kp.seq_group = prefill_seq_group(a, kRowBytes);
  const bool windowed = a.window > 0;
  const bool paged = a.block_table != nullptr;
  (void)hipGetLastError();  // start from a clean per-thread error state
  switch (a.n_q_heads / a.n_kv_heads) {
    case 1: return launch_group<1>(kp, grid, windowed, paged, stream);
    case 2: return launch_group<2>(kp, grid, windowed, paged, stream);
    case 4: return launch_group<4>(kp, grid, windowed, paged, stream);
    case 8: return launch_group<8>(kp, grid, windowed, paged, stream);
    case 16: return launch_group<16>(kp, grid, windowed, paged, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tsmha
