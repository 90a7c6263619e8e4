// prefill_fwd_narrow.hip -- gfx950 (CDNA4) kernels for causal grouped-query
// prefill attention with sliding windows and attention sinks, 32 query rows
// per wave: head_dim 128, and head_dim 64 when the launch is too small to fill
// the GPU with the 256-row work-groups of prefill_fwd.hip.
//
// The same operation as the head_dim 64 kernels (the `mha_prefill` call of the
// TokenSpeed-kernel README, section "Public API"; sinks and sliding windows as
// for the GPT-OSS layers of "TokenSpeed-kernel multi-silicon", section
// "Числа: Gluon на AMD MI355X"); head_dim 128 is the other head width the
// README's kernel traits name.  The design follows the head_dim 64 kernel of
// prefill_fwd.hip, resized:
//
// Work decomposition.  One work-group (4 waves) owns 128 query rows: all G
// query heads of one KV head for P = 128 / G consecutive positions of one
// sequence; each wave holds 32 of them, so that at head_dim 128 the output
// (128 x 32 fp32) and the query operand (32 x 128 bf16) take the registers the
// head_dim 64 kernel spends on 64 rows.  At head_dim 64 the same shape needs
// about 145 VGPRs and 32 KiB of LDS, so three work-groups fit on a compute
// unit, and a launch has twice as many work-groups, each with half the rows:
// that fills the GPU on short or few sequences.  Every K/V tile staged in LDS
// serves the whole head group.
//
// Orientation.  Scores are formed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16 (two 32-key blocks per 64-key tile, D / 16 steps of
// head_dim); lane l holds query l % 32.  The output is accumulated transposed
// too, O^T += V^T P^T (D / 32 blocks of 32 head_dim rows), with V^T read by
// ds_read_b64_tr_b16 from the row-major V tile and P^T taken straight from the
// score accumulators.
//
// Staging.  K and V tiles (64 rows of 2 D bytes) move from HBM to LDS with
// buffer_load_dwordx4 ... lds, double-buffered; the query rows are staged once
// in the second slot before the walk (64 KiB of LDS per work-group at head_dim
// 128, 32 KiB at 64).  A 16-byte chunk c of a 256-byte row r sits at position
// c ^ (((r & 3) << 2) | ((r >> 2) & 3)): 16 consecutive rows reading one chunk
// (K and Q operands) and 4 aligned rows reading two adjacent chunks (the
// transposed V reads) each hit distinct banks of the 64-bank LDS; 128-byte
// rows use the swizzle of cdna4.h, laid out for the same access patterns.
//
// Paged K/V (head_dim 128 only; head_dim 64 uses the 256-row kernel's form):
// the prefill of new rows against a cache, as in prefill_fwd.hip: query
// positions shifted by the cached keys before them, each wave's 16 rows of a
// tile loaded from one page.
//
// Softmax.  As in prefill_fwd.hip: base 2, scale * log2(e) applied to each fp32
// score, every probability exp2 of its scaled score against reference 1,
// row sums on the matrix pipe, and a streaming softmax with running maxima for
// a work-group whose sums leave [2^-64, 2^65).
#include <math.h>

#include <type_traits>

#include "cdna4.h"
#include "prefill_fwd.h"

namespace tsmha {

using namespace cdna4;

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;                        // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;                        // query rows per wave
constexpr int kRows = kQW * kWaves;            // (query head, position) rows per work-group
template <int D>
struct Shape {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kTileBytes = kBK * kRowBytes;
  static constexpr int kTileChunks = kTileBytes / 16;
  static constexpr int kKS = D / 16;
  static constexpr int kDB = D / 32;
  static constexpr int kRPL = 1024 / kRowBytes;       // rows per wave-wide 1 KiB load
  static constexpr int kTileLoads = 16 / kRPL;         // a wave's loads per tile and tensor
  static constexpr int kQLoads = kQW / kRPL;           // a wave's loads of its query rows
};
constexpr int kFastSumBinades = 64;  // the fast pass keeps row sums in [2^-64, 2^65)
constexpr int kMaskCausal = 1;       // mask kinds: key past the row's position
constexpr int kMaskWindow = 2;       // ... key before the row's window

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* sinks;
  const int32_t* cu;
  uint16_t* out;
  int32_t n_kv_heads;
  int32_t n_seqs;
  int32_t n_pblocks;
  int32_t max_seqlen;
  int32_t seq_group;  // sequences per group of the direct order (>= 1)
  int32_t window;
  float c;  // softmax_scale * log2(e)
  // paged K/V only: k and v are the caches [n_pages][page_size][n_kv_heads][D]
  const int32_t* seqlens_k;    // cached keys per sequence, the new rows' own included
  const int32_t* block_table;  // [n_seqs][pages_per_seq] page ids
  int64_t page_elems;          // bf16 elements per page
  int32_t page_bytes;
  int32_t page_shift;
  int32_t pages_per_seq;
  int32_t n_pages;
};

// Position of 16-byte chunk `ch` of row `row` in a tile of 256-byte rows.
__device__ __forceinline__ int key16(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
template <int D>
__device__ __forceinline__ int tkey(int row) {
  if constexpr (D == 128) return key16(row); else return swz_key(row);
}
template <int D>
__device__ __forceinline__ int tpos(int row, int ch) { return row * Shape<D>::kChunks + (ch ^ tkey<D>(row)); }

__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max16(const f32x16& a) {
  float x = fmaxf(fmaxf(a[0], a[1]), a[2]);
  float y = fmaxf(fmaxf(a[3], a[4]), a[5]);
  x = fmaxf(fmaxf(x, a[6]), a[7]);
  y = fmaxf(fmaxf(y, a[8]), a[9]);
  x = fmaxf(fmaxf(x, a[10]), a[11]);
  y = fmaxf(fmaxf(y, a[12]), a[13]);
  return fmaxf(fmaxf(x, a[14]), fmaxf(y, a[15]));
}

template <int D, int G, bool WINDOWED, bool PAGED>
__global__ void __launch_bounds__(kThreads, D == 64 ? 3 : 2) prefill_fwd_narrow(Params p) {
  using S = Shape<D>;
  constexpr int kD = D;
  constexpr int kRowBytes = S::kRowBytes;
  constexpr int kChunks = S::kChunks;
  constexpr int kTileBytes = S::kTileBytes;
  constexpr int kTileChunks = S::kTileChunks;
  constexpr int KS = S::kKS;
  constexpr int DB = S::kDB;
  constexpr int RPL = S::kRPL;
  constexpr int P = kRows / G;  // positions per work-group
  __shared__ u32x4 lds_k[2 * kTileChunks];
  __shared__ u32x4 lds_v[2 * kTileChunks];
  __shared__ int redo_vote[kWaves];

  const int Hkv = p.n_kv_heads;
  const int Hq = Hkv * G;
  const int id = blockIdx.x;
  // KV head fastest (each XCD's L2 serves a fixed set of heads), position
  // blocks last-first (the longest causal work starts first) in groups of
  // sequences whose K/V fit one XCD's L2, and when many blocks lie past their
  // sequence's end, an order that leaves them out.
  const int g = id % Hkv;
  const int item = id / Hkv;
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

  __builtin_amdgcn_s_setprio(2);  // the prologue at raised priority, the walk at normal
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int r16 = lane & 15;
  const int half16 = (lane >> 4) & 1;
  // scale * log2(e) in a VGPR, so that the per-score multiply takes the
  // VGPR-only encoding
  float cv = p.c;
  asm volatile("" : "+v"(cv));

  const int last = qoff + min(L, p0 + P) - 1;
  const int first = WINDOWED ? max(0, qoff + p0 - p.window + 1) : 0;
  const int kt0 = first / kBK;
  const int kt1 = last / kBK;

  // ---- K/V staging: tile t lives in slot (kt1 - t) & 1.  Wave w fills rows
  // 16 w .. 16 w + 15 of a tile with four wave-wide 1 KiB loads (4 rows each)
  // per tensor; each lane fetches the data chunk that belongs at its
  // swizzled LDS position.  Rows past the sequence end read as zeros.
  const int64_t seq_elems = (int64_t)s * Hkv * kD;
  const int nbytes = L * Hkv * kRowBytes;
  const int tile_stride = kBK * Hkv * kRowBytes;
  const i32x4 rk = buffer_rsrc(p.k + seq_elems, nbytes);
  const i32x4 rv = buffer_rsrc(p.v + seq_elems, nbytes);
  int voff[S::kTileLoads], pvoff[S::kTileLoads];
#pragma unroll
  for (int i = 0; i < S::kTileLoads; ++i) {
    const int row = 16 * w + RPL * i + lane / kChunks;
    voff[i] = (row * Hkv + g) * kRowBytes + ((lane % kChunks) ^ tkey<D>(row)) * 16;
    pvoff[i] = g * kRowBytes + ((lane % kChunks) ^ tkey<D>(row)) * 16;
  }
  const uint32_t lds_k_base = lds_addr(lds_k) + w * 16 * kRowBytes;
  const uint32_t lds_v_base = lds_addr(lds_v) + w * 16 * kRowBytes;
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
      for (int i = 0; i < S::kTileLoads; ++i) {
        const int key = t * kBK + 16 * w + RPL * i + lane / kChunks;
        const int vo = key < Lk ? (key & pmask) * Hkv * kRowBytes + pvoff[i] : p.page_bytes;
        lds_dma16(lds_k_base + buf * kTileBytes + i * 1024, rkp, vo);
        lds_dma16(lds_v_base + buf * kTileBytes + i * 1024, rvp, vo);
      }
    } else {
      const int off = t * tile_stride;
#pragma unroll
      for (int i = 0; i < S::kTileLoads; ++i) {
        lds_dma16(lds_k_base + buf * kTileBytes + i * 1024, rk, off + voff[i]);
        lds_dma16(lds_v_base + buf * kTileBytes + i * 1024, rv, off + voff[i]);
      }
    }
  };

  // ---- this lane's query row: 32 w + l32 of the work-group.
  const int r_me = kQW * w + l32;
  const int head = g * G + r_me % G;
  const int pos = p0 + r_me / G;
  // The sink logit: a branch-free buffer load (range 0 without sinks), first
  // used in the epilogue, so no wait for it holds back the loads below.
  const __amdgpu_buffer_rsrc_t rsink =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.sinks, 0, p.sinks ? Hq * 4 : 0, kBufferConfig);
  const float sink_raw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsink, head * 4, 0, 0));
  auto sink_t = [&]() { return p.sinks ? sink_raw * kLog2e : -INFINITY; };

  // The first tile's page id is looked up before any inline-assembly load is
  // in flight (the compiler's wait for it would wait for those too).
  if constexpr (PAGED) {
    (void)tile_page(kt1);
    asm volatile("" : : "v"(pgv));  // the wait for the ids stays ahead of those loads
  }

  // The query rows go through slot 1 of the tiles (waves 0 and 1 in the K
  // slot, 2 and 3 in the V slot; 8 KiB each), with eight wave-wide loads of 4
  // whole rows, then the first tile into slot 0.  Slot 1 receives its first
  // tile only after the walk's first barrier, when every wave holds its
  // query operand in registers.
  const uint32_t q_lds = (w < 2 ? lds_addr(lds_k) : lds_addr(lds_v)) + kTileBytes + (w & 1) * kQW * kRowBytes;
  {
    const i32x4 rq = buffer_rsrc(p.q + (int64_t)s * Hq * kD, L * Hq * kRowBytes);
#pragma unroll
    for (int i = 0; i < S::kQLoads; ++i) {
      const int row = RPL * i + lane / kChunks;  // within the wave's 32 rows
      const int r = kQW * w + row;
      const int data_ch = (lane % kChunks) ^ tkey<D>(row);
      lds_dma16(q_lds + i * 1024, rq, ((p0 + r / G) * Hq + g * G + r % G) * kRowBytes + data_ch * 16);
    }
  }
  issue_tile(kt1, 0);
  wait_vmem<2 * S::kTileLoads>();  // the query rows have landed (the tile's loads may not)
  // Query operand (B of the score MFMA) for the D / 16 steps of head_dim:
  // lane l holds elements 16 ks + 8 hi .. + 7 of its row, the bf16 query
  // itself (the scale is applied to the fp32 scores).
  bf16x8 qf[KS];
  {
    const lds_char* qb = (w < 2 ? (const lds_char*)lds_k : (const lds_char*)lds_v) + kTileBytes + (w & 1) * kQW * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8*)(qb + tpos<D>(l32, 2 * ks + hi) * 16);
  }

  // Per-lane byte offsets of the operand reads within a tile, fixed for the
  // walk: K rows 32 mb + l32 share their swizzle with row l32, and the V rows
  // of PV step s4 with step 0, so the key half and the step add immediates.
  uint32_t koff[KS], vlo_off[DB], vhi_off[DB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = (uint32_t)(tpos<D>(l32, 2 * ks + hi) * 16);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int key_lo = 4 * hi + (r16 >> 2);
    const int key_hi = key_lo + 8;
    const int d = 32 * db + 16 * half16 + 4 * (r16 & 3);
    vlo_off[db] = (uint32_t)(tpos<D>(key_lo, d >> 3) * 16 + (d & 7) * 2);
    vhi_off[db] = (uint32_t)(tpos<D>(key_hi, d >> 3) * 16 + (d & 7) * 2);
  }
  auto read_k = [&](const lds_char* kl, int mb, bf16x8 (&ka)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = *(const bf16x8*)(kl + mb * 32 * kRowBytes + koff[ks]);
  };
  // V^T fragment (A of the PV MFMA) of PV step s4 (keys 16 s4 .. +15) and head_dim block db.
  auto read_v = [&](const lds_char* vb, int s4, int db) -> bf16x8 {
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + s4 * 16 * kRowBytes + vlo_off[db]));
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + s4 * 16 * kRowBytes + vhi_off[db]));
    const u32x2 u0 = __builtin_bit_cast(u32x2, t0);
    const u32x2 u1 = __builtin_bit_cast(u32x2, t1);
    return __builtin_bit_cast(bf16x8, u32x4{u0[0], u0[1], u1[0], u1[1]});
  };
  // Scores of key half mb: element e holds key k0 + 32 mb + 8 (e / 4) + 4 hi + e % 4.
  // Masked tiles start the accumulator from the mask (0 visible, -inf hidden).
  // Mask kinds: 0 none, 1 causal only, 2 window only, 3 both.
  auto qk = [&](auto mask_tag, const bf16x8 (&ka)[KS], int mb, int k0) -> f32x16 {
    constexpr int M = decltype(mask_tag)::value;
    static_assert(WINDOWED || (M & kMaskWindow) == 0, "window mask without a window");
    f32x16 acc = {};
    if constexpr (M != 0) {
      const int di = qoff + pos - k0 - 4 * hi;
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
    for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], acc, 0, 0, 0);
    return acc;
  };
  // bf16 P^T of one score block in the PV B-operand order (plo: PV step 2 mb,
  // phi: step 2 mb + 1): the fast pass's exp2(scale * log2 e * s) against
  // reference 1, and the exact pass's against reference m with the lane's
  // sum of the fp32 values.
  auto probs = [&](const f32x16& sc, bf16x8& plo, bf16x8& phi) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = __builtin_amdgcn_exp2f(sc[e] * cv);
      if (e < 8) plo[e] = (__bf16)pe; else phi[e - 8] = (__bf16)pe;
    }
  };
  auto probs_sum = [&](const f32x16& sc, float m, bf16x8& plo, bf16x8& phi) -> float {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = __builtin_amdgcn_exp2f(fmaf(sc[e], cv, -m));
      if (e < 8) plo[e] = (__bf16)pe; else phi[e - 8] = (__bf16)pe;
      if (e & 1) a1 += pe; else a0 += pe;
    }
    return a0 + a1;
  };
  // Row sums on the matrix pipe: a 16 x 16 x 32 MFMA with a 0/1 selector as A
  // reads a P^T fragment (16 keys x 32 queries) as B; rows 0 and 1 of the
  // result (lanes 0..15, elements 0 and 1) accumulate the sums of queries n
  // and n + 16.
  const int lsel = ((lane & 15) == 0 && ((lane >> 4) & 1) == 0) || ((lane & 15) == 1 && ((lane >> 4) & 1) == 1);
  const bf16x8 sel = __builtin_bit_cast(bf16x8, lsel ? u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}
                                                     : u32x4{0u, 0u, 0u, 0u});
  f32x16 o[DB];  // O^T blocks: head_dim 32 db .. + 31 x the wave's 32 queries
  f32x4 lacc;
  float mref, lsum;
  // V^T fragments of PV steps s0, s0 + 1 (all four head_dim blocks), and
  // O^T += V^T P^T over them.
  auto read_v2 = [&](const lds_char* vb, int s0, bf16x8 (&va)[2][DB]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < DB; ++db) va[j][db] = read_v(vb, s0 + j, db);
  };
  auto pv2 = [&](const bf16x8 (&va)[2][DB], const bf16x8 (&pf)[4], int s0) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j][db], pf[s0 + j], o[db], 0, 0, 0);
  };
  auto interleave = [](auto k_tag, auto n_tag) {
    constexpr int k = decltype(k_tag)::value;
    constexpr int n = decltype(n_tag)::value;
#pragma unroll
    for (int i = 0; i < k; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, n, 0);
    }
  };

  // ---- fast tile: probabilities against reference 1, row sums on the matrix
  // pipe.  Scores of key half 0; scores of half 1 | probabilities of half 0;
  // then the four PV steps with their row sums, the probabilities of half 1
  // interleaved, each step's V^T fragments read one step ahead (16 VGPRs at
  // a time, which leaves the compiler room to keep the K reads ahead of the
  // score MFMAs).
  auto tile_fast = [&](auto mask_tag, const lds_char* kl, const lds_char* vb, int k0) {
    bf16x8 ka[KS], pf[4], va[DB], vn[DB];
    read_k(kl, 0, ka);
    const f32x16 s0 = qk(mask_tag, ka, 0, k0);
    __builtin_amdgcn_sched_barrier(0);
    read_k(kl, 1, ka);
    const f32x16 s1 = qk(mask_tag, ka, 1, k0);
    probs(s0, pf[0], pf[1]);
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = read_v(vb, 0, db);
    interleave(std::integral_constant<int, KS>{}, std::integral_constant<int, 24 / KS>{});
    __builtin_amdgcn_sched_barrier(0);
    auto pv_step = [&](const bf16x8 (&v)[DB], const bf16x8& pfrag) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[db], pfrag, o[db], 0, 0, 0);
      lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pfrag, lacc, 0, 0, 0);
    };
#pragma unroll
    for (int db = 0; db < DB; ++db) vn[db] = read_v(vb, 1, db);
    pv_step(va, pf[0]);
    probs(s1, pf[2], pf[3]);
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = read_v(vb, 2, db);
    pv_step(vn, pf[1]);
    interleave(std::integral_constant<int, 2 * (DB + 1)>{}, std::integral_constant<int, (24 + 2 * DB + 1) / (2 * (DB + 1))>{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) vn[db] = read_v(vb, 3, db);
    pv_step(va, pf[2]);
    pv_step(vn, pf[3]);
  };
  // ---- half tile: only key half mb, masked, for a tile whose other 32 keys
  // are hidden from every row (past every row's position, or before every
  // row's window).
  auto tile_half = [&](auto mb_tag, auto mask_tag, const lds_char* kl, const lds_char* vb, int k0) {
    constexpr int mb = decltype(mb_tag)::value;
    bf16x8 ka[KS], pf[4], va[2][DB];
    read_k(kl, mb, ka);
    const f32x16 sc = qk(mask_tag, ka, mb, k0);
    __builtin_amdgcn_sched_barrier(0);
    read_v2(vb, 2 * mb, va);
    probs(sc, pf[2 * mb], pf[2 * mb + 1]);
    __builtin_amdgcn_sched_barrier(0);
    pv2(va, pf, 2 * mb);
#pragma unroll
    for (int j = 0; j < 2; ++j) lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pf[2 * mb + j], lacc, 0, 0, 0);
  };
  // ---- exact tile (the redo): streaming softmax with running maxima and
  // fp32 row sums on the vector ALU.
  auto tile_exact = [&](const lds_char* kl, const lds_char* vb, int k0) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      bf16x8 ka[KS], pf[4];
      read_k(kl, mb, ka);
      const f32x16 sc = qk(std::integral_constant<int, kMaskCausal | (WINDOWED ? kMaskWindow : 0)>{}, ka, mb, k0);
      // the largest scaled score (c > 0, and rounding is monotonic)
      const float mx = pair_max(max16(sc)) * cv;
      if (mx > mref) {
        const float alpha = __builtin_amdgcn_exp2f(mref - mx);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        mref = mx;
      }
      const float m = (mref == -INFINITY) ? 0.f : mref;
      lsum += probs_sum(sc, m, pf[2 * mb], pf[2 * mb + 1]);
      bf16x8 va[2][DB];
      read_v2(vb, 2 * mb, va);
      pv2(va, pf, 2 * mb);
    }
  };

  // Walk the tiles from the last to the first; tiles [ktB, kt1] hold keys past
  // some row's position, tiles [kt0, ktA) keys that may have left some row's
  // window; only those take the mask, each run in a loop of its own.
  const int ktB = max(kt0, min(kt1 + 1, (qoff + p0 + 1) / kBK));
  const int xa = qoff + p0 + P - p.window;
  const int ktA = (WINDOWED && xa > 0) ? min(ktB, max(kt0, (xa + kBK - 1) / kBK)) : kt0;
  auto walk = [&](auto tile_fn, int kt_hi, int kt_lo) {
    for (int kt = kt_hi; kt >= kt_lo; --kt) {
      const int buf = (kt1 - kt) & 1;
      wait_vmem<0>();   // this wave's loads of tile kt have landed
      __syncthreads();  // every wave's have; the previous tile (or the query rows) fully read
      if (kt > kt0) issue_tile(kt - 1, buf ^ 1);
      tile_fn((const lds_char*)&lds_k[buf * kTileChunks], (const lds_char*)&lds_v[buf * kTileChunks], kt * kBK);
    }
  };
  using MNone = std::integral_constant<int, 0>;
  using MCausal = std::integral_constant<int, kMaskCausal>;
  using MWindow = std::integral_constant<int, WINDOWED ? kMaskWindow : 0>;
  using MBoth = std::integral_constant<int, kMaskCausal | (WINDOWED ? kMaskWindow : 0)>;
  using Lo = std::integral_constant<int, 0>;
  using Hi = std::integral_constant<int, 1>;
  auto fast_both = [&](const lds_char* kl, const lds_char* vb, int k0) { tile_fast(MBoth{}, kl, vb, k0); };
  auto fast_causal = [&](const lds_char* kl, const lds_char* vb, int k0) { tile_fast(MCausal{}, kl, vb, k0); };
  auto fast_window = [&](const lds_char* kl, const lds_char* vb, int k0) { tile_fast(MWindow{}, kl, vb, k0); };
  auto fast_open = [&](const lds_char* kl, const lds_char* vb, int k0) { tile_fast(MNone{}, kl, vb, k0); };
  auto half_lo_both = [&](const lds_char* kl, const lds_char* vb, int k0) { tile_half(Lo{}, MBoth{}, kl, vb, k0); };
  auto half_lo_causal = [&](const lds_char* kl, const lds_char* vb, int k0) { tile_half(Lo{}, MCausal{}, kl, vb, k0); };
  auto half_hi_both = [&](const lds_char* kl, const lds_char* vb, int k0) { tile_half(Hi{}, MBoth{}, kl, vb, k0); };
  auto half_hi_window = [&](const lds_char* kl, const lds_char* vb, int k0) { tile_half(Hi{}, MWindow{}, kl, vb, k0); };
  auto reset = [&](float m0) {
    mref = m0;
    lsum = 0.f;
    lacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  };

  reset(0.f);
  __builtin_amdgcn_s_setprio(0);
  // Tile kt1 (always masked) skips its upper 32 keys when they lie past every
  // row's position; with a window, tile kt0 (then always masked) skips its
  // lower 32 keys when they lie before every row's window (never both on one
  // tile: first <= last).
  const bool hi_half_hidden = (last & (kBK - 1)) < kBK / 2;
  const bool lo_half_hidden = WINDOWED && (first & (kBK - 1)) >= kBK / 2;
  const int top = hi_half_hidden ? kt1 - 1 : kt1;
  const int bot = lo_half_hidden ? kt0 + 1 : kt0;
  // Tiles [ktB, kt1] need the causal test, and the window test only if the
  // window reaches them (kt * kBK <= last - window); tiles below ktA hold no
  // key past any row's position and need the window test alone.
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
  float lrow;
  {
    const float e0 = __shfl(lacc[0], l32 & 15);
    const float e1 = __shfl(lacc[1], l32 & 15);
    lrow = (l32 < 16) ? e0 : e1;
  }
  // The fast pass is kept unless a row's sum left [2^-64, 2^65) or a sum or an
  // output is not finite; then the work-group redoes its rows exactly.
  {
    float osum = pairwise_sum32(o[0], o[1]);
    if constexpr (DB == 4) osum += pairwise_sum32(o[2], o[3]);
    const bool bad = !positive_in_binade_range(lrow, -kFastSumBinades, kFastSumBinades) || !finite_bits(osum);
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) redo_vote[w] = wave_bad ? 1 : 0;
    __syncthreads();
    if ((redo_vote[0] | redo_vote[1] | redo_vote[2] | redo_vote[3]) != 0) {
      reset(sink_t());
      issue_tile(kt1, 0);
      walk(tile_exact, kt1, kt0);
      lrow = pair_sum(lsum);
    }
  }

  // ---- epilogue: the sink's term, 1 / l, bf16, store.  The rows go out
  // through LDS so that each store instruction writes 4 whole 256-byte rows
  // instead of 16-byte pieces of 32 rows: each wave writes its 32 rows, in
  // the staging layout, into its own 8 KiB of the slot that does not hold
  // tile kt0 (every wave finished reading that slot before the barrier that
  // opened tile kt0, or, with a single tile, before the first barrier), and
  // reads them back 16 lanes per row.  Rows past the sequence end fall outside
  // the output descriptor's range and are dropped.  The lane index is
  // laundered so that no address term of the query loads, which share these
  // offsets, is kept live through the walk.
  int el = lane;
  asm volatile("" : "+v"(el));
  const int el32 = el & 31, ehi = el >> 5;
  const int free_slot = ((kt1 - kt0) & 1) ^ 1;
  lds_char* const ob = (w < 2 ? (lds_char*)lds_k : (lds_char*)lds_v) + free_slot * kTileBytes + (w & 1) * kQW * kRowBytes;
  float lt = lrow;
  if (p.sinks) lt += __builtin_amdgcn_exp2f(sink_t() - mref);
  const float inv = __builtin_amdgcn_rcpf(lt);  // v_rcp_f32: 1 ulp, far below the bf16 rounding
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
      // head_dim elements 32 db + 8 vg + 4 hi .. + 3: half hi of chunk 4 db + vg
      bf16x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = (__bf16)(o[db][4 * vg + e] * inv);
      *(u32x2*)(ob + tpos<D>(el32, 4 * db + vg) * 16 + 8 * ehi) = __builtin_bit_cast(u32x2, val);
    }
  {
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.out + (int64_t)s * Hq * kD), 0, L * Hq * kRowBytes, kBufferConfig);
#pragma unroll
    for (int i = 0; i < S::kQLoads; ++i) {
      const int row = RPL * i + el / kChunks;  // within the wave's 32 rows
      const int r = kQW * w + row;
      const int ch = el % kChunks;
      const u32x4 x = *(const u32x4*)(ob + tpos<D>(row, ch) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(x, ro, ((p0 + r / G) * Hq + g * G + r % G) * kRowBytes + ch * 16, 0, kStreamStore);
    }
  }
}

template <int D, int G>
hipError_t launch_g(const Params& kp, int64_t grid, bool windowed, bool paged, hipStream_t stream) {
  const dim3 gd((unsigned)grid), bd(kThreads);
  if constexpr (D == 128) {  // head_dim 64 takes the 256-row kernel's paged form
    if (paged) {
      if (windowed)
        hipLaunchKernelGGL((prefill_fwd_narrow<D, G, true, true>), gd, bd, 0, stream, kp);
      else
        hipLaunchKernelGGL((prefill_fwd_narrow<D, G, false, true>), gd, bd, 0, stream, kp);
      return hipGetLastError();
    }
  }
  if (paged) return hipErrorInvalidValue;
  if (windowed)
    hipLaunchKernelGGL((prefill_fwd_narrow<D, G, true, false>), gd, bd, 0, stream, kp);
  else
    hipLaunchKernelGGL((prefill_fwd_narrow<D, G, false, false>), gd, bd, 0, stream, kp);
  return hipGetLastError();
}
template <int D>
hipError_t launch_d(const Params& kp, int64_t grid, int G, bool windowed, bool paged, hipStream_t stream) {
  switch (G) {
    case 1: return launch_g<D, 1>(kp, grid, windowed, paged, stream);
    case 2: return launch_g<D, 2>(kp, grid, windowed, paged, stream);
    case 4: return launch_g<D, 4>(kp, grid, windowed, paged, stream);
    case 8: return launch_g<D, 8>(kp, grid, windowed, paged, stream);
    case 16: return launch_g<D, 16>(kp, grid, windowed, paged, stream);
    default: return hipErrorInvalidValue;
  }
}

int64_t pblocks128(const PrefillArgs& a) {
  const int P = kRows / (a.n_q_heads / a.n_kv_heads);
  return ((int64_t)a.max_seqlen + P - 1) / P;
}

}  // namespace

int64_t prefill_grid_size_narrow(const PrefillArgs& a, int head_dim) {
  if (a.block_table && head_dim != 128) return -1;  // the paged form is for head_dim 128
  const int64_t row_bytes = 2 * (int64_t)head_dim;
  // each sequence's K (or V) rows must be addressable by one buffer descriptor
  // (a cache is addressed page by page instead)
  if (!a.block_table && ((int64_t)a.max_seqlen + kBK) * a.n_kv_heads * row_bytes > 0x7fffffffLL) return -1;
  if (((int64_t)a.max_seqlen + kRows) * a.n_q_heads * row_bytes > 0x7fffffffLL) return -1;
  const int64_t n = pblocks128(a) * (int64_t)a.n_seqs * (int64_t)a.n_kv_heads;
  if (n > 0x7fffffffLL) return -1;
  return n;
}

hipError_t launch_prefill_narrow(const PrefillArgs& a, int head_dim, hipStream_t stream) {
  const int64_t grid = prefill_grid_size_narrow(a, head_dim);
  if (grid <= 0) return hipSuccess;
  Params kp;
  kp.q = static_cast<const uint16_t*>(a.q);
  kp.k = static_cast<const uint16_t*>(a.k);
  kp.v = static_cast<const uint16_t*>(a.v);
  kp.sinks = a.sinks;
  kp.cu = a.cu_seqlens;
  kp.out = static_cast<uint16_t*>(a.out);
  kp.n_kv_heads = a.n_kv_heads;
  kp.n_seqs = a.n_seqs;
  kp.n_pblocks = (int32_t)pblocks128(a);
  kp.max_seqlen = a.max_seqlen;
  kp.seq_group = prefill_seq_group(a, 2 * head_dim);
  kp.window = a.window > 0 ? a.window : 0;
  kp.c = (float)((double)a.softmax_scale * 1.4426950408889634);
  kp.seqlens_k = a.seqlens_k;
  kp.block_table = a.block_table;
  kp.page_elems = (int64_t)a.page_size * a.n_kv_heads * head_dim;
  kp.page_bytes = a.page_size * a.n_kv_heads * 2 * head_dim;
  kp.page_shift = a.page_size > 0 ? __builtin_ctz((unsigned)a.page_size) : 0;
  kp.pages_per_seq = a.pages_per_seq;
  kp.n_pages = a.n_pages;
  const bool windowed = a.window > 0;
  const bool paged = a.block_table != nullptr;
  (void)hipGetLastError();
  const int G = a.n_q_heads / a.n_kv_heads;
  return head_dim == 128 ? launch_d<128>(kp, grid, G, windowed, paged, stream)
                         : launch_d<64>(kp, grid, G, windowed, paged, stream);
}

}  // namespace tsmha
