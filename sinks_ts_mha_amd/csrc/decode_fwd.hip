// decode_fwd.hip -- gfx950 kernels of decode attention against a paged KV
// cache: one new query row per sequence (all query heads) attends to the
// sequence's cached keys, with the GPT-OSS attention of "TokenSpeed-kernel
// multi-silicon" (aixai.ru blog), section "Числа: Gluon на AMD MI355X":
// grouped query heads, an optional sliding window and an optional per-head
// sink.  This is the `mha_decode_with_kvcache` call of the TokenSpeed-kernel
// README, section "Public API"; the pages give it no signature, and the
// readings taken are stated in include/ts_mha.h.
//
// Decode reads every cached key and value once and does 2 x 64 flops per key
// and query head, so it is bound by HBM bandwidth, not by the matrix cores.
// The design is about keeping enough bytes in flight:
//
// Work decomposition.  One work-group per (sequence, group of HW adjacent KV
// heads, key chunk), HW in {1, 2, 4}; the host picks the chunk length (a
// multiple of 128 keys, at most 8192) so that the grid fills every CU once (a
// work-group takes most of a CU's LDS), and does not split a sequence when
// there are enough (sequence, head group) pairs.  Wave w serves KV head
// w % HW of the group and takes every (4 / HW)-th 32-key tile of the chunk;
// each wave streams its tiles through a private ring of LDS stages with
// wave-wide buffer-to-LDS loads, several tiles ahead, so the walk needs no
// barrier.  A cached key's row holds all KV heads side by side, so with HW
// heads per work-group the waves of one CU read HW * 2 * head_dim contiguous
// bytes of each row at about the same time instead of one head's 2 * head_dim
// bytes at a stride of the whole row: at head_dim 64 and 8 KV heads, 128-byte
// pieces 1 KiB apart reach about 10% less of the HBM bandwidth than 512-byte
// ones.  Every cached row is read once per call, so the loads carry the
// non-temporal hint.
//
// Paging.  A 32-key tile is loaded as four groups of 8 keys; with pages of at
// least 16 keys a group never straddles a page, so each load takes one page
// id (from a copy of the chunk's block-table slice in LDS) and addresses that
// page through its own buffer descriptor.  Keys at or past the sequence end
// fall outside the descriptor's range and read as zeros, so cache slots that
// were never written cannot leak into the result.
//
// Arithmetic.  The G query heads of the KV head are the 16 columns of
// 16 x 16 x 32 bf16 MFMAs (G <= 16; the other columns are zero): S^T = K Q^T
// per 16 keys, then O^T += V^T P^T per 32 keys with V^T read by
// ds_read_b64_tr_b16.  Each lane holds one query (lane % 16), so the running
// maximum, the rescale of O and the probabilities need no lane exchange
// except the tile maximum over the four lane groups.  Softmax in base 2:
// t = s * scale * log2(e).
//
// Merge.  The waves of each KV head combine their (m, l, O) through LDS.  With one chunk
// per sequence the work-group adds the sink's term exp2(sigma - m), normalises
// and stores bf16; otherwise it stores the chunk's (m, l, O) in fp32 and
// decode_merge combines the chunks of each sequence and adds the sink.
#include "decode_fwd.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "cdna4.h"

namespace tsmha {

namespace {

using namespace cdna4;

constexpr int kTileKeys = 32;                     // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunkMax = 8192;                   // keys per work-group at most
constexpr int kMinPage = 16;
constexpr int kPageSlots = kChunkMax / kMinPage + 2;
constexpr int kTargetGroups = 256;                // one work-group per CU
constexpr int kMaxGroupRowBytes = 512;            // a work-group's bytes of one cached row
constexpr int kLongSpanTiles = 64;

// Sizes that follow from head_dim D (64 or 128).
template <int D>
struct DShape {
  static constexpr int kRowBytes = 2 * D;                       // one K or V row
  static constexpr int kChunks = kRowBytes / 16;                // 16-byte chunks per row
  static constexpr int kTileBytes = kTileKeys * kRowBytes;      // one tile of K (or V)
  static constexpr int kLoads = kTileBytes / 1024;              // wave-wide loads per tile and operand
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;
  // LDS tiles per wave (kStages - 1 in flight): four at head_dim 64, two at 128,
  // where four would not fit the LDS (4 waves x 2 x 8 KiB per stage)
  static constexpr int kStages = D == 64 ? 4 : 2;
  static constexpr int kKS = D / 32;                            // 32-wide steps of head_dim (scores)
  static constexpr int kDB = D / 16;                            // 16-row blocks of O^T
};

// XOR key of row r in a tile: 128-byte rows use cdna4.h's key over 8 chunks;
// 256-byte rows c ^ ((r & 3) << 2 | (r >> 2) & 3) over 16 chunks.  Either way
// 16 consecutive rows reading one chunk (the K operand) and 4 aligned rows
// reading two adjacent chunks (the V^T operand) hit distinct bank groups.
template <int D>
__device__ __forceinline__ int dkey(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3); else return swz_key(row);
}
template <int D>
__device__ __forceinline__ int dpos(int row, int ch) { return row * DShape<D>::kChunks + (ch ^ dkey<D>(row)); }

struct DParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const float* sinks;
  const int32_t* seqlens_k;
  const int32_t* block_table;
  uint16_t* out;
  float* ws_ml;          // [n_splits][n_seqs][Hq][2]: (m, l) of each chunk
  float* ws_o;           // [n_splits][n_seqs][Hq][D]: unnormalised O of each chunk
  int64_t page_elems;    // bf16 elements per page: page_size * n_kv_heads * D
  int32_t page_bytes;
  int32_t n_kv_heads;
  int32_t n_seqs;
  int32_t n_pages;
  int32_t page_shift;
  int32_t pages_per_seq;
  int32_t window;
  int32_t chunk;
  int32_t n_splits;
  float c;               // softmax_scale * log2(e)
};

// First key of a sequence's first chunk: the first visible key (window), rounded
// down to a tile boundary.
__device__ __forceinline__ int first_tile_key(int L, int window) {
  const int lo = window > 0 ? max(0, L - window) : 0;
  return lo & ~(kTileKeys - 1);
}

__device__ __forceinline__ float lane_group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float lane_group_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

}  // namespace

template <int D, int G, int HW>
__global__ void __launch_bounds__(kThreads, 1) decode_split(DParams p) {
  static_assert(G >= 1 && G <= 16, "the query heads of a KV head fill at most 16 MFMA columns");
  static_assert(HW == 1 || HW == 2 || HW == 4, "KV heads per work-group");
  constexpr int kWavesPerHead = kWaves / HW;  // waves that share one KV head's tiles
  using S = DShape<D>;
  constexpr int kD = D;
  constexpr int kRowBytes = S::kRowBytes;
  constexpr int kTileBytes = S::kTileBytes;
  constexpr int kLoads = S::kLoads;
  constexpr int kStages = S::kStages;
  constexpr int kWaveRing = kStages * 2 * kTileBytes;  // one wave's part of the ring
  static_assert(G * D * 4 <= kWaveRing, "a wave's O fits its own part of the ring");
  __shared__ u32x4 ring[kWaves * kWaveRing / 16];       // [wave][stage][K, V][tile]
  __shared__ float ml[kWaves][G][2];                    // each wave's (m, l)
  __shared__ int pages[kPageSlots];                     // the chunk's page ids

  const int Hkv = p.n_kv_heads;
  const int Hq = Hkv * G;
  const int id = blockIdx.x;
  const int n_hg = Hkv / HW;
  const int g0 = (id % n_hg) * HW;  // the work-group's first KV head
  const int rest = id / n_hg;
  const int b = rest % p.n_seqs;
  const int split = rest / p.n_seqs;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = g0 + w % HW;        // this wave's KV head
  const int wr = w / HW;            // its rank among the waves of that head
  const int r16 = lane & 15;  // this lane's query (head g * G + r16 when r16 < G)
  const int grp = lane >> 4;

  const int L = p.seqlens_k[b];
  const int lo = p.window > 0 ? max(0, L - p.window) : 0;
  const int start = first_tile_key(L, p.window) + split * p.chunk;
  const int end = min(L, start + p.chunk);
  if (start >= end) {
    // No key in this chunk.  With one chunk per sequence the rows are written
    // here (a sequence without keys has zero output); otherwise decode_merge
    // skips the chunk.
    if (p.n_splits == 1)
      for (int i = tid; i < HW * G * kD / 8; i += kThreads)
        *(u32x4*)(p.out + ((int64_t)b * Hq + g0 * G) * kD + i * 8) = u32x4{0u, 0u, 0u, 0u};
    return;
  }

  // ---- the chunk's page ids into LDS (clamped into the table and the pool, so
  // a malformed table cannot move a load outside the cache), and this lane's
  // query fragments: lane l holds head_dim elements 32 ks + 8 grp .. + 7 of
  // query r16 (ks < D / 32), the B operand of S^T = K Q^T.
  const int pidx0 = start >> p.page_shift;
  const int npg = min(((end - 1) >> p.page_shift) - pidx0 + 1, kPageSlots);
  {
    const int32_t* brow = p.block_table + (int64_t)b * p.pages_per_seq;
    for (int i = tid; i < npg; i += kThreads) {
      const int pg = brow[min(pidx0 + i, p.pages_per_seq - 1)];
      pages[i] = min(max(pg, 0), p.n_pages - 1);
    }
  }
  bf16x8 qf[S::kKS];
  if (r16 < G) {
    const uint16_t* qrow = p.q + ((int64_t)b * Hq + g * G + r16) * kD;
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks) qf[ks] = *(const bf16x8*)(qrow + 32 * ks + 8 * grp);
  } else {
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
  __syncthreads();  // page ids visible to every wave
  // The query loads complete here, before the tile loads below go out, so the
  // compiler's own waits never count those.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- tile loads.  The wave's i-th tile is the work-group's tile w + 4 i and
  // goes to stage i % kStages.  Load `it` brings the R = 1024 / (2 D) keys
  // R it .. R it + R - 1 of the tile: lane l fetches 16 bytes of key
  // R it + l / (D / 8), placed at its swizzled chunk.  Loads past the wave's
  // last tile still go out, with every lane out of range, so the number in
  // flight is the same on every iteration.
  const int nt = (end - start + kTileKeys - 1) / kTileKeys;
  const int my_tiles = nt > wr ? (nt - wr + kWavesPerHead - 1) / kWavesPerHead : 0;
  const int pmask = (1 << p.page_shift) - 1;
  int dch[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int row = S::kRowsPerLoad * it + lane / S::kChunks;
    dch[it] = ((lane % S::kChunks) ^ dkey<D>(row)) * 16 + g * kRowBytes;
  }
  const uint32_t ring_w = lds_addr(ring) + w * kWaveRing;
  auto issue = [&](int i) {
    const int t = wr + kWavesPerHead * i;
    const bool live = i < my_tiles;
    const int tile_key = start + kTileKeys * t;
    const uint32_t dk = ring_w + (i % kStages) * 2 * kTileBytes;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int key0 = tile_key + 16 * half;
      const int slot = min(max((key0 >> p.page_shift) - pidx0, 0), npg - 1);
      const int pg = live ? __builtin_amdgcn_readfirstlane(pages[slot]) : 0;
      const int64_t off = (int64_t)pg * p.page_elems;
      const i32x4 rk = buffer_rsrc(p.kc + off, p.page_bytes);
      const i32x4 rv = buffer_rsrc(p.vc + off, p.page_bytes);
#pragma unroll
      for (int j = 0; j < kLoads / 2; ++j) {
        const int it = (kLoads / 2) * half + j;
        const int key = tile_key + S::kRowsPerLoad * it + lane / S::kChunks;
        const int vo = (live && key < end) ? (key & pmask) * Hkv * kRowBytes + dch[it] : p.page_bytes;
        lds_dma16_nt(dk + it * 1024, rk, vo);
        lds_dma16_nt(dk + kTileBytes + it * 1024, rv, vo);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i) issue(i);

  // Per-lane byte offsets of the V^T reads within a tile: the lanes of group
  // grp read keys 4 grp + r16 / 4 (low half) and 16 more (high half), head_dim
  // columns 16 db + 4 (r16 % 4) .. + 3; the transpose hands lane r16 column
  // 16 db + r16 of those four keys.  Rows 16 apart share their swizzle key.
  uint32_t voff[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) {
    const int row = 4 * grp + (r16 >> 2);
    const int d = 16 * db + 4 * (r16 & 3);
    voff[db] = row * kRowBytes + (((d >> 3) ^ dkey<D>(row)) << 4) + (d & 7) * 2;
  }

  float m = -INFINITY;  // running maximum of t for query r16 (identical across lane groups)
  float lsum = 0.f;     // this lane's share of the row sum
  f32x4 o[S::kDB];      // O^T: element e of block db is head_dim 16 db + 4 grp + e, query r16
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < my_tiles; ++i) {
    issue(i + kStages - 1);
    wait_vmem<(kStages - 1) * 2 * kLoads>();  // tile i has landed
    const lds_char* kt = (const lds_char*)ring + w * kWaveRing + (i % kStages) * 2 * kTileBytes;
    const lds_char* vt = kt + kTileBytes;
    const int tile_key = start + kTileKeys * (wr + kWavesPerHead * i);
    const bool edge = tile_key < lo || tile_key + kTileKeys > L;

    // S^T for keys 16 kb .. 16 kb + 15: element e is key 16 kb + 4 grp + e.
    // Keys outside [lo, L) start from -inf, so the MFMA applies the mask.
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (edge) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = tile_key + 16 * kb + 4 * grp + e;
          acc[e] = (key >= lo && key < L) ? 0.f : -INFINITY;
        }
      }
#pragma unroll
      for (int ks = 0; ks < S::kKS; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(kt + dpos<D>(16 * kb + r16, 4 * ks + grp) * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], acc, 0, 0, 0);
      }
      s[kb] = acc;
    }

    // Streaming softmax of query r16 over the tile's 32 keys.
    float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    const float mn = fmaxf(m, lane_group_max(mt) * p.c);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m - mu);
    m = mn;
    bf16x8 pf;  // P^T, the B operand of the PV MFMA: keys 4 grp + e, then 16 + 4 grp + e
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(s[kb][e], p.c, -mu));
        pf[4 * kb + e] = (__bf16)pe;
        ps += pe;
      }
    lsum = fmaf(lsum, alpha, ps);

    // O^T = alpha O^T + V^T P^T, the A operand's keys in P^T's order.
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) {
      const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + voff[db]));
      const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + voff[db] + 16 * kRowBytes));
      const u32x2 u0 = __builtin_bit_cast(u32x2, t0);
      const u32x2 u1 = __builtin_bit_cast(u32x2, t1);
      const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{u0[0], u0[1], u1[0], u1[1]});
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[db] * alpha, 0, 0, 0);
    }
  }
  // The loads past the last tile land before the wave may leave its LDS.
  wait_vmem<0>();

  // ---- combine the waves of each KV head.  Each wave's O goes into its own part of the
  // ring, which nothing reads or loads into any more: the wave's own reads of
  // it are done and its loads have landed.
  auto mo = [&](int v, int q, int d) -> float& {
    return reinterpret_cast<float*>(reinterpret_cast<char*>(ring) + v * kWaveRing)[q * kD + d];
  };
  lsum = lane_group_sum(lsum);
  if (r16 < G) {
#pragma unroll
    for (int db = 0; db < S::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) mo(w, r16, 16 * db + 4 * grp + e) = o[db][e];
    if (grp == 0) {
      ml[w][r16][0] = m;
      ml[w][r16][1] = lsum;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < HW * G * kD / 4; idx += kThreads) {
    const int hl = idx / (kD / 4);  // query head g0 * G + hl: KV head slot hl / G, query hl % G
    const int q = hl % G;
    const int w0 = hl / G;          // the waves of that KV head: w0, w0 + HW, ...
    const int d0 = 4 * (idx % (kD / 4));
    const int h = g0 * G + hl;
    float M = -INFINITY;
#pragma unroll
    for (int v = w0; v < kWaves; v += HW) M = fmaxf(M, ml[v][q][0]);
    float lt = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = w0; v < kWaves; v += HW) {
      const float f = __builtin_amdgcn_exp2f(ml[v][q][0] - M);  // 0 for a wave without tiles
      lt = fmaf(f, ml[v][q][1], lt);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(f, mo(v, q, d0 + e), acc[e]);
    }
    if (p.n_splits == 1) {
      const float st = p.sinks ? p.sinks[h] * kLog2e : -INFINITY;
      float den = lt;
      float scale = 1.f;
      if (p.sinks) {
        const float M2 = fmaxf(M, st);
        scale = __builtin_amdgcn_exp2f(M - M2);
        den = fmaf(lt, scale, __builtin_amdgcn_exp2f(st - M2));
      }
      const float inv = scale / den;
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (__bf16)(acc[e] * inv);
      *(bf16x4*)(p.out + ((int64_t)b * Hq + h) * kD + d0) = r;
    } else {
      const int64_t row = ((int64_t)split * p.n_seqs + b) * Hq + h;
      *(f32x4*)(p.ws_o + row * kD + d0) = acc;
      if (d0 == 0) {
        p.ws_ml[2 * row] = M;
        p.ws_ml[2 * row + 1] = lt;
      }
    }
  }
}

// Combine the chunks of each (sequence, query head).  S x D / 4 threads per
// (sequence, query head), S a power of two that the host picks from the number
// of chunks (so that few chunks do not leave most threads idle, and many are
// folded by many lanes): thread (sl, dc) folds chunks sl, sl + S, ... of
// head_dim elements 4 dc .. 4 dc + 3 into a running (m, l, O), the S chunk
// lanes (adjacent lanes of one wave) then combine by a butterfly, and the
// sink's term joins the denominator.  A work-group takes 256 threads' worth of
// rows, or one row when a row needs more.
template <int D, int S>
struct MergeShape {
  static_assert(S >= 2 && S <= 16 && (S & (S - 1)) == 0, "chunk lanes");
  static constexpr int kRowThreads = S * D / 4;
  static_assert(kRowThreads <= 1024, "one row per work-group at most");
  static constexpr int kRows = kRowThreads >= 256 ? 1 : 256 / kRowThreads;  // rows per work-group
  static constexpr int kThreads = kRows * kRowThreads;
};

__device__ __forceinline__ void fold(float& m, float& l, f32x4& o, float m2, float l2, const f32x4& o2) {
  const float mn = fmaxf(m, m2);
  const float mu = (mn == -INFINITY) ? 0.f : mn;
  const float a = __builtin_amdgcn_exp2f(m - mu);
  const float b = __builtin_amdgcn_exp2f(m2 - mu);
  l = fmaf(l, a, l2 * b);
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = fmaf(o[e], a, o2[e] * b);
  m = mn;
}

template <int D, int S>
__global__ void __launch_bounds__((MergeShape<D, S>::kThreads)) decode_merge(DParams p, int G) {
  using M = MergeShape<D, S>;
  constexpr int kD = D;
  const int Hq = p.n_kv_heads * G;
  const int bh = (int)blockIdx.x * M::kRows + (int)threadIdx.x / M::kRowThreads;  // b * Hq + h
  if ((int64_t)bh >= (int64_t)p.n_seqs * Hq) return;  // every thread of a row returns together
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int tid = (int)threadIdx.x % M::kRowThreads;
  const int sl = tid & (S - 1);
  const int dc = tid / S;
  const int L = p.seqlens_k[b];
  const int n_valid = L > 0 ? min(p.n_splits, (L - first_tile_key(L, p.window) + p.chunk - 1) / p.chunk) : 0;
  float m = -INFINITY, l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = sl; s < n_valid; s += S) {
    const int64_t row = ((int64_t)s * p.n_seqs + b) * Hq + h;
    fold(m, l, o, p.ws_ml[2 * row], p.ws_ml[2 * row + 1], *(const f32x4*)(p.ws_o + row * kD + 4 * dc));
  }
#pragma unroll
  for (int x = 1; x < S; x <<= 1) {
    f32x4 o2;
#pragma unroll
    for (int e = 0; e < 4; ++e) o2[e] = __shfl_xor(o[e], x);
    fold(m, l, o, __shfl_xor(m, x), __shfl_xor(l, x), o2);
  }
  if (sl != 0) return;
  // the sink's term, then normalise; no key and no sink leaves a zero row
  const float st = p.sinks ? p.sinks[h] * kLog2e : -INFINITY;
  fold(m, l, o, st, 1.f, f32x4{0.f, 0.f, 0.f, 0.f});
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  bf16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (__bf16)(o[e] * inv);
  *(bf16x4*)(p.out + ((int64_t)b * Hq + h) * kD + 4 * dc) = r;
}

namespace {

template <int D, int G>
hipError_t launch_group(const DParams& kp, int64_t grid, int hw, hipStream_t stream) {
  switch (hw) {
    case 1: hipLaunchKernelGGL((decode_split<D, G, 1>), dim3((unsigned)grid), dim3(kThreads), 0, stream, kp); break;
    case 2: hipLaunchKernelGGL((decode_split<D, G, 2>), dim3((unsigned)grid), dim3(kThreads), 0, stream, kp); break;
    case 4: hipLaunchKernelGGL((decode_split<D, G, 4>), dim3((unsigned)grid), dim3(kThreads), 0, stream, kp); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || kp.n_splits == 1) return err;
  const int64_t rows = (int64_t)kp.n_seqs * kp.n_kv_heads * G;
  auto merge = [&](auto lanes) {
    using M = MergeShape<D, decltype(lanes)::value>;
    hipLaunchKernelGGL((decode_merge<D, decltype(lanes)::value>), dim3((unsigned)((rows + M::kRows - 1) / M::kRows)),
                       dim3(M::kThreads), 0, stream, kp, G);
  };
  // chunk lanes: the chunks' count rounded up to a power of two, at most 16
  // (more lanes lengthen the butterfly by more than they shorten the folds:
  // 128 chunks of one sequence merge 5% slower with 64 lanes than with 16)
  const int n = kp.n_splits;
  if (n <= 2) merge(std::integral_constant<int, 2>{});
  else if (n <= 4) merge(std::integral_constant<int, 4>{});
  else if (n <= 8) merge(std::integral_constant<int, 8>{});
  else merge(std::integral_constant<int, 16>{});
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DParams& kp, int64_t grid, int G, int hw, hipStream_t stream) {
  switch (G) {
    case 1: return launch_group<D, 1>(kp, grid, hw, stream);
    case 2: return launch_group<D, 2>(kp, grid, hw, stream);
    case 4: return launch_group<D, 4>(kp, grid, hw, stream);
    case 8: return launch_group<D, 8>(kp, grid, hw, stream);
    case 16: return launch_group<D, 16>(kp, grid, hw, stream);
    default: return hipErrorInvalidValue;
  }
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

DecodePlan decode_plan(const DecodeArgs& a) {
  DecodePlan pl{0, -1, 0, 1};
  int64_t span = a.max_seqlen_k;
  if (a.window > 0) span = std::min<int64_t>(span, (int64_t)a.window + kTileKeys - 1);
  const int64_t tiles = std::max<int64_t>(1, (span + kTileKeys - 1) / kTileKeys);
  // KV heads per work-group: the most (up to 512 contiguous bytes of a cached
  // row) that still fill the grid without splitting the sequences, or, for
  // spans of at least kLongSpanTiles tiles, whose split costs little against
  // the walk, the most regardless.  (64 sequences of 8192 keys at head_dim 64
  // and 8 KV heads: 4 heads and two chunks per sequence beat 2 heads and no
  // split by 2%; with a 128-key window, 4 heads whose 5 tiles split in two
  // ran 2.4 times slower than 2 heads.)
  int hw = 1;
  for (int c = 4; c >= 2; c >>= 1) {
    if (a.n_kv_heads % c != 0 || c * 2 * a.head_dim > kMaxGroupRowBytes) continue;
    if ((int64_t)a.n_seqs * (a.n_kv_heads / c) >= kTargetGroups || tiles >= kLongSpanTiles) {
      hw = c;
      break;
    }
  }
  pl.heads_per_group = hw;
  const int64_t base = std::max<int64_t>(1, (int64_t)a.n_seqs * (a.n_kv_heads / hw));
  const int64_t want = std::max<int64_t>(1, (kTargetGroups + base - 1) / base);
  int64_t ct = (tiles + want - 1) / want;
  ct = std::min<int64_t>(std::max<int64_t>(4, (ct + 3) / 4 * 4), kChunkMax / kTileKeys);
  const int64_t n_splits = (tiles + ct - 1) / ct;
  if (n_splits * base > 0x7fffffffLL) return pl;
  pl.chunk = (int32_t)(ct * kTileKeys);
  pl.n_splits = (int32_t)n_splits;
  if (n_splits > 1) {
    const int64_t rows = n_splits * a.n_seqs * (int64_t)a.n_q_heads;
    pl.workspace_bytes = align_up(rows * 2 * 4, 256) + rows * (int64_t)a.head_dim * 4;
  }
  return pl;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, void* workspace,
                         hipStream_t stream) {
  const int G = a.n_q_heads / a.n_kv_heads;
  DParams kp;
  kp.q = static_cast<const uint16_t*>(a.q);
  kp.kc = static_cast<const uint16_t*>(a.k_cache);
  kp.vc = static_cast<const uint16_t*>(a.v_cache);
  kp.sinks = a.sinks;
  kp.seqlens_k = a.seqlens_k;
  kp.block_table = a.block_table;
  kp.out = static_cast<uint16_t*>(a.out);
  const int64_t rows = (int64_t)plan.n_splits * a.n_seqs * a.n_q_heads;
  kp.ws_ml = plan.n_splits > 1 ? static_cast<float*>(workspace) : nullptr;
  kp.ws_o = plan.n_splits > 1
                ? reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(rows * 2 * 4, 256))
                : nullptr;
  kp.page_elems = (int64_t)a.page_size * a.n_kv_heads * a.head_dim;
  kp.page_bytes = a.page_size * a.n_kv_heads * 2 * a.head_dim;
  kp.n_kv_heads = a.n_kv_heads;
  kp.n_seqs = a.n_seqs;
  kp.n_pages = a.n_pages;
  kp.page_shift = __builtin_ctz((unsigned)a.page_size);
  kp.pages_per_seq = a.pages_per_seq;
  kp.window = a.window;
  kp.chunk = plan.chunk;
  kp.n_splits = plan.n_splits;
  kp.c = a.softmax_scale * kLog2e;
  const int hw = plan.heads_per_group;
  const int64_t grid = (int64_t)a.n_seqs * (a.n_kv_heads / hw) * plan.n_splits;
  if (a.head_dim == 128) return launch_d<128>(kp, grid, G, hw, stream);
  if (a.head_dim == 64) return launch_d<64>(kp, grid, G, hw, stream);
  return hipErrorInvalidValue;
}

}  // namespace tsmha
