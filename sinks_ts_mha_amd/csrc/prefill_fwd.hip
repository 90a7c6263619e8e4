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
// of its rows skip the mask.
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
// Softmax.  Online (streaming) softmax in base 2: t = s * scale * log2(e); the
// running maximum starts at the sink's logit (times log2 e) so the sink takes
// part in the maximum and the denominator, and the sink's own term
// exp2(sigma - m) is added to the denominator once, at the end.  A row whose
// keys are all masked in a tile uses 0 as its reference so no inf - inf occurs.
#include "prefill_fwd.h"

#include <math.h>

namespace tsmha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kD = 64;                 // head_dim
constexpr int kBK = 64;                // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 64 * kWaves;     // (query head, position) rows per work-group
constexpr int kChunksPerRow = kD * 2 / 16;   // 16-byte chunks in one K or V row
constexpr float kLog2e = 1.4426950408889634f;

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
};

// Swizzled position of 16-byte chunk `ch` of tile row `row`: XOR with the row's
// low three bits spreads the 8 chunks of 8 consecutive rows over all banks.
__device__ __forceinline__ int swz(int row, int ch) { return row * kChunksPerRow + (ch ^ (row & 7)); }

template <int G, bool WINDOWED>
__global__ void __launch_bounds__(kThreads, 2) prefill_fwd_d64(KParams p) {
  constexpr int P = kRows / G;  // positions per work-group
  __shared__ u32x4 lds_k[kBK * kChunksPerRow];
  __shared__ u32x4 lds_v[kBK * kChunksPerRow];

  const int Hkv = p.n_kv_heads;
  const int Hq = Hkv * G;
  const int id = blockIdx.x;
  // Consecutive work-group ids go to different XCDs; with the KV head as the
  // fastest index, each XCD's L2 sees the K/V of a fixed set of heads.
  const int g = id % Hkv;
  const int rest = id / Hkv;
  const int b = rest % p.n_seqs;
  // Position blocks are issued last-first: under a causal mask the late blocks
  // carry the most key tiles, so the longest work starts first.
  const int pblk = p.n_pblocks - 1 - rest / p.n_seqs;
  const int s = p.cu[b];
  const int L = p.cu[b + 1] - s;
  const int p0 = pblk * P;
  if (p0 >= L) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int last = min(L, p0 + P) - 1;
  const int first = WINDOWED ? max(0, p0 - p.window + 1) : 0;
  const int kt0 = first / kBK;
  const int kt1 = last / kBK;

  // ---- this lane's two query rows (one per 32-column block nb)
  int pos[2], head[2];
  bf16x8 qf[2][4];
  float m[2], lsum[2];
  f32x16 o[2][2];  // [d block][nb]: O^T, rows = head_dim, columns = queries
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = 64 * w + 32 * nb + l32;
    head[nb] = g * G + r % G;
    pos[nb] = p0 + r / G;
    if (pos[nb] < L) {
      const uint16_t* qrow = p.q + ((int64_t)(s + pos[nb]) * Hq + head[nb]) * kD + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[nb][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * ks));
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[nb][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
    m[nb] = p.sinks ? p.sinks[head[nb]] * kLog2e : -INFINITY;
    lsum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][nb][e] = 0.f;
  }

  // ---- K/V tile staging: each thread moves 2 chunks of K and 2 of V
  u32x4 kreg[2], vreg[2];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + kThreads * it;
      const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
      const int j = kt * kBK + row;
      if (j < L) {
        const int64_t off = ((int64_t)(s + j) * Hkv + g) * kD + ch * 8;
        kreg[it] = *(const u32x4*)(p.k + off);
        vreg[it] = *(const u32x4*)(p.v + off);
      } else {  // past the sequence end: zeros keep the masked products finite
        kreg[it] = u32x4{0, 0, 0, 0};
        vreg[it] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + kThreads * it;
      const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
      lds_k[swz(row, ch)] = kreg[it];
      lds_v[swz(row, ch)] = vreg[it];
    }
  };

  const int r16 = lane & 15;
  const int half16 = (lane >> 4) & 1;
  lds_char* vbase = (lds_char*)(lds_v);

  load_tile(kt0);
  for (int kt = kt0; kt <= kt1; ++kt) {
    __syncthreads();  // all waves are done reading the previous tile
    store_tile();
    __syncthreads();
    if (kt < kt1) load_tile(kt + 1);  // in flight while this tile is consumed

    // ---- S^T = K Q^T for 64 keys x this wave's 64 queries
    f32x16 sacc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[mb][nb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int key = 32 * mb + l32;
        const bf16x8 a = __builtin_bit_cast(bf16x8, lds_k[swz(key, 2 * ks + hi)]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          sacc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[nb][ks], sacc[mb][nb], 0, 0, 0);
      }
    }

    // ---- mask (only tiles not fully visible to every row of the work-group)
    const int k0 = kt * kBK;
    const bool need_mask = (k0 + kBK - 1 > p0) || (WINDOWED && (p0 + P - 1) - k0 >= p.window);
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = k0 + 32 * mb + 8 * (e / 4) + 4 * hi + (e % 4);
            const int i = pos[nb];
            const bool vis = (j <= i) && (!WINDOWED || i - j < p.window);
            if (!vis) sacc[mb][nb][e] = -INFINITY;
          }
    }

    // ---- online softmax; P^T converted to bf16 in the PV B-operand order
    bf16x8 pf[4][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[mb][nb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[nb], mx * p.c);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m[nb] - muse);
      float rs = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[mb][nb][e], p.c, -muse));
          sacc[mb][nb][e] = pe;
          rs += pe;
        }
      lsum[nb] = lsum[nb] * alpha + rs;
      m[nb] = mnew;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][nb][e] *= alpha;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[2 * mb + h2][nb][e] = (__bf16)sacc[mb][nb][8 * h2 + e];
    }

    // ---- O^T += V^T P^T; lane l of step s4 needs keys 16 s4 + 8 (e / 4) + 4 hi + e % 4
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int key_lo = 16 * s4 + 4 * hi + (r16 >> 2);
      const int key_hi = key_lo + 8;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int d = 32 * db + 16 * half16 + 4 * (r16 & 3);
        const int off_lo = key_lo * (kD * 2) + (((d >> 3) ^ (key_lo & 7)) << 4) + (d & 7) * 2;
        const int off_hi = key_hi * (kD * 2) + (((d >> 3) ^ (key_hi & 7)) << 4) + (d & 7) * 2;
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + off_lo));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + off_hi));
        const u32x2 u0 = __builtin_bit_cast(u32x2, t0);
        const u32x2 u1 = __builtin_bit_cast(u32x2, t1);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{u0[0], u0[1], u1[0], u1[1]});
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s4][nb], o[db][nb], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: combine the two half-sums, add the sink's term, normalise, store
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float lt = lsum[nb] + __shfl_xor(lsum[nb], 32);
    if (p.sinks) lt += __builtin_amdgcn_exp2f(p.sinks[head[nb]] * kLog2e - m[nb]);
    const float inv = 1.f / lt;
    if (pos[nb] < L) {
      uint16_t* orow = p.out + ((int64_t)(s + pos[nb]) * Hq + head[nb]) * kD;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int d = 32 * db + 8 * vg + 4 * hi;
          bf16x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = (__bf16)(o[db][nb][4 * vg + e] * inv);
          *(bf16x4*)(orow + d) = val;
        }
    }
  }
}

template <int G>
hipError_t launch_group(const KParams& kp, int64_t grid, bool windowed, hipStream_t stream) {
  if (windowed)
    hipLaunchKernelGGL((prefill_fwd_d64<G, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, kp);
  else
    hipLaunchKernelGGL((prefill_fwd_d64<G, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, kp);
  return hipGetLastError();
}

int64_t pblocks(const PrefillArgs& a) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const int P = kRows / G;
  return ((int64_t)a.max_seqlen + P - 1) / P;
}

}  // namespace

int64_t prefill_grid_size(const PrefillArgs& a) {
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
  const bool windowed = a.window > 0;
  (void)hipGetLastError();  // start from a clean per-thread error state
  switch (a.n_q_heads / a.n_kv_heads) {
    case 1: return launch_group<1>(kp, grid, windowed, stream);
    case 2: return launch_group<2>(kp, grid, windowed, stream);
    case 4: return launch_group<4>(kp, grid, windowed, stream);
    case 8: return launch_group<8>(kp, grid, windowed, stream);
    case 16: return launch_group<16>(kp, grid, windowed, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tsmha
