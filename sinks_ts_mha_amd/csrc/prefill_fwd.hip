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
// Staging.  K and V tiles move from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (no register round trip), double-buffered: the
// loads of tile t+1 are in flight while tile t is consumed, and one barrier per
// tile separates the two.  The buffer descriptor of each work-group spans only
// its own sequence, so rows past the sequence end read as zeros.  Each lane
// picks its source chunk so that the fixed lane-to-LDS order of these loads
// lands in the XOR-swizzled layout the readers expect.  The XOR pattern is laid
// out for an LDS that serves 256 bytes (64 banks) per cycle.
//
// Softmax.  Online (streaming) softmax in base 2: t = s * scale * log2(e).  The
// reference maximum of each row starts at the sink's logit (times log2 e), so
// the sink takes part in the maximum, and the sink's own term exp2(sigma - m)
// is added to the denominator once, at the end.  The reference is raised only
// when a tile's row maximum exceeds it by more than 8 (a factor 256), so the
// rescaling of the accumulators is rare; probabilities stay below 2^8 and fp32
// sums cannot overflow.  Row sums are plain fp32 adds of the probabilities in
// four independent chains (the packed bf16 dot instruction would halve their
// count, but on gfx950 it shares the matrix pipeline and waits behind MFMAs of
// the other wave on the SIMD).  A row with no visible key so far uses 0 as its
// reference, so no inf - inf occurs.
#include "prefill_fwd.h"

#include <math.h>

namespace tsmha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 64;                        // head_dim
constexpr int kBK = 64;                       // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 64 * kWaves;            // (query head, position) rows per work-group
constexpr int kRowBytes = kD * 2;             // one K or V row in bytes
constexpr int kChunks = kRowBytes / 16;       // 16-byte chunks per row
constexpr int kTileChunks = kBK * kChunks;    // 16-byte chunks per tile
constexpr int kTileBytes = kTileChunks * 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;          // log2 units the reference max may lag by
constexpr int kBufferConfig = 0x00020000;     // raw buffer descriptor word 3 (32-bit data)
constexpr int kSlots = 2;                     // LDS buffers for K and for V tiles


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

namespace {

// Position of 16-byte chunk `ch` of tile row `row` in LDS.  The LDS serves 256
// bytes (64 banks of 4 bytes) per cycle, i.e. two 128-byte tile rows, so rows of
// equal parity collide unless their chunks differ.  The XOR key uses row bits 1
// (as chunk bit 2) and 2..3 (as chunk bits 0..1): 16 consecutive rows reading
// one logical chunk (the K operand reads) and 4 consecutive rows reading 4
// adjacent chunks (the V transpose reads) both hit 16 distinct bank groups.
__device__ __forceinline__ int swz_key(int row) { return ((row & 2) << 1) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz(int row, int ch) { return row * kChunks + (ch ^ swz_key(row)); }

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

// Maximum of 32 values: two independent chains of 3-input maxima (v_max3_f32).
__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
  float x = fmaxf(fmaxf(a[0], a[1]), a[2]);
  float y = fmaxf(fmaxf(b[0], b[1]), b[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) {
    x = fmaxf(fmaxf(x, a[i]), a[i + 1]);
    y = fmaxf(fmaxf(y, b[i]), b[i + 1]);
  }
  return fmaxf(fmaxf(x, a[15]), fmaxf(y, b[15]));
}

// Raw buffer descriptor (base, stride 0, byte range n) in scalar registers.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int n) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(n);
  r[3] = kBufferConfig;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const u32x4* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)p);
}

// One wave-wide 16-byte-per-lane load from a buffer straight into LDS: lane i's
// 16 bytes land at lds + 16 i (lds must be wave-uniform).  Written as inline
// assembly so that the compiler does not treat later LDS reads of other ring
// slots as possibly overwritten by this load and stall them on its completion;
// the kernel orders these loads itself (wait_vmem + barrier).  M0 carries the
// LDS address and is used by nothing else in these kernels.
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

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 15, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace

template <int G, bool WINDOWED>
__global__ void __launch_bounds__(kThreads, 2) prefill_fwd_d64(KParams p) {
  constexpr int P = kRows / G;  // positions per work-group
  __shared__ u32x4 lds_k[kSlots * kTileChunks];
  __shared__ u32x4 lds_v[kSlots * kTileChunks];

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
  float mref[2], lsum[2];
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
    mref[nb] = p.sinks ? p.sinks[head[nb]] * kLog2e : -INFINITY;
    lsum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][nb][e] = 0.f;
  }

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
  int voff[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int row = (2 * w + it) * 8 + (lane >> 3);
    const int data_ch = (lane & 7) ^ swz_key(row);
    voff[it] = (row * Hkv + g) * kRowBytes + data_ch * 16;
  }
  const uint32_t lds_k_base = lds_addr(lds_k) + w * 2048;  // this wave's part of slot 0
  const uint32_t lds_v_base = lds_addr(lds_v) + w * 2048;
  auto issue_tile = [&](int t, int buf) {
    const int off = t * tile_stride;  // carried in the VGPR offset, which the range check covers
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      lds_dma16(lds_k_base + buf * kTileBytes + it * 1024, rk, off + voff[it]);
      lds_dma16(lds_v_base + buf * kTileBytes + it * 1024, rv, off + voff[it]);
    }
  };

  const int r16 = lane & 15;
  const int half16 = (lane >> 4) & 1;

  issue_tile(kt0, 0);
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    wait_vmem<0>();   // this wave's loads of tile kt have landed
    __syncthreads();  // every wave's have; tile kt - 1 is fully consumed
    if (kt < kt1) issue_tile(kt + 1, buf ^ 1);
    const u32x4* kl = &lds_k[buf * kTileChunks];
    lds_char* vb = (lds_char*)&lds_v[buf * kTileChunks];

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
        const bf16x8 a = __builtin_bit_cast(bf16x8, kl[swz(key, 2 * ks + hi)]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          sacc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[nb][ks], sacc[mb][nb], 0, 0, 0);
      }
    }

    // ---- mask (only tiles not fully visible to every row of the work-group);
    // element (mb, e) holds key k0 + 4 hi + c with c = 32 mb + 8 (e / 4) + e % 4,
    // compared against this lane's diagonal offset so that c stays an immediate
    const int k0 = kt * kBK;
    const bool need_mask = (k0 + kBK - 1 > p0) || (WINDOWED && (p0 + P - 1) - k0 >= p.window);
    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int di = pos[nb] - k0 - 4 * hi;
        const int dw = di - p.window;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int c = 32 * mb + 8 * (e / 4) + (e % 4);
            const bool vis = (c <= di) && (!WINDOWED || c > dw);
            sacc[mb][nb][e] = vis ? sacc[mb][nb][e] : -INFINITY;
          }
      }
    }

    // ---- raise the reference maxima only when a row outgrows them by > 2^8
    float mcand[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) mcand[nb] = pair_max(max32(sacc[0][nb], sacc[1][nb])) * p.c;
    const bool grow = (mcand[0] > mref[0] + kRescaleSlack) || (mcand[1] > mref[1] + kRescaleSlack);
    if (__any(grow)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float mnew = fmaxf(mref[nb], mcand[nb]);
        const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mref[nb] - mnew);
        lsum[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][nb][e] *= alpha;
        mref[nb] = mnew;
      }
    }

    // ---- probabilities, bf16 P^T in the PV B-operand order, row sums of the bf16 values
    bf16x8 pf[4][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float muse = (mref[nb] == -INFINITY) ? 0.f : mref[nb];
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[mb][nb][8 * h2 + e], p.c, -muse));
            pf[2 * mb + h2][nb][e] = (__bf16)pe;
            part[e & 3] += pe;
          }
      lsum[nb] += (part[0] + part[1]) + (part[2] + part[3]);
    }

    // ---- O^T += V^T P^T; lane l of step s4 needs keys 16 s4 + 8 (e / 4) + 4 hi + e % 4
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int key_lo = 16 * s4 + 4 * hi + (r16 >> 2);
      const int key_hi = key_lo + 8;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int d = 32 * db + 16 * half16 + 4 * (r16 & 3);
        const int off_lo = key_lo * kRowBytes + (((d >> 3) ^ swz_key(key_lo)) << 4) + (d & 7) * 2;
        const int off_hi = key_hi * kRowBytes + (((d >> 3) ^ swz_key(key_hi)) << 4) + (d & 7) * 2;
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + off_lo));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + off_hi));
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
    float lt = pair_sum(lsum[nb]);
    if (p.sinks) lt += __builtin_amdgcn_exp2f(p.sinks[head[nb]] * kLog2e - mref[nb]);
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

namespace {

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
  // each sequence's K (or V) rows must be addressable by one buffer descriptor
  if (((int64_t)a.max_seqlen + kBK) * a.n_kv_heads * kRowBytes > 0x7fffffffLL) return -1;
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
