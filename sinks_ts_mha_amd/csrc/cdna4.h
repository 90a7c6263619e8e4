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

// Position of 16-byte chunk `ch` of row `row` (8 chunks of a 128-byte row) in
// an LDS tile.  The LDS serves 64 banks of 4 bytes per cycle, two 128-byte
// rows; the XOR key (row bit 1 as chunk bit 2, row bits 2..3 as chunk bits
// 0..1) spreads both 16 consecutive rows reading one chunk and 4 consecutive
// rows reading 4 adjacent chunks over 16 distinct bank groups.
__device__ __forceinline__ int swz_key(int row) { return ((row & 2) << 1) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ swz_key(row)); }

}  // namespace cdna4
}  // namespace tsmha
