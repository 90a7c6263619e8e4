// ubench.hip -- microbenchmarks behind the benchmark's third roof: the issue rate
// of the vector-ALU instructions the prefill kernels' softmax spends per score
// (a multiply by scale * log2 e, an exp2, half a bf16 pack), and the sustained
// rate of the bf16 MFMA the kernels use, both on a fully occupied gfx950 at the
// kernels' own occupancy (two waves per SIMD); plus the device's CU count and
// clocks.  Built into its own library (libts_ubench.so), which only the
// benchmark loads; it is not part of the attention library's interface.
//
// Each kernel runs `iters` loop trips of 16 independent instruction chains per
// lane (each chain feeds its next trip, so the compiler can neither remove nor
// hoist them) and writes one float per lane at the end.  Work-groups of 256 lanes that ask for 64 KiB of LDS each
// hold every compute unit to two work-groups, i.e. two waves per SIMD.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Op : int {
  kExp = 0,       // v_exp_f32 with a negated input (x <- 2^-x stays in (0, 1))
  kMul = 1,       // v_mul_f32 with VGPR operands
  kCvtPk = 2,     // v_cvt_pk_bf16_f32
  kSoftmax = 3,   // per score: v_mul_f32, v_exp_f32, half a v_cvt_pk_bf16_f32
  kMfma = 4,      // v_mfma_f32_32x32x16_bf16, four independent accumulators
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (one v_cvt_pk_bf16_f32) and the pair's bits read as one float.
__device__ __forceinline__ float pack_as_float(float lo, float hi) {
  const bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(float, p);
}

template <int OP>
__global__ void __launch_bounds__(256) valu_loop(float* out, int iters) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 0.25f + 0.01f * (float)((tid + i) & 15);
  float c = -1.0f;
  asm volatile("" : "+v"(c));
  if constexpr (OP == kMfma) {
    f32x16 acc[4] = {};
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(x[e] * 0.0f);
      b[e] = (__bf16)(x[e + 8] * 0.0f);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][e];
    out[tid] = s;
    return;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (OP == kExp) {
        x[i] = __builtin_amdgcn_exp2f(-x[i]);
      } else if constexpr (OP == kMul) {
        x[i] = x[i] * c;
      } else if constexpr (OP == kCvtPk) {
        x[i] = pack_as_float(x[i], x[(i + 1) & 15]);
      } else {
        x[i] = __builtin_amdgcn_exp2f(x[i] * c);
        // the pair's packed bf16 read back as a float is close to its upper
        // value, which keeps every chain in (0, 1) with no extra instruction
        if (i & 1) x[i - 1] = pack_as_float(x[i - 1], x[i]);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += x[i];
  out[tid] = s;
}

// Dynamic LDS each work-group reserves and never touches: with 160 KiB per
// compute unit, two work-groups fit and a third does not.
constexpr int kPadBytes = 64 * 1024;

template <int OP>
hipError_t launch(float* out, int n_groups, int iters, hipStream_t st) {
  hipLaunchKernelGGL(valu_loop<OP>, dim3(n_groups), dim3(256), kPadBytes, st, out, iters);
  return hipGetLastError();
}

}  // namespace

// CU count and clocks (kHz) of the current device, from hipDeviceGetAttribute.
extern "C" int ts_ubench_device_info(int* cus, int* clock_khz, int* mem_clock_khz, int* mem_bus_bits) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(mem_clock_khz, hipDeviceAttributeMemoryClockRate, dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(mem_bus_bits, hipDeviceAttributeMemoryBusWidth, dev) != hipSuccess) return -1;
  return 0;
}

// Enqueue one microbenchmark launch: n_groups work-groups of 256 lanes, `iters`
// loop trips of 16 instructions of kind `op` (0 exp2, 1 multiply, 2 bf16 pack,
// 3 softmax score, 4 MFMA 32x32x16 bf16) per lane; out holds n_groups * 256
// floats.  Returns 0, or -1 for a bad argument or a failed launch.
extern "C" int ts_ubench_valu(int op, int n_groups, int iters, float* out, void* stream) {
  if (!out || n_groups <= 0 || iters <= 0) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (op) {
    case kExp: e = launch<kExp>(out, n_groups, iters, st); break;
    case kMul: e = launch<kMul>(out, n_groups, iters, st); break;
    case kCvtPk: e = launch<kCvtPk>(out, n_groups, iters, st); break;
    case kSoftmax: e = launch<kSoftmax>(out, n_groups, iters, st); break;
    case kMfma: e = launch<kMfma>(out, n_groups, iters, st); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -1;
}
