// Measurement helper for the benchmark (not part of the attention path): the
// bf16 MFMA throughput this GPU sustains on a loop of nothing but
// v_mfma_f32_32x32x16_bf16, with operands that are either all 1.0 or
// pseudo-random.  The matrix cores draw more power on random bits than on
// constant ones, and under a power limit the clock follows, so the random
// figure is the practical ceiling for a kernel fed with real activations,
// next to the vendor's 2516.6 TFLOP/s dense bf16 peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vitattn_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;  // independent accumulators per wave

// 32-bit xorshift step (Marsaglia), for operand bits only
__device__ __forceinline__ uint32_t xorshift(uint32_t x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

// two bf16 values with random sign and mantissa and an exponent drawn from
// [2^-7, 2^0], roughly the spread of unit-variance activations (no sum of a
// launch can overflow)
__device__ __forceinline__ uint32_t random_pair(uint32_t x) {
  const uint32_t y = xorshift(x ^ 0x5bd1e995u);
  const uint32_t e0 = 120u + (x >> 29), e1 = 120u + (y >> 29);
  return (x & 0x807fu) | (e0 << 7) | (((y & 0x807fu) | (e1 << 7)) << 16);
}

__global__ __launch_bounds__(256) void mfma_loop(float* out, int iters, int random) {
  uint32_t x = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 0x9e3779b9u;
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    u32x4 ua, ub;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x = xorshift(x);
      ua[i] = random ? random_pair(x) : 0x3f803f80u;
      x = xorshift(x);
      ub[i] = random ? random_pair(x) : 0x3f803f80u;
    }
    a[j] = __builtin_bit_cast(bf16x8, ua);
    b[j] = __builtin_bit_cast(bf16x8, ub);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * 256u + threadIdx.x] = s;
}

}  // namespace

extern "C" int vitattn_probe_mfma_loop(float* out, int blocks, int iters, int random,
                                       void* stream) {
  if (!out) return -1;
  if (blocks < 1 || iters < 1) return -2;
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                     iters, random);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

extern "C" double vitattn_probe_mfma_loop_flops(int blocks, int iters) {
  // 4 waves per block, kChains MFMAs per iteration, 2*32*32*16 flops each
  return static_cast<double>(blocks) * 4.0 * iters * kChains * 2.0 * 32 * 32 * 16;
}
