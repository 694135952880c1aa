// MFMA rate probe (a measurement aid of the benchmark, not part of the attention path): every wave issues
// back-to-back v_mfma_f32_32x32x16_bf16 on random bf16 operands, cycling through eight operand pairs so that
// consecutive products see different data, into four independent accumulators.  The host times the launch;
// each wave also reports the shader-clock cycles it ran, so the clock the chip held can be read off.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sattn_probe.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int PAIRS = 8;

__global__ __launch_bounds__(256) void k_mfma_rate(const uint32_t* __restrict__ data, float* __restrict__ sink,
                                                   long long* __restrict__ cycles, int iters) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a[PAIRS], b[PAIRS];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p) {
    // 16 random bytes per operand and lane; the buffer holds 1024 lanes' worth of every pair
    const int slot = (t & 1023) * 2 * PAIRS + 2 * p;
    a[p] = __builtin_bit_cast(bf16x8, *(const u32x4*)(data + 4 * slot));
    b[p] = __builtin_bit_cast(bf16x8, *(const u32x4*)(data + 4 * (slot + 1)));
  }
  f32x16 acc[4] = {};
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m)
      acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % PAIRS], b[(m + 3) % PAIRS], acc[m & 3], 0, 0, 0);
  }
  const long long t1 = clock64();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  sink[t] = s;
  if ((threadIdx.x & 63) == 0) cycles[t >> 6] = t1 - t0;
}

extern "C" int sattn_probe_mfma_rate(const uint32_t* data, float* sink, long long* cycles, int workgroups, int iters,
                                     void* stream) {
  if (!data || !sink || !cycles || workgroups < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(k_mfma_rate, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, data, sink, cycles, iters);
  return (int)hipGetLastError();
}
