// Token permutation (voxel order) and index-list validation kernels.
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace sattn {

// dst[bh, i] = src[bh, perm[i]] (inverse = 0) or dst[bh, perm[i]] = src[bh, i] (inverse = 1).
// One 16-byte chunk per thread; rows are D*2 bytes.
__global__ __launch_bounds__(256) void k_permute_tokens(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                        const int32_t* __restrict__ perm, int N, int D, int inverse,
                                                        size_t total_chunks) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total_chunks) return;
  const int nc = D / 8;
  const size_t row = t / nc;
  const int chunk = (int)(t % nc);
  const size_t bh = row / N;
  const int i = (int)(row % N);
  int p = perm[i];
  if (p < 0 || p >= N) return;   // not a permutation entry: leave the row alone
  const size_t s_row = inverse ? row : bh * N + p;
  const size_t d_row = inverse ? bh * N + p : row;
  *(u32x4*)(dst + d_row * D + chunk * 8) = *(const u32x4*)(src + s_row * D + chunk * 8);
}

int launch_permute_tokens(const void* src, void* dst, const int32_t* perm, int BH, int N, int D, int inverse,
                          void* stream) {
  const size_t total = (size_t)BH * N * (D / 8);
  const size_t blocks = (total + 255) / 256;
  log_launch("k_permute_tokens%s: %zu workgroups x 256 threads", inverse ? " (inverse)" : "", blocks);
  hipLaunchKernelGGL(k_permute_tokens, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)src, (uint16_t*)dst, perm, N, D, inverse, total);
  return (int)hipGetLastError();
}

// Result word of the validation kernel: bit 0 counts out of [0,cap], bit 1 index out of range,
// bit 2 list not strictly ascending (a duplicate or out of order).
__device__ int g_validate_flag;

__global__ __launch_bounds__(256) void k_validate_lists(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ counts, int cap, int Nk) {
  const size_t unit = blockIdx.x;
  const int c = counts[unit];
  int bad = 0;
  if (c < 0 || c > cap) bad |= 1;
  const int n = c < 0 ? 0 : (c > cap ? cap : c);
  const int32_t* l = idx + unit * (size_t)cap;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int j = l[i];
    if (j < 0 || j >= Nk) bad |= 2;
    if (i > 0 && l[i - 1] >= j) bad |= 4;
  }
  if (bad) atomicOr(&g_validate_flag, bad);
}

// The flag is one word per device, so validating calls are serialised: each one clears it, launches the
// check and reads it back before the next one starts (the call synchronises its stream anyway).
static std::mutex g_validate_mutex;

int validate_index_lists(const int32_t* idx, const int32_t* counts, int cap, int BHG, int Nk, void* stream,
                         int* flag_host) {
  std::lock_guard<std::mutex> lock(g_validate_mutex);
  hipStream_t st = (hipStream_t)stream;
  static const int zero = 0;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_validate_flag), &zero, sizeof(int), 0,
                                        hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(k_validate_lists, dim3(BHG), dim3(256), 0, st, idx, counts, cap, Nk);
  e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  e = hipMemcpyFromSymbolAsync(flag_host, HIP_SYMBOL(g_validate_flag), sizeof(int), 0, hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return (int)e;
  return (int)hipStreamSynchronize(st);
}

const char* hip_error_string(int e) { return hipGetErrorString((hipError_t)e); }

}  // namespace sattn
