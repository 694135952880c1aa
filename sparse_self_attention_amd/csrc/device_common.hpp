// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sattn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

#define SATTN_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Buffer resource over [base, base + bytes): loads past the end return zeros instead of faulting.
// Third dword 0x00020000 selects raw 32-bit data for the CDNA buffer unit.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16-byte buffer load of one lane straight into LDS at (wave-uniform lds_base + 16 * lane).
__device__ inline void buffer_load_lds_x4(__amdgpu_buffer_rsrc_t rsrc, void* lds_base, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, SATTN_LDS_PTR(void, lds_base), 16, voffset, 0, 0, 0);
}

__device__ inline u32x4 buffer_load_x4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc, voffset, 0, 0);
}

// s_waitcnt vmcnt(0) only (expcnt / lgkmcnt left at their no-wait maxima; gfx9 encoding).
__device__ inline void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Max / sum of a value with the same value in the partner lane (lane ^ 32).
// v_permlane32_swap exchanges the upper half of the first operand with the lower half of the
// second; with both operands equal to x the two results hold x and its partner in some order,
// so a symmetric reduction of the two is the pair reduction in every lane.
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  f32x2 p = {a, b};
  bf16x2 r = __builtin_convertvector(p, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Sum of the two bf16 halves of a packed word, accumulated in fp32 (v_dot2_f32_bf16 with ones).
__device__ inline float add_bf16x2(uint32_t packed, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
}

// Workgroup id remap so that consecutive logical work items share one XCD (and its L2).
// The hardware deals workgroups to the 8 XCDs round robin; this bijection gives XCD x the
// contiguous logical range [x*q + min(x,r), ... + q + (x<r)) where n = 8q + r.
__device__ inline uint32_t xcd_contiguous(uint32_t bid, uint32_t n) {
  const uint32_t q = n >> 3, r = n & 7u;
  const uint32_t x = bid & 7u, pos = bid >> 3;
  return x * q + (x < r ? x : r) + pos;
}

// Workgroup id remap for the attention kernels: the logical range is cut into stripes of 8*S items
// and XCD x takes the x-th run of S items of each stripe, so at any moment the eight XCDs work on
// neighbouring items (one head's K/V stays hot in the shared last-level cache) while each XCD's own
// L2 still sees runs of S adjacent items.  Past the last whole stripe the remainder is dealt out as
// in xcd_contiguous.  A bijection of [0, n) for the round-robin dealing of workgroups to XCDs.
__device__ inline uint32_t xcd_striped(uint32_t bid, uint32_t n, uint32_t S) {
  const uint32_t x = bid & 7u, pos = bid >> 3;
  const uint32_t C = 8u * S, K = n / C, k = pos / S;
  if (k < K) return k * C + x * S + (pos - k * S);
  const uint32_t R = n - K * C, q = R >> 3, r = R & 7u;
  return K * C + x * q + (x < r ? x : r) + (pos - K * S);
}

}  // namespace sattn
