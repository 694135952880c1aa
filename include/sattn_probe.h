/*
 * sattn_probe.h - measurement aid of the benchmark (libsattn_probe.so), not part of the attention ABI.
 *
 * sattn_probe_mfma_rate - launch `workgroups` workgroups of 256 threads (4 waves) on `stream`; every wave
 * issues iters x 16 back-to-back v_mfma_f32_32x32x16_bf16 (32,768 flops each) on random bf16 operands,
 * into four independent accumulators.  Device pointers, owned by the caller:
 *   data    16 KiB x 16 = 256 KiB of random bits (operand pairs of 1024 lanes), 16-byte aligned;
 *   sink    one float per thread (workgroups * 256), written so the products are not optimised away;
 *   cycles  one int64 per wave (workgroups * 4): the shader-clock cycles the wave ran its loop.
 * The caller times the launch (HIP events on `stream`).  Returns 0, 1 for a bad argument, or a HIP error.
 */
#ifndef SATTN_PROBE_H
#define SATTN_PROBE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
int sattn_probe_mfma_rate(const uint32_t* data, float* sink, long long* cycles, int workgroups, int iters,
                          void* stream);
#ifdef __cplusplus
}
#endif
#endif /* SATTN_PROBE_H */
