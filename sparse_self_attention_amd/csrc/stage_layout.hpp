// Layout of the fp32 per-(group, key) values that the mask kernels stage in the workspace for the
// per-group selection: one padded row per group, plus a contiguous row of every 16th value.
#pragma once

#include <stddef.h>

namespace sattn {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// fp32 rows are padded to a multiple of 32 floats: every row starts on a 128-byte cache line, so the
// 32-key runs the scores kernels store, and the 16-byte loads of the select, cover whole lines
static inline __host__ __device__ int score_stride(int Nk) { return (Nk + 31) & ~31; }
// Every SAMPLE_STEP-th score of a row is also written to a short contiguous sample row.
constexpr int SAMPLE_STEP = 16;
static inline __host__ __device__ int sample_len(int Nk) { return (Nk + SAMPLE_STEP - 1) / SAMPLE_STEP; }
static inline __host__ __device__ int sample_stride(int Nk) { return (sample_len(Nk) + 31) & ~31; }

}  // namespace sattn
