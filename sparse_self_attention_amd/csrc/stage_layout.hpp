// Layout of the fp32 per-(group, key) values that the mask kernels stage in the workspace for the
// per-group selection: one padded row per group, plus a contiguous row of every 16th value.
// Plain constexpr C++ (no HIP header): the host-side sizing in mask_sizes.cpp and the kernels share it.
#pragma once

#include <stddef.h>

namespace sattn {

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// fp32 rows are padded to a multiple of 32 floats: every row starts on a 128-byte cache line, so the
// 32-key runs the scores kernels store, and the 16-byte loads of the select, cover whole lines
constexpr int score_stride(int Nk) { return (Nk + 31) & ~31; }
// Every SAMPLE_STEP-th score of a row is also written to a short contiguous sample row.
constexpr int SAMPLE_STEP = 16;
constexpr int sample_len(int Nk) { return (Nk + SAMPLE_STEP - 1) / SAMPLE_STEP; }
constexpr int sample_stride(int Nk) { return (sample_len(Nk) + 31) & ~31; }

}  // namespace sattn
