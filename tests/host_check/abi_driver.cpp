// Host-only driver of the C ABI, built with AddressSanitizer and UBSan by tests/test_host_sanitizers.py.
// It makes every entry point fail each of its host-side checks (null pointers, shapes, sizes at the edge of
// the 32-bit index range, alignment, modes, workspace), reach the launcher with valid arguments, and runs the
// host-only calls (workspace sizes, voxel permutation, strerror, last_error) on edge cases.  Any
// out-of-bounds access, leak of the error-string buffer or undefined arithmetic aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/sattn.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(expr, want)                                                                           \
  do {                                                                                               \
    const int got_ = (int)(expr);                                                                    \
    if (got_ != (want)) {                                                                            \
      fprintf(stderr, "line %d: %s returned %d, want %d (%s)\n", __LINE__, #expr, got_, (int)(want), \
              sattn_last_error());                                                                   \
      ++failures;                                                                                    \
    }                                                                                                \
  } while (0)

int main() {
  alignas(256) static char buf[1 << 16];
  void* P = buf;                  // aligned, non-NULL, never dereferenced by the ABI layer
  void* U = buf + 2;              // misaligned
  int32_t* I = (int32_t*)buf;
  float* F = (float*)buf;
  uint8_t* B8 = (uint8_t*)buf;
  const int BIG = 0x7fffffff;

  for (int s = -1; s <= 9; ++s) EXPECT(sattn_strerror(s) != nullptr, 1);

  // workspace sizes: valid, invalid and the largest shapes
  EXPECT(sattn_mask_workspace_bytes(1, 24, 70200, 70200, 128, 128) > 0, 1);
  EXPECT(sattn_mask_workspace_bytes(0, 1, 1, 1, 128, 128), 0);
  EXPECT(sattn_mask_workspace_bytes(1, 1, 1, SATTN_MASK_MAX_NK + 1, 128, 128), 0);
  EXPECT(sattn_mask_workspace_bytes(1, 1, BIG, SATTN_MASK_MAX_NK, 128, 16), 0);          // a Q head over 2 GiB
  EXPECT(sattn_mask_workspace_bytes(1, 1, (1 << 23) - 1, SATTN_MASK_MAX_NK, 128, 16) > 0, 1);
  EXPECT(sattn_mask_workspace_bytes(1000, 1000, 1000, 1000, 64, 17), 0);
  EXPECT(sattn_vsmooth_workspace_bytes(1, 24, 70200, 128) > 0, 1);
  EXPECT(sattn_vsmooth_workspace_bytes(BIG, BIG, BIG, 128), 0);
  EXPECT(sattn_vsmooth_mean_stride(0), 0);
  EXPECT(sattn_vsmooth_mean_stride(BIG) > 0, 1);

  // sattn_mask
  const size_t ws = sattn_mask_workspace_bytes(1, 2, 300, 500, 128, 64);
  EXPECT(sattn_mask(nullptr, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_NULL);
  EXPECT(sattn_mask(P, P, 0, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_SHAPE);
  EXPECT(sattn_mask(P, P, 1, 2, BIG, BIG, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_SHAPE);
  EXPECT(sattn_mask(P, P, BIG, BIG, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_SHAPE);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 96, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_UNSUPPORTED);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 24, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_UNSUPPORTED);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 0, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 501, 0, 0.1f, I, I, 600, P, ws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 9, P, ws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_THRESH, 0, 1.5f, 0.1f, I, I, 500, P, ws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_THRESH, 0, 0.5f, 0.1f, I, I, 499, P, ws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, 7, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, -1.0f, I, I, 10, P, ws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask(U, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws - 1, nullptr), SATTN_ERR_WORKSPACE);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, nullptr, ws, nullptr), SATTN_ERR_WORKSPACE);
  EXPECT(sattn_mask(P, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_colsum_mask(P, P, F, 1, 2, 300, 500, 128, 64, 10, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_mask_noalloc(P, P, 2, 24, 70200, 70200, 128, 128, SATTN_TOPK, 14040, 0, 0.1f, I, I, 14040, nullptr),
         SATTN_ERR_HIP);
  EXPECT(sattn_mask_noalloc(P, P, 1, 1, 131072, 131072, 64, 16, SATTN_TOPK, 64, 0, 0.1f, I, I, 64, nullptr),
         SATTN_ERR_UNSUPPORTED);                                                 // one head exceeds the scratch
  EXPECT(sattn_mask_noalloc(P, P, 1, 2, 300, 500, 128, 64, SATTN_THRESH, 0, 2.0f, 0.1f, I, I, 500, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_mask_noalloc(nullptr, P, 1, 2, 300, 500, 128, 64, SATTN_TOPK, 10, 0, 0.1f, I, I, 10, nullptr), SATTN_ERR_NULL);
  EXPECT(sattn_colsum_mask(P, P, nullptr, 1, 2, 300, 500, 128, 64, 10, 0.1f, I, I, 10, P, ws, nullptr), SATTN_ERR_NULL);
  EXPECT(sattn_cached_mask(P, P, F, 1, 2, 300, 500, 128, 64, 1e-3f, 0.1f, I, I, 500, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_cached_mask(P, P, F, 1, 2, 300, 500, 128, 64, 0.0f / 0.0f, 0.1f, I, I, 500, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_cached_mask(P, P, F, 1, 2, 300, 500, 128, 64, 1e-3f, 0.1f, I, I, 0, nullptr), SATTN_ERR_ARG);

  // forward family
  EXPECT(sattn_forward(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, P, SATTN_F32, F, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_forward(P, P, P, I, I, 0, 1, 2, 300, 500, 128, 64, 0.1f, P, SATTN_F32, F, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_forward(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, P, 5, F, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_forward(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f / 0.0f, P, SATTN_F32, F, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_forward(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 272, 0.1f, P, SATTN_F32, F, nullptr), SATTN_ERR_UNSUPPORTED);
  EXPECT(sattn_forward(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, U, SATTN_F32, F, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_forward(P, P, P, I, I, 64, BIG / 2, 4, BIG / 1024, 500, 128, 16, 0.1f, P, SATTN_F32, F, nullptr),
         SATTN_ERR_SHAPE);
  EXPECT(sattn_forward(P, P, nullptr, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, P, SATTN_F32, F, nullptr), SATTN_ERR_NULL);
  const size_t sws = sattn_forward_split_workspace_bytes(1, 2, 300, 128, 3);
  EXPECT(sattn_forward_split(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, 3, P, sws, P, SATTN_F32, F, nullptr),
         SATTN_ERR_HIP);
  EXPECT(sattn_forward_split(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, 3, P, sws - 1, P, SATTN_F32, F, nullptr),
         SATTN_ERR_WORKSPACE);
  EXPECT(sattn_forward_split(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, 40, P, sws, P, SATTN_F32, F, nullptr),
         SATTN_ERR_ARG);
  EXPECT(sattn_delta_forward(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, F, F, F, P, SATTN_F32, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_delta_forward(P, P, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, F, F, nullptr, P, SATTN_F32, nullptr),
         SATTN_ERR_NULL);
  EXPECT(attn_forward(P, P, P, 1, 2, 300, 500, 128, 0.1f, P, SATTN_BF16, nullptr, nullptr), SATTN_ERR_HIP);
  EXPECT(attn_forward(P, P, P, 1, 2, 300, 500, 80, 0.1f, P, SATTN_BF16, nullptr, nullptr), SATTN_ERR_UNSUPPORTED);

  // FP8 / FP4 paths
  const size_t vws = sattn_vsmooth_workspace_bytes(1, 2, 500, 128);
  EXPECT(sattn_vsmooth_quantize(P, 1, 2, 500, 128, B8, F, P, P, vws, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_vsmooth_quantize(P, 1, 2, 500, 128, B8, F, P, P, vws - 1, nullptr), SATTN_ERR_WORKSPACE);
  EXPECT(sattn_vsmooth_quantize(P, 1, 2, 500, 128, B8 + 1, F, P, P, vws, nullptr), SATTN_ERR_ARG);
  EXPECT(sattn_fp8_forward(P, P, B8, F, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, P, SATTN_F32, F, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_fp8_forward(P, P, nullptr, F, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, P, SATTN_F32, F, nullptr),
         SATTN_ERR_NULL);
  EXPECT(sattn_mx4_quantize(P, 1, 2, 300, 128, B8, B8, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_mx4_quantize(P, BIG, BIG, BIG, 128, B8, B8, nullptr), SATTN_ERR_SHAPE);
  EXPECT(sattn_fp4_forward(B8, B8, B8, B8, B8, F, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, P, SATTN_F32, F, nullptr),
         SATTN_ERR_HIP);
  EXPECT(sattn_fp4_forward(B8, B8 + 1, B8, B8, B8, F, P, I, I, 64, 1, 2, 300, 500, 128, 64, 0.1f, P, SATTN_F32, F, nullptr),
         SATTN_ERR_ARG);

  // voxel permutation on the host: a permutation of [0, N), edges longer than the grid, the largest values
  {
    std::vector<int32_t> perm(30 * 45 * 52);
    EXPECT(sattn_voxel_permutation(30, 45, 52, 4, 6, 8, perm.data()), SATTN_OK);
    std::vector<char> seen(perm.size(), 0);
    for (int32_t p : perm) {
      if (p < 0 || (size_t)p >= perm.size() || seen[(size_t)p]) { ++failures; break; }
      seen[(size_t)p] = 1;
    }
    EXPECT(sattn_voxel_permutation(30, 45, 52, BIG, BIG, BIG, perm.data()), SATTN_OK);
    for (size_t i = 0; i < perm.size(); ++i)
      if (perm[i] != (int32_t)i) { ++failures; break; }      // one voxel holds the whole grid: raster order
    EXPECT(sattn_voxel_permutation(BIG, BIG, 2, 1, 1, 1, perm.data()), SATTN_ERR_SHAPE);
    EXPECT(sattn_voxel_permutation(3, 4, 5, 0, 1, 1, perm.data()), SATTN_ERR_SHAPE);
    EXPECT(sattn_voxel_permutation(3, 4, 5, 1, 1, 1, nullptr), SATTN_ERR_NULL);
  }
  EXPECT(sattn_permute_tokens(P, buf + 4096, I, 1, 2, 500, 128, 0, nullptr), SATTN_ERR_HIP);
  EXPECT(sattn_permute_tokens(P, P, I, 1, 2, 500, 128, 0, nullptr), SATTN_ERR_ARG);          // src == dst
  EXPECT(sattn_permute_tokens(P, buf + 4096, I, 1, 2, 500, 128, 2, nullptr), SATTN_ERR_ARG);

  // the detail string is bounded whatever the message
  EXPECT(strlen(sattn_last_error()) < 512, 1);
  if (g_launches == 0) ++failures;
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host ABI checks passed (%d launcher calls reached)\n", g_launches);
  return 0;
}
