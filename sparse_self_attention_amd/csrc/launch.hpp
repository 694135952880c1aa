// Internal launcher interface between the C-ABI layer (api.cpp, plain C++) and the HIP kernels.
// Every launcher returns 0 or a hipError_t value; pointers are device pointers; stream is a
// hipStream_t passed as void*.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  const int32_t* counts;
  int cap;
  int B, H, Nq, Nk, D, group;
  float scale;
  void* out;
  bool out_f32;
  float* lse;
  bool dense;
  void* stream;
  // sparse-delta update (sattn_delta_forward): stale lse, cached output, running fresh part
  bool delta = false;
  const float* lse_in = nullptr;
  const float* out_prev = nullptr;
  float* fresh = nullptr;
};
int launch_attn_fwd(const FwdArgs& a);

// Validation of index lists: writes 0 into *flag_host when every list is unique, ascending and in
// range with 0 <= counts <= cap, else a non-zero code.  Synchronises the stream.
int validate_index_lists(const int32_t* idx, const int32_t* counts, int cap, int BHG, int Nk, void* stream,
                         int* flag_host);

struct MaskArgs {
  const void* q;
  const void* k;
  int B, H, Nq, Nk, D, group;
  int mode;        // 0 top-k, 1 threshold (both on the group-mean scores), 2 top-k of column sums
  int topk;
  float thresh;
  float scale;
  int32_t* idx;
  int32_t* counts;
  int cap;
  void* workspace;
  size_t ws_bytes;
  void* stream;
  const float* lse = nullptr;   // mode 2: row lse of the step whose normalisation is reused
};
// Number of (batch, head) pairs whose scores are held in the workspace at once.
int mask_heads_per_pass(int BH, int G, int Nk);
size_t mask_workspace_bytes(int BH, int G, int Nk, int D);
int launch_mask(const MaskArgs& a);

struct CachedMaskArgs {
  const void* q;
  const void* k;
  const float* lse;
  int B, H, Nq, Nk, D, group;
  float tau;
  float scale;
  int32_t* idx;
  int32_t* counts;
  int cap;
  void* stream;
};
int launch_cached_mask(const CachedMaskArgs& a);

// Column sums of attention probabilities with a given lse, c[g][j] = sum_{i in g} exp(scale q_i.k_j - lse_i),
// for heads [bh0, bh0 + nheads), written in the staging layout of stage_layout.hpp (rows and samples).
struct ColsumArgs {
  const void* q;
  const void* k;
  const float* lse;
  int Nq, Nk, D, group;
  float scale;
  float* scores;
  float* samples;
  int bh0, nheads;
  void* stream;
};
int launch_colsum_scores(const ColsumArgs& a);

int launch_permute_tokens(const void* src, void* dst, const int32_t* perm, int BH, int N, int D, int inverse,
                          void* stream);

const char* hip_error_string(int e);

}  // namespace sattn
