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
  // pipeline depth 1 (SATTN_SERIAL_GATHER=1): each block's gather lands before the previous block computes
  bool serial = false;
};
int launch_attn_fwd(const FwdArgs& a);

// Split-list forward (sattn_forward_split): workspace = per (row, part) the unnormalised fp32 output
// (D floats) then, from a 256-byte boundary, the part's running max and normaliser (2 floats).
inline size_t split_partials_bytes(int B, int H, int Nq, int D, int nsplit) {
  return ((size_t)B * H * Nq * nsplit * D * 4 + 255) & ~(size_t)255;
}
inline size_t split_workspace_bytes(int B, int H, int Nq, int D, int nsplit) {
  return split_partials_bytes(B, H, Nq, D, nsplit) + (((size_t)B * H * Nq * nsplit * 8 + 255) & ~(size_t)255);
}
constexpr int SPLIT_MAX_PARTS = 32;
int launch_attn_fwd_split(const FwdArgs& a, int nsplit, void* ws);

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
// sattn_mask_noalloc: launch_mask over ranges of heads_per_call heads with the library's device scratch as
// the workspace (noalloc.hip).
int launch_mask_noalloc(const MaskArgs& a, int heads_per_call);

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

// V-Smooth quantisation of V (fp8_attn.hip): E4M3 codes [B,H,Nk,D], power-of-two channel scales
// [B,H,D] and channel-major scaled block means [B,H,D,vsmooth_mean_stride(Nk)] (bf16 mean / scale).
constexpr int VSMOOTH_BLOCK = 128;
inline int vsmooth_blocks(int Nk) { return (int)(((int64_t)Nk + VSMOOTH_BLOCK - 1) / VSMOOTH_BLOCK); }
inline int vsmooth_mean_stride(int Nk) { return (vsmooth_blocks(Nk) + 3) & ~3; }
inline size_t vsmooth_mean_ws_bytes(int BH, int Nk, int D) {
  return ((size_t)BH * vsmooth_blocks(Nk) * D * 2 + 255) & ~(size_t)255;
}
inline size_t vsmooth_workspace_bytes(int BH, int Nk, int D) {
  return vsmooth_mean_ws_bytes(BH, Nk, D) + (((size_t)BH * vsmooth_blocks(Nk) * D * 4 + 255) & ~(size_t)255);
}
struct VsmoothArgs {
  const void* v;
  int B, H, Nk, D;
  uint8_t* codes;
  float* vscale;
  void* vmean;
  void* workspace;
  void* stream;
};
int launch_vsmooth(const VsmoothArgs& a);

struct Fp8FwdArgs {
  const void* q;                  // bf16 Q, or E2M1 codes of Q when q_scales is set
  const void* k;                  // bf16 K, or E2M1 codes of K when k_scales is set
  const uint8_t* q_scales;        // E8M0 block scales of Q and K (4-bit QK^T), else nullptr
  const uint8_t* k_scales;
  const uint8_t* codes;
  const float* vscale;
  const void* vmean;
  const int32_t* idx;
  const int32_t* counts;
  int cap;
  int B, H, Nq, Nk, D, group;
  float scale;
  void* out;
  bool out_f32;
  float* lse;
  void* stream;
};
int launch_fp8_fwd(const Fp8FwdArgs& a);

// MXFP4 codes [B,H,N,D/2] (two per byte, even element low) and E8M0 scales [B,H,N,4] (block b at byte b,
// D/32 blocks used) of bf16 rows.
struct Mx4QuantArgs {
  const void* x;
  int B, H, N, D;
  uint8_t* codes;
  uint8_t* scales;
  void* stream;
};
int launch_mx4_quant(const Mx4QuantArgs& a);

int launch_permute_tokens(const void* src, void* dst, const int32_t* perm, int BH, int N, int D, int inverse,
                          void* stream);

const char* hip_error_string(int e);

// With SATTN_LOG=1 in the environment: one line on stderr per kernel launch (printf format).
void log_launch(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

}  // namespace sattn
