// C ABI of libsattn: host-side argument validation and dispatch to the HIP launchers.
// Plain C++ (no HIP headers): every check here runs before any HIP call, so the validation
// paths can be exercised on a machine without a GPU.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "../../include/sattn.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(int err, const char* where) {
  return fail(SATTN_ERR_HIP, "%s: HIP error %d (%s)", where, err, sattn::hip_error_string(err));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int MAX_GROUP = 256;
constexpr int64_t I32_MAX = 0x7fffffff;

// Common shape checks of the attention inputs.
int check_shapes(const char* fn, int B, int H, int Nq, int Nk, int D) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return fail(SATTN_ERR_SHAPE, "%s: B, H, Nq, Nk must be >= 1", fn);
  if (D != 64 && D != 128) return fail(SATTN_ERR_UNSUPPORTED, "%s: D = %d, only 64 and 128 are supported", fn, D);
  // per-head byte offsets are 32-bit inside the kernels
  if ((int64_t)Nq * D * 2 >= I32_MAX || (int64_t)Nk * D * 2 >= I32_MAX)
    return fail(SATTN_ERR_SHAPE, "%s: one head of Q, K or V exceeds 2 GiB", fn);
  if ((int64_t)B * H >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: B*H too large", fn);
  return SATTN_OK;
}

int check_group(const char* fn, int group) {
  if (group < 16 || group > MAX_GROUP || group % 16 != 0)
    return fail(SATTN_ERR_UNSUPPORTED, "%s: group = %d must be a multiple of 16 in [16, %d]", fn, group, MAX_GROUP);
  return SATTN_OK;
}

int check_scale(const char* fn, float scale) {
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(SATTN_ERR_ARG, "%s: scale must be finite and > 0", fn);
  return SATTN_OK;
}

bool log_mode() {
  static const bool on = [] {
    const char* e = getenv("SATTN_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

bool serial_gather() {
  const char* e = getenv("SATTN_SERIAL_GATHER");
  return e != nullptr && e[0] != '\0' && e[0] != '0';
}

bool validate_mode() {
  const char* e = getenv("SATTN_VALIDATE");
  return e != nullptr && e[0] != '\0' && e[0] != '0';
}

}  // namespace

namespace sattn {
void log_launch(const char* fmt, ...) {
  if (!log_mode()) return;
  char line[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof(line), fmt, ap);
  va_end(ap);
  fprintf(stderr, "[sattn] %s\n", line);
}
}  // namespace sattn

extern "C" {

const char* sattn_strerror(int status) {
  switch (status) {
    case SATTN_OK: return "ok";
    case SATTN_ERR_NULL: return "a required pointer is NULL";
    case SATTN_ERR_SHAPE: return "invalid or too large shape";
    case SATTN_ERR_UNSUPPORTED: return "unsupported head dimension, group size or key count";
    case SATTN_ERR_ARG: return "invalid argument";
    case SATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case SATTN_ERR_HIP: return "HIP runtime error";
    case SATTN_ERR_INDEX: return "index list violates the preconditions";
    default: return "unknown status";
  }
}

const char* sattn_last_error(void) { return g_last_error; }

size_t sattn_mask_workspace_bytes(int B, int H, int Nq, int Nk, int D, int group) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (D != 64 && D != 128) || group < 16 || group > MAX_GROUP ||
      group % 16 != 0 || Nk > SATTN_MASK_MAX_NK || (int64_t)Nq * D * 2 >= I32_MAX || (int64_t)B * H >= I32_MAX)
    return 0;
  const int G = (int)(((int64_t)Nq + group - 1) / group);
  if ((int64_t)B * H * G >= I32_MAX) return 0;
  return sattn::mask_workspace_bytes(B * H, G, Nk, D);
}

}  // extern "C"

namespace {
// Host checks shared by sattn_mask and sattn_mask_noalloc.
int check_mask_args(const char* fn, const void* q, const void* k, int B, int H, int Nq, int Nk, int D, int group,
                    int mode, int topk, float thresh, float scale, const int32_t* idx, const int32_t* counts, int cap) {
  if (!q || !k || !idx || !counts) return fail(SATTN_ERR_NULL, "%s: q, k, idx and counts must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_group(fn, group)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (Nk > SATTN_MASK_MAX_NK) return fail(SATTN_ERR_UNSUPPORTED, "%s: Nk = %d > %d", fn, Nk, SATTN_MASK_MAX_NK);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(idx, 4) || !aligned(counts, 4))
    return fail(SATTN_ERR_ARG, "%s: q and k must be 16-byte aligned, idx and counts 4-byte aligned", fn);
  if (mode == SATTN_TOPK) {
    if (topk < 1 || topk > Nk) return fail(SATTN_ERR_ARG, "%s: topk = %d not in [1, Nk = %d]", fn, topk, Nk);
    if (cap < topk) return fail(SATTN_ERR_ARG, "%s: cap = %d < topk = %d", fn, cap, topk);
  } else if (mode == SATTN_THRESH) {
    if (!(thresh >= 0.0f && thresh <= 1.0f)) return fail(SATTN_ERR_ARG, "%s: thresh must be in [0, 1]", fn);
    if (cap < Nk) return fail(SATTN_ERR_ARG, "%s: cap = %d < Nk = %d in threshold mode", fn, cap, Nk);
  } else {
    return fail(SATTN_ERR_ARG, "%s: mode = %d is neither SATTN_TOPK nor SATTN_THRESH", fn, mode);
  }
  if ((int64_t)B * H * ((Nq + group - 1) / group) >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many groups", fn);
  return SATTN_OK;
}
}  // namespace

extern "C" {

int sattn_mask(const void* q, const void* k, int B, int H, int Nq, int Nk, int D, int group, int mode, int topk,
               float thresh, float scale, int32_t* idx, int32_t* counts, int cap, void* workspace, size_t ws_bytes,
               void* stream) {
  static const char* fn = "sattn_mask";
  if (int r = check_mask_args(fn, q, k, B, H, Nq, Nk, D, group, mode, topk, thresh, scale, idx, counts, cap)) return r;
  const size_t need = sattn_mask_workspace_bytes(B, H, Nq, Nk, D, group);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256))
    return fail(SATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-byte aligned), got %zu", fn, need, ws_bytes);
  sattn::MaskArgs a{q, k, B, H, Nq, Nk, D, group, mode, topk, thresh, scale, idx, counts, cap,
                    workspace, ws_bytes, stream};
  const int err = sattn::launch_mask(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_mask_noalloc(const void* q, const void* k, int B, int H, int Nq, int Nk, int D, int group, int mode,
                       int topk, float thresh, float scale, int32_t* idx, int32_t* counts, int cap, void* stream) {
  static const char* fn = "sattn_mask_noalloc";
  if (int r = check_mask_args(fn, q, k, B, H, Nq, Nk, D, group, mode, topk, thresh, scale, idx, counts, cap)) return r;
  const int G = (Nq + group - 1) / group;
  const size_t one = sattn::mask_workspace_bytes(1, G, Nk, D);
  if (one > SATTN_MASK_SCRATCH_BYTES)
    return fail(SATTN_ERR_UNSUPPORTED, "%s: one head needs %zu bytes of workspace, the device scratch holds %u "
                "(fewer groups or keys, or sattn_mask with a caller's workspace)", fn, one, SATTN_MASK_SCRATCH_BYTES);
  // the most heads per call whose workspace fits (the size grows with the head count)
  int lo = 1, hi = B * H;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (sattn::mask_workspace_bytes(mid, G, Nk, D) <= SATTN_MASK_SCRATCH_BYTES) lo = mid;
    else hi = mid - 1;
  }
  sattn::MaskArgs a{q, k, B, H, Nq, Nk, D, group, mode, topk, thresh, scale, idx, counts, cap, nullptr, 0, stream};
  const int err = sattn::launch_mask_noalloc(a, lo);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_colsum_mask(const void* q, const void* k, const float* lse, int B, int H, int Nq, int Nk, int D,
                      int group, int topk, float scale, int32_t* idx, int32_t* counts, int cap, void* workspace,
                      size_t ws_bytes, void* stream) {
  static const char* fn = "sattn_colsum_mask";
  if (!q || !k || !lse || !idx || !counts)
    return fail(SATTN_ERR_NULL, "%s: q, k, lse, idx and counts must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_group(fn, group)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (Nk > SATTN_MASK_MAX_NK) return fail(SATTN_ERR_UNSUPPORTED, "%s: Nk = %d > %d", fn, Nk, SATTN_MASK_MAX_NK);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4) || !aligned(idx, 4) || !aligned(counts, 4))
    return fail(SATTN_ERR_ARG, "%s: q and k must be 16-byte aligned, lse, idx and counts 4-byte aligned", fn);
  if (topk < 1 || topk > Nk) return fail(SATTN_ERR_ARG, "%s: topk = %d not in [1, Nk = %d]", fn, topk, Nk);
  if (cap < topk) return fail(SATTN_ERR_ARG, "%s: cap = %d < topk = %d", fn, cap, topk);
  const size_t need = sattn_mask_workspace_bytes(B, H, Nq, Nk, D, group);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256))
    return fail(SATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-byte aligned), got %zu", fn, need, ws_bytes);
  sattn::MaskArgs a{q, k, B, H, Nq, Nk, D, group, 2, topk, 0.0f, scale, idx, counts, cap, workspace, ws_bytes, stream};
  a.lse = lse;
  const int err = sattn::launch_mask(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_cached_mask(const void* q, const void* k, const float* lse, int B, int H, int Nq, int Nk, int D,
                      int group, float tau, float scale, int32_t* idx, int32_t* counts, int cap, void* stream) {
  static const char* fn = "sattn_cached_mask";
  if (!q || !k || !lse || !idx || !counts)
    return fail(SATTN_ERR_NULL, "%s: q, k, lse, idx and counts must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_group(fn, group)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (Nk > SATTN_MASK_MAX_NK) return fail(SATTN_ERR_UNSUPPORTED, "%s: Nk = %d > %d", fn, Nk, SATTN_MASK_MAX_NK);
  if (tau != tau) return fail(SATTN_ERR_ARG, "%s: tau is NaN", fn);
  if (cap < 1) return fail(SATTN_ERR_ARG, "%s: cap = %d must be >= 1", fn, cap);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4) || !aligned(idx, 4) || !aligned(counts, 4))
    return fail(SATTN_ERR_ARG, "%s: q and k must be 16-byte aligned, lse, idx and counts 4-byte aligned", fn);
  if ((int64_t)B * H * ((Nq + group - 1) / group) >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many groups", fn);
  sattn::CachedMaskArgs a{q, k, lse, B, H, Nq, Nk, D, group, tau, scale, idx, counts, cap, stream};
  const int err = sattn::launch_cached_mask(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_forward(const void* q, const void* k, const void* v, const int32_t* idx, const int32_t* counts, int cap,
                  int B, int H, int Nq, int Nk, int D, int group, float scale, void* out, int out_dtype, float* lse,
                  void* stream) {
  static const char* fn = "sattn_forward";
  if (!q || !k || !v || !idx || !counts || !out)
    return fail(SATTN_ERR_NULL, "%s: q, k, v, idx, counts and out must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_group(fn, group)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (cap < 1) return fail(SATTN_ERR_ARG, "%s: cap = %d must be >= 1", fn, cap);
  if (out_dtype != SATTN_BF16 && out_dtype != SATTN_F32) return fail(SATTN_ERR_ARG, "%s: bad out_dtype", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(idx, 4) ||
      !aligned(counts, 4) || !aligned(lse, 4))
    return fail(SATTN_ERR_ARG, "%s: q, k, v, out must be 16-byte aligned; idx, counts, lse 4-byte aligned", fn);
  const int64_t G = (Nq + group - 1) / group;
  if ((int64_t)B * H * G >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many groups", fn);
  if (validate_mode()) {
    int flag = 0;
    const int err = sattn::validate_index_lists(idx, counts, cap, (int)(B * H * G), Nk, stream, &flag);
    if (err) return hip_fail(err, fn);
    if (flag)
      return fail(SATTN_ERR_INDEX, "%s: index lists invalid (%s%s%s)", fn, (flag & 1) ? "counts out of [0,cap] " : "",
                  (flag & 2) ? "index out of [0,Nk) " : "", (flag & 4) ? "not strictly ascending" : "");
  }
  sattn::FwdArgs a{q, k, v, idx, counts, cap, B, H, Nq, Nk, D, group, scale, out, out_dtype == SATTN_F32, lse,
                   false, stream};
  a.serial = serial_gather();
  const int err = sattn::launch_attn_fwd(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

size_t sattn_forward_split_workspace_bytes(int B, int H, int Nq, int D, int splits) {
  if (B < 1 || H < 1 || Nq < 1 || (D != 64 && D != 128) || splits < 1 || splits > sattn::SPLIT_MAX_PARTS ||
      (int64_t)B * H * Nq * splits >= I32_MAX)
    return 0;
  return sattn::split_workspace_bytes(B, H, Nq, D, splits);
}

int sattn_forward_split(const void* q, const void* k, const void* v, const int32_t* idx, const int32_t* counts,
                        int cap, int B, int H, int Nq, int Nk, int D, int group, float scale, int splits,
                        void* workspace, size_t ws_bytes, void* out, int out_dtype, float* lse, void* stream) {
  static const char* fn = "sattn_forward_split";
  if (!q || !k || !v || !idx || !counts || !out)
    return fail(SATTN_ERR_NULL, "%s: q, k, v, idx, counts and out must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_group(fn, group)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (cap < 1) return fail(SATTN_ERR_ARG, "%s: cap = %d must be >= 1", fn, cap);
  if (splits < 1 || splits > sattn::SPLIT_MAX_PARTS)
    return fail(SATTN_ERR_ARG, "%s: splits = %d must be in 1 .. %d", fn, splits, sattn::SPLIT_MAX_PARTS);
  if (out_dtype != SATTN_BF16 && out_dtype != SATTN_F32) return fail(SATTN_ERR_ARG, "%s: bad out_dtype", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(idx, 4) ||
      !aligned(counts, 4) || !aligned(lse, 4) || !aligned(workspace, 16))
    return fail(SATTN_ERR_ARG, "%s: q, k, v, out, workspace must be 16-byte aligned; idx, counts, lse 4-byte aligned",
                fn);
  const int64_t G = (Nq + group - 1) / group;
  if ((int64_t)B * H * G * splits >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many groups x splits", fn);
  const size_t need = sattn_forward_split_workspace_bytes(B, H, Nq, D, splits);
  if (need == 0) return fail(SATTN_ERR_SHAPE, "%s: too many rows x splits", fn);
  if (!workspace || ws_bytes < need)
    return fail(SATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  if (validate_mode()) {
    int flag = 0;
    const int err = sattn::validate_index_lists(idx, counts, cap, (int)(B * H * G), Nk, stream, &flag);
    if (err) return hip_fail(err, fn);
    if (flag)
      return fail(SATTN_ERR_INDEX, "%s: index lists invalid (%s%s%s)", fn, (flag & 1) ? "counts out of [0,cap] " : "",
                  (flag & 2) ? "index out of [0,Nk) " : "", (flag & 4) ? "not strictly ascending" : "");
  }
  sattn::FwdArgs a{q, k, v, idx, counts, cap, B, H, Nq, Nk, D, group, scale, out, out_dtype == SATTN_F32, lse,
                   false, stream};
  a.serial = serial_gather();
  const int err = sattn::launch_attn_fwd_split(a, splits, workspace);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_delta_forward(const void* q, const void* k, const void* v, const int32_t* idx, const int32_t* counts,
                        int cap, int B, int H, int Nq, int Nk, int D, int group, float scale, const float* lse,
                        const float* out_prev, float* fresh, void* out, int out_dtype, void* stream) {
  static const char* fn = "sattn_delta_forward";
  if (!q || !k || !v || !idx || !counts || !lse || !out_prev || !fresh || !out)
    return fail(SATTN_ERR_NULL, "%s: q, k, v, idx, counts, lse, out_prev, fresh and out must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_group(fn, group)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (cap < 1) return fail(SATTN_ERR_ARG, "%s: cap = %d must be >= 1", fn, cap);
  if (out_dtype != SATTN_BF16 && out_dtype != SATTN_F32) return fail(SATTN_ERR_ARG, "%s: bad out_dtype", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(out_prev, 16) ||
      !aligned(fresh, 16) || !aligned(idx, 4) || !aligned(counts, 4) || !aligned(lse, 4))
    return fail(SATTN_ERR_ARG, "%s: q, k, v, out, out_prev, fresh must be 16-byte aligned; idx, counts, lse 4-byte",
                fn);
  const int64_t G = (Nq + group - 1) / group;
  if ((int64_t)B * H * G >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many groups", fn);
  if (validate_mode()) {
    int flag = 0;
    const int err = sattn::validate_index_lists(idx, counts, cap, (int)(B * H * G), Nk, stream, &flag);
    if (err) return hip_fail(err, fn);
    if (flag) return fail(SATTN_ERR_INDEX, "%s: index lists invalid (code %d)", fn, flag);
  }
  sattn::FwdArgs a{q, k, v, idx, counts, cap, B, H, Nq, Nk, D, group, scale, out, out_dtype == SATTN_F32, nullptr,
                   false, stream};
  a.delta = true;
  a.lse_in = lse;
  a.out_prev = out_prev;
  a.fresh = fresh;
  a.serial = serial_gather();
  const int err = sattn::launch_attn_fwd(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

size_t sattn_vsmooth_workspace_bytes(int B, int H, int Nk, int D) {
  if (B < 1 || H < 1 || Nk < 1 || (D != 64 && D != 128) || (int64_t)B * H >= I32_MAX || (int64_t)Nk * D * 2 >= I32_MAX)
    return 0;
  return sattn::vsmooth_workspace_bytes(B * H, Nk, D);
}

int sattn_vsmooth_mean_stride(int Nk) { return Nk < 1 ? 0 : sattn::vsmooth_mean_stride(Nk); }

int sattn_vsmooth_quantize(const void* v, int B, int H, int Nk, int D, uint8_t* codes, float* vscale, void* vmean,
                           void* workspace, size_t ws_bytes, void* stream) {
  static const char* fn = "sattn_vsmooth_quantize";
  if (!v || !codes || !vscale || !vmean) return fail(SATTN_ERR_NULL, "%s: v, codes, vscale and vmean must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, 1, Nk, D)) return r;
  if ((int64_t)B * H * sattn::vsmooth_blocks(Nk) >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many blocks", fn);
  if (!aligned(v, 16) || !aligned(codes, 16) || !aligned(vscale, 16) || !aligned(vmean, 16))
    return fail(SATTN_ERR_ARG, "%s: v, codes, vscale and vmean must be 16-byte aligned", fn);
  const size_t need = sattn_vsmooth_workspace_bytes(B, H, Nk, D);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256))
    return fail(SATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-byte aligned), got %zu", fn, need, ws_bytes);
  sattn::VsmoothArgs a{v, B, H, Nk, D, codes, vscale, vmean, workspace, stream};
  const int err = sattn::launch_vsmooth(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_fp8_forward(const void* q, const void* k, const uint8_t* codes, const float* vscale, const void* vmean,
                      const int32_t* idx, const int32_t* counts, int cap, int B, int H, int Nq, int Nk, int D,
                      int group, float scale, void* out, int out_dtype, float* lse, void* stream) {
  static const char* fn = "sattn_fp8_forward";
  if (!q || !k || !codes || !vscale || !vmean || !idx || !counts || !out)
    return fail(SATTN_ERR_NULL, "%s: q, k, codes, vscale, vmean, idx, counts and out must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_group(fn, group)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (cap < 1) return fail(SATTN_ERR_ARG, "%s: cap = %d must be >= 1", fn, cap);
  if (out_dtype != SATTN_BF16 && out_dtype != SATTN_F32) return fail(SATTN_ERR_ARG, "%s: bad out_dtype", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(codes, 16) || !aligned(vscale, 16) || !aligned(vmean, 16) ||
      !aligned(out, 16) || !aligned(idx, 4) || !aligned(counts, 4) || !aligned(lse, 4))
    return fail(SATTN_ERR_ARG, "%s: q, k, codes, vscale, vmean, out must be 16-byte aligned; idx, counts, lse 4-byte",
                fn);
  const int64_t G = (Nq + group - 1) / group;
  if ((int64_t)B * H * G >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many groups", fn);
  if (validate_mode()) {
    int flag = 0;
    const int err = sattn::validate_index_lists(idx, counts, cap, (int)(B * H * G), Nk, stream, &flag);
    if (err) return hip_fail(err, fn);
    if (flag) return fail(SATTN_ERR_INDEX, "%s: index lists invalid (code %d)", fn, flag);
  }
  sattn::Fp8FwdArgs a{q, k, nullptr, nullptr, codes, vscale, vmean, idx, counts, cap, B, H, Nq, Nk, D, group, scale, out,
                      out_dtype == SATTN_F32, lse, stream};
  const int err = sattn::launch_fp8_fwd(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_mx4_quantize(const void* x, int B, int H, int N, int D, uint8_t* codes, uint8_t* scales, void* stream) {
  static const char* fn = "sattn_mx4_quantize";
  if (!x || !codes || !scales) return fail(SATTN_ERR_NULL, "%s: x, codes and scales must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, N, 1, D)) return r;
  if ((int64_t)B * H * N * (D / 32) >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many blocks", fn);
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(SATTN_ERR_ARG, "%s: x and codes must be 16-byte aligned, scales 4-byte aligned", fn);
  sattn::Mx4QuantArgs a{x, B, H, N, D, codes, scales, stream};
  const int err = sattn::launch_mx4_quant(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_fp4_forward(const uint8_t* q4, const uint8_t* q_scales, const uint8_t* k4, const uint8_t* k_scales,
                      const uint8_t* codes, const float* vscale, const void* vmean, const int32_t* idx,
                      const int32_t* counts, int cap, int B, int H, int Nq, int Nk, int D, int group, float scale,
                      void* out, int out_dtype, float* lse, void* stream) {
  static const char* fn = "sattn_fp4_forward";
  if (!q4 || !q_scales || !k4 || !k_scales || !codes || !vscale || !vmean || !idx || !counts || !out)
    return fail(SATTN_ERR_NULL, "%s: every input and out must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_group(fn, group)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (cap < 1) return fail(SATTN_ERR_ARG, "%s: cap = %d must be >= 1", fn, cap);
  if (out_dtype != SATTN_BF16 && out_dtype != SATTN_F32) return fail(SATTN_ERR_ARG, "%s: bad out_dtype", fn);
  if (!aligned(q4, 16) || !aligned(k4, 16) || !aligned(q_scales, 4) || !aligned(k_scales, 4) || !aligned(codes, 16) ||
      !aligned(vscale, 16) || !aligned(vmean, 16) || !aligned(out, 16) || !aligned(idx, 4) || !aligned(counts, 4) ||
      !aligned(lse, 4))
    return fail(SATTN_ERR_ARG, "%s: q4, k4, codes, vscale, vmean, out 16-byte; scales, idx, counts, lse 4-byte aligned",
                fn);
  const int64_t G = (Nq + group - 1) / group;
  if ((int64_t)B * H * G >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: too many groups", fn);
  if (validate_mode()) {
    int flag = 0;
    const int err = sattn::validate_index_lists(idx, counts, cap, (int)(B * H * G), Nk, stream, &flag);
    if (err) return hip_fail(err, fn);
    if (flag) return fail(SATTN_ERR_INDEX, "%s: index lists invalid (code %d)", fn, flag);
  }
  sattn::Fp8FwdArgs a{q4, k4, q_scales, k_scales, codes, vscale, vmean, idx, counts, cap, B, H, Nq, Nk, D, group,
                      scale, out, out_dtype == SATTN_F32, lse, stream};
  const int err = sattn::launch_fp8_fwd(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int attn_forward(const void* q, const void* k, const void* v, int B, int H, int Nq, int Nk, int D, float scale,
                 void* out, int out_dtype, float* lse, void* stream) {
  static const char* fn = "attn_forward";
  if (!q || !k || !v || !out) return fail(SATTN_ERR_NULL, "%s: q, k, v and out must be non-NULL", fn);
  if (int r = check_shapes(fn, B, H, Nq, Nk, D)) return r;
  if (int r = check_scale(fn, scale)) return r;
  if (out_dtype != SATTN_BF16 && out_dtype != SATTN_F32) return fail(SATTN_ERR_ARG, "%s: bad out_dtype", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return fail(SATTN_ERR_ARG, "%s: q, k, v, out must be 16-byte aligned; lse 4-byte aligned", fn);
  sattn::FwdArgs a{q, k, v, nullptr, nullptr, 1, B, H, Nq, Nk, D, 128, scale, out, out_dtype == SATTN_F32, lse,
                   true, stream};
  a.serial = serial_gather();
  const int err = sattn::launch_attn_fwd(a);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

int sattn_voxel_permutation(int T, int Hg, int Wg, int vt, int vy, int vx, int32_t* perm) {
  static const char* fn = "sattn_voxel_permutation";
  if (!perm) return fail(SATTN_ERR_NULL, "%s: perm must be non-NULL", fn);
  if (T < 1 || Hg < 1 || Wg < 1 || vt < 1 || vy < 1 || vx < 1)
    return fail(SATTN_ERR_SHAPE, "%s: grid and voxel sizes must be >= 1", fn);
  const int64_t n = (int64_t)T * Hg * Wg;
  if (n >= I32_MAX) return fail(SATTN_ERR_SHAPE, "%s: grid too large", fn);
  // an edge longer than the grid acts as the grid's own extent (t / vt = 0, t % vt = t); clamping keeps the
  // composite key below T * Hg * Wg
  vt = std::min(vt, T);
  vy = std::min(vy, Hg);
  vx = std::min(vx, Wg);
  const int64_t ny = (Hg + vy - 1) / vy, nx = (Wg + vx - 1) / vx;
  // composite key of (t/vt, y/vy, x/vx, t%vt, y%vy, x%vx): unique per token and order-preserving
  std::vector<std::pair<int64_t, int32_t>> keyed((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = i / ((int64_t)Hg * Wg), y = (i / Wg) % Hg, x = i % Wg;
    const int64_t cell = ((t / vt) * ny + y / vy) * nx + x / vx;
    const int64_t inner = ((t % vt) * vy + y % vy) * vx + x % vx;
    keyed[(size_t)i] = {cell * ((int64_t)vt * vy * vx) + inner, (int32_t)i};
  }
  std::sort(keyed.begin(), keyed.end());
  for (int64_t i = 0; i < n; ++i) perm[i] = keyed[(size_t)i].second;
  return SATTN_OK;
}

int sattn_permute_tokens(const void* src, void* dst, const int32_t* perm, int B, int H, int N, int D, int inverse,
                         void* stream) {
  static const char* fn = "sattn_permute_tokens";
  if (!src || !dst || !perm) return fail(SATTN_ERR_NULL, "%s: src, dst and perm must be non-NULL", fn);
  if (B < 1 || H < 1 || N < 1) return fail(SATTN_ERR_SHAPE, "%s: B, H, N must be >= 1", fn);
  if (D != 64 && D != 128) return fail(SATTN_ERR_UNSUPPORTED, "%s: D must be 64 or 128", fn);
  if (inverse != 0 && inverse != 1) return fail(SATTN_ERR_ARG, "%s: inverse must be 0 or 1", fn);
  if (src == dst) return fail(SATTN_ERR_ARG, "%s: src and dst must not alias", fn);
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(perm, 4))
    return fail(SATTN_ERR_ARG, "%s: src and dst must be 16-byte aligned", fn);
  const int err = sattn::launch_permute_tokens(src, dst, perm, B * H, N, D, inverse, stream);
  return err ? hip_fail(err, fn) : SATTN_OK;
}

}  // extern "C"
