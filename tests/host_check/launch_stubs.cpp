// Stand-ins for the HIP launchers of launch.hpp, so that the C-ABI layer (api.cpp) and the host sizing
// (mask_sizes.cpp) can be built and run on the host alone, under AddressSanitizer and UBSan.  Every
// launcher records that it was reached and returns a non-zero "HIP error", so a call whose arguments pass
// validation comes back as SATTN_ERR_HIP without touching a device.
#include <stdio.h>

#include "../../sparse_self_attention_amd/csrc/launch.hpp"

int g_launches = 0;
constexpr int FAKE_HIP_ERROR = 999;

namespace sattn {
int launch_attn_fwd(const FwdArgs&) { ++g_launches; return FAKE_HIP_ERROR; }
int launch_attn_fwd_split(const FwdArgs&, int, void*) { ++g_launches; return FAKE_HIP_ERROR; }
int validate_index_lists(const int32_t*, const int32_t*, int, int, int, void*, int* flag_host) {
  ++g_launches;
  *flag_host = 0;
  return FAKE_HIP_ERROR;
}
int launch_mask(const MaskArgs&) { ++g_launches; return FAKE_HIP_ERROR; }
int launch_mask_noalloc(const MaskArgs&, int heads_per_call) {
  ++g_launches;
  return heads_per_call >= 1 ? FAKE_HIP_ERROR : 1;
}
int launch_cached_mask(const CachedMaskArgs&) { ++g_launches; return FAKE_HIP_ERROR; }
int launch_colsum_scores(const ColsumArgs&) { ++g_launches; return FAKE_HIP_ERROR; }
int launch_vsmooth(const VsmoothArgs&) { ++g_launches; return FAKE_HIP_ERROR; }
int launch_fp8_fwd(const Fp8FwdArgs&) { ++g_launches; return FAKE_HIP_ERROR; }
int launch_mx4_quant(const Mx4QuantArgs&) { ++g_launches; return FAKE_HIP_ERROR; }
int launch_permute_tokens(const void*, void*, const int32_t*, int, int, int, int, void*) {
  ++g_launches;
  return FAKE_HIP_ERROR;
}
const char* hip_error_string(int) { return "stand-in launcher (host-only build)"; }
}  // namespace sattn
