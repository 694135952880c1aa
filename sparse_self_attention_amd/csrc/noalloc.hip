// Allocation-free pooling mask: sattn_mask with its workspace in a fixed device array of this library
// instead of a caller's buffer, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array; every GPU the library runs on holds its own copy until the
// process ends.  In host code its name is only a host-side stand-in, so its device address is looked up
// once per device (with that device current) and only that address is passed to the kernels.  Every call
// on a device shares that device's array: calls that overlap on one GPU (other streams or threads) race.
// Nothing in it has to start at zero: each pass writes every part of it that it later reads.
#include <mutex>

#include "../../include/sattn.h"
#include "device_common.hpp"
#include "launch.hpp"

namespace sattn {

__device__ __align__(256) char scratch[SATTN_MASK_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device (null until looked up)
}  // namespace

// Device address of `scratch` on the current device, looked up on the first call there.
static int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= MAX_DEVICES) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

int launch_mask_noalloc(const MaskArgs& a, int heads_per_call) {
  void* ws = nullptr;
  int err = scratch_address(&ws);
  if (err) return err;
  const int BH = a.B * a.H;
  const int G = (a.Nq + a.group - 1) / a.group;
  log_launch("sattn_mask_noalloc: %d heads in calls of %d on the %d-byte device scratch", BH, heads_per_call,
             (int)SATTN_MASK_SCRATCH_BYTES);
  // the heads are independent: each call takes a contiguous range of the flattened (b, h) heads
  for (int bh0 = 0; bh0 < BH; bh0 += heads_per_call) {
    MaskArgs c = a;
    c.B = 1;
    c.H = BH - bh0 < heads_per_call ? BH - bh0 : heads_per_call;
    c.q = (const char*)a.q + (size_t)bh0 * a.Nq * a.D * 2;
    c.k = (const char*)a.k + (size_t)bh0 * a.Nk * a.D * 2;
    c.idx = a.idx + (size_t)bh0 * G * a.cap;
    c.counts = a.counts + (size_t)bh0 * G;
    c.workspace = ws;
    c.ws_bytes = SATTN_MASK_SCRATCH_BYTES;
    err = launch_mask(c);
    if (err) return err;
  }
  return 0;
}

}  // namespace sattn
