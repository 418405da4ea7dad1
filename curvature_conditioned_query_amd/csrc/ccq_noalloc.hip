// ccq_fwd_chunked_noalloc: the chunked prefill with its workspace in a device array the library
// owns, for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  The kernels and the launch are those of
// ccq_fwd_chunked; only where the workspace comes from differs.
#include <mutex>

#include "ccq.h"
#include "ccq_internal.hpp"

namespace {

constexpr size_t kScratchBytes = CCQ_NOALLOC_SCRATCH_BYTES;

// The workspace of every ccq_fwd_chunked_noalloc call on a device.  Its name is only a host-side
// stand-in: host code uses the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// This device's address of `scratch`, looked up on the first call on the device (with that
// device current) and kept for the life of the process.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int ccq_fwd_chunked_noalloc(const ccq_fwd_params* p, void* hip_stream) {
  int seg = 0, cps = 0;
  const int st = ccq::fwd_resolve(p, &seg, &cps);
  if (st != CCQ_OK) return st;
  if (p->segments == 0) {
    // the library's own segment choice, with longer segments until the workspace fits
    const int nchunks = (p->T + 63) / 64;
    while (seg > 1 && ccq::fwd_workspace_for(p, seg) > kScratchBytes) {
      ++cps;
      seg = (nchunks + cps - 1) / cps;
    }
  }
  if (ccq::fwd_workspace_for(p, seg) > kScratchBytes) return CCQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return CCQ_ERR_LAUNCH;
  // nothing in the workspace has to start at zero: every slot and count the kernels read is
  // written earlier in the same call
  return ccq::fwd_launch(p, seg, cps, ws, static_cast<hipStream_t>(hip_stream));
}
