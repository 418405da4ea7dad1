// Chunked prefill of the CCQ read step on a Gated DeltaNet backbone: main kernel, carry scans
// and launch (the kernels and their description are in ccq_prefill_gdn_kernels.hpp; the segment
// summary is instantiated in ccq_prefill_gdn_summary.hip).
#include "ccq_prefill_gdn_kernels.hpp"

namespace ccq {

// ---------------------------------------------------------------- launch

template <int D, typename T>
static hipError_t launch_gdn_t(const FwdArgs& a, hipStream_t s) {
  const int chains = a.B * a.H;
  const int P = a.segments;
  auto rec = [&](int i) -> hipError_t {
    return a.events ? hipEventRecord(static_cast<hipEvent_t>(a.events[i]), s) : hipSuccess;
  };
  if (rec(0) != hipSuccess) return hipErrorLaunchFailure;
  if (P > 1) {
    const hipError_t es = launch_gdn_summary(a, s);
    if (es != hipSuccess) return es;
    if (rec(1) != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((gdn_scan_state_kernel<D>), dim3(D / 16, (unsigned)chains), dim3(2 * D), 0, s, a);
    hipLaunchKernelGGL((gdn_scan_sum_kernel<D>), dim3((unsigned)((D * D + D + 255) / 256), (unsigned)chains), dim3(256),
                       0, s, a);
  } else if (rec(1) != hipSuccess) {
    return hipErrorLaunchFailure;
  }
  if (rec(2) != hipSuccess) return hipErrorLaunchFailure;
  if (a.chunk_carry != nullptr)
    hipLaunchKernelGGL((gdn_main_kernel<D, T, true>), dim3((unsigned)(chains * P)), dim3(4 * D), 0, s, a);
  else
    hipLaunchKernelGGL((gdn_main_kernel<D, T, false>), dim3((unsigned)(chains * P)), dim3(4 * D), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return rec(3);
}

size_t gdn_slot_bytes(int d) { return gdn_slot_floats(d) * sizeof(float); }

hipError_t launch_gdn(const FwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) return launch_gdn_t<128, __bf16>(a, s);
    if (a.d == 64) return launch_gdn_t<64, __bf16>(a, s);
  } else {
    if (a.d == 64) return launch_gdn_t<64, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
