// Segment summary of the Gated DeltaNet chunked prefill (the kernel is in
// ccq_prefill_gdn_kernels.hpp), in a translation unit of its own for its scheduler setting.
#include "ccq_prefill_gdn_kernels.hpp"

namespace ccq {

hipError_t launch_gdn_summary(const FwdArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * a.H * (a.segments - 1));
  if (a.dtype == 1) {
    if (a.d == 128) {
      hipLaunchKernelGGL((gdn_summary_kernel<128, __bf16>), dim3(grid), dim3(4 * 128), 0, s, a);
      return hipGetLastError();
    }
    if (a.d == 64) {
      hipLaunchKernelGGL((gdn_summary_kernel<64, __bf16>), dim3(grid), dim3(4 * 64), 0, s, a);
      return hipGetLastError();
    }
  } else if (a.d == 64) {
    hipLaunchKernelGGL((gdn_summary_kernel<64, float>), dim3(grid), dim3(4 * 64), 0, s, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
