// Segment summary of the Gated DeltaNet chunked prefill (the kernel is in
// ccq_prefill_gdn_kernels.hpp), in a translation unit of its own for its scheduler setting.
#include "ccq_prefill_gdn_kernels.hpp"

namespace ccq {

template <int D, typename T>
static void launch_gdn_summary_t(const FwdArgs& a, hipStream_t s) {
  const int nS = a.B * a.H * (a.segments - 1);
  const int Wc = summary_c_groups(nS);
  if (Wc > 0)
    hipLaunchKernelGGL((gdn_summary_split_kernel<D, T>), dim3((unsigned)(nS + Wc)), dim3(4 * D), 0, s, a);
  else
    hipLaunchKernelGGL((gdn_summary_kernel<D, T>), dim3((unsigned)nS), dim3(4 * D), 0, s, a);
}

hipError_t launch_gdn_summary(const FwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) {
      launch_gdn_summary_t<128, __bf16>(a, s);
      return hipGetLastError();
    }
    if (a.d == 64) {
      launch_gdn_summary_t<64, __bf16>(a, s);
      return hipGetLastError();
    }
  } else if (a.d == 64) {
    launch_gdn_summary_t<64, float>(a, s);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
