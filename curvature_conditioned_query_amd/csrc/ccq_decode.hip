// Decode step of the CCQ read with the full second-moment matrix C (the kernel and its
// description are in ccq_decode_kernel.hpp), and the entry that dispatches on the packed flag.
#include "ccq_decode_kernel.hpp"

namespace ccq {

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.flags & kFlagPackedCov) return launch_decode_packed(a, s);
  return launch_decode_dtype<false>(a, s);
}

}  // namespace ccq
