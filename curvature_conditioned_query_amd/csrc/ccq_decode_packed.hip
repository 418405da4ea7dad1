// Decode step of the CCQ read with C as its packed upper triangle (the kernel and its
// description are in ccq_decode_kernel.hpp).
#include "ccq_decode_kernel.hpp"

namespace ccq {

hipError_t launch_decode_packed(const DecodeArgs& a, hipStream_t s) { return launch_decode_dtype<true>(a, s); }

}  // namespace ccq
