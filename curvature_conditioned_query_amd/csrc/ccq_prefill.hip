// placeholder: replaced by the chunked prefill kernels
#include "ccq_internal.hpp"
namespace ccq {
size_t fwd_slot_bytes(int d) { return (size_t)(2 * d * d + 2 * d + 4) * sizeof(float); }
hipError_t launch_fwd(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ccq
