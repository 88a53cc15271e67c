// Backward ring step (placeholder until the MFMA kernels land).
#include "ra_internal.h"

namespace ra {
hipError_t launch_bwd_bf16(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ra
