// Backward kernels (placeholder until the gradient kernels land).
#include "kernels.h"

namespace nomas {
hipError_t launch_attn_bwd(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace nomas
