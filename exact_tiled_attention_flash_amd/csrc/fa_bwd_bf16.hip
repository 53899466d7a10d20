// fa_bwd_bf16.hip -- placeholder until the backward kernels land.
#include "fa_kernels.h"
namespace fa {
hipError_t launch_bwd_bf16(const BwdArgs&, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fa
