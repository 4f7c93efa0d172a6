// Backward attention (bf16 storage): kernels under construction.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t launch_bwd_bf16(const BwdParams&, int, bool, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa
