// FlashAttention forward pass with block-scaled fp8 (E4M3FN) inputs.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

hipError_t launch_fwd_fp8(const FwdArgs&) { return hipErrorNotSupported; }

}  // namespace fa
