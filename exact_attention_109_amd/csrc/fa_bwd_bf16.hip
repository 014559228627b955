// Attention backward for bf16 inputs: dispatch.
#include "fa_internal.h"

namespace fa {

hipError_t launch_bwd_bf16_valu(const BwdParams& p, hipStream_t stream);

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) { return launch_bwd_bf16_valu(p, stream); }

}  // namespace fa
