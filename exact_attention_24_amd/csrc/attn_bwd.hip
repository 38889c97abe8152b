// Attention backward kernels for gfx950 (recompute-based).
#include "attn_common.h"
#include "attn_kernels.h"

namespace attn {

hipError_t launch_bwd_bf16(const BwdArgs&, int, bool, hipStream_t) { return hipErrorNotSupported; }

}  // namespace attn
