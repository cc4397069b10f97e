// FP8 E4M3 forward kernel for gfx950 (placeholder until the kernel lands).
#include "attn_internal.h"

namespace mi355attn {

hipError_t run_fwd_fp8(const Fp8FwdParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mi355attn
