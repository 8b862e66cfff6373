// attn_fwd_fp8.hip -- fp8 forward kernel (not yet implemented).
#include "attn_kernels.hpp"
namespace attn {
hipError_t launch_fwd_fp8(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
