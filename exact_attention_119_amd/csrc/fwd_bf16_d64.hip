// Forward-pass kernels: bf16 inputs, head dim 64.
#include "fwd_kernel.hpp"

namespace attn119 {
template hipError_t launch_fwd_family<64, kInBf16>(const FwdArgs&, bool, bool, bool, hipStream_t);
}  // namespace attn119
