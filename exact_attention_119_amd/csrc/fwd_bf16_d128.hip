// Forward-pass kernels: bf16 inputs, head dim 128.
#include "fwd_kernel.hpp"

namespace attn119 {
template hipError_t launch_fwd_family<128, kInBf16>(const FwdArgs&, bool, bool, bool, hipStream_t);
}  // namespace attn119
