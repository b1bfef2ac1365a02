// Forward-pass kernels: e4m3 inputs, exact bf16 Q.K^T, head dim 128.
#include "fwd_kernel.hpp"

namespace attn119 {
template hipError_t launch_fwd_family<128, kInFp8>(const FwdArgs&, bool, bool, bool, hipStream_t);
}  // namespace attn119
