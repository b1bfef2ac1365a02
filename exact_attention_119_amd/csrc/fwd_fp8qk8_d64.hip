// Forward-pass kernels: e4m3 inputs, Q.K^T on the fp8 MFMA, head dim 64.
#include "fwd_kernel.hpp"

namespace attn119 {
template hipError_t launch_fwd_family<64, kInFp8Qk8>(const FwdArgs&, bool, bool, bool, hipStream_t);
}  // namespace attn119
