// Forward-pass kernels: bf16 inputs, head dim 128 (the software-pipelined kernel).
#include "fwd_bf16.hpp"

namespace attn119 {
namespace bf16path {
template hipError_t launch<128, false, false, false, 0>(const FwdArgs&, bool, int, bool, bool, hipStream_t);
}  // namespace bf16path
}  // namespace attn119
