// Forward-pass kernels that also count rescale events per query row (bf16 inputs, head
// dim 128): the instantiation behind attn_fwd_rescale_counts.
#include "fwd_bf16.hpp"

namespace attn119 {
namespace bf16path {
template hipError_t launch<128, false, false, true, 0>(const FwdArgs&, bool, int, bool, bool, hipStream_t);
}  // namespace bf16path
}  // namespace attn119
