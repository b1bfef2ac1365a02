// Forward-pass kernels: e4m3 inputs with block scales, head dim 64 (the software-pipelined
// kernel; Q.K^T on the bf16 MFMA from exactly widened codes, P.V on the fp16 MFMA).
#include "fwd_bf16.hpp"

namespace attn119 {
namespace bf16path {
template hipError_t launch<64, true, false, false, 0>(const FwdArgs&, bool, int, bool, bool, hipStream_t);
}  // namespace bf16path
}  // namespace attn119
