// Forward-pass kernels: e4m3 inputs, Q.K^T on the e4m3 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4),
// P.V on the fp16 MFMA, head dim 128 (the software-pipelined kernel).
#include "fwd_bf16.hpp"

namespace attn119 {
namespace bf16path {
template hipError_t launch<128, true, true, false, 0>(const FwdArgs&, bool, int, bool, bool, hipStream_t);
}  // namespace bf16path
}  // namespace attn119
