// Forward-pass kernels: e4m3 inputs, Q.K^T and P.V both on the f8f6f4 MFMA, head dim 128,
// no positional mask: P rounded to e4m3, or to E2M1 with one E8M0 scale per 32 keys
// (measured variants, see attn119.h ATTN_PV_E4M3 / ATTN_PV_FP4).
#include "fwd_bf16.hpp"

namespace attn119 {
namespace bf16path {
template hipError_t launch<128, true, true, false, kPvE4m3>(const FwdArgs&, bool, int, bool, bool, hipStream_t);
template hipError_t launch<128, true, true, false, kPvFp4>(const FwdArgs&, bool, int, bool, bool, hipStream_t);
}  // namespace bf16path
}  // namespace attn119
