// Quantised (fp8 e4m3) forward RMSNorm launches for bf16 activations (bf16 or
// fp32 gamma).
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_fwd_quant_bf16(const FwdCall& c) {
  return c.gamma_dtype == kDtF32 ? fwd_quant_typed<BF16, F32>(c) : fwd_quant_typed<BF16, BF16>(c);
}

}  // namespace rmsn
