// Quantised (fp8 e4m3) forward RMSNorm launches for f16 activations (f16 or
// fp32 gamma).
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_fwd_quant_f16(const FwdCall& c) {
  return c.gamma_dtype == kDtF32 ? fwd_quant_typed<F16, F32>(c) : fwd_quant_typed<F16, F16>(c);
}

}  // namespace rmsn
