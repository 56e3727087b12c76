// Forward RMSNorm launches for fp16 activations (fp16 or fp32 gamma).
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_fwd_f16(const FwdCall& c) {
  return c.gamma_dtype == kDtF32 ? fwd_gamma_typed<F16, F32, kOutAct>(c)
                                 : fwd_gamma_typed<F16, F16, kOutAct>(c);
}

}  // namespace rmsn
