// Forward RMSNorm launches for bf16 activations (bf16 or fp32 gamma).
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_fwd_bf16(const FwdCall& c) {
  return c.gamma_dtype == kDtF32 ? fwd_gamma_typed<BF16, F32, kOutAct>(c)
                                 : fwd_gamma_typed<BF16, BF16, kOutAct>(c);
}

}  // namespace rmsn
