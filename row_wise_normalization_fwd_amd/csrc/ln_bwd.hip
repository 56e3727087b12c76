// Backward LayerNorm launches for every activation type.
#include "bwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_ln_bwd(const BwdCall& c) {
  switch (c.x_dtype) {
    case kDtF32:
      return bwd_typed<F32, F32, false, true>(c);
    case kDtF16:
      return c.gamma_dtype == kDtF32 ? bwd_typed<F16, F32, false, true>(c)
                                     : bwd_typed<F16, F16, false, true>(c);
    default:
      return c.gamma_dtype == kDtF32 ? bwd_typed<BF16, F32, false, true>(c)
                                     : bwd_typed<BF16, BF16, false, true>(c);
  }
}

}  // namespace rmsn
