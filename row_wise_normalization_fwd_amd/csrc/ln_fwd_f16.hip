// LayerNorm forward launches for f16 activations (f16 or fp32 gamma and beta).
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_ln_fwd_f16(const FwdCall& c) {
  return c.gamma_dtype == kDtF32 ? ln_fwd_typed<F16, F32>(c) : ln_fwd_typed<F16, F16>(c);
}

}  // namespace rmsn
