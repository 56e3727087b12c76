// LayerNorm forward launches for bf16 activations (bf16 or fp32 gamma and beta).
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_ln_fwd_bf16(const FwdCall& c) {
  return c.gamma_dtype == kDtF32 ? ln_fwd_typed<BF16, F32>(c) : ln_fwd_typed<BF16, BF16>(c);
}

}  // namespace rmsn
