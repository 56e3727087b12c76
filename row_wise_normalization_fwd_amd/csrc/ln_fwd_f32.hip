// LayerNorm forward launches for fp32 activations (fp32 gamma and beta).
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_ln_fwd_f32(const FwdCall& c) { return ln_fwd_typed<F32, F32>(c); }

}  // namespace rmsn
