// Forward RMSNorm launches for fp32 activations (fp32 gamma).
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_fwd_f32(const FwdCall& c) { return fwd_gamma_typed<F32, F32, kOutAct>(c); }

}  // namespace rmsn
