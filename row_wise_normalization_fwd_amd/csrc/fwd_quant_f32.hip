// Quantised (fp8 e4m3) forward RMSNorm launches for fp32 activations.
#include "fwd_dispatch.hpp"

namespace rmsn {

hipError_t launch_fwd_quant_f32(const FwdCall& c) { return fwd_quant_typed<F32, F32>(c); }

}  // namespace rmsn
