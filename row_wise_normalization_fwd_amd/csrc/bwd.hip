// Backward RMSNorm launches (plain and fused-add) for every activation type.
#include "bwd_dispatch.hpp"

namespace rmsn {

template <class T, class G>
hipError_t bwd_res(const BwdCall& c) {
  return c.dres ? bwd_typed<T, G, true, false>(c) : bwd_typed<T, G, false, false>(c);
}

hipError_t launch_bwd(const BwdCall& c) {
  switch (c.x_dtype) {
    case kDtF32:
      return bwd_res<F32, F32>(c);
    case kDtF16:
      return c.gamma_dtype == kDtF32 ? bwd_res<F16, F32>(c) : bwd_res<F16, F16>(c);
    default:
      return c.gamma_dtype == kDtF32 ? bwd_res<BF16, F32>(c) : bwd_res<BF16, BF16>(c);
  }
}

}  // namespace rmsn
