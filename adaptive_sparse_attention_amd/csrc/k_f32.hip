// fp32 instantiations of the forward and backward kernels.
#include "ea_launch_impl.hpp"

namespace ea {

hipError_t launch_fwd_f32(const FwdArgs& a, int d, unsigned phases, hipStream_t st) {
  return d == 64 ? launch_fwd_t<F32, 64>(a, phases, st) : launch_fwd_t<F32, 128>(a, phases, st);
}

hipError_t launch_bwd_f32(const BwdArgs& a, int d, unsigned phases, hipStream_t st) {
  return d == 64 ? launch_bwd_t<F32, 64>(a, phases, st) : launch_bwd_t<F32, 128>(a, phases, st);
}

hipError_t launch_sm_fwd_f32(const SmArgs& a, int d, hipStream_t st) {
  return d == 64 ? launch_sm_fwd_t<F32, 64>(a, st) : launch_sm_fwd_t<F32, 128>(a, st);
}

hipError_t launch_sm_bwd_f32(const BwdArgs& a, uint32_t* rowmask, int d, hipStream_t st) {
  return d == 64 ? launch_sm_bwd_t<F32, 64>(a, rowmask, st) : launch_sm_bwd_t<F32, 128>(a, rowmask, st);
}

}  // namespace ea
