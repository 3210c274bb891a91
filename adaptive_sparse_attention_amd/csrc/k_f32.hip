// fp32 instantiations of the forward and backward kernels.
#include "ea_launch_impl.hpp"

namespace ea {

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t st) {
  return d == 64 ? launch_fwd_t<F32, 64>(a, st) : launch_fwd_t<F32, 128>(a, st);
}

hipError_t launch_bwd_f32(const BwdArgs& a, int d, hipStream_t st) {
  return d == 64 ? launch_bwd_t<F32, 64>(a, st) : launch_bwd_t<F32, 128>(a, st);
}

}  // namespace ea
