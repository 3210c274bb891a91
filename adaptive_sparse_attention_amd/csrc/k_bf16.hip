// bfloat16 instantiations of the forward and backward kernels.
#include "ea_launch_impl.hpp"

namespace ea {

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, unsigned phases, hipStream_t st) {
  return d == 64 ? launch_fwd_t<BF16, 64>(a, phases, st) : launch_fwd_t<BF16, 128>(a, phases, st);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, unsigned phases, hipStream_t st) {
  return d == 64 ? launch_bwd_t<BF16, 64>(a, phases, st) : launch_bwd_t<BF16, 128>(a, phases, st);
}

}  // namespace ea
