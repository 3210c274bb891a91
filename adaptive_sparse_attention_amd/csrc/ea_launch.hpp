// Host-side launch entry points of the kernels (one translation unit per
// element type). Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>

#include "ea_bwd.hpp"
#include "ea_fwd.hpp"
#include "ea_softmax.hpp"

namespace ea {

// Solver chosen from alpha: Halley for alpha <= 1.5, Newton for
// 1.5 < alpha <= 2, secant above (gist.science Hindi page, section 2).
inline int solver_of(float alpha) {
  if (alpha <= 1.5f) return SV_HALLEY;
  if (alpha <= 2.0f) return SV_NEWTON;
  return SV_SECANT;
}

inline int host_pow_mode(float kappa) {
  if (kappa == 1.f) return PM_K1;
  if (kappa == 2.f) return PM_K2;
  if (kappa == 4.f) return PM_K4;
  return PM_GEN;
}

// phases: bit 0 row max, bit 1 histogram, bit 2 refinement, bit 3 output (forward);
// bit 0 mask transpose, bit 1 rows (delta, dQ), bit 2 columns (dK, dV) (backward)
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, unsigned phases, hipStream_t st);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, unsigned phases, hipStream_t st);
hipError_t launch_bwd_bf16(const BwdArgs& a, int d, unsigned phases, hipStream_t st);
hipError_t launch_bwd_f32(const BwdArgs& a, int d, unsigned phases, hipStream_t st);
hipError_t launch_mask_transpose(const uint32_t* mask, uint32_t* colmask, int BH, int nb, int W, hipStream_t st);
// gathered rows in the backward: the tile rows' mask (and its key-major copy);
// the key counters cleared before the rows kernels count the entries; after
// them, the entries grouped by key
hipError_t launch_gather_prep(const BwdArgs& a, int D, hipStream_t st);
hipError_t launch_gather_buckets(const BwdArgs& a, int D, hipStream_t st);
hipError_t launch_clear_counts(const BwdArgs& a, hipStream_t st);

// softmax comparator: forward; backward over the full visible mask, which it
// writes into `rowmask` (the backward's workspace) first
hipError_t launch_sm_fwd_bf16(const SmArgs& a, int d, hipStream_t st);
hipError_t launch_sm_fwd_f32(const SmArgs& a, int d, hipStream_t st);
hipError_t launch_sm_bwd_bf16(const BwdArgs& a, uint32_t* rowmask, int d, hipStream_t st);
hipError_t launch_sm_bwd_f32(const BwdArgs& a, uint32_t* rowmask, int d, hipStream_t st);

}  // namespace ea
