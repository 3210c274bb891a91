// Template launchers shared by the per-dtype translation units.
#pragma once

#include "ea_launch.hpp"

namespace ea {

// Histogram-pass layout per (type, d, 32-bit counters): waves per workgroup
// (two per group of 32 rows) and whether the key tile is double-buffered,
// chosen so the histograms (516 B per row with 16-bit counters, 1028 B with
// 32-bit ones) and the key tile leave room for two or more workgroups per CU
// (160 KiB of LDS) where possible. 32-bit counters are used when a row can
// hold more than 65536 scores (with 16-bit ones a row of 65536 can fill only
// the top bin, whose count then reads 0: the solve takes that as 65536).
template <class E, int D, bool H32> struct InitCfg;
template <> struct InitCfg<BF16, 64, false> { static constexpr int NW = 8; static constexpr bool DB = false; };
template <> struct InitCfg<BF16, 64, true> { static constexpr int NW = 8; static constexpr bool DB = false; };
template <> struct InitCfg<BF16, 128, false> { static constexpr int NW = 4; static constexpr bool DB = false; };
template <> struct InitCfg<BF16, 128, true> { static constexpr int NW = 8; static constexpr bool DB = false; };
template <> struct InitCfg<F32, 64, false> { static constexpr int NW = 4; static constexpr bool DB = false; };
template <> struct InitCfg<F32, 64, true> { static constexpr int NW = 4; static constexpr bool DB = false; };
template <> struct InitCfg<F32, 128, false> { static constexpr int NW = 4; static constexpr bool DB = false; };
template <> struct InitCfg<F32, 128, true> { static constexpr int NW = 4; static constexpr bool DB = false; };

// Tile buffers of the streaming kernels: 2 unless the double-buffered tiles
// would not fit in LDS.
template <class E, int D> struct NBuf { static constexpr int value = (sizeof(typename E::storage) == 4 && D == 128) ? 1 : 2; };

// Row groups of 32 per wave in the row-max pass: two at bf16 (at d = 128 in
// 168 VGPRs, three waves per SIMD, with a few spilled: measured faster than
// one group per wave or two at 176 VGPRs and two waves per SIMD).
template <class E, int D> struct MaxRG { static constexpr int value = (sizeof(typename E::storage) == 2) ? 2 : 1; };

// Row groups of 32 per wave in the list pass (a workgroup takes 128 RG rows,
// which must cover whole groups of the histogram kernel: 64 or 128 rows).
// One: two (each key fragment feeding two products, three waves per SIMD
// instead of four) measured no faster at bf16 d = 64 and slower where the
// windows are shortest.
template <class E, int D> struct ListRG { static constexpr int value = 1; };

template <class E, int D>
hipError_t launch_max(const FwdArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.B * a.H * a.N;
  hipLaunchKernelGGL((fwd_max_init_kernel<E, D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RG = MaxRG<E, D>::value;
  const int grid = a.B * a.H * ((a.nb + 2 * RG - 1) / (2 * RG)) * max_chunks(a.nb);
  hipLaunchKernelGGL((fwd_max_kernel<E, D, NBuf<E, D>::value, RG>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class E, int D, bool H32>
hipError_t launch_init(const FwdArgs& a, hipStream_t st) {
  constexpr int NW = InitCfg<E, D, H32>::NW;
  constexpr int NBLKS = NW / 4;   // 64-row blocks per workgroup
  constexpr bool DB = InitCfg<E, D, H32>::DB;
  const int groups = (a.nb + NBLKS - 1) / NBLKS;
  const dim3 grid(a.B * a.H * groups), block(NW * 64);
  // other histogram sizes than 256 bins per unit: bf16, 16-bit counters
  if constexpr (sizeof(typename E::storage) == 2 && !H32) {
    switch (a.bins) {
      case 32: hipLaunchKernelGGL((fwd_init_kernel<E, D, NW, H32, DB, 32>), grid, block, 0, st, a); return hipGetLastError();
      case 64: hipLaunchKernelGGL((fwd_init_kernel<E, D, NW, H32, DB, 64>), grid, block, 0, st, a); return hipGetLastError();
      case 128: hipLaunchKernelGGL((fwd_init_kernel<E, D, NW, H32, DB, 128>), grid, block, 0, st, a); return hipGetLastError();
      case 512: hipLaunchKernelGGL((fwd_init_kernel<E, D, NW, H32, DB, 512>), grid, block, 0, st, a); return hipGetLastError();
      default: break;
    }
  }
  hipLaunchKernelGGL((fwd_init_kernel<E, D, NW, H32, DB, HIST_BINS>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <class E, int D, int PM, int SV>
hipError_t launch_refine(const FwdArgs& a, hipStream_t st) {
  const int grid = a.B * a.H * ((a.nb + 1) / 2);
  hipLaunchKernelGGL((fwd_refine_kernel<E, D, PM, SV, NBuf<E, D>::value>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class E, int D, int PM>
hipError_t launch_out(const FwdArgs& a, hipStream_t st) {
  const int grid = a.B * a.H * ((a.nb + 1) / 2);
  if (a.state)
    hipLaunchKernelGGL((fwd_out_kernel<E, D, PM, NBuf<E, D>::value, true>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_out_kernel<E, D, PM, NBuf<E, D>::value, false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_fwd_t(const FwdArgs& a, unsigned phases, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (phases & 1u) {
    e = launch_max<E, D>(a, st);
    if (e != hipSuccess) return e;
  }
  if ((phases & 2u) && !a.nohist) {
    // rows whose windows are short first (default mode and histogram size,
    // keys that fit the lists); the histogram kernel takes the groups left
    FwdArgs b = a;
    b.listpass = (!a.plain && a.bins == HIST_BINS && a.N <= LIST_MAX_N) ? 1 : 0;
    if (b.listpass) {
      constexpr int RG = ListRG<E, D>::value;
      const int grid = a.B * a.H * ((a.nb + 2 * RG - 1) / (2 * RG));
      hipLaunchKernelGGL((fwd_list_kernel<E, D, NBuf<E, D>::value, RG>), dim3(grid), dim3(256), 0, st, b);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      // the single rows it flagged
      hipLaunchKernelGGL((fwd_rowhist_kernel<E, D, RG>), dim3(grid), dim3(256), 0, st, b);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    e = (a.N > 65536) ? launch_init<E, D, true>(b, st) : launch_init<E, D, false>(b, st);
    if (e != hipSuccess) return e;
  }
  if (phases & 4u) {
    const int sv = solver_of(a.alpha);
    switch (a.pow_mode) {
      case PM_K2: e = launch_refine<E, D, PM_K2, SV_HALLEY>(a, st); break;
      case PM_K1: e = launch_refine<E, D, PM_K1, SV_NEWTON>(a, st); break;
      case PM_K4: e = launch_refine<E, D, PM_K4, SV_HALLEY>(a, st); break;
      default:
        if (sv == SV_HALLEY) e = launch_refine<E, D, PM_GEN, SV_HALLEY>(a, st);
        else if (sv == SV_NEWTON) e = launch_refine<E, D, PM_GEN, SV_NEWTON>(a, st);
        else e = launch_refine<E, D, PM_GEN, SV_SECANT>(a, st);
    }
    if (e != hipSuccess) return e;
  }
  if (phases & 8u) {
    switch (a.pow_mode) {
      case PM_K2: return launch_out<E, D, PM_K2>(a, st);
      case PM_K1: return launch_out<E, D, PM_K1>(a, st);
      case PM_K4: return launch_out<E, D, PM_K4>(a, st);
      default: return launch_out<E, D, PM_GEN>(a, st);
    }
  }
  return e;
}

template <class E, int D, int PM>
hipError_t launch_bwd_pm(const BwdArgs& a, unsigned phases, hipStream_t st) {
  const int grid = a.B * a.H * ((a.nb + 1) / 2);
  constexpr int NB = NBuf<E, D>::value;
  if (phases & 2u) {
    if constexpr (PM != PM_SOFTMAX) {
      if (a.gather) {
        // rows the forward gathered: one workgroup per 128 rows
        hipError_t e0 = launch_clear_counts(a, st);
        if (e0 != hipSuccess) return e0;
        const int grid_g = a.B * a.H * ((a.N + 127) / 128);
        hipLaunchKernelGGL((bwd_rows_gather_kernel<E, D, PM>), dim3(grid_g), dim3(256), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
    hipLaunchKernelGGL((bwd_rows_kernel<E, D, PM, NB>), dim3(grid), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 4u) {
    if (PM != PM_SOFTMAX && a.gather) {
      // the gathered rows' entries, grouped and summed by key
      hipError_t e = launch_gather_buckets(a, D, st);
      if (e != hipSuccess) return e;
      const size_t nk = (size_t)a.B * (a.H / a.G) * a.N;
      // the workgroups that sum the long keys first, then one per 16 keys
      hipLaunchKernelGGL((bwd_kv_gather_kernel<E, D>), dim3((unsigned)(kv_heavy_blocks(nk) + (nk + 15) / 16)), dim3(256),
                         0, st, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    // one workgroup per key/value head and pair of key blocks
    const int grid_kv = a.B * (a.H / a.G) * ((a.nb + 1) / 2);
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, PM, NB>), dim3(grid_kv), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <class E, int D>
hipError_t launch_bwd_t(const BwdArgs& a, unsigned phases, hipStream_t st) {
  if (phases & 1u) {
    hipError_t e = a.gather ? launch_gather_prep(a, D, st) : launch_mask_transpose(a.mask, a.colmask, a.B * a.H, a.nb, a.W, st);
    if (e != hipSuccess) return e;
  }
  switch (host_pow_mode(a.kappa)) {
    case PM_K2: return launch_bwd_pm<E, D, PM_K2>(a, phases, st);
    case PM_K1: return launch_bwd_pm<E, D, PM_K1>(a, phases, st);
    case PM_K4: return launch_bwd_pm<E, D, PM_K4>(a, phases, st);
    default: return launch_bwd_pm<E, D, PM_GEN>(a, phases, st);
  }
}

template <class E, int D>
hipError_t launch_sm_fwd_t(const SmArgs& a, hipStream_t st) {
  const int grid = a.B * a.H * ((a.nb + 1) / 2);
  hipLaunchKernelGGL((sm_fwd_kernel<E, D, NBuf<E, D>::value>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_sm_bwd_t(const BwdArgs& a, uint32_t* rowmask, hipStream_t st) {
  const size_t words = (size_t)a.B * a.H * a.nb * a.W;
  hipLaunchKernelGGL(sm_fill_mask_kernel<0>, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st, rowmask,
                     a.B * a.H, a.nb, a.W, a.causal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_mask_transpose(rowmask, a.colmask, a.B * a.H, a.nb, a.W, st);
  if (e != hipSuccess) return e;
  return launch_bwd_pm<E, D, PM_SOFTMAX>(a, 6u, st);
}

}  // namespace ea
