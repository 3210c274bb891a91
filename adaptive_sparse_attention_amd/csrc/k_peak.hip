// The achievable dense bf16 MFMA rate of the device: every wave issues
// PEAK_CHAINS independent chains of v_mfma_f32_32x32x16_bf16 on register
// operands, with no memory traffic, on enough workgroups to fill every CU.
// It is the rate the attention kernels' MFMA work is compared with, beside the
// published peak.
#include <hip/hip_runtime.h>

#include "../../include/entmax_attn.h"
#include "ea_common.hpp"

namespace {

constexpr int PEAK_CHAINS = 8;

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  ea::bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  ea::floatx16 acc[PEAK_CHAINS];
#pragma unroll
  for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = ea::floatx16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PEAK_CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  // one word per workgroup (keeps the products live)
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

}  // namespace

extern "C" {

double ea_mfma_peak_flop(int workgroups, int iters) {
  if (workgroups < 1 || iters < 1) return 0.0;
  return 32.0 * 32.0 * 16.0 * 2.0 * PEAK_CHAINS * (double)iters * 4.0 * (double)workgroups;
}

ea_status ea_mfma_peak(float* out, int workgroups, int iters, void* stream) {
  if (out == nullptr || workgroups < 1 || iters < 1) return EA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_LAUNCH;
}

}  // extern "C"
