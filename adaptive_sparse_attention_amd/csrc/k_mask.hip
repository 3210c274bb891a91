// Key-major copy of the block mask, used by the column-parallel backward.
#include "ea_launch.hpp"

namespace ea {

// ---------------------------------------------------------------------------
// key-major mask: colmask[(bh, J), w'] bit t  <=>  mask[(bh, I = 32 w' + t), J]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mask_transpose_kernel(const uint32_t* __restrict__ mask, uint32_t* __restrict__ colmask,
                                      int BH, int nb, int W) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)BH * nb * W;
  if (idx >= total) return;
  const int w2 = (int)(idx % W);
  const int J = (int)((idx / W) % nb);
  const size_t bh = idx / ((size_t)W * nb);
  uint32_t out = 0;
  for (int t = 0; t < 32; ++t) {
    const int I = 32 * w2 + t;
    if (I < nb) out |= ((mask[(bh * nb + I) * W + (J >> 5)] >> (J & 31)) & 1u) << t;
  }
  colmask[(bh * nb + J) * W + w2] = out;
}

hipError_t launch_mask_transpose(const uint32_t* mask, uint32_t* colmask, int BH, int nb, int W, hipStream_t st) {
  const size_t total = (size_t)BH * nb * W;
  const int threads = 256;
  const int blocks = (int)((total + threads - 1) / threads);
  hipLaunchKernelGGL(mask_transpose_kernel, dim3(blocks), dim3(threads), 0, st, mask, colmask, BH, nb, W);
  return hipGetLastError();
}

}  // namespace ea
