// Mask and bookkeeping kernels of the backward: the key-major copy of the
// block mask, and, for rows the forward formed from their support lists, the
// mask of the remaining rows and the grouping of the list entries by key.
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

// ---------------------------------------------------------------------------
// Block mask of the rows that take the tile path, one wave per 64-row query
// block: the final mask when none of the block's rows was gathered, nothing
// when all were, else the mask the forward stored after the list of its
// gathered rows (words 32 .. 32 + W of their state record).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_mask_kernel(const uint32_t* __restrict__ mask, const float* __restrict__ state,
                                                        uint32_t* __restrict__ tmask, uint32_t* __restrict__ gblk, int BH,
                                                        int N, int nb, int W, int D) {
  const int wave = wave_index(threadIdx.x), lane = threadIdx.x & 63;
  const size_t blk = (size_t)blockIdx.x * 4 + wave;   // (bh, I)
  if (blk >= (size_t)BH * nb) return;                  // whole waves
  const int I = (int)(blk % nb);
  const size_t bh = blk / nb;
  const int row = I * BLK + lane;
  const bool valid = row < N;
  const uint32_t* vr = reinterpret_cast<const uint32_t*>(state) + (bh * N + (valid ? row : 0)) * D;
  const bool gathered = valid && list_marked(vr[0]);
  const uint64_t mg = __ballot(gathered), mv = __ballot(valid);
  const uint32_t* src = mask + blk * W;
  if (mg != 0 && mg != mv)
    src = reinterpret_cast<const uint32_t*>(state) + (bh * N + (size_t)I * BLK + __builtin_ctzll(mg)) * D + 32;
  for (int w = lane; w < W; w += 64) tmask[blk * W + w] = (mg != 0 && mg == mv) ? 0u : src[w];
  if (lane == 0) gblk[blk] = mg != 0 ? 1u : 0u;
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---------------------------------------------------------------------------
// Exclusive prefix sums of the per-key entry counts (three passes over
// blocks of SCAN_B counts): out[k] = sum of cnt[0 .. k), out[n] = total.
// ---------------------------------------------------------------------------
constexpr int SCAN_T = 256, SCAN_E = 8, SCAN_B = SCAN_T * SCAN_E;

// inclusive prefix sum over the 256 threads of the workgroup
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* sh) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; ++w) add += sh[w];
  __syncthreads();
  return v + add;
}

__global__ __launch_bounds__(SCAN_T) void scan_sums_kernel(const uint32_t* __restrict__ cnt, size_t n,
                                                           uint32_t* __restrict__ part) {
  __shared__ uint32_t sh[4];
  const size_t base = (size_t)blockIdx.x * SCAN_B + (size_t)threadIdx.x * SCAN_E;
  uint32_t s = 0;
#pragma unroll
  for (int e = 0; e < SCAN_E; ++e) s += (base + e < n) ? cnt[base + e] : 0u;
  const uint32_t incl = block_incl_scan(s, sh);
  if (threadIdx.x == SCAN_T - 1) part[blockIdx.x] = incl;
}

// one workgroup: exclusive prefix sums of the block totals, in place
__global__ __launch_bounds__(SCAN_T) void scan_parts_kernel(uint32_t* __restrict__ part, int nparts) {
  __shared__ uint32_t sh[4];
  __shared__ uint32_t tot;
  uint32_t carry = 0;
  for (int b0 = 0; b0 < nparts; b0 += SCAN_T) {
    const int i = b0 + (int)threadIdx.x;
    const uint32_t v = i < nparts ? part[i] : 0u;
    const uint32_t incl = block_incl_scan(v, sh);
    if (i < nparts) part[i] = carry + incl - v;
    if (threadIdx.x == SCAN_T - 1) tot = incl;
    __syncthreads();
    carry += tot;
    __syncthreads();
  }
}

__global__ __launch_bounds__(SCAN_T) void scan_out_kernel(const uint32_t* __restrict__ cnt, size_t n,
                                                          const uint32_t* __restrict__ part, uint32_t* __restrict__ out) {
  __shared__ uint32_t sh[4];
  const size_t base = (size_t)blockIdx.x * SCAN_B + (size_t)threadIdx.x * SCAN_E;
  uint32_t v[SCAN_E];
  uint32_t s = 0;
#pragma unroll
  for (int e = 0; e < SCAN_E; ++e) {
    v[e] = (base + e < n) ? cnt[base + e] : 0u;
    s += v[e];
  }
  const uint32_t incl = block_incl_scan(s, sh);
  uint32_t run = part[blockIdx.x] + incl - s;
#pragma unroll
  for (int e = 0; e < SCAN_E; ++e) {
    if (base + e <= n) out[base + e] = run;   // out[n] = the total
    run += v[e];
  }
}

// ---------------------------------------------------------------------------
// Entry slots grouped by key, one thread per slot: slot s with key k goes to
// bucket[off[k] + rank[s]], its place among k's entries as the counting
// atomics handed it out (an order the sums over a bucket do not depend on).
// Slots without an entry hold key ~0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bucket_fill_kernel(const uint32_t* __restrict__ ent_key,
                                                          const uint32_t* __restrict__ ent_rank,
                                                          const uint32_t* __restrict__ off,
                                                          uint32_t* __restrict__ bucket, size_t nslots) {
  const size_t slot = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= nslots) return;
  const uint32_t k = ent_key[slot];
  if (k == 0xFFFFFFFFu) return;
  const size_t pos = (size_t)off[k] + ent_rank[slot];
  if (pos < nslots) bucket[pos] = (uint32_t)slot;   // (counts from one rows pass never exceed the slots)
}

hipError_t launch_gather_prep(const BwdArgs& a, int D, hipStream_t st) {
  const int BH = a.B * a.H;
  const size_t nblk = (size_t)BH * a.nb;
  hipLaunchKernelGGL(tile_mask_kernel, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st, a.mask, a.state, a.tmask,
                     a.gblk, BH, a.N, a.nb, a.W, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mask_transpose(a.tmask, a.colmask, BH, a.nb, a.W, st);
}

hipError_t launch_clear_counts(const BwdArgs& a, hipStream_t st) {
  const size_t nk = (size_t)a.B * (a.H / a.G) * a.N;
  const size_t nslots = (size_t)a.B * a.H * a.N * LIST_CAP;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1024), dim3(256), 0, st, a.kcnt, nk, 0u);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(2048), dim3(256), 0, st, a.ent_key, nslots, 0xFFFFFFFFu);
  return hipGetLastError();
}

hipError_t launch_gather_buckets(const BwdArgs& a, int D, hipStream_t st) {
  const size_t nk = (size_t)a.B * (a.H / a.G) * a.N;
  const int nparts = (int)((nk + 1 + SCAN_B - 1) / SCAN_B);
  hipLaunchKernelGGL(scan_sums_kernel, dim3(nparts), dim3(SCAN_T), 0, st, a.kcnt, nk, a.kpart);
  hipLaunchKernelGGL(scan_parts_kernel, dim3(1), dim3(SCAN_T), 0, st, a.kpart, nparts);
  hipLaunchKernelGGL(scan_out_kernel, dim3(nparts), dim3(SCAN_T), 0, st, a.kcnt, nk, a.kpart, a.koff);
  const size_t nslots = (size_t)a.B * a.H * a.N * LIST_CAP;
  hipLaunchKernelGGL(bucket_fill_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, st, a.ent_key, a.ent_rank,
                     a.koff, a.bucket, nslots);
  return hipGetLastError();
}

}  // namespace ea
