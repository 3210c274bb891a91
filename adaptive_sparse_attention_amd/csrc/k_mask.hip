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
// gathered rows (words 32 .. 32 + W of their state record). Also each row's
// list length where it was gathered (0 where not), for the bucket fill.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_mask_kernel(const uint32_t* __restrict__ mask, const float* __restrict__ state,
                                                        uint32_t* __restrict__ tmask, uint32_t* __restrict__ gblk,
                                                        uint8_t* __restrict__ rown, int BH, int N, int nb, int W, int D) {
  const int wave = wave_index(threadIdx.x), lane = threadIdx.x & 63;
  const size_t blk = (size_t)blockIdx.x * 4 + wave;   // (bh, I)
  if (blk >= (size_t)BH * nb) return;                  // whole waves
  const int I = (int)(blk % nb);
  const size_t bh = blk / nb;
  const int row = I * BLK + lane;
  const bool valid = row < N;
  const uint32_t* vr = reinterpret_cast<const uint32_t*>(state) + (bh * N + (valid ? row : 0)) * D;
  const uint32_t w0 = vr[0];
  const bool gathered = valid && list_marked(w0);
  const uint64_t mg = __ballot(gathered), mv = __ballot(valid);
  if (valid) rown[bh * N + row] = gathered ? (uint8_t)min(w0 & 0xFFFFu, (uint32_t)LIST_CAP) : (uint8_t)0;
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

// the sum over the 256 threads of the workgroup
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  const uint32_t s = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return s;
}

// With own_prefix set, part holds the blocks' totals and each workgroup adds
// up those before its own (few blocks); else part holds their exclusive sums.
__global__ __launch_bounds__(SCAN_T) void scan_out_kernel(const uint32_t* __restrict__ cnt, size_t n,
                                                          const uint32_t* __restrict__ part, uint32_t* __restrict__ out,
                                                          int own_prefix) {
  __shared__ uint32_t sh[4];
  uint32_t pre;
  if (own_prefix) {
    uint32_t s = 0;
    for (int i = (int)threadIdx.x; i < (int)blockIdx.x; i += SCAN_T) s += part[i];
    pre = block_sum(s, sh);
  } else {
    pre = part[blockIdx.x];
  }
  const size_t base = (size_t)blockIdx.x * SCAN_B + (size_t)threadIdx.x * SCAN_E;
  uint32_t v[SCAN_E];
  uint32_t s = 0;
#pragma unroll
  for (int e = 0; e < SCAN_E; ++e) {
    v[e] = (base + e < n) ? cnt[base + e] : 0u;
    s += v[e];
  }
  const uint32_t incl = block_incl_scan(s, sh);
  uint32_t run = pre + incl - s;
#pragma unroll
  for (int e = 0; e < SCAN_E; ++e) {
    if (base + e <= n) out[base + e] = run;   // out[n] = the total
    run += v[e];
  }
}

// ---------------------------------------------------------------------------
// Entry slots grouped by key, one thread per row: of a row formed from its
// list (n = its list length, 0 for the other rows), the rows gather wrote
// entries 0 .. n; entry i with key k goes to
// bucket[off[k] + rank_i], its place among k's entries as the counting
// atomics handed it out (an order the sums over a bucket do not depend on).
// Entries without a key hold ~0. Slots past n are never read, so they need no
// clearing.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bucket_fill_kernel(const uint8_t* __restrict__ rown,
                                                          const uint32_t* __restrict__ ent_key,
                                                          const uint32_t* __restrict__ ent_rank,
                                                          const uint32_t* __restrict__ off,
                                                          uint32_t* __restrict__ bucket, size_t nrows) {
  static_assert(LIST_CAP % 4 == 0, "a row's entries are read 16 bytes at a time");
  constexpr int NQ = LIST_CAP / 4;
  const size_t row = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= nrows) return;
  const int n = min((int)rown[row], LIST_CAP);
  if (n == 0) return;
  const size_t slot0 = row * LIST_CAP;
  const size_t nslots = nrows * LIST_CAP;
  // (slot0 is a multiple of 4 entries: 16-byte aligned)
  const uint4* kq = reinterpret_cast<const uint4*>(ent_key + slot0);
  const uint4* rq = reinterpret_cast<const uint4*>(ent_rank + slot0);
  uint32_t k[LIST_CAP], rk[LIST_CAP];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    uint4 kv = make_uint4(~0u, ~0u, ~0u, ~0u), rv = make_uint4(0u, 0u, 0u, 0u);
    if (4 * q < n) {
      kv = kq[q];
      rv = rq[q];
    }
    k[4 * q] = kv.x, k[4 * q + 1] = kv.y, k[4 * q + 2] = kv.z, k[4 * q + 3] = kv.w;
    rk[4 * q] = rv.x, rk[4 * q + 1] = rv.y, rk[4 * q + 2] = rv.z, rk[4 * q + 3] = rv.w;
  }
  uint32_t base[LIST_CAP];
#pragma unroll
  for (int i = 0; i < LIST_CAP; ++i) {
    if (i >= n) k[i] = ~0u;   // (read with their group of four, never written)
    base[i] = k[i] != ~0u ? off[k[i]] : 0u;
  }
#pragma unroll
  for (int i = 0; i < LIST_CAP; ++i) {
    if (k[i] == ~0u) continue;
    const size_t pos = (size_t)base[i] + rk[i];
    if (pos < nslots) bucket[pos] = (uint32_t)(slot0 + i);   // (counts from one rows pass never exceed the slots)
  }
}

hipError_t launch_gather_prep(const BwdArgs& a, int D, hipStream_t st) {
  const int BH = a.B * a.H;
  const size_t nblk = (size_t)BH * a.nb;
  hipLaunchKernelGGL(tile_mask_kernel, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st, a.mask, a.state, a.tmask,
                     a.gblk, a.rown, BH, a.N, a.nb, a.W, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mask_transpose(a.tmask, a.colmask, BH, a.nb, a.W, st);
}

hipError_t launch_clear_counts(const BwdArgs& a, hipStream_t st) {
  const size_t nk = (size_t)a.B * (a.H / a.G) * a.N;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1024), dim3(256), 0, st, a.kcnt, nk, 0u);
  return hipGetLastError();
}

hipError_t launch_gather_buckets(const BwdArgs& a, int D, hipStream_t st) {
  const size_t nk = (size_t)a.B * (a.H / a.G) * a.N;
  const int nparts = (int)((nk + 1 + SCAN_B - 1) / SCAN_B);
  // up to 256 blocks (524 288 keys), each workgroup of the last pass sums the
  // totals before its block itself (at most 1 KB read, from L2) instead of a
  // pass between
  const int own = nparts <= 256 ? 1 : 0;
  hipLaunchKernelGGL(scan_sums_kernel, dim3(nparts), dim3(SCAN_T), 0, st, a.kcnt, nk, a.kpart);
  if (!own) hipLaunchKernelGGL(scan_parts_kernel, dim3(1), dim3(SCAN_T), 0, st, a.kpart, nparts);
  hipLaunchKernelGGL(scan_out_kernel, dim3(nparts), dim3(SCAN_T), 0, st, a.kcnt, nk, a.kpart, a.koff, own);
  const size_t nrows = (size_t)a.B * a.H * a.N;
  hipLaunchKernelGGL(bucket_fill_kernel, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, st,
                     a.rown, a.ent_key, a.ent_rank, a.koff, a.bucket, nrows);
  return hipGetLastError();
}

}  // namespace ea
