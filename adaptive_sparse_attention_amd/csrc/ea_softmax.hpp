// Dense softmax attention on the same tile pipeline: the comparator the
// entmax kernels are measured against (the pages set alpha-entmax against
// softmax kernels of the FlashAttention kind: gist.science German page,
// section 1 "Problemstellung", and section 4 "Ergebnisse").
//
//  sm_fwd : one pass per query block over every visible key block with the
//           online softmax: running row max m of x = s log2(e)/sqrt(d),
//           running sum l of 2^(x - m), O rescaled by 2^(m_old - m_new) when
//           the max grows; writes O = sum p v / l, the base-2 log-sum-exp
//           lse2 = m + log2(l) per row and, on request, O in fp32 (the
//           backward's delta = dO . O).
//  The backward is the entmax backward with p = u = 2^(x - lse2)
//  (PM_SOFTMAX) over the full visible mask (sm_fill_mask).
#pragma once

#include "ea_common.hpp"

namespace ea {

struct SmArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse2;       // [B,H,N]
  float* o32;        // optional [B,H,N,D]
  int B, H, N, nb;
  int G;             // query heads per key/value head
  Lay lq, lkv;       // strides of q, o and of k, v
  int causal;
  float c;           // log2(e) / sqrt(d)
};

template <class E, int D, int NBUF>
__global__ __launch_bounds__(256) void sm_fwd_kernel(SmArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = 256, NBLKS = 2;
  constexpr int LDK = Ld<E, D>::value;
  constexpr bool TR = E::TR_READ;
  constexpr int LDV = TR ? LDK : Ld<E, BLK>::value;
  __shared__ __attribute__((aligned(16))) S ktile[NBUF][BLK * LDK];
  __shared__ __attribute__((aligned(16))) S vtile[NBUF][TR ? BLK * LDK : D * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid), h = lane >> 5, l32 = lane & 31;
  const int ngroups = (a.nb + NBLKS - 1) / NBLKS;
  const int wg = xcd_remap(blockIdx.x, a.B * a.H * ngroups);
  const int bh = wg / ngroups;
  const int grp = ngroups - 1 - (wg % ngroups);   // longest rows first when causal
  const int blk0 = grp * NBLKS;
  const int myblk = blk0 + (wave >> 1);
  const int qrow = myblk * BLK + (wave & 1) * 32 + l32;
  const bool qvalid = qrow < a.N;
  const bool blk_valid = myblk < a.nb;

  const S* Q = reinterpret_cast<const S*>(a.q) + a.lq.head(bh, a.H);
  const S* K = reinterpret_cast<const S*>(a.k) + a.lkv.head(bh / a.G, a.H / a.G);
  const S* V = reinterpret_cast<const S*>(a.v) + a.lkv.head(bh / a.G, a.H / a.G);
  typename E::frag bq[D / E::KPI];
  load_row_frags<E, D>(bq, Q + (size_t)qrow * a.lq.sn, qvalid, h);

  const float c = a.c;
  float m = -INFINITY, l = 0.f;
  floatx16 acc_o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc_o[db] = floatx16{};
  const int tr_off = tr_lane_off(lane, LDV);

  const int jmax = a.causal ? min(blk0 + NBLKS - 1, a.nb - 1) : a.nb - 1;
  TileIO<E, D, NTHR> iok, iov;
  iok.load(K, jmax * BLK, a.N, tid, a.lkv.sn);
  iov.load(V, jmax * BLK, a.N, tid, a.lkv.sn);
  wait_vmem();
  iok.template store_rows<LDK>(ktile[0], tid);
  if constexpr (TR) iov.template store_rows<LDV>(vtile[0], tid);
  else iov.template store_trans<LDV>(vtile[0], tid);
  __syncthreads();
  int buf = 0;
  for (int J = jmax; J >= 0; --J) {
    if (J > 0) {
      iok.load(K, (J - 1) * BLK, a.N, tid, a.lkv.sn);
      iov.load(V, (J - 1) * BLK, a.N, tid, a.lkv.sn);
    }
    if (blk_valid && (!a.causal || J <= myblk)) {
      floatx16 acc[2];
      tile_x_frags<E, D, LDK>(acc, ktile[buf], bq, l32, h);
      if (J * BLK + BLK > a.N || (a.causal && J == myblk)) mask_keys(acc, J * BLK, a.N, a.causal, qrow, h);
      // the first tile a row visits holds a visible key (its own block, or
      // a full block), so m is finite from then on. The reference point m
      // moves only when the tile max exceeds it by more than RESCALE (log2
      // units): p = 2^(x - m) then stays at most 2^RESCALE, and O and l are
      // rescaled on few tiles; O / l and m + log2(l) do not depend on m.
      constexpr float RESCALE = 8.f;
      const float tm = pair_max(tile_max(acc) * c);
      const bool grow = tm > m + RESCALE;   // always on the first tile (m = -inf)
      if (__ballot(grow) != 0) {
        const float mn = grow ? tm : m;
        const float scale = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first tile, 1 where m stays
        m = mn;
        l *= scale;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[db][r] *= scale;
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        floatx16 pv;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pv[r] = __builtin_amdgcn_exp2f(fmaf(acc[kh][r], c, -m));
          l += pv[r];
        }
#pragma unroll
        for (int st = 0; st < E::ACC_KSTEPS; ++st) {
          const typename E::frag bp = E::from_acc(pv, st);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            typename E::frag av;
            if constexpr (TR) av = E::ld_tr(vtile[buf] + tr_off + (32 * kh + 16 * st) * LDV + 32 * db, LDV);
            else av = E::ld_kacc(vtile[buf] + (32 * db + sigma32(l32)) * LDV + 32 * kh, st, h);
            acc_o[db] = E::mma(av, bp, acc_o[db]);
          }
        }
      }
    }
    wait_vmem();
    if (J > 0) {
      if (NBUF == 1) __syncthreads();
      iok.template store_rows<LDK>(ktile[NBUF - 1 - buf], tid);
      if constexpr (TR) iov.template store_rows<LDV>(vtile[NBUF - 1 - buf], tid);
      else iov.template store_trans<LDV>(vtile[NBUF - 1 - buf], tid);
      __syncthreads();
      buf = NBUF - 1 - buf;
    }
  }

  l = pair_sum(l);
  const float rinv = l > 0.f ? 1.f / l : 0.f;
  if (qvalid) {
    if (h == 0) a.lse2[(size_t)bh * a.N + qrow] = m + __builtin_amdgcn_logf(l);
    S* orow = reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) + (size_t)qrow * a.lq.sn;
    float* o32row = a.o32 ? a.o32 + ((size_t)bh * a.N + qrow) * D : nullptr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int col = 32 * db + 16 * half + 8 * h;
        float ov[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = acc_o[db][8 * half + e] * rinv;
        if constexpr (sizeof(S) == 2) {
          uint32_t wv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            wv[e] = (uint32_t)E::from_f(ov[2 * e]) | ((uint32_t)E::from_f(ov[2 * e + 1]) << 16);
          *reinterpret_cast<uint4*>(orow + col) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        } else {
          *reinterpret_cast<float4*>(orow + col) = make_float4(ov[0], ov[1], ov[2], ov[3]);
          *reinterpret_cast<float4*>(orow + col + 4) = make_float4(ov[4], ov[5], ov[6], ov[7]);
        }
        if (o32row) {
          *reinterpret_cast<float4*>(o32row + col) = make_float4(ov[0], ov[1], ov[2], ov[3]);
          *reinterpret_cast<float4*>(o32row + col + 4) = make_float4(ov[4], ov[5], ov[6], ov[7]);
        }
      }
  }
}

// Row-major mask of every visible key block: J <= I (causal) or J < nb.
template <int U = 0>   // a template, so every translation unit shares one instance
__global__ __launch_bounds__(256) void sm_fill_mask_kernel(uint32_t* mask, int BH, int nb, int W, int causal) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)BH * nb * W) return;
  const int w = (int)(idx % W);
  const int I = (int)((idx / W) % nb);
  const int last = (causal ? I : nb - 1) - 32 * w;
  mask[idx] = last >= 31 ? 0xFFFFFFFFu : (last >= 0 ? (2u << last) - 1u : 0u);
}

}  // namespace ea
