// Backward kernels of alpha-entmax attention.
//
// With x = z - tau on the support, p = x^kappa and u = x^(kappa-1), the
// gradient of a score is dS = u (dP - delta), dP = dO . v, delta =
// sum(u dP) / sum(u) per query row (derivative of the entmax map; the pages
// only state that the backward forms gradients over the non-zero blocks alone,
// AdaSplash-2 summary, gist.science German page, section 4 "Ergebnisse").
//
//  bwd_rows : row-parallel over query blocks, walking the block mask. delta
//             is dO . vbar when the forward's state holds vbar = sum(u v) /
//             sum(u) (sum(u dP) = dO . sum(u v)); otherwise sweep 1 accumulates
//             sum(u) and sum(u dP). It writes delta, then sweep 2 forms dS
//             and accumulates dQ = dS K / sqrt(d).
//  mask_transpose : key-major copy of the block mask.
//  bwd_dkdv : column-parallel over key blocks, walking the key-major mask:
//             dV = P^T dO and dK = dS^T Q / sqrt(d).
// Only blocks whose bit is set are loaded or multiplied (find-first-set walk;
// gist.science Hindi page, section 2, efficient traversal).
#pragma once

#include "ea_common.hpp"

namespace ea {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* tau;
  const uint32_t* mask;
  // optional: the forward's state, one record of D fp32 words per row: vbar
  // (delta = dO . vbar) for rows formed by tiles, the support list for rows
  // formed by gathering (see fwd_out_kernel)
  const float* state;
  void* dq;
  void* dk;
  void* dv;
  float* delta;        // workspace [B,H,N]
  uint32_t* colmask;   // workspace [B,H,nb,W]
  // Rows the forward formed from their support list keep that list in their
  // state record (with the block mask of their block's other rows); with
  // `gather` set, those rows take the gather path here and the tile kernels
  // run over the other rows' mask alone. Workspace:
  int gather;          // state given and N <= LIST_MAX_N
  uint32_t* tmask;     // [B,H,nb,W]: block mask of the rows taking the tile path
  uint32_t* gblk;      // [B,H,nb]: nonzero where the 64-row block has gathered rows
  uint8_t* rown;       // [B,H,N]: entries in the row's list where it was gathered, else 0
  uint32_t* ent_key;   // [B,H,N,LIST_CAP]: key id (b, kv head, key) of each entry, or ~0 (the row's first n only)
  float* ent_ds;       // [B,H,N,LIST_CAP]: dS of each entry
  float* ent_p;        // [B,H,N,LIST_CAP]: p of each entry
  uint32_t* kcnt;      // [B*Hkv*N]: entries per key
  uint32_t* koff;      // [B*Hkv*N + 1]: their exclusive prefix sums
  uint32_t* ent_rank;  // [B,H,N,LIST_CAP]: an entry's place among its key's entries
  uint32_t* kpart;     // [scan blocks]: prefix-sum partials
  uint32_t* bucket;    // [B*H*N*LIST_CAP]: entry slots grouped by key
  float* part;         // [B*Hkv*N, 2, D]: gathered sums of dS q (dK before 1/sqrt(d)) and p dO (dV)
  int B, H, N, nb, W;
  int G;               // query heads per key/value head (grouped-query attention; 1 = one each)
  Lay lq, lkv;         // strides of q, dout, dq and of k, v, dk, dv
  int causal;
  float kappa;
  float zscale;        // (alpha - 1) / sqrt(d)
  float rscale;        // 1 / sqrt(d)
};

// Walk of the union of two blocks' mask words held in LDS (wave-uniform).
struct UnionIterB {
  const uint32_t* m0;
  const uint32_t* m1;
  int use1, W, w;
  uint32_t bits;
  __device__ __forceinline__ void init(const uint32_t* a0, const uint32_t* a1, bool u1, int nw) {
    m0 = a0; m1 = a1; use1 = u1; W = nw; w = -1; bits = 0;
  }
  __device__ __forceinline__ int next() {
    while (bits == 0) {
      if (++w >= W) return -1;
      uint32_t x = m0[w] | (use1 ? m1[w] : 0u);
      bits = __builtin_amdgcn_readfirstlane(x);
    }
    const int t = __builtin_ctz(bits);
    bits &= bits - 1;
    return w * 32 + t;
  }
};

template <class E, int D>
__device__ __forceinline__ void store_row_acc(typename E::storage* rowp, const floatx16* acc, float scale, int h) {
  using S = typename E::storage;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      S* dst = rowp + 32 * db + 16 * half + 8 * h;
      if constexpr (sizeof(S) == 2) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wv[e] = (uint32_t)E::from_f(acc[db][8 * half + 2 * e] * scale) |
                  ((uint32_t)E::from_f(acc[db][8 * half + 2 * e + 1] * scale) << 16);
        *reinterpret_cast<uint4*>(dst) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      } else {
        *reinterpret_cast<float4*>(dst) =
            make_float4(acc[db][8 * half + 0] * scale, acc[db][8 * half + 1] * scale,
                        acc[db][8 * half + 2] * scale, acc[db][8 * half + 3] * scale);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(acc[db][8 * half + 4] * scale, acc[db][8 * half + 5] * scale,
                        acc[db][8 * half + 6] * scale, acc[db][8 * half + 7] * scale);
      }
    }
}

__device__ __forceinline__ void mask_keys_b(floatx16 acc[2], int key0, int N, int causal, int qrow, int h) {
  const int lim = (causal ? min(qrow, N - 1) : N - 1) - key0 - 8 * h;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 32 * kh + 16 * (r >> 3) + (r & 7);
      if (off > lim) acc[kh][r] = -INFINITY;
    }
}

// Whether some row of the wave has p > 0 in a 32-key half of scores s
// (lane rows at threshold t; wave-uniform).
template <int PM>
__device__ __forceinline__ bool half_active(const floatx16& s, float zs, float t, bool qvalid) {
  float m = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
  return __ballot(qvalid && pos_arg<PM>(xarg<PM>(m, zs, t))) != 0;
}

// ---------------------------------------------------------------------------
// bwd_rows: delta and dQ
// ---------------------------------------------------------------------------
// 3 waves per SIMD at d = 64 (at most 168 VGPRs), as in the output kernel
template <class E, int D, int PM, int NBUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 1)))
void bwd_rows_kernel(BwdArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = 256, NBLKS = 2;
  constexpr int LDK = Ld<E, D>::value;
  constexpr int LDT = Ld<E, BLK>::value;
  constexpr bool TR = E::TR_READ;   // K^T read transposed from the K tile
  __shared__ __attribute__((aligned(16))) S ktile[NBUF][BLK * LDK];
  __shared__ __attribute__((aligned(16))) S vtile[NBUF][BLK * LDK];
  __shared__ __attribute__((aligned(16))) S kttile[TR ? 1 : NBUF][TR ? 8 : D * LDT];
  __shared__ uint32_t mk[NBLKS][WMAX];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid), h = lane >> 5, l32 = lane & 31;
  const int ngroups = (a.nb + NBLKS - 1) / NBLKS;
  const int total = a.B * a.H * ngroups;
  const int wg = xcd_remap(blockIdx.x, total);
  int bh, rank;
  xcd_split(wg, total, ngroups, bh, rank);
  const int grp = ngroups - 1 - rank;
  const int blk0 = grp * NBLKS;
  const int lb = wave >> 1;
  const int myblk = blk0 + lb;
  const int qrow = myblk * BLK + (wave & 1) * 32 + l32;
  const bool qvalid = qrow < a.N;
  const bool blk_valid = myblk < a.nb;
  const int W = a.W;
  const bool has1 = blk0 + 1 < a.nb;

  const size_t hoff = a.lq.head(bh, a.H);
  const size_t kvoff = a.lkv.head(bh / a.G, a.H / a.G);
  const S* Q = reinterpret_cast<const S*>(a.q) + hoff;
  const S* K = reinterpret_cast<const S*>(a.k) + kvoff;
  const S* V = reinterpret_cast<const S*>(a.v) + kvoff;
  const S* DO = reinterpret_cast<const S*>(a.dout) + hoff;

  if (a.gather) {
    // every tile row sets at least its maximum's block in the tile rows'
    // mask, so a workgroup whose blocks have none set has no tile rows (the
    // gathered rows' dQ and delta come from the rows gather)
    uint32_t any = 0u;
    for (int i = tid; i < NBLKS * W; i += NTHR)
      if (blk0 + i / W < a.nb) any |= a.tmask[((size_t)bh * a.nb + blk0 + i / W) * W + i % W];
    if (__syncthreads_or(any != 0u) == 0) return;
  }

  typename E::frag bq[D / E::KPI], bdo[D / E::KPI];
  load_row_frags<E, D>(bq, Q + (size_t)qrow * a.lq.sn, qvalid, h);
  load_row_frags<E, D>(bdo, DO + (size_t)qrow * a.lq.sn, qvalid, h);
  // rows whose state record holds their support list take the gather path; the
  // others the tile path over the mask of those rows alone
  const uint32_t vw0 =
      (a.gather && qvalid) ? reinterpret_cast<const uint32_t*>(a.state)[((size_t)bh * a.N + qrow) * D] : 0u;
  const bool marked = a.gather && qvalid && list_marked(vw0);
  const bool tile_row = qvalid && !marked;
  const float tq = qvalid ? a.tau[(size_t)bh * a.N + qrow] : INFINITY;
  const float t = tile_row ? tq : INFINITY;   // gathered rows take p = 0 on the tiles
  const float zs = a.zscale, kappa = a.kappa;
  const uint32_t* MK = a.gather ? a.tmask : a.mask;

  for (int i = tid; i < NBLKS * W; i += NTHR) {
    const int b = i / W, w = i % W;
    mk[b][w] = (blk0 + b < a.nb) ? MK[((size_t)bh * a.nb + blk0 + b) * W + w] : 0u;
  }
  __syncthreads();

  TileIO<E, D, NTHR> iok, iov;

  // ---- delta: from vbar in the state, or sweep 1 ----
  float su = 0.f, sud = 0.f;
  if (a.state) {
    // this lane holds dO at the columns of its fragments; the two lanes of a
    // row cover all D columns
    su = 1.f;
    if (tile_row) {
      const float* vb = a.state + ((size_t)bh * a.N + qrow) * D;   // [B, H, N, D]
#pragma unroll
      for (int ks = 0; ks < D / E::KPI; ++ks) {
        if constexpr (sizeof(S) == 2) {
          const float4 v0 = *reinterpret_cast<const float4*>(vb + ks * 16 + 8 * h);
          const float4 v1 = *reinterpret_cast<const float4*>(vb + ks * 16 + 8 * h + 4);
          const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) sud = fmaf((float)bdo[ks][j], vv[j], sud);
        } else {
          sud = fmaf(bdo[ks], vb[ks * 2 + h], sud);
        }
      }
    }
  } else {
    UnionIterB itr;
    itr.init(mk[0], mk[1], has1, W);
    int J = itr.next();
    int buf = 0;
    if (J >= 0) {
      iok.load(K, J * BLK, a.N, tid, a.lkv.sn);
      iov.load(V, J * BLK, a.N, tid, a.lkv.sn);
    }
    wait_vmem();
    if (J >= 0) {
      iok.template store_rows<LDK>(ktile[0], tid);
      iov.template store_rows<LDK>(vtile[0], tid);
    }
    __syncthreads();
    while (J >= 0) {
      const int Jn = itr.next();
      if (Jn >= 0) {
        iok.load(K, Jn * BLK, a.N, tid, a.lkv.sn);
        iov.load(V, Jn * BLK, a.N, tid, a.lkv.sn);
      }
      if (blk_valid && ((mk[lb][J >> 5] >> (J & 31)) & 1u)) {
        floatx16 s[2];
        tile_x_frags<E, D, LDK>(s, ktile[buf], bq, l32, h);
        if (J * BLK + BLK > a.N || (a.causal && J == myblk)) mask_keys_b(s, J * BLK, a.N, a.causal, qrow, h);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          if (!half_active<PM>(s[kh], zs, t, tile_row)) continue;   // u = 0 on the whole half
          const floatx16 dp = tile_x_half<E, D, LDK>(vtile[buf], bdo, l32, h, kh);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float u = uk01<PM>(xarg<PM>(s[kh][r], zs, t), kappa);
            su += u;
            sud = fmaf(u, dp[r], sud);
          }
        }
      }
      wait_vmem();
      if (Jn >= 0) {
        if (NBUF == 1) __syncthreads();
        iok.template store_rows<LDK>(ktile[NBUF - 1 - buf], tid);
        iov.template store_rows<LDK>(vtile[NBUF - 1 - buf], tid);
      }
      __syncthreads();
      buf = NBUF - 1 - buf;
      J = Jn;
    }
  }
  if (!a.state) su += __shfl_xor(su, 32);
  sud += __shfl_xor(sud, 32);
  const float delta = su > 0.f ? sud / su : 0.f;
  if (tile_row && h == 0) a.delta[(size_t)bh * a.N + qrow] = delta;


  // ---- sweep 2: dQ ----
  const int tr_off = tr_lane_off(lane, LDK);
  floatx16 acc_dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc_dq[db] = floatx16{};
  {
    UnionIterB itr;
    itr.init(mk[0], mk[1], has1, W);
    int J = itr.next();
    int buf = 0;
    if (J >= 0) {
      iok.load(K, J * BLK, a.N, tid, a.lkv.sn);
      iov.load(V, J * BLK, a.N, tid, a.lkv.sn);
    }
    wait_vmem();
    if (J >= 0) {
      iok.template store_rows<LDK>(ktile[0], tid);
      if constexpr (!TR) iok.template store_trans<LDT>(kttile[0], tid);
      iov.template store_rows<LDK>(vtile[0], tid);
    }
    __syncthreads();
    while (J >= 0) {
      const int Jn = itr.next();
      if (Jn >= 0) {
        iok.load(K, Jn * BLK, a.N, tid, a.lkv.sn);
        iov.load(V, Jn * BLK, a.N, tid, a.lkv.sn);
      }
      if (blk_valid && ((mk[lb][J >> 5] >> (J & 31)) & 1u)) {
        floatx16 s[2];
        tile_x_frags<E, D, LDK>(s, ktile[buf], bq, l32, h);
        if (J * BLK + BLK > a.N || (a.causal && J == myblk)) mask_keys_b(s, J * BLK, a.N, a.causal, qrow, h);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          // dP and the dQ products of a 32-key half run only where some row
          // of the wave has p > 0 in it (dS = 0 elsewhere)
          if (!half_active<PM>(s[kh], zs, t, tile_row)) continue;
          const floatx16 dp = tile_x_half<E, D, LDK>(vtile[buf], bdo, l32, h, kh);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kh][r] = uk01<PM>(xarg<PM>(s[kh][r], zs, t), kappa) * (dp[r] - delta);
          if constexpr (TR) {
            const S* kt = ktile[buf] + tr_off;
#pragma unroll
            for (int st = 0; st < E::ACC_KSTEPS; ++st)
#pragma unroll
              for (int db = 0; db < D / 32; ++db)
                acc_dq[db] = E::mma(E::ld_tr(kt + (32 * kh + 16 * st) * LDK + 32 * db, LDK),
                                    E::from_acc(s[kh], st), acc_dq[db]);
          } else {
            const S* kt = kttile[buf];
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              const S* krow = kt + (32 * db + sigma32(l32)) * LDT;
#pragma unroll
              for (int st = 0; st < E::ACC_KSTEPS; ++st)
                acc_dq[db] = E::mma(E::ld_kacc(krow + 32 * kh, st, h), E::from_acc(s[kh], st), acc_dq[db]);
            }
          }
        }
      }
      wait_vmem();
      if (Jn >= 0) {
        if (NBUF == 1) __syncthreads();
        iok.template store_rows<LDK>(ktile[NBUF - 1 - buf], tid);
        if constexpr (!TR) iok.template store_trans<LDT>(kttile[NBUF - 1 - buf], tid);
        iov.template store_rows<LDK>(vtile[NBUF - 1 - buf], tid);
      }
      __syncthreads();
      buf = NBUF - 1 - buf;
      J = Jn;
    }
  }
  if (tile_row) {
    S* rowp = reinterpret_cast<S*>(a.dq) + hoff + (size_t)qrow * a.lq.sn;
    store_row_acc<E, D>(rowp, acc_dq, a.rscale, h);
  }
}

// ---------------------------------------------------------------------------
// bwd_rows_gather: the rows the forward formed from their support lists (kept
// in their state records): dP over the listed keys, delta, dS, dQ, one row per
// lane pair; the entries (key, dS, p) are left for the key side
// ---------------------------------------------------------------------------
template <class E, int D, int PM>
__global__ __launch_bounds__(256) void bwd_rows_gather_kernel(BwdArgs a) {
  using S = typename E::storage;
  constexpr int DH = D / 2;   // elements of the row this lane takes
  __shared__ uint32_t lists[128 * LIST_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid), h = lane >> 5, l32 = lane & 31;
  const int ngroups = (a.N + 127) / 128;
  const int wg = xcd_remap(blockIdx.x, a.B * a.H * ngroups);
  const int bh = wg / ngroups;
  const int r128 = 32 * wave + l32;   // row within the workgroup
  const int qrow = (wg % ngroups) * 128 + r128;
  const bool qvalid = qrow < a.N;
  const uint32_t vw0 = qvalid ? reinterpret_cast<const uint32_t*>(a.state)[((size_t)bh * a.N + qrow) * D] : 0u;
  const bool marked = qvalid && list_marked(vw0);
  if (__ballot(marked) == 0) return;   // (whole waves; no barrier follows)
  const size_t hoff = a.lq.head(bh, a.H);
  const size_t kvoff = a.lkv.head(bh / a.G, a.H / a.G);
  const S* K = reinterpret_cast<const S*>(a.k) + kvoff;
  const S* V = reinterpret_cast<const S*>(a.v) + kvoff;
  const S* DO = reinterpret_cast<const S*>(a.dout) + hoff;
  const float zs = a.zscale, kappa = a.kappa;
  const float tq = marked ? a.tau[(size_t)bh * a.N + qrow] : 0.f;
  // the list, staged in LDS (each lane of the row copies half of it)
  uint32_t* lds_l = lists + LIST_LDS * r128;
  if (marked) stage_list(lds_l, reinterpret_cast<const uint32_t*>(a.state + ((size_t)bh * a.N + qrow) * D), h);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();   // (rows are read only by the wave that staged them)
  const int n = marked ? (int)(vw0 & 0xFFFFu) : 0;
  const int kmax = a.causal ? qrow : a.N - 1;
  const uint32_t* lkw = lds_l + 2 + LIST_CAP;   // keys, two per word
  RowChunk<E, DH> dor;
  if (marked) dor.load(DO + (size_t)qrow * a.lq.sn + DH * h);
  // the row's x_j replace its scores in the staged list (0 for entries not
  // used); keys of unused entries read as row 0 with weight 0
  auto key_of = [&](int i) -> int {
    return __uint_as_float(lds_l[2 + i]) > 0.f ? (int)((lkw[i / 2] >> (16 * (i & 1))) & 0xFFFFu) : 0;
  };
  float dpv[LIST_CAP];
#pragma unroll
  for (int i = 0; i < LIST_CAP; ++i) dpv[i] = 0.f;
  constexpr int CH = 2;   // rows in flight per step
  // dP_ij = dO_i . v_j, each lane over its half of d
#pragma unroll
  for (int i = 0; i < LIST_CAP; i += CH) {
    if (i < n) {
      RowChunk<E, DH> rc[CH];
      bool use[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const float xc = xclamp(__uint_as_float(lds_l[2 + i + c]), zs, tq);
        const int kc = (int)((lkw[(i + c) / 2] >> (16 * ((i + c) & 1))) & 0xFFFFu);
        use[c] = i + c < n && xc > 0.f && kc <= kmax;
        rc[c].load(V + (size_t)(use[c] ? kc : 0) * a.lkv.sn + DH * h);
        lds_l[2 + i + c] = __float_as_uint(use[c] ? xc : 0.f);   // (both lanes store the same)
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) dpv[i + c] = use[c] ? rc[c].dot(dor) : 0.f;
    }
  }
  // entries past n read x = 0
#pragma unroll
  for (int i = 0; i < LIST_CAP; ++i)
    if (i >= n) lds_l[2 + i] = 0u;
  float gsu = 0.f, gsud = 0.f;
#pragma unroll
  for (int i = 0; i < LIST_CAP; ++i) {
    dpv[i] += __shfl_xor(dpv[i], 32);
    const float u = uk01<PM>(__uint_as_float(lds_l[2 + i]), kappa);
    gsu += u;
    gsud = fmaf(u, dpv[i], gsud);
  }
  const float gdel = gsu > 0.f ? gsud / gsu : 0.f;
  // dS_ij = u_ij (dP_ij - delta_i); dQ_i = sum_j dS_ij k_j / sqrt(d)
  float dqv[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) dqv[e] = 0.f;
#pragma unroll
  for (int i = 0; i < LIST_CAP; i += CH) {
    if (i < n) {
      RowChunk<E, DH> rc[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) rc[c].load(K + (size_t)key_of(i + c) * a.lkv.sn + DH * h);
#pragma unroll
      for (int c = 0; c < CH; ++c)
        rc[c].fma(dqv, uk01<PM>(__uint_as_float(lds_l[2 + i + c]), kappa) * (dpv[i + c] - gdel));
    }
  }
  if (marked) {
    S* dqrow = reinterpret_cast<S*>(a.dq) + hoff + (size_t)qrow * a.lq.sn + DH * h;
    if constexpr (sizeof(S) == 2) {
#pragma unroll
      for (int c = 0; c < DH / 8; ++c) {
        uint32_t ww[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ww[e] = (uint32_t)E::from_f(dqv[8 * c + 2 * e] * a.rscale) |
                  ((uint32_t)E::from_f(dqv[8 * c + 2 * e + 1] * a.rscale) << 16);
        *reinterpret_cast<uint4*>(dqrow + 8 * c) = make_uint4(ww[0], ww[1], ww[2], ww[3]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < DH / 4; ++c)
        *reinterpret_cast<float4*>(dqrow + 4 * c) = make_float4(dqv[4 * c] * a.rscale, dqv[4 * c + 1] * a.rscale,
                                                                dqv[4 * c + 2] * a.rscale, dqv[4 * c + 3] * a.rscale);
    }
    if (h == 0) {
      a.delta[(size_t)bh * a.N + qrow] = gdel;
      const size_t slot0 = ((size_t)bh * a.N + qrow) * LIST_CAP;
      const uint32_t kbase = (uint32_t)(bh / a.G) * (uint32_t)a.N;   // key ids of this row's kv head
#pragma unroll
      for (int i = 0; i < LIST_CAP; ++i)
        if (i < n) {
          const float x = __uint_as_float(lds_l[2 + i]);
          const bool use = x > 0.f;
          const uint32_t kid = use ? kbase + (uint32_t)key_of(i) : 0xFFFFFFFFu;
          a.ent_key[slot0 + i] = kid;
          a.ent_ds[slot0 + i] = uk01<PM>(x, kappa) * (dpv[i] - gdel);
          a.ent_p[slot0 + i] = pk01<PM>(x, kappa);
          if (use) a.ent_rank[slot0 + i] = atomicAdd(a.kcnt + kid, 1u);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Gathered rows, key side: for each key, the sums over the entries listing it
// of dS q (dK before the 1/sqrt(d) scale) and p dO (dV), one key per 16
// lanes (one per workgroup past 64 entries). The order of a key's entries in
// its bucket follows the atomics that placed them, so the sums are formed
// independently of it: up to 64 entries are sorted by slot (a bitonic network
// over the lanes: one entry per lane up to 16, four per lane up to 64) and
// added in that order in fp32; more are added as integers. For the integer
// sums a first
// sweep over the entries finds, per element, the largest |term| < 2^e; each
// term is then rounded to a multiple of 2^(e - 31) (|term| < 2^31 units) and
// the multiples are added in 64 bits, exactly, so the result does not depend
// on the order and is relative to the data's own scale (the rounding is at
// most 2^-31 of the largest term, finer than fp32 accumulation).
// ---------------------------------------------------------------------------
// the unit exponent of elements whose largest |term| is m: 31 - e with
// m < 2^e (frexp), so |term| * 2^(31 - e) < 2^31
__device__ __forceinline__ int fixp_shift(float m) {
  int e;
  frexpf(m, &e);
  return 31 - e;
}
// a term in units of 2^-sh, rounded to nearest (|x| < 2^31 by the shift)
__device__ __forceinline__ long long fixp_units(float x, int sh) {
  return (long long)(int)rintf(ldexpf(x, sh));
}

// Bitonic sort, ascending, of 64 keys held four per lane by a group of 16
// lanes (element 4 l + j in register j of lane l).
__device__ __forceinline__ void bitonic64(uint32_t (&v)[4], int l) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int jd = k >> 1; jd > 0; jd >>= 1) {
      if (jd >= 4) {   // partner in lane l ^ (jd / 4), same register
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * l + j;
          const uint32_t o = __shfl_xor(v[j], jd >> 2, 16);
          const bool up = (i & k) == 0, lower = (i & jd) == 0;
          v[j] = (up == lower) ? min(v[j], o) : max(v[j], o);
        }
      } else {         // partner in this lane, register j ^ jd
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * l + j;
          const uint32_t o = v[j ^ jd];
          const bool up = (i & k) == 0, lower = (i & jd) == 0;
          w[j] = (up == lower) ? min(v[j], o) : max(v[j], o);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = w[j];
      }
    }
  }
}

template <class E, int EL>
__device__ __forceinline__ void load_el(float (&x)[EL], const typename E::storage* p) {
  if constexpr (sizeof(typename E::storage) == 2) {
#pragma unroll
    for (int c = 0; c < EL / 2; ++c) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(p)[c];
      x[2 * c] = __uint_as_float(w << 16);
      x[2 * c + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int c = 0; c < EL; ++c) x[c] = p[c];
  }
}

// Keys with more than KV_HEAVY entries are summed by whole workgroups: the
// first workgroups of the launch each look for them among KV_RANGE keys and
// sum each one with 16 groups of 16 lanes over its entries (in the integer
// form, whose sum does not depend on how the entries are split); the rest
// take one key per 16 lanes. A long key thus spreads over 256 lanes and
// starts with the launch instead of ending it.
constexpr uint32_t KV_HEAVY = 64;
constexpr int KV_RANGE = 256;

__host__ __device__ inline int kv_heavy_blocks(size_t nk) { return (int)((nk + KV_RANGE - 1) / KV_RANGE); }

template <class E, int D>
__global__ __launch_bounds__(256) void bwd_kv_gather_kernel(BwdArgs a) {
  using S = typename E::storage;
  constexpr int EL = D / 16;   // elements of the row per lane
  __shared__ uint32_t hk[KV_RANGE];                 // this workgroup's long keys
  __shared__ uint32_t nh;
  __shared__ int redm[2][D];                        // per element: largest |term| (bits of a float >= 0)
  __shared__ unsigned long long reds[2][D];         // per element: the sums in units of 2^-sh
  const int g = threadIdx.x >> 4, l = threadIdx.x & 15;
  const size_t nk = (size_t)a.B * (a.H / a.G) * a.N;
  const int nhb = kv_heavy_blocks(nk);
  const int hkv = a.H / a.G;
  const uint32_t nslots = (uint32_t)((size_t)a.B * a.H * a.N * LIST_CAP);
  const double rn = 1.0 / (double)a.N;
  // an entry's slot -> the offset of its query row in q and dO (a valid row,
  // with weights 0, for slots past the end)
  auto rowoff = [&](uint32_t slot) -> long long {
    if (slot >= nslots) return 0;
    const uint32_t row = slot / LIST_CAP;
    uint32_t bh = (uint32_t)((double)row * rn);
    if ((size_t)bh * a.N > row) --bh;
    else if ((size_t)(bh + 1) * a.N <= row) ++bh;
    const uint32_t i = row - bh * (uint32_t)a.N;
    return (long long)(a.lq.head((int)bh, a.H) + (size_t)i * a.lq.sn);
  };
  // one lane's entry: its query row offset and weights
  auto fetch = [&](uint32_t slot, long long& off, float& ds, float& p) {
    off = rowoff(slot);
    ds = slot < nslots ? a.ent_ds[slot] : 0.f;
    p = slot < nslots ? a.ent_p[slot] : 0.f;
  };
  // the key's final rows, as the column kernel stores them: dK scaled by
  // 1/sqrt(d), dV as is
  auto store_final = [&](size_t kid, const float (&fk)[EL], const float (&fv)[EL]) {
    const int bhkv = (int)(kid / (size_t)a.N), key = (int)(kid % (size_t)a.N);
    const size_t roff = a.lkv.head(bhkv, hkv) + (size_t)key * a.lkv.sn + EL * l;
    S* dkrow = reinterpret_cast<S*>(a.dk) + roff;
    S* dvrow = reinterpret_cast<S*>(a.dv) + roff;
#pragma unroll
    for (int k = 0; k < EL; ++k) {
      dkrow[k] = E::from_f(fk[k] * a.rscale);
      dvrow[k] = E::from_f(fv[k]);
    }
  };
  const S* Qb = reinterpret_cast<const S*>(a.q) + EL * l;
  const S* Db = reinterpret_cast<const S*>(a.dout) + EL * l;

  if ((int)blockIdx.x < nhb) {
    // ---- long keys: one at a time over the whole workgroup ----
    const size_t k0 = (size_t)blockIdx.x * KV_RANGE;
    if (threadIdx.x == 0) nh = 0u;
    __syncthreads();
    {
      const size_t kid = k0 + threadIdx.x;
      if (kid < nk && a.kcnt[kid] > KV_HEAVY) hk[atomicAdd(&nh, 1u)] = threadIdx.x;
    }
    __syncthreads();
    const uint32_t n = nh;
    for (uint32_t t = 0; t < n; ++t) {
      const size_t kid = k0 + hk[t];
      const uint32_t cnt = a.kcnt[kid], beg = a.koff[kid];
      const int bhkv = (int)(kid / (size_t)a.N), kb = (int)(kid % (size_t)a.N) / BLK;
      uint32_t tw = 0u;
      for (int i = threadIdx.x; i < a.G * a.W; i += 256)
        tw |= a.colmask[((size_t)(bhkv * a.G + i / a.W) * a.nb + kb) * a.W + i % a.W];
      for (int i = threadIdx.x; i < 2 * D; i += 256) {
        (&redm[0][0])[i] = 0;
        (&reds[0][0])[i] = 0ull;
      }
      const bool tiles = __syncthreads_or(tw != 0u) != 0;
      // group g takes entries g, g + 16, ...; in each round of 256 entries
      // lane j of the group holds the slot and weights of its j-th
      auto sweep = [&](auto&& term) {
        for (uint32_t e0 = 0; e0 < cnt; e0 += 256) {
          const uint32_t e = e0 + (uint32_t)g + 16u * (uint32_t)l;
          const uint32_t ms = (e < cnt && beg + e < nslots) ? a.bucket[beg + e] : 0xFFFFFFFFu;
          long long moff;
          float mds, mp;
          fetch(ms, moff, mds, mp);
          const uint32_t ne = e0 + (uint32_t)g < cnt ? min(16u, (cnt - e0 - (uint32_t)g + 15u) / 16u) : 0u;
#pragma unroll 4
          for (uint32_t j = 0; j < ne; ++j) {
            const long long off = __shfl(moff, (int)j, 16);
            const float ds = __shfl(mds, (int)j, 16), p = __shfl(mp, (int)j, 16);
            float qv[EL], dv[EL];
            load_el<E, EL>(qv, Qb + off);
            load_el<E, EL>(dv, Db + off);
            term(ds, p, qv, dv);
          }
        }
      };
      // sweep 1: per element, the largest |term| of the key's entries
      float mk[EL], mv[EL];
#pragma unroll
      for (int k = 0; k < EL; ++k) mk[k] = mv[k] = 0.f;
      sweep([&](float ds, float p, const float (&qv)[EL], const float (&dv)[EL]) {
#pragma unroll
        for (int k = 0; k < EL; ++k) {
          mk[k] = fmaxf(mk[k], fabsf(ds * qv[k]));
          mv[k] = fmaxf(mv[k], fabsf(p * dv[k]));
        }
      });
#pragma unroll
      for (int k = 0; k < EL; ++k) {
        atomicMax(&redm[0][EL * l + k], __float_as_int(mk[k]));
        atomicMax(&redm[1][EL * l + k], __float_as_int(mv[k]));
      }
      __syncthreads();
      int shk[EL], shv[EL];
      long long sk[EL], sv[EL];
#pragma unroll
      for (int k = 0; k < EL; ++k) {
        shk[k] = fixp_shift(__int_as_float(redm[0][EL * l + k]));
        shv[k] = fixp_shift(__int_as_float(redm[1][EL * l + k]));
        sk[k] = sv[k] = 0;
      }
      // sweep 2: the terms as integer multiples of 2^-sh, summed exactly
      sweep([&](float ds, float p, const float (&qv)[EL], const float (&dv)[EL]) {
#pragma unroll
        for (int k = 0; k < EL; ++k) {
          sk[k] += fixp_units(ds * qv[k], shk[k]);
          sv[k] += fixp_units(p * dv[k], shv[k]);
        }
      });
#pragma unroll
      for (int k = 0; k < EL; ++k) {
        atomicAdd(&reds[0][EL * l + k], (unsigned long long)sk[k]);
        atomicAdd(&reds[1][EL * l + k], (unsigned long long)sv[k]);
      }
      __syncthreads();
      if (g == 0) {
        float fk[EL], fv[EL];
#pragma unroll
        for (int k = 0; k < EL; ++k) {
          fk[k] = (float)ldexp((double)(long long)reds[0][EL * l + k], -shk[k]);
          fv[k] = (float)ldexp((double)(long long)reds[1][EL * l + k], -shv[k]);
        }
        if (tiles) {
          float* pk = a.part + kid * 2 * D + EL * l;
#pragma unroll
          for (int k = 0; k < EL; ++k) {
            pk[k] = fk[k];
            pk[D + k] = fv[k];
          }
        } else {
          store_final(kid, fk, fv);
        }
      }
      __syncthreads();   // (the reductions are cleared for the next key)
    }
    return;
  }

  // ---- the other keys: one per 16 lanes ----
  // consecutive keys on one XCD: the rows they read share its L2
  const size_t kid = (size_t)xcd_remap((int)blockIdx.x - nhb, (int)gridDim.x - nhb) * 16 + g;
  if (kid >= nk) return;   // (whole 16-lane groups)
  const uint32_t cnt = a.kcnt[kid], beg = a.koff[kid];
  if (cnt > KV_HEAVY) return;   // (a long key: summed above)
  // Whether the key's block has tile rows in some query head of its group
  // (a bit in their key-major masks): if so the column kernel forms the
  // key's dK, dV and adds these sums from the partials; if not, it skips the
  // block and the rows are stored here (zeros for a key without entries).
  const int bhkv = (int)(kid / (size_t)a.N), key = (int)(kid % (size_t)a.N), kb = key / BLK;
  uint32_t tw = 0u;
  for (int i = l; i < a.G * a.W; i += 16)
    tw |= a.colmask[((size_t)(bhkv * a.G + i / a.W) * a.nb + kb) * a.W + i % a.W];
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) tw |= __shfl_xor(tw, o, 16);
  const bool tiles = tw != 0u;
  if (cnt == 0u && tiles) return;
  float fk[EL], fv[EL];
#pragma unroll
  for (int k = 0; k < EL; ++k) fk[k] = fv[k] = 0.f;
  if (cnt == 0u) {
    // (no entries: zero rows)
  } else if (cnt <= 16u) {
    uint32_t ms = ((uint32_t)l < cnt && beg + l < nslots) ? a.bucket[beg + l] : 0xFFFFFFFFu;
#pragma unroll
    for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
      for (int j = k >> 1; j > 0; j >>= 1) {
        const uint32_t o = __shfl_xor(ms, j, 16);
        ms = (((l & j) == 0) == ((l & k) == 0)) ? min(ms, o) : max(ms, o);
      }
    long long moff;
    float mds, mp;
    fetch(ms, moff, mds, mp);
#pragma unroll 4
    for (uint32_t e = 0; e < cnt; ++e) {
      const long long off = __shfl(moff, (int)e, 16);
      const float ds = __shfl(mds, (int)e, 16), p = __shfl(mp, (int)e, 16);
      float qv[EL], dv[EL];
      load_el<E, EL>(qv, Qb + off);
      load_el<E, EL>(dv, Db + off);
#pragma unroll
      for (int k = 0; k < EL; ++k) {
        fk[k] = fmaf(ds, qv[k], fk[k]);
        fv[k] = fmaf(p, dv[k], fv[k]);
      }
    }
  } else if (cnt <= 64u) {
    uint32_t ms[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e = 4u * (uint32_t)l + (uint32_t)j;
      ms[j] = (e < cnt && beg + e < nslots) ? a.bucket[beg + e] : 0xFFFFFFFFu;
    }
    bitonic64(ms, l);
    long long moff[4];
    float mds[4], mp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fetch(ms[j], moff[j], mds[j], mp[j]);
    // entry e (in slot order) sits in register e % 4 of lane e / 4
    for (uint32_t e0 = 0; e0 < cnt; e0 += 4) {
      const int src = (int)(e0 >> 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (e0 + (uint32_t)j < cnt) {
          const long long off = __shfl(moff[j], src, 16);
          const float ds = __shfl(mds[j], src, 16), p = __shfl(mp[j], src, 16);
          float qv[EL], dv[EL];
          load_el<E, EL>(qv, Qb + off);
          load_el<E, EL>(dv, Db + off);
#pragma unroll
          for (int k = 0; k < EL; ++k) {
            fk[k] = fmaf(ds, qv[k], fk[k]);
            fv[k] = fmaf(p, dv[k], fv[k]);
          }
        }
      }
    }
  }
  if (tiles) {
    float* pk = a.part + kid * 2 * D + EL * l;
#pragma unroll
    for (int k = 0; k < EL; ++k) {
      pk[k] = fk[k];
      pk[D + k] = fv[k];
    }
  } else {
    store_final(kid, fk, fv);
  }
}

// ---------------------------------------------------------------------------
// bwd_dkdv
// ---------------------------------------------------------------------------
template <class E, int D, int PM, int NBUF>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = 256, NBLKS = 2;
  constexpr int LDK = Ld<E, D>::value;
  constexpr int LDT = Ld<E, BLK>::value;
  constexpr bool TR = E::TR_READ;   // Q^T, dO^T read transposed from the row tiles
  __shared__ __attribute__((aligned(16))) S qtile[NBUF][BLK * LDK];
  __shared__ __attribute__((aligned(16))) S dotile[NBUF][BLK * LDK];
  __shared__ __attribute__((aligned(16))) S qttile[TR ? 1 : NBUF][TR ? 8 : D * LDT];
  __shared__ __attribute__((aligned(16))) S dottile[TR ? 1 : NBUF][TR ? 8 : D * LDT];
  __shared__ __attribute__((aligned(16))) float taus[NBUF][BLK];
  __shared__ __attribute__((aligned(16))) float dels[NBUF][BLK];
  __shared__ uint32_t cm[NBLKS][WMAX];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid), h = lane >> 5, l32 = lane & 31;
  const int ngroups = (a.nb + NBLKS - 1) / NBLKS;
  const int hkv = a.H / a.G;                      // key/value heads
  const int total = a.B * hkv * ngroups;
  const int wg = xcd_remap(blockIdx.x, total);
  int bhkv, grp;
  xcd_split(wg, total, ngroups, bhkv, grp);   // causal: low key blocks see the most query blocks
  const int blk0 = grp * NBLKS;
  const int lb = wave >> 1;
  const int kblk = blk0 + lb;
  const int krow = kblk * BLK + (wave & 1) * 32 + l32;
  const bool kvalid = krow < a.N;
  const bool blk_valid = kblk < a.nb;
  const int W = a.W;
  const bool has1 = blk0 + 1 < a.nb;

  const size_t kvoff = a.lkv.head(bhkv, hkv);
  const S* K = reinterpret_cast<const S*>(a.k) + kvoff;
  const S* V = reinterpret_cast<const S*>(a.v) + kvoff;

  if (a.gather) {
    // a workgroup whose key blocks have no tile rows in any query head of the
    // group has nothing to add: the key gather stored those keys' rows
    uint32_t any = 0u;
    for (int i = tid; i < a.G * NBLKS * W; i += NTHR) {
      const int g = i / (NBLKS * W), b = (i / W) % NBLKS, w = i % W;
      if (blk0 + b < a.nb) any |= a.colmask[((size_t)(bhkv * a.G + g) * a.nb + blk0 + b) * W + w];
    }
    if (__syncthreads_or(any != 0u) == 0) return;
  }

  typename E::frag bk[D / E::KPI], bv[D / E::KPI];
  load_row_frags<E, D>(bk, K + (size_t)krow * a.lkv.sn, kvalid, h);
  load_row_frags<E, D>(bv, V + (size_t)krow * a.lkv.sn, kvalid, h);
  const float zs = a.zscale, kappa = a.kappa;

  floatx16 acc_dk[D / 32], acc_dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    acc_dk[db] = floatx16{};
    acc_dv[db] = floatx16{};
  }
  const int tr_off = tr_lane_off(lane, LDK);
  bool tile_rows = false;   // the wave's key block has tile rows in some query head
  // dK and dV of a key/value head sum over the query heads that share it
  for (int g = 0; g < a.G; ++g) {
    const int bh = bhkv * a.G + g;
    const size_t hoff = a.lq.head(bh, a.H);
    const S* Q = reinterpret_cast<const S*>(a.q) + hoff;
    const S* DO = reinterpret_cast<const S*>(a.dout) + hoff;
    const float* TAU = a.tau + (size_t)bh * a.N;
    const float* DEL = a.delta + (size_t)bh * a.N;
    // gathered rows take p = 0 here (their entries are summed separately):
    // a row's first state word is read only in blocks holding gathered rows
    // (a flag per block, a wave-uniform load), and tested when tau is staged,
    // so the tile loads in flight are not waited for
    const uint32_t* VB0 = a.gather ? reinterpret_cast<const uint32_t*>(a.state) + (size_t)bh * a.N * D : nullptr;
    const uint32_t* GB = a.gather ? a.gblk + (size_t)bh * a.nb : nullptr;
    uint32_t vw = 0u;
    auto stage_load = [&](int blk, float& t_, float& d_, uint32_t& w_) {
      const int qr = blk * BLK + tid;
      t_ = qr < a.N ? TAU[qr] : INFINITY;
      d_ = qr < a.N ? DEL[qr] : 0.f;
      w_ = (VB0 != nullptr && GB[blk] != 0u && qr < a.N) ? VB0[(size_t)qr * D] : 0u;
    };
    __syncthreads();   // the previous head's tiles and mask words are no longer read
    for (int i = tid; i < NBLKS * W; i += NTHR) {
      const int b = i / W, w = i % W;
      cm[b][w] = (blk0 + b < a.nb) ? a.colmask[((size_t)bh * a.nb + blk0 + b) * W + w] : 0u;
    }
    __syncthreads();
    for (int w = 0; w < W; ++w) tile_rows = tile_rows || cm[lb][w] != 0u;

    TileIO<E, D, NTHR> ioq, iod;
    UnionIterB itr;
    itr.init(cm[0], cm[1], has1, W);
    int I = itr.next();
    int buf = 0;
    float tv = 0.f, dlv = 0.f;
    if (I >= 0) {
      ioq.load(Q, I * BLK, a.N, tid, a.lq.sn);
      iod.load(DO, I * BLK, a.N, tid, a.lq.sn);
      if (tid < BLK) stage_load(I, tv, dlv, vw);
    }
    wait_vmem();
    if (I >= 0) {
      ioq.template store_rows<LDK>(qtile[0], tid);
      iod.template store_rows<LDK>(dotile[0], tid);
      if constexpr (!TR) {
        ioq.template store_trans<LDT>(qttile[0], tid);
        iod.template store_trans<LDT>(dottile[0], tid);
      }
      if (tid < BLK) {
        taus[0][tid] = list_marked(vw) ? INFINITY : tv;
        dels[0][tid] = dlv;
      }
    }
    __syncthreads();
    while (I >= 0) {
      const int In = itr.next();
      if (In >= 0) {
        ioq.load(Q, In * BLK, a.N, tid, a.lq.sn);
        iod.load(DO, In * BLK, a.N, tid, a.lq.sn);
        if (tid < BLK) stage_load(In, tv, dlv, vw);
      }
      if (blk_valid && ((cm[lb][I >> 5] >> (I & 31)) & 1u)) {
        // query q = I*64 + q0 + e is invisible to key krow when q < krow
        // (causal) and every query is invisible to a key past N: compare the
        // in-tile offset q0 + e against one per-lane limit
        int qlim = -1;
        if (!kvalid) qlim = BLK;
        else if (a.causal && I == kblk) qlim = krow - I * BLK;
        // the limit can only bite on the diagonal block or the last key block
        const bool edge = (a.causal && I == kblk) || kblk * BLK + BLK > a.N;
        // one 32-query half at a time keeps a single half's S and dP live;
        // dP and the dV, dK products of a half run only where some score of
        // it has p > 0 (P = dS = 0 elsewhere)
  #pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          floatx16 s = tile_x_half<E, D, LDK>(qtile[buf], bk, l32, h, qb);
          if (edge) {
            // register r holds query 32 qb + 16 (r >> 3) + 8 h + (r & 7)
  #pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * qb + 16 * (r >> 3) + 8 * h + (r & 7) < qlim) s[r] = -INFINITY;
          }
          float xm = -INFINITY;
  #pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int q0 = 32 * qb + 16 * half + 8 * h;   // 8 consecutive query rows
            const float4 ta = *reinterpret_cast<const float4*>(&taus[buf][q0]);
            const float4 tb = *reinterpret_cast<const float4*>(&taus[buf][q0 + 4]);
            const float tq[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
  #pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * half + e;
              s[r] = xarg<PM>(s[r], zs, tq[e]);
              xm = fmaxf(xm, s[r]);
            }
          }
          if (__ballot(pos_arg<PM>(xm)) == 0) continue;
          floatx16 dp = tile_x_half<E, D, LDK>(dotile[buf], bv, l32, h, qb);
  #pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int q0 = 32 * qb + 16 * half + 8 * h;
            const float4 da = *reinterpret_cast<const float4*>(&dels[buf][q0]);
            const float4 dbv = *reinterpret_cast<const float4*>(&dels[buf][q0 + 4]);
            const float dl[8] = {da.x, da.y, da.z, da.w, dbv.x, dbv.y, dbv.z, dbv.w};
  #pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * half + e;
              const float x = s[r];
              const float u = uk01<PM>(x, kappa);
              s[r] = pk01<PM>(x, kappa);
              dp[r] = u * (dp[r] - dl[e]);
            }
          }
  #pragma unroll
          for (int st = 0; st < E::ACC_KSTEPS; ++st) {
            const typename E::frag bp = E::from_acc(s, st);
            const typename E::frag bd = E::from_acc(dp, st);
  #pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              typename E::frag ado, aq;
              if constexpr (TR) {
                const int off = tr_off + (32 * qb + 16 * st) * LDK + 32 * db;
                ado = E::ld_tr(dotile[buf] + off, LDK);
                aq = E::ld_tr(qtile[buf] + off, LDK);
              } else {
                const int off = (32 * db + sigma32(l32)) * LDT + 32 * qb;
                ado = E::ld_kacc(dottile[buf] + off, st, h);
                aq = E::ld_kacc(qttile[buf] + off, st, h);
              }
              acc_dv[db] = E::mma(ado, bp, acc_dv[db]);
              acc_dk[db] = E::mma(aq, bd, acc_dk[db]);
            }
          }
        }
      }
      wait_vmem();
      if (In >= 0) {
        if (NBUF == 1) __syncthreads();
        const int nbuf = NBUF - 1 - buf;
        ioq.template store_rows<LDK>(qtile[nbuf], tid);
        iod.template store_rows<LDK>(dotile[nbuf], tid);
        if constexpr (!TR) {
          ioq.template store_trans<LDT>(qttile[nbuf], tid);
          iod.template store_trans<LDT>(dottile[nbuf], tid);
        }
        if (tid < BLK) {
          taus[nbuf][tid] = list_marked(vw) ? INFINITY : tv;
          dels[nbuf][tid] = dlv;
        }
      }
      __syncthreads();
      buf = NBUF - 1 - buf;
      I = In;
    }
  }
  // with the gather path, a key block without tile rows was stored by the key
  // gather (its sums are the whole gradient)
  const bool stored = a.gather && !tile_rows;
  if (a.gather && kvalid && !stored) {
    // the gathered rows' sums for this key (dK before the 1/sqrt(d) scale)
    const size_t kid = (size_t)bhkv * a.N + krow;
    if (a.kcnt[kid] != 0u) {
      const float* pk = a.part + kid * 2 * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int d0 = 32 * db + 16 * half + 8 * h;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            acc_dk[db][8 * half + e] += pk[d0 + e];
            acc_dv[db][8 * half + e] += pk[D + d0 + e];
          }
        }
    }
  }
  if (kvalid && !stored) {
    S* dkrow = reinterpret_cast<S*>(a.dk) + kvoff + (size_t)krow * a.lkv.sn;
    S* dvrow = reinterpret_cast<S*>(a.dv) + kvoff + (size_t)krow * a.lkv.sn;
    store_row_acc<E, D>(dkrow, acc_dk, a.rscale, h);
    store_row_acc<E, D>(dvrow, acc_dv, 1.f, h);
  }
}

}  // namespace ea
