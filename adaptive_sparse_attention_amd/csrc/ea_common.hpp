// Shared device code for the alpha-entmax attention kernels (gfx950).
//
// Tile geometry. Queries and keys are cut into blocks of 64 rows. A wave owns
// 32 rows of its side (query rows in the row-parallel kernels, key rows in the
// column-parallel one) and multiplies them against a 64-row tile of the other
// side staged in LDS, with the 32x32x16 bf16 MFMA (32x32x2 for fp32 inputs).
//
// MFMA lane layout (checked on gfx950): for a 32x32 result, lane l holds
// column l % 32 and, in register r, row 8*(r/4) + 4*(l/32) + r%4. The A operand
// of the bf16 instruction holds A[l%32][8*(l/32) + j], j < 8; the B operand
// holds B[8*(l/32) + j][l%32].
//
// Row permutation. Every A operand reads logical row rho from physical row
// sigma(rho) (bits 2 and 3 of rho swapped). The result row of register r in
// lane half h is then the physical row 16*(r/8) + 8*h + r%8: registers 0..7
// hold 8 consecutive rows and 8..15 the next run 16 rows on. Those runs are
// exactly the k-slices the B operand of the next MFMA needs, so a score tile
// feeds the following product (P.V, dS.K, ...) straight from registers, and
// the A operand of that product reads 16 contiguous bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <type_traits>

namespace ea {

constexpr int BLK = 64;            // query / key block size
constexpr int HIST_BINS = 256;     // bins per unit of z
constexpr int HIST_SLOTS = 257;    // window [ktop - 256, ktop]
constexpr int MAX_PASSES = 8;
constexpr int MAX_PASSES_NOHIST = 40;   // without the histogram start (bisection from a bracket of width < 1)
constexpr int WMAX = 128;          // mask words per block for N <= 2^18
// Support lists of rows solved on the histogram kernel's kept keys: 2
// header words (word 0: LIST_GATHER | count once the refinement has solved
// the row), LIST_CAP scores, LIST_CAP 16-bit keys: 128 bytes, kept in the
// row of o by the forward and in the row's state record for the backward.
constexpr int LIST_CAP = 20;                 // 8 + 20 * (4 + 2) = 128 bytes
constexpr uint32_t LIST_GATHER = 0xFFFF0000u;
constexpr int LIST_MAX_N = 65536;            // key indices in 16 bits
__device__ __forceinline__ bool list_marked(uint32_t w0) {
  return (w0 & 0xFFFF0000u) == LIST_GATHER && (w0 & 0xFFFFu) <= (uint32_t)LIST_CAP;
}
// Lists staged in LDS one row per LIST_LDS words (odd: the lanes' rows fall
// in different banks). Each of the two lanes of a row copies half of it.
constexpr int LIST_LDS = 33;
__device__ __forceinline__ void stage_list(uint32_t* lds_row, const uint32_t* src, int h) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src) + 4 * h;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 v = s4[c];
    lds_row[16 * h + 4 * c] = v.x;
    lds_row[16 * h + 4 * c + 1] = v.y;
    lds_row[16 * h + 4 * c + 2] = v.z;
    lds_row[16 * h + 4 * c + 3] = v.w;
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ int sigma32(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// physical row (within a 32-row half) of accumulator register r in lane half h
__device__ __forceinline__ int acc_row(int r, int h) {
  return 16 * (r >> 3) + 8 * h + (r & 7);
}

// Transposed LDS reads (ds_read_b64_tr_b16, checked on gfx950): within each
// group of 16 lanes, lane i receives element (i & 3) of the 8-byte chunks
// addressed by lanes 4j + (i >> 2), j = 0..3. Lane L = 16g + 4j + q of the
// wave therefore addresses row 8*(g >> 1) + j and column chunk
// sigma(4*(g & 1) + q) of a row-major tile X[k][m]; two such reads (rows +0
// and +4) give every lane l the A-operand slice X[8h + t][sigma(l % 32)],
// t < 8, h = l / 32, of the 32x32x16 MFMA with A[m][k] = X[k][m]. This is
// the element offset of that pattern for a tile with row stride ld.
__device__ __forceinline__ int tr_lane_off(int lane, int ld) {
  const int g = lane >> 4, i = lane & 15;
  const int chunk = 4 * (g & 1) + (i & 3);
  const int sch = (chunk & 4) | ((chunk & 1) << 1) | ((chunk & 2) >> 1);
  return (8 * (g >> 1) + (i >> 2)) * ld + 4 * sch;
}

// ---------------------------------------------------------------------------
// Element types
// ---------------------------------------------------------------------------

struct BF16 {
  using storage = uint16_t;
  using frag = bf16x8;
  static constexpr int KPI = 16;     // k per MFMA instruction
  static constexpr int VEC = 8;      // elements per lane per operand
  static constexpr int ACC_KSTEPS = 2;   // k-steps covering 32 accumulator rows
  static constexpr int CHUNK = 8;    // elements per 16-byte chunk
  static constexpr bool TR_READ = true;  // A operands of transposed tiles via ds_read_b64_tr_b16

  __device__ static __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // operand whose k runs along a contiguous row: k-step ks, lane half h
  __device__ static __forceinline__ frag ld_k(const storage* row, int ks, int h) {
    return *reinterpret_cast<const frag*>(row + ks * 16 + 8 * h);
  }
  // operand matching an accumulator-fed partner: k-step s over 32 rows
  __device__ static __forceinline__ frag ld_kacc(const storage* row, int s, int h) {
    return *reinterpret_cast<const frag*>(row + 16 * s + 8 * h);
  }
  // A operand read transposed from a row-major LDS tile: p = tile + lane
  // offset (tr_lane_off) + k0 * ld + m0 gives X[k0 + 8h + t][m0 + sigma(l%32)]
  __device__ static __forceinline__ frag ld_tr(const storage* p, int ld) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * ld));
    const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag, both);
  }
  // B operand from accumulator registers 8s .. 8s+7
  __device__ static __forceinline__ frag from_acc(const floatx16& a, int s) {
    frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (__bf16)a[8 * s + j];
    return f;
  }
  __device__ static __forceinline__ float to_f(storage x) {
    return __uint_as_float(((uint32_t)x) << 16);
  }
  __device__ static __forceinline__ storage from_f(float x) {
    __bf16 b = (__bf16)x;
    return *reinterpret_cast<storage*>(&b);
  }
};

struct F32 {
  using storage = float;
  using frag = float;
  static constexpr int KPI = 2;
  static constexpr int VEC = 1;
  static constexpr int ACC_KSTEPS = 16;
  static constexpr int CHUNK = 4;
  static constexpr bool TR_READ = false;  // no 32-bit transposed read: transposed LDS tiles

  __device__ static __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag ld_k(const storage* row, int ks, int h) {
    return row[ks * 2 + h];
  }
  __device__ static __forceinline__ frag ld_kacc(const storage* row, int s, int h) {
    return row[16 * (s >> 3) + 8 * h + (s & 7)];
  }
  __device__ static __forceinline__ frag from_acc(const floatx16& a, int s) { return a[s]; }
  __device__ static __forceinline__ float to_f(storage x) { return x; }
  __device__ static __forceinline__ storage from_f(float x) { return x; }
};

// The wave's index in its workgroup as a scalar: every value derived from it
// (the wave's rows and blocks, the branches on them) then stays in scalar
// registers and scalar branches instead of taking vector registers.
__device__ __forceinline__ int wave_index(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

// Max and sum of a value over the lane pair (l, l ^ 32), equal on both lanes,
// through v_permlane32_swap (a VALU exchange of the wave's halves, no LDS
// round trip). With both operands v it returns the lower lane's value first
// and the upper lane's second on either lane, so the sum's order is the same
// on both. Every lane of the wave must be active.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of the elements of an operand fragment, in fp32 (bf16 pairs through
// v_dot2 with (1, 1): exact products, one fp32 accumulation per pair).
template <class E>
__device__ __forceinline__ float frag_sum(const typename E::frag& f) {
  if constexpr (sizeof(typename E::storage) == 2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x2 p = {f[2 * j], f[2 * j + 1]};
      s = __builtin_amdgcn_fdot2_f32_bf16(p, one, s, false);
    }
    return s;
  } else {
    return f;
  }
}

// LDS row strides (elements) with a 16-byte pad against bank conflicts
template <class E, int COLS>
struct Ld {
  static constexpr int value = COLS + 16 / (int)sizeof(typename E::storage);
};

// Wait for every outstanding vector-memory load (s_waitcnt vmcnt(0)). Placed
// unconditionally before the LDS stores that consume prefetched tile
// registers, so the compiler's wait analysis sees no load pending at loop
// heads and puts no memory wait inside the MFMA sequences.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// Workgroup id -> work item
// ---------------------------------------------------------------------------

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs. Give
// each XCD a contiguous range of logical ids, so that the blocks of one head
// (which share K and V) run under one L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  int xcd = id & 7, slot = id >> 3;
  int q = total >> 3, r = total & 7;
  return xcd * q + min(xcd, r) + slot;
}

// A logical id from xcd_remap as (head, rank) over ngroups items per head.
// When every XCD's range holds whole heads, the ids run rank-major over
// the XCD's heads: it starts the items of rank 0 (the longest, where the
// caller orders them so) of all its heads before any of rank 1, which keeps
// its slots evenly loaded to the end. Otherwise head-major.
__device__ __forceinline__ void xcd_split(int wg, int total, int ngroups, int& bh, int& rank) {
  const int per = total >> 3;
  if ((total & 7) == 0 && per % ngroups == 0) {
    const int hpx = per / ngroups, x = wg / per, t = wg - x * per;
    bh = x * hpx + t % hpx;
    rank = t / hpx;
  } else {
    bh = wg / ngroups;
    rank = wg % ngroups;
  }
}

// Element strides of a [B, H, N, D] tensor view with D contiguous: batch,
// head, row. [B, H, N, D] storage has (H N D, N D, D); token-major
// [B, N, H, D] storage has (N H D, D, H D).
struct Lay {
  long long sb, sh;
  int sn;
  // offset of head bh = b H + h
  __device__ __forceinline__ size_t head(int bh, int H) const {
    return (size_t)((long long)(bh / H) * sb + (long long)(bh % H) * sh);
  }
};

// ---------------------------------------------------------------------------
// Global <-> LDS tile movement (64 rows x D columns)
// ---------------------------------------------------------------------------

// One task = a pair of rows (2rp, 2rp+1) x one 16-byte column chunk.
template <class E, int D, int NTHR>
struct TileIO {
  using S = typename E::storage;
  static constexpr int CPR = D / E::CHUNK;          // chunks per row
  static constexpr int NTASK = 32 * CPR;
  static constexpr int TPT = (NTASK + NTHR - 1) / NTHR;   // tasks per thread
  uint4 r0[TPT], r1[TPT];

  // Rows row0 .. row0 + 63 of an [nrows][D] array whose rows are rs
  // elements apart (D contiguous). The address is a wave-uniform tile base
  // plus a 32-bit per-thread byte offset, so the loads take the scalar-base
  // form; rows past the end repeat the last row (finite values that every
  // kernel masks or weights by zero).
  __device__ __forceinline__ void load(const S* base, int row0, int nrows, int tid, int rs) {
    const int RB = rs * (int)sizeof(S);       // bytes per row
    const char* tb = reinterpret_cast<const char*>(base + (size_t)row0 * rs);
    const int lastb = min(nrows - 1 - row0, 63) * RB;   // byte offset of the last valid row of the tile
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      int task = tid + t * NTHR;
      // defined on every path, so the registers are never demoted to scratch
      r0[t] = make_uint4(0, 0, 0, 0);
      r1[t] = make_uint4(0, 0, 0, 0);
      if (NTASK % NTHR == 0 || task < NTASK) {
        const int rp = task / CPR, c = task % CPR;
        const int cb = c * E::CHUNK * (int)sizeof(S);
        const uint32_t oa = (uint32_t)(min(2 * rp * RB, lastb) + cb);
        const uint32_t ob = (uint32_t)(min((2 * rp + 1) * RB, lastb) + cb);
        r0[t] = *reinterpret_cast<const uint4*>(tb + oa);
        r1[t] = *reinterpret_cast<const uint4*>(tb + ob);
      }
    }
  }
  // row-major tile [64][LD]
  template <int LD>
  __device__ __forceinline__ void store_rows(S* tile, int tid) const {
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      int task = tid + t * NTHR;
      if (NTASK % NTHR == 0 || task < NTASK) {
        int rp = task / CPR, c = task % CPR;
        *reinterpret_cast<uint4*>(tile + (2 * rp) * LD + c * E::CHUNK) = r0[t];
        *reinterpret_cast<uint4*>(tile + (2 * rp + 1) * LD + c * E::CHUNK) = r1[t];
      }
    }
  }
  // transposed tile [D][LDT]: element (row, col) at tile[col * LDT + row]
  template <int LDT>
  __device__ __forceinline__ void store_trans(S* tile, int tid) const {
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      int task = tid + t * NTHR;
      if (NTASK % NTHR == 0 || task < NTASK) {
        int rp = task / CPR, c = task % CPR;
        if constexpr (sizeof(S) == 2) {
          const uint32_t* a = reinterpret_cast<const uint32_t*>(&r0[t]);
          const uint32_t* b = reinterpret_cast<const uint32_t*>(&r1[t]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t lo = (a[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            uint32_t hi = (b[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            *reinterpret_cast<uint32_t*>(tile + (c * 8 + e) * LDT + 2 * rp) = lo | (hi << 16);
          }
        } else {
          const float* a = reinterpret_cast<const float*>(&r0[t]);
          const float* b = reinterpret_cast<const float*>(&r1[t]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<float2*>(tile + (c * 4 + e) * LDT + 2 * rp) = make_float2(a[e], b[e]);
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA tile products
// ---------------------------------------------------------------------------

// acc[kh] (kh = 0, 1) = T[32kh + sigma(rho)][:] . F^T over D, where T is a
// row-major LDS tile [64][LD] (k along the row) and F the caller's B operand
// fragments (one per k-step).
template <class E, int D, int LD>
__device__ __forceinline__ void tile_x_frags(floatx16 acc[2], const typename E::storage* tile,
                                             const typename E::frag* fr, int l32, int h) {
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    floatx16 c = {};
    const typename E::storage* row = tile + (32 * kh + sigma32(l32)) * LD;
#pragma unroll
    for (int ks = 0; ks < D / E::KPI; ++ks) c = E::mma(E::ld_k(row, ks, h), fr[ks], c);
    acc[kh] = c;
  }
}

// tile_x_frags for RG groups of 32 rows at once: each A fragment read from
// LDS feeds RG products (acc[g][kh] for row group g), so LDS reads per
// product drop by RG.
template <class E, int D, int LD, int RG>
__device__ __forceinline__ void tile_x_frags_rg(floatx16 (&acc)[RG][2], const typename E::storage* tile,
                                                const typename E::frag (&fr)[RG][D / E::KPI], int l32, int h) {
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g][kh] = floatx16{};
    const typename E::storage* row = tile + (32 * kh + sigma32(l32)) * LD;
#pragma unroll
    for (int ks = 0; ks < D / E::KPI; ++ks) {
      const typename E::frag a = E::ld_k(row, ks, h);
#pragma unroll
      for (int g = 0; g < RG; ++g) acc[g][kh] = E::mma(a, fr[g][ks], acc[g][kh]);
    }
  }
}

// One 32-row half kh of tile_x_frags.
template <class E, int D, int LD>
__device__ __forceinline__ floatx16 tile_x_half(const typename E::storage* tile, const typename E::frag* fr,
                                                int l32, int h, int kh) {
  floatx16 c = {};
  const typename E::storage* row = tile + (32 * kh + sigma32(l32)) * LD;
#pragma unroll
  for (int ks = 0; ks < D / E::KPI; ++ks) c = E::mma(E::ld_k(row, ks, h), fr[ks], c);
  return c;
}

// Load the B operand fragments of one row (k along the row) from global memory.
template <class E, int D>
__device__ __forceinline__ void load_row_frags(typename E::frag* fr, const typename E::storage* rowp,
                                               bool valid, int h) {
#pragma unroll
  for (int ks = 0; ks < D / E::KPI; ++ks) {
    if (valid) {
      fr[ks] = E::ld_k(rowp, ks, h);
    } else {
      fr[ks] = typename E::frag{};
    }
  }
}

// ---------------------------------------------------------------------------
// One lane's NE consecutive elements of a row: 16-byte loads kept raw, and
// acc += c x accumulated from them in fp32
// ---------------------------------------------------------------------------
template <class E, int NE>
struct RowChunk {
  static constexpr int NV = NE * (int)sizeof(typename E::storage) / 16;
  uint4 w[NV];
  __device__ __forceinline__ void load(const typename E::storage* p) {
#pragma unroll
    for (int c = 0; c < NV; ++c) w[c] = *reinterpret_cast<const uint4*>(p + c * (16 / sizeof(typename E::storage)));
  }
  __device__ __forceinline__ float elem(int i) const {   // element i (compile-time index)
    const uint4 v = w[i / (16 / (int)sizeof(typename E::storage))];
    const int e = i % (16 / (int)sizeof(typename E::storage));
    uint32_t u;
    if constexpr (sizeof(typename E::storage) == 2) {
      const int wi = e >> 1;
      u = wi == 0 ? v.x : (wi == 1 ? v.y : (wi == 2 ? v.z : v.w));
      return __uint_as_float((e & 1) ? (u & 0xFFFF0000u) : (u << 16));
    } else {
      u = e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
      return __uint_as_float(u);
    }
  }
  // sum of this chunk's elements times another's, in fp32
  __device__ __forceinline__ float dot(const RowChunk& o) const {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i) s = fmaf(elem(i), o.elem(i), s);
    return s;
  }
  __device__ __forceinline__ void fma(float (&acc)[NE], float c) const {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const uint32_t ww[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(typename E::storage) == 2) {
          acc[8 * k + 2 * e] = fmaf(c, __uint_as_float(ww[e] << 16), acc[8 * k + 2 * e]);
          acc[8 * k + 2 * e + 1] = fmaf(c, __uint_as_float(ww[e] & 0xFFFF0000u), acc[8 * k + 2 * e + 1]);
        } else {
          acc[4 * k + e] = fmaf(c, __uint_as_float(ww[e]), acc[4 * k + e]);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Powers of positive parts, specialised for kappa = 1, 2, 4
// ---------------------------------------------------------------------------

enum PowMode { PM_K1 = 0, PM_K2 = 1, PM_K4 = 2, PM_GEN = 3, PM_SOFTMAX = 4 };

// x^e for x > 0 via the hardware base-2 exp / log
__device__ __forceinline__ float powpos(float x, float e) {
  return __builtin_amdgcn_exp2f(e * __builtin_amdgcn_logf(x));
}

// x = min(max(s c - t, 0), 1) in one fused multiply-add with the clamp
// modifier. At the final threshold every x lies in [0, 1]: tau >= max z - 1
// for the exact root, so only rounding can take x past 1, by a few ulp.
__device__ __forceinline__ float xclamp(float s, float c, float t) {
  return __builtin_amdgcn_fmed3f(fmaf(s, c, -t), 0.f, 1.f);
}

// The argument of p and u in the backward: the clamped x of entmax, or
// x = s c - lse2 (c = log2(e)/sqrt(d)) of the softmax comparator.
template <int PM>
__device__ __forceinline__ float xarg(float s, float c, float t) {
  if constexpr (PM == PM_SOFTMAX) return fmaf(s, c, -t);
  else return xclamp(s, c, t);
}

// Whether p > 0 at an argument from xarg: x > 0 on the entmax support; any
// finite x for softmax (masked scores are -inf).
template <int PM>
__device__ __forceinline__ bool pos_arg(float x) {
  if constexpr (PM == PM_SOFTMAX) return x > -INFINITY;
  else return x > 0.f;
}

// p and u of a clamped x in [0, 1] (x = 0 off the support); for the softmax
// comparator p = u = 2^x.
template <int PM>
__device__ __forceinline__ float pk01(float x, float kappa) {
  if constexpr (PM == PM_SOFTMAX) return __builtin_amdgcn_exp2f(x);
  else if constexpr (PM == PM_K1) return x;
  else if constexpr (PM == PM_K2) return x * x;
  else if constexpr (PM == PM_K4) { const float y = x * x; return y * y; }
  else return __builtin_amdgcn_exp2f(kappa * __builtin_amdgcn_logf(x));   // 0 at x = 0 (kappa > 0)
}
template <int PM>
__device__ __forceinline__ float uk01(float x, float kappa) {
  if constexpr (PM == PM_SOFTMAX) return __builtin_amdgcn_exp2f(x);
  else if constexpr (PM == PM_K1) return x > 0.f ? 1.f : 0.f;
  else if constexpr (PM == PM_K2) return x;
  else if constexpr (PM == PM_K4) return x * x * x;
  else return x > 0.f ? __builtin_amdgcn_exp2f((kappa - 1.f) * __builtin_amdgcn_logf(x)) : 0.f;
}

__device__ __forceinline__ int pow_mode_of(float kappa) {
  if (kappa == 1.f) return PM_K1;
  if (kappa == 2.f) return PM_K2;
  if (kappa == 4.f) return PM_K4;
  return PM_GEN;
}

}  // namespace ea
