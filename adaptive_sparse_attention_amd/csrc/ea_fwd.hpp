// Forward kernels of alpha-entmax attention.
//
//  fwd_max  : the row max m of the scores (one sweep over the visible keys).
//  fwd_init : histogram pass. Streams every visible key block through LDS
//             and counts the scores within 1 of m into a (B + 1)-bin left-
//             edge histogram (z units, B = 256 bins per unit unless the caller
//             picks 32 .. 512) held in LDS. Solving the
//             entmax equation on the histogram gives the lower bound tau_h of
//             each row. It also records the key blocks that hold any such
//             score; every support member is among them, since
//             tau >= max z - 1.
//             (AdaSplash-2 summary, gist.science German page, section 2
//             "Kernidee", steps 1-2.)
//  fwd_list : the same bound and kept keys for groups of rows whose windows
//             hold few scores, from short per-lane lists instead of the
//             histogram (which then takes only the other groups).
//  fwd_refine : starting from tau_h, each pass evaluates
//             f(t) = sum_j (z_j - t)_+^kappa - 1 and its derivatives over the
//             candidate blocks and takes one safeguarded step (Halley for
//             alpha <= 1.5, Newton for 1.5 < alpha <= 2, secant for alpha > 2,
//             bisection when the step leaves the bracket), until the stop
//             rule holds; pass 1 also builds the block mask at tau_h.
//             (gist.science Hindi page, section 2, hybrid solver strategy;
//             German page, section 2 "Kernidee", step 3.)
//  fwd_out  : P.V over the set mask bits only, walked with find-first-set,
//             and the mask at the final tau. (Hindi page, section 2,
//             efficient traversal.) When the caller asks for the
//             backward's state, the same walk also forms, for rows formed
//             by tiles, vbar = sum_j u_j v_j / sum_j u_j with
//             u = x_+^(kappa-1): the backward then gets the per-row
//             delta = sum_j u_j dP_j / sum_j u_j as dO . vbar, since
//             dP_j = dO . v_j, without a sweep of its own; rows formed by
//             gathering leave their support list there instead.
#pragma once

#include "ea_common.hpp"

namespace ea {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* tau;
  uint32_t* mask;
  float* state;              // optional [B,H,N] records of D fp32 words: the backward's state
  float* tau_h_out;          // optional
  uint8_t* passes_out;       // optional
  uint8_t* iters_out;        // optional: solver steps per row (each safeguarded step)
  uint32_t* tiles_per_pass;  // optional [MAX_PASSES + 2]
  uint32_t* unconverged;     // optional [1]
  uint32_t* halves_out;      // optional [1]: 32x32 sub-tiles holding some p > 0
  uint32_t* gathered;        // optional [2]: rows the output pass gathered, and their sub-tiles
  int B, H, N, nb, W;
  int G;                     // query heads per key/value head (grouped-query attention; 1 = one each)
  Lay lq, lkv;               // strides of q, o and of k, v
  int causal;
  int pow_mode;              // PowMode of kappa (histogram solve)
  int nohist;                // solver mode without the histogram pass
  int plain;                 // every solver step takes a streamed pass (no kept scores, shifted
                             // sums or top-k steps)
  int pass_cap;              // streamed passes allowed per row (the mode's default when 0)
  int listpass;              // the list pass ran before the histogram kernel (fwd_list_kernel)
  float alpha, kappa;
  float zscale;              // (alpha - 1) / sqrt(d)
  float zscaleB;             // bins * zscale (bins per unit of z of the histogram)
  float delta_h;             // 1 / bins: histogram bin width (z units)
  int bins;                  // histogram bins per unit of z
};

enum Solver { SV_HALLEY = 0, SV_NEWTON = 1, SV_SECANT = 2 };

constexpr float BRACKET_PAD = 1.0f / 4096;    // widening of [tau_h, tau_h + 1/B]
constexpr float MASK_PAD = 1.0f / 4096;       // mask at tau_h is taken at tau_h - pad
constexpr float STEP_TOL = 1e-6f;
constexpr float F_TOL = 1e-6f;
constexpr int TOPK = 4;             // x > 0 values a pass keeps per row (other kappa)
constexpr int XK = 4;               // smallest x > 0 a pass keeps per row (kappa = 1, 2, 4)
// The histogram pass also keeps, per lane, the keys of the LIST_LANE
// largest window scores it bins (ranked by the score rounded down to a
// quantum of about 1.5e-5 in z). A lane's list holds every key of the lane
// with a score above t when the lane binned at most LIST_LANE scores or the
// quantum of its smallest kept score ends below t; a lane stops keeping
// after LIST_SCAN scores, which bounds the cost where windows are dense and
// the lists would go unused. After the solve, the four lanes of a row pool
// the kept keys whose scores may lie above lo = max(tau_h - BRACKET_PAD, the
// window's lower edge) (the refinement's bracket never goes below it) into
// the row of o, free until the output pass writes it (every o row holds at
// least 128 bytes):
//   word 0: the pooled count n <= LIST_CAP, or LIST_NONE when some lane's
//           list may miss a key above lo, or more than LIST_CAP may lie
//           above it, or key indices do not fit 16 bits;
//   word 1: lo (float);
//   words 2 .. 2 + LIST_CAP: the n scores, written by the refinement;
//   bytes 8 + 4 LIST_CAP ..: the n keys (uint16).
// The refinement forms the n scores, solves the row on them, and stores
// them; where it does so for every row of a workgroup it also sets
// LIST_GATHER in word 0 of each of its rows, and the output pass then forms
// those rows by gathering the rows of V of the support instead of streaming
// tiles. Word 0 with LIST_GATHER set reads as a NaN in o's element type,
// which the output pass never writes.
constexpr int LIST_LANE = 7;
constexpr int LIST_SCAN = 16;
constexpr uint32_t LIST_NONE = 0xFFu;
constexpr int MAX_VSTEPS = 40;      // solver steps on those values without a new pass

// Set scores of invalid keys (key >= N, or key > query when causal) to -inf.
// Score register r of key half kh, lane half h, belongs to key
// key0 + 32 kh + acc_row(r, h).
__device__ __forceinline__ void mask_keys(floatx16 acc[2], int key0, int N, int causal, int qrow, int h) {
  // key = key0 + 8h + off(kh, r) with a compile-time offset; invalid past lim
  const int lim = (causal ? min(qrow, N - 1) : N - 1) - key0 - 8 * h;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 32 * kh + 16 * (r >> 3) + (r & 7);
      if (off > lim) acc[kh][r] = -INFINITY;
    }
}

__device__ __forceinline__ float tile_max(const floatx16 acc[2]) {
  float m = acc[0][0];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[kh][r]);
  return m;
}

__device__ __forceinline__ float half_max(const floatx16& x) {
  float m = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, x[r]);
  return m;
}

// maxima of the four groups of 8 scores (registers 8*(g&1) .. +7 of half g>>1).
// The IEEE maximum (NaN-propagating; the scores hold none, masked keys -inf)
// goes to v_maximum3_f32 without quieting its operands first, four
// instructions per group where fmaxf takes six; for these scores it returns
// the same values.
__device__ __forceinline__ void group_max(const floatx16 acc[2], float gm[4]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int kh = g >> 1, r0 = 8 * (g & 1);
    float m = __builtin_elementwise_maximum(acc[kh][r0], acc[kh][r0 + 1]);
#pragma unroll
    for (int r = 2; r < 8; ++r) m = __builtin_elementwise_maximum(m, acc[kh][r0 + r]);
    gm[g] = m;
  }
}

// Words of one row's histogram, padded so every row starts 16-byte aligned.
template <bool H32, int NB> struct HistRow {
  static constexpr int SLOTS_PER_WORD = H32 ? 1 : 2;
  static constexpr int WORDS = ((NB + 1 + SLOTS_PER_WORD - 1) / SLOTS_PER_WORD + 3) & ~3;
  static constexpr int PER_BLOCK = 4 * SLOTS_PER_WORD;   // slots per 16-byte block
};

template <bool H32>
__device__ __forceinline__ uint32_t hist_get(const uint32_t* row, int s) {
  if constexpr (H32) return row[s];
  else return reinterpret_cast<const uint16_t*>(row)[s];
}

// The top bin (depth 0) holds at least the row's maximum, so a 16-bit count
// of 0 there can only be 65536 wrapped (a row of 65536 scores, all in it).
template <bool H32, int NB>
__device__ __forceinline__ uint32_t hist_top(const uint32_t* row) {
  const uint32_t c = hist_get<H32>(row, NB);
  return (!H32 && c == 0u) ? 65536u : c;
}

// Calls f(y, c) for every non-empty bin of quarter qd of the depths 1..NB
// (depths qd Q + 1 .. qd Q + Q, Q = NB / 4, at slots NB - y), in increasing
// depth, until f returns true. Empty stretches are skipped 16 bytes at a
// time. Depth 0 (slot NB, the top bin) belongs to no quarter.
template <bool H32, int NB, class F>
__device__ __forceinline__ void for_quarter_bins(const uint32_t* row, int qd, F&& f) {
  constexpr int PER = HistRow<H32, NB>::PER_BLOCK;
  constexpr int QB = NB / 4 / PER;          // 16-byte blocks per quarter
  const int b0 = (3 - qd) * QB;             // lowest block of the quarter
#pragma unroll 1
  for (int b = b0 + QB - 1; b >= b0; --b) {
    const uint4 w = reinterpret_cast<const uint4*>(row)[b];
    if ((w.x | w.y | w.z | w.w) == 0) continue;
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      const uint32_t c = H32 ? ws[j] : ((ws[j >> 1] >> (16 * (j & 1))) & 0xffffu);
      if (c && f(NB - (b * PER + j), c)) return;
    }
  }
}

// sums over the four lanes of a quad (lane order = quarter order)
__device__ __forceinline__ double quad_prefix(double v, int qd) {   // inclusive
  double t = __shfl_up(v, 1, 4);
  if (qd >= 1) v += t;
  t = __shfl_up(v, 2, 4);
  if (qd >= 2) v += t;
  return v;
}
__device__ __forceinline__ uint32_t quad_prefix_u(uint32_t v, int qd) {   // inclusive
  uint32_t t = __shfl_up(v, 1, 4);
  if (qd >= 1) v += t;
  t = __shfl_up(v, 2, 4);
  if (qd >= 2) v += t;
  return v;
}
__device__ __forceinline__ double quad_sum(double v) {
  v += __shfl_xor(v, 1, 4);
  v += __shfl_xor(v, 2, 4);
  return v;
}

// ---------------------------------------------------------------------------
// Histogram solve: tau_h = root of sum_bins c (e - t)_+^kappa - 1, e = k/B.
// The histogram holds the B + 1 bins k = ktop - y, y = 0..B, of one row at
// slots B - y. A bin at depth y contributes c_y ((T - y)/B)^kappa for
// T > y, and tau = (ktop - T) / B. Going down from the top, the root lies
// in the first gap (y_prev, y] where the sum at T = y reaches 1, with the
// bins above y as the fixed active set.
// The four lanes of a quad solve one row together, each over a quarter of
// the depths: power sums c y^m (m = 0..4) per quarter, an exclusive prefix
// over the quad, then each lane looks for the first crossing in its own
// quarter; the first quarter with one (else the last, with every bin
// active) gives the active set. Every lane of the quad returns the same T.
// ---------------------------------------------------------------------------
// Sums c, c y, c y^2 over the L bins at depths ya .. ya + L - 1 of a row
// of 16-bit counters (slots NB - ya - L + 1 .. NB - ya; the callers' ranges
// start at a multiple of L slots, so the L / 2 words load aligned), without
// branches: the depth offsets within the range are constants. Exact in 32
// bits while the row holds at most 65536 scores (so at most 65535 below the
// top bin, which no range includes) and y <= 256.
template <int NB, int L>
__device__ __forceinline__ void range_sums16(const uint32_t* row, int ya, uint32_t& C, uint32_t& S1, uint32_t& S2) {
  static_assert(L % 2 == 0, "whole words");
  constexpr int NWD = L / 2;
  const uint32_t* wp = row + (NB - ya - L + 1) / 2;
  uint32_t w[NWD];
  if constexpr (NWD % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NWD / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(wp)[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (NWD == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(wp);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NWD; ++i) w[i] = wp[i];
  }
  uint32_t cp = 0, a = 0, b = 0;   // cp: both halves at once (neither half carries)
#pragma unroll
  for (int k = 0; k < NWD; ++k) {
    const uint32_t lo = w[k] & 0xFFFFu, hi = w[k] >> 16;
    const uint32_t vlo = (uint32_t)(L - 1 - 2 * k), vhi = (uint32_t)(L - 2 - 2 * k);   // depth - ya
    cp += w[k];
    a += lo * vlo + hi * vhi;
    b += lo * (vlo * vlo) + hi * (vhi * vhi);
  }
  C = (cp & 0xFFFFu) + (cp >> 16);
  const uint32_t y0 = (uint32_t)ya;
  S1 = y0 * C + a;
  S2 = y0 * y0 * C + 2u * y0 * a + b;
}

template <bool H32, int NB>
__device__ __forceinline__ double hist_solve_quad(const uint32_t* row, int lane, int pm, float kappa) {
  constexpr double B1 = NB, B2 = (double)NB * NB, B4 = B2 * B2;
  const int qd = lane & 3, qbase = lane & ~3;
  const double ctop = (double)hist_top<H32, NB>(row);   // depth 0
  if constexpr (!H32 && NB == 256) {
    if (pm == PM_K1 || pm == PM_K2) {
      // H(y) = sum over bins y' <= y of c (y - y')^kappa grows with y, and
      // the root lies in (y* - 1, y*] for the least depth y* with
      // H(y*) >= B^kappa, with the bins above y* as the active set: the same
      // set a scan down the non-empty bins stops with. The quad finds y* in
      // four rounds of four: quarters of 64 depths, then 16, 4 and single
      // depths of the chosen one, each round from the sums of its four
      // ranges and their prefix over the lanes.
      auto reach = [&](uint32_t C, uint32_t S1, uint32_t S2, long long y) -> bool {   // H(y) >= B^kappa
        if (pm == PM_K1) return (long long)C * y - (long long)S1 - (long long)NB >= 0;
        return ((long long)C * y - 2 * (long long)S1) * y + (long long)S2 - (long long)NB * NB >= 0;
      };
      uint32_t bC = hist_top<false, NB>(row), bS1 = 0, bS2 = 0;   // sums above the current range
      int ya = 1;                                                 // its first depth
      // one round over four ranges of L depths from ya, lane qd taking the
      // qd-th: the first range (in depth order) whose end reaches becomes
      // the current one; if none does, every bin is active
      auto narrow = [&](auto lc) -> bool {
        constexpr int L = decltype(lc)::value;
        const int y0 = ya + qd * L;
        uint32_t C, S1, S2;
        if constexpr (L == 1) {
          C = hist_get<false>(row, NB - y0);
          S1 = C * (uint32_t)y0;
          S2 = S1 * (uint32_t)y0;
        } else {
          range_sums16<NB, L>(row, y0, C, S1, S2);
        }
        const uint32_t iC = quad_prefix_u(C, qd), iS1 = quad_prefix_u(S1, qd), iS2 = quad_prefix_u(S2, qd);
        const bool hit = reach(bC + iC, bS1 + iS1, bS2 + iS2, (long long)(y0 + L - 1));
        const unsigned qb = (unsigned)(__ballot(hit) >> qbase) & 0xFu;
        const bool none = qb == 0u;
        const int sel = none ? 3 : __builtin_ctz(qb);
        // from lane sel: the sums through its range (none) or above it
        const uint32_t xC = none ? iC : iC - C, xS1 = none ? iS1 : iS1 - S1, xS2 = none ? iS2 : iS2 - S2;
        bC += __shfl(xC, qbase + sel, 64);
        bS1 += __shfl(xS1, qbase + sel, 64);
        bS2 += __shfl(xS2, qbase + sel, 64);
        ya += sel * L;
        return !none;
      };
      if (narrow(std::integral_constant<int, 64>{})) {
        narrow(std::integral_constant<int, 16>{});
        narrow(std::integral_constant<int, 4>{});
        narrow(std::integral_constant<int, 1>{});   // ya = y*; b* = the bins above it
      }
      const double c0 = bC, s1 = bS1, s2 = bS2;
      if (pm == PM_K1) return (s1 + B1) / c0;
      const double disc = fmax(s1 * s1 - c0 * (s2 - B2), 0.0);
      return (s1 + sqrt(disc)) / c0;
    }
  }
  if (!H32 && NB <= 256 && (pm == PM_K1 || pm == PM_K2)) {
    // 16-bit counters: at most 65536 scores, at most 65535 of them below the
    // top bin, so the sums of c, c y and c y^2 (y <= 256) stay below 2^32 and
    // add exactly in 32-bit integers
    // the quarter's 16-byte blocks, read at once (no chain of dependent reads)
    constexpr int PER = HistRow<H32, NB>::PER_BLOCK;
    constexpr int QB = NB / 4 / PER;
    const int b0 = (3 - qd) * QB;
    uint4 blk[QB];
#pragma unroll
    for (int i = 0; i < QB; ++i) blk[i] = reinterpret_cast<const uint4*>(row)[b0 + i];
    // visits the non-empty bins in increasing depth while go() holds
    auto scan = [&](auto&& f) {
#pragma unroll
      for (int i = QB - 1; i >= 0; --i) {
        const uint4 w = blk[i];
        if ((w.x | w.y | w.z | w.w) == 0) continue;
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = PER - 1; j >= 0; --j) {
          const uint32_t c = (ws[j >> 1] >> (16 * (j & 1))) & 0xffffu;
          if (c) f(NB - ((b0 + i) * PER + j), c);
        }
      }
    };
    uint32_t C = 0, S1 = 0, S2 = 0;
    scan([&](int y, uint32_t c) {
      C += c;
      S1 += c * (uint32_t)y;
      S2 += c * (uint32_t)(y * y);
    });
    C = quad_prefix_u(C, qd) - C;
    S1 = quad_prefix_u(S1, qd) - S1;
    S2 = quad_prefix_u(S2, qd) - S2;
    C += hist_top<H32, NB>(row);
    // the binned sum at T = y (times B^kappa) minus B^kappa, active set C, S1, S2
    auto g = [&](long long y) -> long long {
      if (pm == PM_K1) return (long long)C * y - (long long)S1 - (long long)NB;
      return ((long long)C * y - 2 * (long long)S1) * y + (long long)S2 - (long long)NB * NB;
    };
    int yc = -1;
    scan([&](int y, uint32_t c) {
      if (yc >= 0) return;
      if (C > 0 && g(y) >= 0) {
        yc = y;
        return;
      }
      C += c;
      S1 += c * (uint32_t)y;
      S2 += c * (uint32_t)(y * y);
    });
    const unsigned qb = (unsigned)(__ballot(yc >= 0) >> qbase) & 0xFu;
    const int src = qb ? __builtin_ctz(qb) : 3;
    const double c0 = C, s1 = S1, s2 = S2;
    double T;
    if (pm == PM_K1) {
      T = (s1 + B1) / c0;
    } else {
      const double disc = fmax(s1 * s1 - c0 * (s2 - B2), 0.0);
      T = (s1 + sqrt(disc)) / c0;
    }
    return __shfl(T, qbase + src, 64);
  }
  if (pm == PM_K1 || pm == PM_K2 || pm == PM_K4) {
    double S[5] = {0, 0, 0, 0, 0};
    for_quarter_bins<H32, NB>(row, qd, [&](int y, uint32_t c) {
      double p = c;
#pragma unroll
      for (int m = 0; m < 5; ++m) { S[m] += p; p *= y; }
      return false;
    });
#pragma unroll
    for (int m = 0; m < 5; ++m) S[m] = quad_prefix(S[m], qd) - S[m];
    S[0] += ctop;
    // the binned sum at T = y (times B^kappa) minus B^kappa, active set S
    auto g = [&](double y) {
      if (pm == PM_K1) return S[0] * y - S[1] - B1;
      if (pm == PM_K2) return (S[0] * y - 2.0 * S[1]) * y + S[2] - B2;
      const double y2 = y * y;
      return y2 * y2 * S[0] - 4 * y2 * y * S[1] + 6 * y2 * S[2] - 4 * y * S[3] + S[4] - B4;
    };
    int yc = -1;
    for_quarter_bins<H32, NB>(row, qd, [&](int y, uint32_t c) {
      if (S[0] > 0 && g((double)y) >= 0) { yc = y; return true; }
      double p = c;
#pragma unroll
      for (int m = 0; m < 5; ++m) { S[m] += p; p *= y; }
      return false;
    });
    const unsigned qb = (unsigned)(__ballot(yc >= 0) >> qbase) & 0xFu;
    const int src = qb ? __builtin_ctz(qb) : 3;
    double T;
    if (pm == PM_K1) {
      T = (S[1] + B1) / S[0];
    } else if (pm == PM_K2) {
      const double disc = fmax(S[1] * S[1] - S[0] * (S[2] - B2), 0.0);
      T = (S[1] + sqrt(disc)) / S[0];
    } else {
      // the quartic is convex and increasing on the gap: Newton from its
      // right end converges monotonically from above
      auto dg = [&](double y) {
        const double y2 = y * y;
        return 4 * y2 * y * S[0] - 12 * y2 * S[1] + 12 * y * S[2] - 4 * S[3];
      };
      T = yc >= 0 ? (double)yc : B1;
      for (int it = 0; it < 40; ++it) {
        const double gv = g(T), dv = dg(T);
        if (!(dv > 0)) break;
        const double Tn = T - gv / dv;
        if (!(Tn < T)) break;
        T = Tn;
        if (gv < 1e-9 * B4) break;
      }
    }
    return __shfl(T, qbase + src, 64);
  }
  // general kappa: the binned sum over the bins above depth ylim, summed over
  // the quad; first the integer depth y with G(y) >= 0 (binary search, G
  // increasing), then bisection on [y - 1, y] with that active set
  auto G = [&](double T, int ylim) {
    double acc = 0;
    for_quarter_bins<H32, NB>(row, qd, [&](int y, uint32_t c) {
      if (y >= ylim) return true;
      acc += (double)c * (double)powpos((float)((T - y) * (1.0 / B1)), kappa);
      return false;
    });
    if (qd == 0) acc += ctop * (double)powpos((float)(T * (1.0 / B1)), kappa);
    return quad_sum(acc) - 1.0;
  };
  int ylo = 0, yhi = NB;   // G(ylo, ylo) < 0; yhi: the first y with G >= 0, or NB
  while (yhi - ylo > 1) {
    const int ym = (ylo + yhi) >> 1;
    if (G((double)ym, ym) >= 0) yhi = ym;
    else ylo = ym;
  }
  double lo = yhi - 1, hi = yhi;
  for (int it = 0; it < 18; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (G(mid, yhi) >= 0) hi = mid;
    else lo = mid;
  }
  return hi;
}

// Safeguard and stop rule of one solver step from te (f = f(te)) to tn: a
// step outside the bracket [lo, hi] (or NaN, or one the caller rejects)
// becomes the bracket midpoint, except when f already meets the tolerance at
// te, which then stands. Returns whether the row has converged; tn is the
// next threshold either way.
__device__ __forceinline__ bool safeguard_step(float& tn, float te, float f, float lo, float hi, bool ok) {
  const bool inside = (tn >= lo) && (tn <= hi) && ok;
  const bool fsmall = fabsf(f) <= F_TOL;
  if (!inside) tn = fsmall ? te : 0.5f * (lo + hi);
  return fsmall || fabsf(tn - te) <= STEP_TOL * fmaxf(1.f, fabsf(te));
}

// ---------------------------------------------------------------------------
// fwd_max: the row max m of the raw scores q.k over the visible keys. A
// workgroup takes 128 query rows and one chunk of at most MAX_CHUNK key
// blocks, so long causal rows are split over several workgroups and no long
// workgroup is left running alone at the end of the launch; the chunks of a
// row combine with integer atomic maxima on an order-preserving encoding of
// the floats (fwd_max_init_kernel fills the targets with the encoding of -inf
// first).
//
// With the histogram pass to follow, the sweep keeps the maxima of four
// classes of the row's keys (the lane half and the 32-key half of each tile
// that holds them) in the row of o, which is free until the output pass:
// four of the row's scores, the largest of them the row max. Each chunk
// stores its four in words 4c .. 4c + 3 while the row has room for every
// chunk (class_slots), which needs no atomics; otherwise the chunks combine
// in words 0-3 by atomic maxima.
// f(t) = sum_i (z_i - t)_+^kappa - 1 over any of the row's scores is at most
// the row's own f, and both fall with t, so a t where the four give f >= 0
// lies at or below tau: the histogram pass raises its window's lower edge
// above max z - 1 to that bound wherever the top scores are close together,
// bins fewer scores, and finds the same bound tau_h and support. Without the
// histogram pass the row max goes to tau.
// ---------------------------------------------------------------------------
constexpr int MAX_CHUNK = 32;
__host__ __device__ inline int max_chunks(int nb) { return (nb + MAX_CHUNK - 1) / MAX_CHUNK; }

// float <-> int with the same order, for atomic max on floats
__device__ __forceinline__ int ord_of(float f) {
  const int i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float float_of_ord(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF); }

// whether a row of o (D elements of E) holds the class maxima of every key
// chunk, four words each
template <class E, int D>
__host__ __device__ inline bool class_slots(int nb) {
  return 4 * max_chunks(nb) <= D * (int)sizeof(typename E::storage) / 4;
}

// the max pass's atomic targets at -inf: the four class maxima in words 0-3
// of each row of o when the chunks combine there, or the row max in tau
// without the histogram pass
template <class E, int D>
__global__ __launch_bounds__(256) void fwd_max_init_kernel(FwdArgs a) {
  using S = typename E::storage;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)a.B * a.H * a.N) return;
  const int ninf = ord_of(-INFINITY);
  if (a.nohist) {
    reinterpret_cast<int*>(a.tau)[i] = ninf;
  } else if (!class_slots<E, D>(a.nb)) {
    const int bh = (int)(i / a.N), row = (int)(i % a.N);
    *reinterpret_cast<int4*>(reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) + (size_t)row * a.lq.sn) =
        make_int4(ninf, ninf, ninf, ninf);
  }
}

// x^kappa for x > 0 in the pass's power mode
__device__ __forceinline__ float pow_kappa(float x, int pm, float kappa) {
  if (pm == PM_K1) return x;
  if (pm == PM_K2) return x * x;
  if (pm == PM_K4) {
    const float x2 = x * x;
    return x2 * x2;
  }
  return __builtin_amdgcn_exp2f(kappa * __builtin_amdgcn_logf(x));
}

// A lower bound of tau from four of a row's raw scores v (-inf where
// absent): bisection for the root of sum_i (zs v_i - t)_+^kappa = 1 on
// [max z - 1, max z], keeping the end where the sum is at least 1, then
// lowered by BRACKET_PAD, which covers the rounding of the fp32 sums.
__device__ __forceinline__ float class_bound(const float (&v)[4], float zs, int pm, float kappa) {
  float z[4];
  float zm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = v[i] * zs;
    zm = fmaxf(zm, z[i]);
  }
  float lo = zm - 1.f, hi = zm;
#pragma unroll 1
  for (int it = 0; it < 16; ++it) {
    const float mid = 0.5f * (lo + hi);
    float f = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = z[i] - mid;
      if (x > 0.f) f += pow_kappa(x, pm, kappa);
    }
    if (f >= 1.f) lo = mid; else hi = mid;
  }
  return lo - BRACKET_PAD;
}


// RG row groups of 32 per wave: 4 waves cover 2 RG query blocks, and every K
// fragment read from LDS feeds RG products.
template <class E, int D, int NBUF, int RG>
__global__ __launch_bounds__(256, 3) void fwd_max_kernel(FwdArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = 256, NBLKS = 2 * RG;
  constexpr int LDK = Ld<E, D>::value;
  __shared__ __attribute__((aligned(16))) S ktile[NBUF][BLK * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid), h = lane >> 5, l32 = lane & 31;
  const int ngroups = (a.nb + NBLKS - 1) / NBLKS;
  const int nch = max_chunks(a.nb);
  const int per_head = ngroups * nch;
  const int wg = xcd_remap(blockIdx.x, a.B * a.H * per_head);
  const int bh = wg / per_head;
  const int rem = wg % per_head;
  const int chunk = rem / ngroups;                  // consecutive workgroups share a key chunk
  const int grp = ngroups - 1 - rem % ngroups;
  const int blk0 = grp * NBLKS;
  const int jmax = a.causal ? min(blk0 + NBLKS - 1, a.nb - 1) : a.nb - 1;
  const int jlo = chunk * MAX_CHUNK;
  if (jlo > jmax) return;                           // no visible key block in this chunk
  const int jhi = min(jlo + MAX_CHUNK - 1, jmax);
  // row group g of this wave: rows 32 (RG wave + g) .. of the workgroup
  const int myblk = blk0 + ((RG * wave) >> 1);      // the wave's groups share one block when RG = 2
  const bool blk_valid = myblk < a.nb;
  int qrow[RG];
  bool qvalid[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    qrow[g] = blk0 * BLK + (RG * wave + g) * 32 + l32;
    qvalid[g] = qrow[g] < a.N;
  }

  const S* Q = reinterpret_cast<const S*>(a.q) + a.lq.head(bh, a.H);
  const S* K = reinterpret_cast<const S*>(a.k) + a.lkv.head(bh / a.G, a.H / a.G);
  typename E::frag bq[RG][D / E::KPI];
#pragma unroll
  for (int g = 0; g < RG; ++g) load_row_frags<E, D>(bq[g], Q + (size_t)qrow[g] * a.lq.sn, qvalid[g], h);

  float mlane[RG][2];   // the maxima of this lane's keys in each 32-key half of the tiles
#pragma unroll
  for (int g = 0; g < RG; ++g) mlane[g][0] = mlane[g][1] = -INFINITY;
  TileIO<E, D, NTHR> io;
  io.load(K, jhi * BLK, a.N, tid, a.lkv.sn);
  wait_vmem();
  io.template store_rows<LDK>(ktile[0], tid);
  __syncthreads();
  int buf = 0;
  for (int J = jhi; J >= jlo; --J) {
    if (J > jlo) io.load(K, (J - 1) * BLK, a.N, tid, a.lkv.sn);
    if (blk_valid && (!a.causal || J <= myblk)) {
      floatx16 acc[RG][2];
      tile_x_frags_rg<E, D, LDK, RG>(acc, ktile[buf], bq, l32, h);
      const bool edge = J * BLK + BLK > a.N || (a.causal && J == myblk);
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        if (edge) mask_keys(acc[g], J * BLK, a.N, a.causal, qrow[g], h);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) mlane[g][kh] = fmaxf(mlane[g][kh], half_max(acc[g][kh]));
      }
    }
    wait_vmem();
    if (J > jlo) {
      if (NBUF == 1) __syncthreads();
      io.template store_rows<LDK>(ktile[NBUF - 1 - buf], tid);
      __syncthreads();
      buf = NBUF - 1 - buf;
    }
  }
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    if (a.nohist) {
      const float ml = fmaxf(mlane[g][0], mlane[g][1]);
      const float m = fmaxf(ml, __shfl_xor(ml, 32));
      if (qvalid[g] && h == 0 && m > -INFINITY)
        atomicMax(reinterpret_cast<int*>(a.tau) + (size_t)bh * a.N + qrow[g], ord_of(m));
    } else if (qvalid[g]) {
      // classes 2 h and 2 h + 1: this lane's keys in each 32-key half
      int* cls = reinterpret_cast<int*>(reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) + (size_t)qrow[g] * a.lq.sn);
      if (class_slots<E, D>(a.nb)) {
        // every chunk holding visible keys of the row stores its own (-inf
        // for a class with none)
        if (!a.causal || jlo <= myblk)
          *reinterpret_cast<int2*>(cls + 4 * chunk + 2 * h) = make_int2(ord_of(mlane[g][0]), ord_of(mlane[g][1]));
      } else {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          if (mlane[g][kh] > -INFINITY) atomicMax(cls + 2 * h + kh, ord_of(mlane[g][kh]));
      }
    }
  }
}

// The histogram window of one row, from the max pass's class maxima: bins k
// in [ktop - NB, ktop], ktop = floor(NB c m), slot k - kbase; of those, the
// bins from kwin up: kwin is raised above kbase to the bin of the max pass's
// lower bound of tau where that is higher (the default solver mode), since
// no score below tau is in the support or in the root's equation at or above
// the bound. lo_raw is the least float x with fl(x * zscaleB) >= kwin, so
// that testing a raw score against it decides window membership exactly as
// the scaled score would; +inf for rows past N.
struct RowWindow {
  int kbase, kwin;
  float lo_raw;
};

template <class E, int D, int NB>
__device__ __forceinline__ RowWindow row_window(const FwdArgs& a, int bh, int qrow, int myblk, bool qvalid) {
  using S = typename E::storage;
  float cv[4] = {0.f, 0.f, 0.f, 0.f};   // the max pass's class maxima (raw)
  if (qvalid) {
    const int4* cls = reinterpret_cast<const int4*>(reinterpret_cast<const S*>(a.o) + a.lq.head(bh, a.H) +
                                                    (size_t)qrow * a.lq.sn);
    // per chunk (those holding visible keys of the row), or combined
    const int nc = !class_slots<E, D>(a.nb) ? 1 : (a.causal ? (myblk / MAX_CHUNK) + 1 : max_chunks(a.nb));
    int4 cw = cls[0];
    for (int c = 1; c < nc; ++c) {
      const int4 x = cls[c];
      cw = make_int4(max(cw.x, x.x), max(cw.y, x.y), max(cw.z, x.z), max(cw.w, x.w));
    }
    cv[0] = float_of_ord(cw.x);
    cv[1] = float_of_ord(cw.y);
    cv[2] = float_of_ord(cw.z);
    cv[3] = float_of_ord(cw.w);
  }
  const float m = fmaxf(fmaxf(cv[0], cv[1]), fmaxf(cv[2], cv[3]));
  RowWindow w;
  w.kbase = (int)floorf(m * a.zscaleB) - NB;
  w.kwin = w.kbase;
  if (qvalid && !a.plain) {
    const float lb = class_bound(cv, a.zscale, a.pow_mode, a.kappa);
    if (lb * (float)NB > (float)w.kbase) w.kwin = (int)floorf(lb * (float)NB);   // NB a power of two: exact
  }
  const float win_f = (float)w.kwin;
  float lo_raw = win_f / a.zscaleB;
  while (lo_raw * a.zscaleB < win_f) lo_raw = nextafterf(lo_raw, INFINITY);
  for (float p = nextafterf(lo_raw, -INFINITY); p * a.zscaleB >= win_f; p = nextafterf(p, -INFINITY)) lo_raw = p;
  w.lo_raw = qvalid ? lo_raw : INFINITY;
  return w;
}

// ---------------------------------------------------------------------------
// fwd_list: the histogram pass for rows whose windows hold few scores. Where
// a row has at most WL_CAP window scores (over its two lanes), the binned
// window is that short list, and the histogram's root follows from it alone:
// the same equation over the same left edges. So this kernel sweeps the keys like the max pass, with no
// histogram in LDS (a small footprint, four waves per SIMD), appends each
// window score, binned and with its key, to its row's list (in LDS), and
// solves sum_j (e_j - t)_+^kappa = 1 over the list's left edges e_j from the
// window's lower edge: by Newton's method for kappa >= 1 (the sum is then
// convex and falls with t, so the iterates rise to the root and stay below
// it), by bisection keeping the lower end for kappa < 1. tau_h, the kept
// keys above max(tau_h - 2^-12, window edge) and the candidate mask are
// then written as the histogram kernel would write them; a row with more
// than LIST_CAP keys above that point is left to the refinement's passes
// from tau_h, over the key blocks of its window scores, as the histogram
// kernel leaves the rows it cannot list. A row with more than WL_CAP window
// scores is left to fwd_rowhist (its tau set to -inf). A group whose windows
// are dense (more than 2 WL_FLAGS lanes past WL_CAP / 2 window scores, or
// past WL_CAP / 4 within the first quarter of their key blocks) stops its
// sweep after that key block; one with more than WL_FLAGS rows past
// WL_CAP, or where a row's root search does not settle, stops after the
// solve: either
// writes NaN into the tau of its rows and leaves the rest (class maxima
// included) untouched, and the histogram kernel then takes the group.
// (gist.science German page, section 2 "Kernidee", steps 1-2: the histogram
// bound; this is the same bound where the window is short.)
// ---------------------------------------------------------------------------
constexpr int WL_CAP = 32;   // window scores a row of the list pass keeps (its two lanes together)
constexpr int WL_FLAGS = 4;  // rows of a group that may pass WL_CAP (they go to fwd_rowhist)

template <class E, int D, int NBUF, int RG>
__global__ __launch_bounds__(256) void fwd_list_kernel(FwdArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = 256, NBLKS = 2 * RG, NB = HIST_BINS;
  constexpr int LDK = Ld<E, D>::value;
  constexpr uint32_t QB = 65535u / (uint32_t)(NB + 1);   // steps per bin, as in the histogram pass
  __shared__ __attribute__((aligned(16))) S ktile[NBUF][BLK * LDK];
  // bail_s[J & 1]: some lane of the group saw more than WL_CAP window scores
  // in the sweep step of key block J (read after that step's barrier, so a
  // wave already in the next step writes the other slot); bail2_s: some row
  // keeps too many keys, or its root search did not settle
  __shared__ int bail_s[2], bail2_s, nflag_s, nflag_early_s, nrow_s;
  // row r of the group (32 (RG wave + g) + l32) owns slots s = 0 .. WL_CAP - 1
  // at lists[s][r]: its lane 0 fills them upward, its lane 1 downward
  __shared__ uint32_t lists[WL_CAP][128 * RG];
  __shared__ uint32_t cand_s[NBLKS][WMAX];   // window blocks of the rows the refinement will stream

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid), h = lane >> 5, l32 = lane & 31;
  const int ngroups = (a.nb + NBLKS - 1) / NBLKS;
  const int total = a.B * a.H * ngroups;
  const int wg = xcd_remap(blockIdx.x, total);
  int bh, rank;
  xcd_split(wg, total, ngroups, bh, rank);
  const int grp = ngroups - 1 - rank;   // longest rows first when causal
  const int blk0 = grp * NBLKS;
  // row group g of this wave: rows 32 (RG wave + g) .. of the workgroup
  const int myblk = blk0 + ((RG * wave) >> 1);
  const bool blk_valid = myblk < a.nb;
  int qrow[RG];
  bool qvalid[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    qrow[g] = blk0 * BLK + (RG * wave + g) * 32 + l32;
    qvalid[g] = qrow[g] < a.N;
  }
  if (tid == 0) bail_s[0] = bail_s[1] = bail2_s = nflag_s = nflag_early_s = nrow_s = 0;
  for (int i = tid; i < NBLKS * WMAX; i += NTHR) (&cand_s[0][0])[i] = 0u;

  const S* Q = reinterpret_cast<const S*>(a.q) + a.lq.head(bh, a.H);
  const S* K = reinterpret_cast<const S*>(a.k) + a.lkv.head(bh / a.G, a.H / a.G);
  typename E::frag bq[RG][D / E::KPI];
  RowWindow rw[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    load_row_frags<E, D>(bq[g], Q + (size_t)qrow[g] * a.lq.sn, qvalid[g], h);
    rw[g] = row_window<E, D, NB>(a, bh, qrow[g], myblk, qvalid[g]);
  }

  // each row's window scores met by this lane, in the order met, in the
  // row's LDS slots (lane 0 from the first up, lane 1 from the last down, so
  // they meet only when the row holds more than WL_CAP; each slot in bounds
  // either way): bin above the window's lower edge times QB plus the place in
  // the bin in steps of 1/QB (high half), key (low half)
  uint32_t lc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) lc[g] = 0u;
  auto slot_of = [&](uint32_t i) { return h ? (uint32_t)WL_CAP - 1u - i : i; };
  auto take = [&](int g, float val, uint32_t key) {
    const float v = val * a.zscaleB;
    const float fv = floorf(v);
    const uint32_t sb = (uint32_t)min((int)fv - rw[g].kbase, NB);
    const uint32_t st = min((uint32_t)((v - fv) * (float)QB), QB - 1u);
    if (lc[g] < (uint32_t)WL_CAP)
      lists[slot_of(lc[g])][(RG * wave + g) * 32 + l32] = ((__umul24(sb, QB) + st) << 16) | (key & 0xFFFFu);
    ++lc[g];
  };

  const int jmax = a.causal ? min(blk0 + NBLKS - 1, a.nb - 1) : a.nb - 1;
  const int nvis = a.causal ? myblk + 1 : a.nb;   // key blocks this wave's rows see
  uint32_t tiles = 0;
  TileIO<E, D, NTHR> io;
  io.load(K, jmax * BLK, a.N, tid, a.lkv.sn);
  wait_vmem();
  io.template store_rows<LDK>(ktile[0], tid);
  __syncthreads();
  int buf = 0;
  for (int J = jmax; J >= 0; --J) {
    if (J > 0) io.load(K, (J - 1) * BLK, a.N, tid, a.lkv.sn);
    if (blk_valid && (!a.causal || J <= myblk)) {
      floatx16 acc[RG][2];
      tile_x_frags_rg<E, D, LDK, RG>(acc, ktile[buf], bq, l32, h);
      const bool edge = J * BLK + BLK > a.N || (a.causal && J == myblk);
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        if (edge) mask_keys(acc[g], J * BLK, a.N, a.causal, qrow[g], h);
        float gm[4];
        group_max(acc[g], gm);
        const bool mine = __builtin_elementwise_maximum(__builtin_elementwise_maximum(gm[0], gm[1]),
                                                        __builtin_elementwise_maximum(gm[2], gm[3])) >= rw[g].lo_raw;
        if (__ballot(mine) != 0) {
          // the workgroup's next barrier waits for the waves that take this
          // branch: they issue ahead of the other waves of their SIMD until
          // it ends
          __builtin_amdgcn_s_setprio(2);
          const uint32_t lc0 = lc[g];
          const uint32_t key0 = (uint32_t)(J * BLK + 8 * h);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            if (__ballot(gm[q4] >= rw[g].lo_raw) == 0) continue;
            const int kh = q4 >> 1, r0 = 8 * (q4 & 1);
            const uint32_t kg = key0 + 32 * kh + 16 * (q4 & 1);
            if (gm[q4] >= rw[g].lo_raw) {
              // one window score in the group of 8 (the common case): its
              // value is the group max
              int ne = 0, ri = 0;
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const bool wr = acc[g][kh][r0 + r] >= rw[g].lo_raw;
                ne += wr ? 1 : 0;
                ri = wr ? r : ri;
              }
              if (ne == 1) {
                take(g, gm[q4], kg + ri);
              } else {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                  if (acc[g][kh][r0 + r] >= rw[g].lo_raw) take(g, acc[g][kh][r0 + r], kg + r);
              }
            }
          }
          // dense windows: past 2 WL_FLAGS lanes of the group with more than
          // WL_CAP / 2 window scores each, or with more than WL_CAP / 4 within
          // the first quarter of their key blocks, the group goes to the
          // histogram kernel at once (the rows' totals decide the rest after
          // the sweep)
          if (lc0 <= (uint32_t)WL_CAP / 2 && lc[g] > (uint32_t)WL_CAP / 2 && atomicAdd(&nflag_s, 1) >= 2 * WL_FLAGS)
            bail_s[J & 1] = 1;
          if (4 * (int)tiles < nvis && lc0 <= (uint32_t)WL_CAP / 4 && lc[g] > (uint32_t)WL_CAP / 4 &&
              atomicAdd(&nflag_early_s, 1) >= 2 * WL_FLAGS)
            bail_s[J & 1] = 1;
          __builtin_amdgcn_s_setprio(0);
        }
      }
      tiles++;
    }
    wait_vmem();
    if (J > 0) {
      if (NBUF == 1) __syncthreads();
      io.template store_rows<LDK>(ktile[NBUF - 1 - buf], tid);
      __syncthreads();
      buf = NBUF - 1 - buf;
      if (bail_s[J & 1]) break;   // (uniform) the histogram kernel takes this group
    }
  }
  if (a.tiles_per_pass && lane == 0 && ((RG * wave) & 1) == 0 && tiles) atomicAdd(a.tiles_per_pass, tiles);
  __syncthreads();
  if (bail_s[0] | bail_s[1]) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
      if (qvalid[g] && h == 0) a.tau[(size_t)bh * a.N + qrow[g]] = __builtin_nanf("");
    return;
  }

  float th[RG], lo[RG], lo_q[RG];
  int nab[RG], nab_o[RG];
  bool flagged[RG];   // a lane of the row passed WL_CAP: its list is not whole
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    // (the shuffle outside any condition: both lanes of the row take part)
    const uint32_t lc_o = (uint32_t)__shfl_xor((int)lc[g], 32);
    flagged[g] = lc[g] + lc_o > (uint32_t)WL_CAP;
    // a row past WL_CAP goes to fwd_rowhist; past WL_FLAGS such rows the
    // group goes to the histogram kernel
    if (flagged[g] && qvalid[g] && h == 0 && atomicAdd(&nrow_s, 1) >= WL_FLAGS) bail2_s = 1;
    // the histogram root over the two lanes' lists, in bins above kbase:
    // sum_j (sb_j - u)_+^kappa = B^kappa, with x_j = (sb_j - u) / B
    const int lrw = (RG * wave + g) * 32 + l32;
    // (the lane's own entries, read from LDS: a row holds a few)
    const int n = flagged[g] ? 0 : (int)lc[g];
    auto sums = [&](float u, float& f0, float& f1) {
      f0 = f1 = 0.f;
#pragma unroll 1
      for (int i = 0; i < n; ++i) {
        const float x = ((float)((lists[slot_of(i)][lrw] >> 16) / QB) - u) * (1.0f / NB);
        if (x > 0.f) {
          if (a.pow_mode == PM_K1) {
            f0 += x;
            f1 += 1.f;
          } else if (a.pow_mode == PM_K2) {
            f0 = fmaf(x, x, f0);
            f1 += x;
          } else if (a.pow_mode == PM_K4) {
            const float x2 = x * x;
            f0 = fmaf(x2, x2, f0);
            f1 = fmaf(x2, x, f1);
          } else {
            const float lx = __builtin_amdgcn_logf(x);
            f0 += __builtin_amdgcn_exp2f(a.kappa * lx);
            f1 += __builtin_amdgcn_exp2f((a.kappa - 1.f) * lx);
          }
        }
      }
      // (the row's two lanes hold the same qrow: both run this or neither)
      f0 += __shfl_xor(f0, 32);
      f1 += __shfl_xor(f1, 32);
    };
    const float uwin = (float)(rw[g].kwin - rw[g].kbase);
    float u = uwin;
    bool ok = true;
    if (qvalid[g] && !flagged[g]) {
      float f0, f1;
      sums(u, f0, f1);
      if (f0 > 1.f) {
        if (a.kappa >= 1.f) {
          // each term (sb - u)_+^kappa is convex in u: Newton from below,
          // u += (f0 - 1) B / (kappa f1), rises to the root and stays below it
          bool conv = false;
#pragma unroll 1
          for (int it = 0; it < 32 && !conv; ++it) {
            const float du = (f0 - 1.f) * (float)NB / (a.kappa * f1);
            u += du;
            conv = !(du > 1e-4f);
            if (!conv) sums(u, f0, f1);
          }
          ok = conv;
        } else {
          // concave terms (alpha > 2): bisection on [uwin, B], keeping the end
          // where the sum is at least 1 (2^-16 bins after 24 halvings)
          float hi = (float)NB;
#pragma unroll 1
          for (int it = 0; it < 24; ++it) {
            const float mid = 0.5f * (u + hi);
            sums(mid, f0, f1);
            if (f0 >= 1.f) u = mid; else hi = mid;
          }
        }
      }
      // else the root lies at or below the window's edge
    }
    // tau_h, raised to the window's edge, and the kept keys above lo
    const float wedge = (float)rw[g].kwin * (1.0f / NB);
    th[g] = fmaxf(((float)rw[g].kbase + u) * (1.0f / NB), wedge);
    lo[g] = fmaxf(th[g] - BRACKET_PAD, wedge);
    lo_q[g] = (lo[g] * (float)NB - (float)rw[g].kbase) * (float)QB;
    int c = 0;
#pragma unroll 1
    for (int i = 0; i < n; ++i) c += ((float)((lists[slot_of(i)][lrw] >> 16) + 2u) > lo_q[g]) ? 1 : 0;
    nab[g] = c;
    nab_o[g] = __shfl_xor(c, 32);
    if (qvalid[g] && (!ok || a.N > LIST_MAX_N)) bail2_s = 1;
  }
  __syncthreads();
  if (bail2_s) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
      if (qvalid[g] && h == 0) a.tau[(size_t)bh * a.N + qrow[g]] = __builtin_nanf("");
    return;
  }
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    if (!qvalid[g]) continue;
    if (flagged[g]) {
      // (the class maxima in the row of o stay for fwd_rowhist)
      if (h == 0) a.tau[(size_t)bh * a.N + qrow[g]] = -INFINITY;
      continue;
    }
    uint32_t* lrow =
        reinterpret_cast<uint32_t*>(reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) + (size_t)qrow[g] * a.lq.sn);
    uint16_t* lidx = reinterpret_cast<uint16_t*>(lrow + 2 + LIST_CAP);
    // more kept keys than a row of o holds: the row takes the refinement's
    // passes from tau_h over the key blocks of its window scores, as the
    // histogram kernel leaves the rows it cannot list
    const bool over = nab[g] + nab_o[g] > LIST_CAP;
    if (h == 0) {
      a.tau[(size_t)bh * a.N + qrow[g]] = th[g];
      if (a.tau_h_out) a.tau_h_out[(size_t)bh * a.N + qrow[g]] = th[g];
      lrow[0] = over ? LIST_NONE : (uint32_t)(nab[g] + nab_o[g]);
      lrow[1] = __float_as_uint(lo[g]);
    }
    if (over) {
      uint32_t* cw = cand_s[(RG * wave) >> 1];
      for (int i = 0; i < (int)lc[g]; ++i) {
        const int J = (int)(lists[slot_of(i)][(RG * wave + g) * 32 + l32] & 0xFFFFu) / BLK;
        atomicOr(cw + (J >> 5), 1u << (J & 31));
      }
    } else {
      // lane 0 of the row first, then lane 1; each in the order met
      int off = h ? nab_o[g] : 0;
      for (int i = 0; i < (int)lc[g]; ++i) {
        const uint32_t w = lists[slot_of(i)][(RG * wave + g) * 32 + l32];
        if ((float)((w >> 16) + 2u) > lo_q[g]) lidx[off++] = (uint16_t)(w & 0xFFFFu);
      }
    }
  }
  // the candidate mask the refinement streams: the window blocks of the
  // rows it solves by passes
  __syncthreads();
  for (int i = tid; i < NBLKS * a.W; i += NTHR) {
    const int b = i / a.W, w = i % a.W;
    if (blk0 + b < a.nb) a.mask[((size_t)bh * a.nb + blk0 + b) * a.W + w] = cand_s[b][w];
  }
}

// ---------------------------------------------------------------------------
// fwd_rowhist: the histogram of the single rows the list pass flagged (the
// row has more than WL_CAP window scores, in a group with few such rows;
// their tau holds -inf). One workgroup per list-pass group takes
// its flagged rows in turn: the row's scores as fp32 dot products, one key
// per thread; those in the window binned into a one-row left-edge histogram
// in LDS (the histogram kernel's bins and counters) and kept with their
// keys; the histogram solved as the histogram kernel solves a row (one quad
// of lanes); then, like the histogram kernel, tau_h, and the keys above
// max(tau_h - 2^-12, window edge) in key order where they are at most
// LIST_CAP (and every window score was kept), else the key blocks of the
// window scores added to the block's candidate mask for the refinement's
// passes. (gist.science German page, section 2 "Kernidee", steps 1-2.)
// ---------------------------------------------------------------------------
template <class E, int D, int RG>
__global__ __launch_bounds__(256) void fwd_rowhist_kernel(FwdArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = 256, ROWS = 128 * RG, NBLKS = 2 * RG, NB = HIST_BINS;
  constexpr int HW = HistRow<false, NB>::WORDS;
  constexpr int CAND = 1024;   // window scores a row keeps (key, raw score)
  __shared__ __attribute__((aligned(16))) uint32_t hist[HW];
  __shared__ __attribute__((aligned(16))) float qs[D];
  __shared__ int rows_s[ROWS];
  __shared__ uint32_t ckey[CAND];
  __shared__ float cs[CAND];
  __shared__ uint32_t wblk[WMAX];   // key blocks holding window scores of the row
  __shared__ int nrows_s, ncand_s, nkeep_s;
  __shared__ float th_s;

  const int tid = threadIdx.x;
  const int ngroups = (a.nb + NBLKS - 1) / NBLKS;
  const int total = a.B * a.H * ngroups;
  const int wg = xcd_remap(blockIdx.x, total);
  int bh, rank;
  xcd_split(wg, total, ngroups, bh, rank);
  const int blk0 = (ngroups - 1 - rank) * NBLKS;
  if (tid == 0) nrows_s = 0;
  __syncthreads();
  for (int i = tid; i < ROWS; i += NTHR) {
    const int r = blk0 * BLK + i;
    if (r < a.N && a.tau[(size_t)bh * a.N + r] == -INFINITY) rows_s[atomicAdd(&nrows_s, 1)] = r;
  }
  __syncthreads();
  const int nr = nrows_s;
  if (nr == 0) return;
  const S* Q = reinterpret_cast<const S*>(a.q) + a.lq.head(bh, a.H);
  const S* K = reinterpret_cast<const S*>(a.k) + a.lkv.head(bh / a.G, a.H / a.G);
#pragma unroll 1
  for (int ri = 0; ri < nr; ++ri) {
    // (the rows in increasing order, whatever order the atomics left)
    int qrow = 0x7fffffff;
    for (int i = 0; i < nr; ++i) {
      const int r = rows_s[i];
      int rk = 0;
      for (int i2 = 0; i2 < nr; ++i2) rk += rows_s[i2] < r ? 1 : 0;
      if (rk == ri) qrow = r;
    }
    const int myblk = qrow / BLK;
    const RowWindow rw = row_window<E, D, NB>(a, bh, qrow, myblk, true);
    for (int e = tid; e < D; e += NTHR) {
      if constexpr (sizeof(S) == 2)
        qs[e] = __uint_as_float((uint32_t)Q[(size_t)qrow * a.lq.sn + e] << 16);
      else
        qs[e] = (float)Q[(size_t)qrow * a.lq.sn + e];
    }
    for (int i = tid; i < HW; i += NTHR) hist[i] = 0u;
    for (int i = tid; i < WMAX; i += NTHR) wblk[i] = 0u;
    if (tid == 0) ncand_s = nkeep_s = 0;
    __syncthreads();
    const int nk = a.causal ? qrow + 1 : a.N;
    for (int j = tid; j < nk; j += NTHR) {
      const uint4* kr = reinterpret_cast<const uint4*>(K + (size_t)j * a.lkv.sn);
      float sc = 0.f;
#pragma unroll
      for (int c = 0; c < D / E::CHUNK; ++c) {
        const uint4 w = kr[c];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (sizeof(S) == 2) {
            sc = fmaf(qs[c * 8 + 2 * e], __uint_as_float(ws[e] << 16), sc);
            sc = fmaf(qs[c * 8 + 2 * e + 1], __uint_as_float(ws[e] & 0xFFFF0000u), sc);
          } else {
            sc = fmaf(qs[c * 4 + e], __uint_as_float(ws[e]), sc);
          }
        }
      }
      if (sc >= rw.lo_raw) {
        const int sb = min((int)floorf(sc * a.zscaleB) - rw.kbase, NB);
        atomicAdd(hist + (sb >> 1), 1u << ((sb & 1) * 16));
        const int c = atomicAdd(&ncand_s, 1);
        if (c < CAND) {
          ckey[c] = (uint32_t)j;
          cs[c] = sc;
        }
        atomicOr(&wblk[(j / BLK) >> 5], 1u << ((j / BLK) & 31));
      }
    }
    __syncthreads();
    if (tid < 4) {
      const double T = hist_solve_quad<false, NB>(hist, tid, a.pow_mode, a.kappa);
      if (tid == 0) th_s = (float)(((double)rw.kbase + NB - T) * (1.0 / NB));
    }
    __syncthreads();
    const float wedge = (float)rw.kwin * (1.0f / NB);
    const float th = fmaxf(th_s, wedge);
    const float lo = fmaxf(th - BRACKET_PAD, wedge);
    // kept: window scores whose scaled value lies above lo, less 1/32 bin
    // for the rounding of these dot products against the refinement's
    const float keep_v = lo * (float)NB - (1.0f / 32);
    const int nc = ncand_s;
    const bool whole = nc <= CAND;
    int mine = 0;
    for (int i = tid; i < min(nc, CAND); i += NTHR) mine += (cs[i] * a.zscaleB > keep_v) ? 1 : 0;
    if (mine) atomicAdd(&nkeep_s, mine);
    __syncthreads();
    const int tot = nkeep_s;
    const bool listed = whole && tot <= LIST_CAP;
    uint32_t* lrow = reinterpret_cast<uint32_t*>(reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) + (size_t)qrow * a.lq.sn);
    if (listed) {
      // each kept key at its rank among the kept keys
      uint16_t* lidx = reinterpret_cast<uint16_t*>(lrow + 2 + LIST_CAP);
      for (int i = tid; i < nc; i += NTHR) {
        if (!(cs[i] * a.zscaleB > keep_v)) continue;
        int rk = 0;
        for (int i2 = 0; i2 < nc; ++i2) rk += (cs[i2] * a.zscaleB > keep_v && ckey[i2] < ckey[i]) ? 1 : 0;
        lidx[rk] = (uint16_t)ckey[i];
      }
    } else {
      for (int w = tid; w < a.W; w += NTHR)
        if (wblk[w]) atomicOr(&a.mask[((size_t)bh * a.nb + myblk) * a.W + w], wblk[w]);
    }
    if (tid == 0) {
      a.tau[(size_t)bh * a.N + qrow] = th;
      if (a.tau_h_out) a.tau_h_out[(size_t)bh * a.N + qrow] = th;
      lrow[0] = listed ? (uint32_t)tot : LIST_NONE;
      lrow[1] = __float_as_uint(lo);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// fwd_init: with the row max m from fwd_max, one sweep bins every score with
// floor(B z) >= kwin at slot floor(B z) - (ktop - B) (ktop = floor(B m),
// B = NB bins per unit; kwin = ktop - B, or the bin of the lower bound of tau
// from the max pass's class maxima where that is higher), and marks the key
// blocks that hold such a score. Knowing m first makes the window fixed, so
// no bin is ever evicted.
// Two waves share each group of 32 rows, one per 32-key half of every key
// tile: the histograms (the bulk of the LDS) then serve twice the waves, so
// more waves per CU hide the latency of the compares and LDS atomics.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mask_keys_half(floatx16& c, int kh, int key0, int N, int causal, int qrow, int h) {
  const int lim = (causal ? min(qrow, N - 1) : N - 1) - key0 - 8 * h;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = 32 * kh + 16 * (r >> 3) + (r & 7);
    if (off > lim) c[r] = -INFINITY;
  }
}

template <class E, int D, int NW, bool H32, bool DBUF, int NB>
__global__ __launch_bounds__(NW * 64) void fwd_init_kernel(FwdArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = NW * 64;
  constexpr int ROWS = NW * 16;          // NW / 2 groups of 32 rows
  constexpr int NBLKS = ROWS / BLK;
  constexpr int LDK = Ld<E, D>::value;
  constexpr int HWORDS = HistRow<H32, NB>::WORDS;
  constexpr int NBUF = DBUF ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t hist[ROWS * HWORDS];
  __shared__ __attribute__((aligned(16))) S ktile[NBUF][BLK * LDK];
  __shared__ uint32_t cand[NBLKS][WMAX];
  __shared__ uint32_t cand2[NBLKS][WMAX];  // window blocks of the rows whose lists are not complete
  __shared__ int kb_s[ROWS];             // kbase per row, for the solve
  __shared__ float th_s[ROWS];           // tau_h per row, for the lists
  __shared__ uint32_t lcnt_s[ROWS];      // byte j: kept scores of lane j above lo

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid), h = lane >> 5, l32 = lane & 31;
  const int kh = wave & 1;               // key half of this wave
  const int rg = wave >> 1;              // row group of this wave
  const int ngroups = (a.nb + NBLKS - 1) / NBLKS;
  const int total = a.B * a.H * ngroups;
  const int wg = xcd_remap(blockIdx.x, total);
  int bh, rank;
  xcd_split(wg, total, ngroups, bh, rank);
  const int grp = ngroups - 1 - rank;  // longest rows first when causal
  const int blk0 = grp * NBLKS;
  const int myblk = blk0 + (rg >> 1);
  const int qrow = myblk * BLK + (rg & 1) * 32 + l32;
  const bool qvalid = qrow < a.N;
  const bool blk_valid = myblk < a.nb;

  if (a.listpass) {
    // the list pass has finished the groups whose rows hold their tau_h and
    // left NaN in the rows of the others
    int need = 0;
    for (int i = tid; i < ROWS; i += NTHR) {
      const int r = blk0 * BLK + i;
      if (r < a.N && __builtin_isnan(a.tau[(size_t)bh * a.N + r])) need = 1;
    }
    if (!__syncthreads_or(need)) return;
  }

  const S* Q = reinterpret_cast<const S*>(a.q) + a.lq.head(bh, a.H);
  const S* K = reinterpret_cast<const S*>(a.k) + a.lkv.head(bh / a.G, a.H / a.G);

  typename E::frag bq[D / E::KPI];
  load_row_frags<E, D>(bq, Q + (size_t)qrow * a.lq.sn, qvalid, h);
  const RowWindow rw = row_window<E, D, NB>(a, bh, qrow, myblk, qvalid);
  const int kbase = rw.kbase, kwin = rw.kwin;
  const float lo_f = (float)kbase;
  const float lo_raw = rw.lo_raw;

  for (int i = tid; i < ROWS * HWORDS; i += NTHR) hist[i] = 0;
  for (int i = tid; i < NBLKS * WMAX; i += NTHR) (&cand[0][0])[i] = (&cand2[0][0])[i] = 0;
  // the key blocks holding window scores of this lane's row (up to 32 RBW
  // blocks; past that the candidate mask stays the union over all rows)
  constexpr int RBW = 8;
  const bool track = a.nb <= 32 * RBW;
  uint32_t rb[RBW];
#pragma unroll
  for (int i = 0; i < RBW; ++i) rb[i] = 0u;
  // the sweep collects the bits of one word (wcur, wave-uniform; the key
  // blocks go down, so each word is visited once) in rcur
  uint32_t rcur = 0u;
  int wcur = -1;
  auto flush_rb = [&]() {
    if (track) {
#pragma unroll
      for (int i = 0; i < RBW; ++i)
        if (i == wcur) rb[i] |= rcur;
    }
    rcur = 0u;
  };
  if (kh == 0 && h == 0) kb_s[rg * 32 + l32] = kbase;
  // this lane's LIST_LANE largest window scores among the first LIST_SCAN it
  // sees, descending, each as one word: its bin above the window's lower
  // edge times QB plus its place in the bin in steps of 1/QB (high half;
  // truncated), and its key (low half); and the count of window scores the
  // lane has seen. Every window score is binned as it comes.
  constexpr uint32_t QB = 65535u / (uint32_t)(NB + 1);   // steps per bin (bin NB, step QB - 1 fit 16 bits)
  uint32_t lp[LIST_LANE];
#pragma unroll
  for (int i = 0; i < LIST_LANE; ++i) lp[i] = 0u;
  uint32_t lc = 0;

  const int jmax = a.causal ? min(blk0 + NBLKS - 1, a.nb - 1) : a.nb - 1;
  uint32_t* myhist = hist + (rg * 32 + l32) * HWORDS;
  uint32_t tiles = 0;
  auto bin_s = [&](int sb) {   // one count into bin sb
    if constexpr (H32) atomicAdd(myhist + sb, 1u);
    else atomicAdd(myhist + (sb >> 1), 1u << ((sb & 1) * 16));
  };
  auto insert = [&](uint32_t w) {   // into the descending list
    uint32_t x = w;
#pragma unroll
    for (int i = 0; i < LIST_LANE; ++i) {
      const uint32_t m = max(lp[i], x);
      x = min(lp[i], x);
      lp[i] = m;
    }
  };
  // a window score of this lane; score register r of group g holds key
  // J BLK + 32 kh + 16 g + 8 h + r. It is binned; while the lane has seen
  // fewer than LIST_SCAN window scores it also enters the list (past that
  // the row takes the refinement's passes). The key takes the low 16 bits of
  // the word: past 65536 keys the lists are never used (rows are not gathered
  // there), so it is cut to 16 bits and never reaches the bin's half.
  auto take = [&](float val, uint32_t key) {
    const float v = val * a.zscaleB;
    const float fv = floorf(v);
    const int sb = min((int)fv - kbase, NB);   // 0 .. NB
    bin_s(sb);
    if (lc < (uint32_t)LIST_SCAN) {
      const uint32_t st = min((uint32_t)((v - fv) * (float)QB), QB - 1u);
      insert(((__umul24((uint32_t)sb, QB) + st) << 16) | (key & 0xFFFFu));
    }
    ++lc;
  };
  // past LIST_SCAN window scores (dense windows) a score is only binned
  auto bin = [&](float val) { bin_s(min((int)floorf(val * a.zscaleB) - kbase, NB)); };

  TileIO<E, D, NTHR> io;
  io.load(K, jmax * BLK, a.N, tid, a.lkv.sn);
  wait_vmem();
  io.template store_rows<LDK>(ktile[0], tid);
  __syncthreads();

  int buf = 0;
  for (int J = jmax; J >= 0; --J) {
    if ((J >> 5) != wcur) {   // (uniform) the next word of window blocks
      flush_rb();
      wcur = J >> 5;
    }
    if (J > 0) io.load(K, (J - 1) * BLK, a.N, tid, a.lkv.sn);
    if (blk_valid && (!a.causal || J <= myblk)) {
      floatx16 acc = tile_x_half<E, D, LDK>(ktile[buf], bq, l32, h, kh);
      if (J * BLK + BLK > a.N || (a.causal && J == myblk)) mask_keys_half(acc, kh, J * BLK, a.N, a.causal, qrow, h);
      float gm[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float mx = fmaxf(acc[8 * g], acc[8 * g + 1]);
#pragma unroll
        for (int r = 2; r < 8; ++r) mx = fmaxf(mx, acc[8 * g + r]);
        gm[g] = mx;
      }
      const bool mine = fmaxf(gm[0], gm[1]) >= lo_raw;
      rcur |= mine ? 1u << (J & 31) : 0u;
      if (__ballot(mine) != 0) {
        // The workgroup's next barrier waits for the waves that take this
        // branch: they issue ahead of the other waves of their SIMD until it
        // ends.
        __builtin_amdgcn_s_setprio(2);
        // A group of 8 scores no lane needs costs one compare and a branch.
        // A lane with one window score in a group takes the group's max; a
        // lane with several takes each.
        const uint32_t key0 = (uint32_t)(J * BLK + 32 * kh + 8 * h);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const bool in_g = gm[g] >= lo_raw;
          if (__ballot(in_g) == 0) continue;
          const int r0 = 8 * g;
          if (in_g) {
            if (lc >= (uint32_t)LIST_SCAN) {
#pragma unroll
              for (int r = 0; r < 8; ++r)
                if (acc[r0 + r] >= lo_raw) {
                  bin(acc[r0 + r]);
                  ++lc;
                }
            } else {
              // one window score in the group (the common case): its value
              // is the group max
              int ne = 0, ri = 0;
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const bool wr = acc[r0 + r] >= lo_raw;
                ne += wr ? 1 : 0;
                ri = wr ? r : ri;
              }
              if (ne == 1) {
                take(gm[g], key0 + 16 * g + ri);
              } else {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                  if (acc[r0 + r] >= lo_raw) take(acc[r0 + r], key0 + 16 * g + r);
              }
            }
          }
        }
        if (lane == 0) atomicOr(&cand[rg >> 1][J >> 5], 1u << (J & 31));
        __builtin_amdgcn_s_setprio(0);
      }
      tiles++;
    }
    wait_vmem();
    if (J > 0) {
      if (!DBUF) __syncthreads();
      io.template store_rows<LDK>(ktile[DBUF ? (buf ^ 1) : 0], tid);
      __syncthreads();
      buf = DBUF ? (buf ^ 1) : 0;
    }
  }
  flush_rb();
  __syncthreads();   // both key halves binned
  // histogram solve: four lanes per row, 16 rows per wave
  if (blk_valid) {
    const int r = 16 * kh + (lane >> 2);   // row within the group
    const double T = hist_solve_quad<H32, NB>(hist + (rg * 32 + r) * HWORDS, lane, a.pow_mode, a.kappa);
    const int qr = myblk * BLK + (rg & 1) * 32 + r;
    if ((lane & 3) == 0 && qr < a.N) th_s[rg * 32 + r] = (float)(((double)kb_s[rg * 32 + r] + NB - T) * (1.0 / NB));
  }

  // pool the four lanes' kept keys whose scores may lie above lo into the
  // row of o. An entry's score is below the upper end of its quantum; one
  // more quantum covers the rounding of the scaled score.
  __syncthreads();   // tau_h of every row; the histograms are no longer read
  const int lrw = rg * 32 + l32;   // this lane's row in the workgroup
  const int j = 2 * kh + h;        // lane of the row
  uint32_t* rbs = hist + RBW * lrw;   // the row's window blocks, over the four lanes
  if (track && qvalid && j == 0) {
#pragma unroll
    for (int i = 0; i < RBW; ++i) rbs[i] = rb[i];
  }
  float lo = 0.f;
  int nab = 0;                     // kept entries that may lie above lo (a prefix of the list)
  if (qvalid) {
    // tau_h: the root over the binned window, at least the window's lower
    // edge (the root over bins from kwin up can fall below it, by less than
    // a bin; the edge is itself a bound)
    const float wedge = (float)kwin * (1.0f / NB);
    const float th = fmaxf(th_s[lrw], wedge);
    if (j == 0) {
      a.tau[(size_t)bh * a.N + qrow] = th;
      if (a.tau_h_out) a.tau_h_out[(size_t)bh * a.N + qrow] = th;
    }
    lo = fmaxf(th - BRACKET_PAD, wedge);
    const float lo_q = (lo * (float)NB - lo_f) * (float)QB;   // lo in steps above the window's edge
#pragma unroll
    for (int i = 0; i < LIST_LANE; ++i)
      nab += ((uint32_t)i < lc && (float)((lp[i] >> 16) + 2u) > lo_q) ? 1 : 0;
    const bool complete =
        lc <= (uint32_t)LIST_LANE || (lc <= (uint32_t)LIST_SCAN && (float)((lp[LIST_LANE - 1] >> 16) + 2u) <= lo_q);
    reinterpret_cast<uint8_t*>(&lcnt_s[lrw])[j] = (uint8_t)(complete ? nab : 255);
  }
  __syncthreads();
  if (track && qvalid && j != 0) {
#pragma unroll
    for (int i = 0; i < RBW; ++i)
      if (rb[i]) atomicOr(rbs + i, rb[i]);
  }
  bool row_ok = false;
  if (qvalid) {
    const uint32_t c4 = lcnt_s[lrw];
    bool ok = a.N <= LIST_MAX_N;
    int tot = 0, off = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = (int)((c4 >> (8 * jj)) & 0xFFu);
      ok = ok && c != 255;
      tot += c;
      off += (jj < j) ? c : 0;
    }
    ok = ok && tot <= LIST_CAP;
    row_ok = ok;
    uint32_t* lrow = reinterpret_cast<uint32_t*>(reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) + (size_t)qrow * a.lq.sn);
    uint16_t* lidx = reinterpret_cast<uint16_t*>(lrow + 2 + LIST_CAP);
    if (j == 0) {
      lrow[0] = ok ? (uint32_t)tot : LIST_NONE;
      lrow[1] = __float_as_uint(lo);
    }
    if (ok) {
#pragma unroll
      for (int i = 0; i < LIST_LANE; ++i)
        if (i < nab) lidx[off + i] = (uint16_t)(lp[i] & 0xFFFFu);
    }
  }
  if (a.tiles_per_pass && lane == 0 && (wave & 3) == 0 && tiles) atomicAdd(a.tiles_per_pass, tiles);
  // the candidate mask the refinement streams: the window blocks of the rows
  // its passes solve (those whose kept lists are not complete)
  __syncthreads();
  if (track && qvalid && j == 0 && !row_ok) {
#pragma unroll
    for (int i = 0; i < RBW; ++i)
      if (rbs[i]) atomicOr(&cand2[lrw >> 6][i], rbs[i]);
  }
  __syncthreads();
  for (int i = tid; i < NBLKS * a.W; i += NTHR) {
    const int b = i / a.W, w = i % a.W;
    // (every row streams in the plain solver mode: the union over all rows)
    if (blk0 + b < a.nb) a.mask[((size_t)bh * a.nb + blk0 + b) * a.W + w] = (track && !a.plain) ? cand2[b][w] : cand[b][w];
  }
}

// ---------------------------------------------------------------------------
// One lane's half of a row's dot product with a key row read from memory:
// the k-slices the lane's operand fragments hold (the other lane of the row
// holds the rest)
// ---------------------------------------------------------------------------
template <class E, int D>
__device__ __forceinline__ float row_dot(const typename E::frag* bq, const typename E::storage* krow, int h) {
  typename E::frag kf[D / E::KPI];
#pragma unroll
  for (int ks = 0; ks < D / E::KPI; ++ks) kf[ks] = E::ld_k(krow, ks, h);
  float s = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / E::KPI; ++ks) {
    if constexpr (sizeof(typename E::storage) == 2) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 x = {bq[ks][2 * e], bq[ks][2 * e + 1]};
        const bf16x2 y = {kf[ks][2 * e], kf[ks][2 * e + 1]};
        s = __builtin_amdgcn_fdot2_f32_bf16(x, y, s, false);
      }
    } else {
      s = fmaf(bq[ks], kf[ks], s);
    }
  }
  return s;
}

// ---------------------------------------------------------------------------
// Mask walker over the union of up to two blocks' words in LDS (wave-uniform)
// ---------------------------------------------------------------------------
struct UnionIter {
  const uint32_t* m0;
  const uint32_t* m1;
  int use0, use1, W, w;
  uint32_t bits;
  __device__ __forceinline__ void init(const uint32_t* a0, const uint32_t* a1, bool u0, bool u1, int nw) {
    m0 = a0; m1 = a1; use0 = u0; use1 = u1; W = nw; w = -1; bits = 0;
  }
  __device__ __forceinline__ int next() {
    while (bits == 0) {
      if (++w >= W) return -1;
      uint32_t x = (use0 ? m0[w] : 0u) | (use1 ? m1[w] : 0u);
      bits = __builtin_amdgcn_readfirstlane(x);
    }
    const int t = __builtin_ctz(bits);
    bits &= bits - 1;
    return w * 32 + t;
  }
};

// ---------------------------------------------------------------------------
// fwd_refine: the refinement passes
// ---------------------------------------------------------------------------
template <class E, int D, int PM, int SV, int NBUF>
__global__ __launch_bounds__(256) void fwd_refine_kernel(FwdArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = 256, NBLKS = 2;
  constexpr int LDK = Ld<E, D>::value;
  __shared__ __attribute__((aligned(16))) S ktile[NBUF][BLK * LDK];
  __shared__ uint32_t m0[NBLKS][WMAX], m1[NBLKS][WMAX];
  __shared__ int wave_busy[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(tid), h = lane >> 5, l32 = lane & 31;
  const int ngroups = (a.nb + NBLKS - 1) / NBLKS;
  const int total = a.B * a.H * ngroups;
  const int wg = xcd_remap(blockIdx.x, total);
  int bh, rank;
  xcd_split(wg, total, ngroups, bh, rank);
  const int grp = ngroups - 1 - rank;
  const int blk0 = grp * NBLKS;
  const int lb = wave >> 1;                 // local block of this wave
  const int myblk = blk0 + lb;
  const int qrow = myblk * BLK + (wave & 1) * 32 + l32;
  const bool qvalid = qrow < a.N;
  const bool blk_valid = myblk < a.nb;
  const int W = a.W;

  const S* Q = reinterpret_cast<const S*>(a.q) + a.lq.head(bh, a.H);
  const S* K = reinterpret_cast<const S*>(a.k) + a.lkv.head(bh / a.G, a.H / a.G);

  typename E::frag bq[D / E::KPI];
  load_row_frags<E, D>(bq, Q + (size_t)qrow * a.lq.sn, qvalid, h);

  for (int i = tid; i < NBLKS * W; i += NTHR) {
    const int b = i / W, w = i % W;
    const int I = blk0 + b;
    uint32_t bits = 0u;
    if (I < a.nb) {
      if (a.nohist) {
        // every visible key block: J <= I (causal) or J < nb
        const int last = (a.causal ? I : a.nb - 1) - 32 * w;   // highest bit of this word
        bits = last >= 31 ? 0xFFFFFFFFu : (last >= 0 ? (2u << last) - 1u : 0u);
      } else {
        bits = a.mask[((size_t)bh * a.nb + I) * W + w];
      }
    }
    m0[b][w] = bits;
    m1[b][w] = 0u;
  }

  const float zs = a.zscale;
  const float kappa = a.kappa;
  float t0, lo, hi;
  if (a.nohist) {
    // without the histogram: the bracket [max z - 1, max z - n^(1 - alpha)]
    // (f(max z - 1) >= 0 from the max term alone; at max z - n^(1 - alpha)
    // each of the n terms is at most 1/n), started from its lower end
    const float zmax = qvalid ? float_of_ord(reinterpret_cast<const int*>(a.tau)[(size_t)bh * a.N + qrow]) * zs : 0.f;
    const float n = (float)(a.causal ? qrow + 1 : a.N);
    t0 = zmax - 1.f;
    lo = t0 - BRACKET_PAD;
    hi = zmax - __builtin_amdgcn_exp2f((1.f - a.alpha) * __builtin_amdgcn_logf(n)) + BRACKET_PAD;
    if (qvalid && h == 0 && a.tau_h_out) a.tau_h_out[(size_t)bh * a.N + qrow] = t0;
  } else {
    t0 = qvalid ? a.tau[(size_t)bh * a.N + qrow] : 0.f;
    lo = t0 - BRACKET_PAD;
    hi = t0 + a.delta_h + BRACKET_PAD;
  }
  float t = t0;
  float tp = 0.f, fprev = 0.f;    // previous point (secant)
  bool done = !qvalid;
  int npass = 0;

  // ---- rows whose keys with scores above lo the histogram pass kept ----
  // f(t) for t >= lo sums over those scores alone, so the solver's steps
  // (the ones the passes would take) run on them exactly, without streaming
  // the tiles. The scores are formed here, each lane of a row taking the dot
  // product over its half of d, in the order the keys were stored (the same
  // in every run), and written beside the keys for the output pass.
  bool listed = false;
  uint32_t* lrow = nullptr;
  uint32_t lnum = LIST_NONE;
  float lv[LIST_CAP];               // the listed scores
  uint32_t kws[LIST_CAP / 2];       // their keys, two per word
  int nsteps = 0;                   // solver steps this row took
  if (!a.nohist && !a.plain) {
    lrow = reinterpret_cast<uint32_t*>(reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) +
                                       (size_t)(qvalid ? qrow : 0) * a.lq.sn);
    if (qvalid) {
      lnum = lrow[0];
      if ((lnum & 0xFFFF0000u) == LIST_GATHER) lnum &= 0xFFFFu;   // marked by an earlier run of this pass
      lo = fmaxf(lo, __uint_as_float(lrow[1]));   // the root is not below the window
    }
    listed = qvalid && lnum <= (uint32_t)LIST_CAP;
    if (__ballot(listed) != 0) {
      const uint32_t* lkw = lrow + 2 + LIST_CAP;   // keys, two per word
      const int kmax = a.causal ? qrow : a.N - 1;
#pragma unroll
      for (int i = 0; i < LIST_CAP; i += 2) {
        const uint32_t kw = (listed && i < (int)lnum) ? lkw[i / 2] : 0u;
        kws[i / 2] = kw;
        float part[2] = {0.f, 0.f};
        bool use[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int key = (int)((kw >> (16 * c)) & 0xFFFFu);
          use[c] = listed && i + c < (int)lnum && key <= kmax;
        }
        if (use[0]) {
          const int k0 = (int)(kw & 0xFFFFu), k1 = use[1] ? (int)(kw >> 16) : k0;
          part[0] = row_dot<E, D>(bq, K + (size_t)k0 * a.lkv.sn, h);
          part[1] = row_dot<E, D>(bq, K + (size_t)k1 * a.lkv.sn, h);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          part[c] += __shfl_xor(part[c], 32);
          lv[i + c] = use[c] ? part[c] : -INFINITY;
        }
      }
      auto lsums = [&](float e, float& g0, float& g1, float& g2) {
        g0 = g1 = g2 = 0.f;
#pragma unroll
        for (int i = 0; i < LIST_CAP; ++i) {
          const float x = lv[i] * zs - e;
          if (x > 0.f) {
            if constexpr (PM == PM_K1) {
              g0 += x;
              g1 += 1.f;
            } else if constexpr (PM == PM_K2) {
              g0 = fmaf(x, x, g0);
              g1 += x;
              g2 += 1.f;
            } else if constexpr (PM == PM_K4) {
              const float x2 = x * x;
              g0 = fmaf(x2, x2, g0);
              g1 = fmaf(x2, x, g1);
              g2 += x2;
            } else {
              const float lx = __builtin_amdgcn_logf(x);
              g0 += __builtin_amdgcn_exp2f(kappa * lx);
              g1 += __builtin_amdgcn_exp2f((kappa - 1.f) * lx);
              g2 += __builtin_amdgcn_exp2f((kappa - 2.f) * lx);
            }
          }
        }
      };
      bool ldone = !listed;
      // A secant through a change of support (a score entering between its
      // two points) can be much steeper than f near the root, so a step below
      // the tolerance does not bound the error there: such a step stands only
      // where f changes sign within the tolerance of the new point (values in
      // registers, so the two extra evaluations are cheap); else both points
      // narrow the bracket and the steps go on.
      auto confirm = [&](float tn, float f) {
        if (fabsf(f) <= F_TOL) return true;
        const float eps = STEP_TOL * fmaxf(1.f, fabsf(tn));
        float m0, m1, m2, p0, p1, p2;
        lsums(tn - eps, m0, m1, m2);
        lsums(tn + eps, p0, p1, p2);
        if (m0 >= 1.f && p0 <= 1.f) return true;
        if (m0 >= 1.f) lo = fmaxf(lo, tn - eps); else hi = fminf(hi, tn - eps);
        if (p0 >= 1.f) lo = fmaxf(lo, tn + eps); else hi = fminf(hi, tn + eps);
        return false;
      };
      if constexpr (SV == SV_SECANT) {
        // first step from tau_h and tau_h + 1/B, as the first pass would take it
        float g0, g1, g2, h0, h1, h2;
        const float t1 = t + a.delta_h;
        lsums(t, g0, g1, g2);
        lsums(t1, h0, h1, h2);
        if (!ldone) {
          const float f = g0 - 1.f, f1 = h0 - 1.f;
          if (f >= 0.f) lo = fmaxf(lo, t); else hi = fminf(hi, t);
          if (f1 >= 0.f) lo = fmaxf(lo, t1); else hi = fminf(hi, t1);
          float tn = t1 - f1 * (t1 - t) / (f1 - f);
          ldone = safeguard_step(tn, t, f, lo, hi, true);
          if (ldone) ldone = confirm(tn, f);
          ++nsteps;
          tp = t1;
          fprev = f1;
          t = tn;
        }
      }
#pragma unroll 1
      for (int vs = 0; vs < MAX_VSTEPS && __ballot(!ldone) != 0; ++vs) {
        const float e = t;
        float g0, g1, g2;
        lsums(e, g0, g1, g2);
        if (!ldone) {
          const float f = g0 - 1.f;
          if (f >= 0.f) lo = fmaxf(lo, e); else hi = fminf(hi, e);
          float tn;
          bool ok = true;
          if constexpr (SV == SV_SECANT) {
            tn = e - f * (e - tp) / (f - fprev);
            ok = fabsf(tn - e) <= 0.5f * fabsf(e - tp);
            tp = e;
            fprev = f;
          } else if constexpr (SV == SV_HALLEY) {
            const float d1 = -kappa * g1, d2 = kappa * (kappa - 1.f) * g2;
            tn = e - 2.f * f * d1 / (2.f * d1 * d1 - f * d2);
          } else {
            tn = e + f / (kappa * g1);
          }
          ldone = safeguard_step(tn, e, f, lo, hi, ok);
          if constexpr (SV == SV_SECANT) {
            if (ldone) ldone = confirm(tn, f);
          }
          ++nsteps;
          t = tn;
        }
      }
      if (listed) {
        if (!ldone) t = 0.5f * (lo + hi);   // the bracket has closed around the root
        done = true;
      }
    }
  }

  TileIO<E, D, NTHR> iok;
  __syncthreads();

  bool act0 = true, act1 = true;   // blocks with unconverged rows (their tiles are streamed)
  bool my_busy = true;             // this wave has unconverged rows (it computes)
  if (!a.nohist) {
    // rows solved on their kept keys take no pass: only the waves (and
    // blocks) holding other rows stream and compute, and the mask at tau_h
    // covers only those rows. The output pass gathers the solved rows: their
    // support at the final t (x > 0 as the output pass evaluates it),
    // compacted, scores and keys, marked in word 0.
    if (listed && h == 0) {
      uint16_t* lk = reinterpret_cast<uint16_t*>(lrow + 2 + LIST_CAP);
      int pos = 0;
#pragma unroll
      for (int i = 0; i < LIST_CAP; ++i)
        if (i < (int)lnum && xclamp(lv[i], zs, t) > 0.f) {
          lrow[2 + pos] = __float_as_uint(lv[i]);
          lk[pos] = (uint16_t)((kws[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
          ++pos;
        }
#pragma unroll
      for (int i = 0; i < LIST_CAP; ++i)   // the unused slots cleared (the list is copied whole)
        if (i >= pos) {
          lrow[2 + i] = 0u;
          lk[i] = 0;
        }
      lrow[0] = LIST_GATHER | (uint32_t)pos;
    }
    my_busy = __ballot(!done) != 0;
    if (lane == 0) wave_busy[wave] = my_busy ? 1 : 0;
    __syncthreads();
    act0 = wave_busy[0] || wave_busy[1];
    act1 = wave_busy[2] || wave_busy[3];
    __syncthreads();
  }
  // the start without the histogram can be far from the root, and plain
  // secant steps converge slowly where a score sits just above the root:
  // those modes get the larger cap
  const int cap = (!act0 && !act1) ? 0
                : (a.pass_cap ? a.pass_cap : ((a.nohist || a.plain) ? MAX_PASSES_NOHIST : MAX_PASSES));
  for (int pass = 1; pass <= cap; ++pass) {
    const uint32_t* tm0 = (pass == 1) ? m0[0] : m1[0];
    const uint32_t* tm1 = (pass == 1) ? m0[1] : m1[1];
    const uint32_t* mymask = (pass == 1) ? m0[lb] : m1[lb];
    const bool wave_act = my_busy && blk_valid;
    float F0 = 0.f, F1 = 0.f, F2 = 0.f, F0b = 0.f;
    float F3 = 0.f, F4 = 0.f;                  // sum x and count (kappa = 4)
    int npos_k = 0;                            // count of x > 0 (kappa = 1, 2, 4), an integer add per score
    float xs[XK];                              // the XK smallest x > 0, ascending (kappa = 1, 2, 4)
#pragma unroll
    for (int i = 0; i < XK; ++i) xs[i] = INFINITY;
    // other kappa, pass 1: the TOPK largest x > 0 (descending) and how many x > 0
    float L[TOPK];
#pragma unroll
    for (int i = 0; i < TOPK; ++i) L[i] = 0.f;
    int npos = 0;
    uint32_t tiles_pass = 0;
    const float te = t;                     // evaluation point of this pass
    const float te_lo = (SV == SV_SECANT && pass == 1) ? t : te;
    // integer powers: the least raw score v with fma(v, c, -te) > 0, so that
    // comparing raw scores against it finds the x > 0 exactly as the sums
    // form x (-inf where it cannot be found: every score is then formed)
    float xr_first = -INFINITY;
    if constexpr (PM == PM_K1 || PM == PM_K2 || PM == PM_K4) {
      float v = te / zs;
      bool ok = isfinite(v);
#pragma unroll 1
      for (int i = 0; ok && i < 8 && fmaf(v, zs, -te) > 0.f; ++i) v = nextafterf(v, -INFINITY);
      ok = ok && !(fmaf(v, zs, -te) > 0.f);
#pragma unroll 1
      for (int i = 0; ok && i < 8 && !(fmaf(v, zs, -te) > 0.f); ++i) v = nextafterf(v, INFINITY);
      ok = ok && fmaf(v, zs, -te) > 0.f;
      if (ok) xr_first = v;
    }

    UnionIter itr;
    itr.init(tm0, tm1, act0, act1 && (blk0 + 1 < a.nb), W);
    int J = itr.next();
    int buf = 0;
    if (J >= 0) {
      iok.load(K, J * BLK, a.N, tid, a.lkv.sn);
    }
    wait_vmem();
    if (J >= 0) {
      iok.template store_rows<LDK>(ktile[0], tid);
    }
    __syncthreads();
    while (J >= 0) {
      const int Jn = itr.next();
      if (Jn >= 0) iok.load(K, Jn * BLK, a.N, tid, a.lkv.sn);
      if (wave_act && ((mymask[J >> 5] >> (J & 31)) & 1u)) {
        floatx16 acc[2];
        tile_x_frags<E, D, LDK>(acc, ktile[buf], bq, l32, h);
        if (J * BLK + BLK > a.N || (a.causal && J == myblk)) mask_keys(acc, J * BLK, a.N, a.causal, qrow, h);
        float gm[4];
        group_max(acc, gm);
        const float lm = fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3]));
        const float xmax = lm * zs - te_lo;
        if (pass == 1) {
          const bool mb = qvalid && !listed && (xmax > -MASK_PAD);
          if (__ballot(mb) != 0 && lane == 0) atomicOr(&m1[lb][J >> 5], 1u << (J & 31));
        }
        if (__ballot(!done && xmax > 0.f) != 0) {
          // groups of 8 scores where no lane has x > 0 add nothing: skip them
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (__ballot(!done && gm[g] * zs - te_lo > 0.f) == 0) continue;
            const int kh = g >> 1;
            if constexpr (PM == PM_K1 || PM == PM_K2 || PM == PM_K4) {
              // one score's terms; x <= 0 adds zeros and leaves the minima
              auto add = [&](float v) {
                const float x = fmaf(v, zs, -te);
                const bool pos = x > 0.f;
                npos_k += pos ? 1 : 0;
                float xp = pos ? x : INFINITY;
#pragma unroll
                for (int i = 0; i < XK; ++i) {
                  const float m = fminf(xs[i], xp);
                  xp = fmaxf(xs[i], xp);
                  xs[i] = m;
                }
                if constexpr (PM == PM_K2) {
                  const float y = fmaxf(x, 0.f);
                  F0 = fmaf(y, y, F0);
                  F1 += y;
                } else if constexpr (PM == PM_K1) {
                  F0 += fmaxf(x, 0.f);
                } else {
                  const float y = fmaxf(x, 0.f);
                  const float y2 = y * y;
                  F0 = fmaf(y2, y2, F0);
                  F1 = fmaf(y2, y, F1);
                  F2 += y2;
                  F3 += y;
                }
              };
              // A lane with one x > 0 in the group adds the group max's
              // terms alone (the other seven add zeros); one with several
              // adds each score's; one with none adds nothing.
              int ne = 0;
#pragma unroll
              for (int rr = 0; rr < 8; ++rr) ne += acc[kh][8 * (g & 1) + rr] >= xr_first ? 1 : 0;
              if (ne == 1) {
                add(gm[g]);
              } else if (ne > 1) {
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) add(acc[kh][8 * (g & 1) + rr]);
              }
              continue;
            }
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
              const int r = 8 * (g & 1) + rr;
              const float x = acc[kh][r] * zs - te;
              if (pass == 1 && x > 0.f) {
                ++npos;
                float v = x;
#pragma unroll
                for (int i = 0; i < TOPK; ++i) {
                  const float m = fmaxf(L[i], v);
                  v = fminf(L[i], v);
                  L[i] = m;
                }
              }
              if constexpr (SV == SV_SECANT) {
                if (x > 0.f) F0 += powpos(x, kappa);
                if (pass == 1) {
                  const float xb = x - a.delta_h;
                  if (xb > 0.f) F0b += powpos(xb, kappa);
                }
              } else {
                if (x > 0.f) {
                  const float lx = __builtin_amdgcn_logf(x);
                  F0 += __builtin_amdgcn_exp2f(kappa * lx);
                  F1 += __builtin_amdgcn_exp2f((kappa - 1.f) * lx);
                  if constexpr (SV == SV_HALLEY) F2 += __builtin_amdgcn_exp2f((kappa - 2.f) * lx);
                }
              }
            }
          }
        }
        if ((wave & 1) == 0) tiles_pass++;
      }
      wait_vmem();
      if (Jn >= 0) {
        if (NBUF == 1) __syncthreads();
        iok.template store_rows<LDK>(ktile[NBUF - 1 - buf], tid);
      }
      __syncthreads();
      buf = NBUF - 1 - buf;
      J = Jn;
    }

    if (a.tiles_per_pass && lane == 0 && (wave & 1) == 0 && tiles_pass) atomicAdd(a.tiles_per_pass + min(pass, MAX_PASSES), tiles_pass);
    if constexpr (PM == PM_K1) F1 = (float)npos_k;
    if constexpr (PM == PM_K2) F2 = (float)npos_k;
    if constexpr (PM == PM_K4) F4 = (float)npos_k;
    F0 += __shfl_xor(F0, 32);
    F1 += __shfl_xor(F1, 32);
    F2 += __shfl_xor(F2, 32);
    F0b += __shfl_xor(F0b, 32);
    if constexpr (PM == PM_K4) {
      F3 += __shfl_xor(F3, 32);
      F4 += __shfl_xor(F4, 32);
    }
    if constexpr (PM == PM_GEN) {
      if (pass == 1) {   // the row's TOPK largest x > 0: merge the two lanes' lists
        float o[TOPK];
#pragma unroll
        for (int i = 0; i < TOPK; ++i) o[i] = __shfl_xor(L[i], 32);
        npos += __shfl_xor(npos, 32);
#pragma unroll
        for (int j = 0; j < TOPK; ++j) {
          float v = o[j];
#pragma unroll
          for (int i = 0; i < TOPK; ++i) {
            const float m = fmaxf(L[i], v);
            v = fminf(L[i], v);
            L[i] = m;
          }
        }
      }
    }
    {   // the row's XK smallest over its two lanes
      float o[XK];
#pragma unroll
      for (int i = 0; i < XK; ++i) o[i] = __shfl_xor(xs[i], 32);
#pragma unroll
      for (int j = 0; j < XK; ++j) {
        float v = o[j];
#pragma unroll
        for (int i = 0; i < XK; ++i) {
          const float m = fminf(xs[i], v);
          v = fmaxf(xs[i], v);
          xs[i] = m;
        }
      }
    }

    if (!done && wave_act) {
      npass = pass;
      if constexpr (SV == SV_SECANT) {
        const float f = F0 - 1.f;
        float tn;
        bool shrink_ok;   // the step must at least halve the previous one
        if (pass == 1) {
          const float t1 = te + a.delta_h, f1 = F0b - 1.f;
          if (f >= 0.f) lo = fmaxf(lo, te); else hi = fminf(hi, te);
          if (f1 >= 0.f) lo = fmaxf(lo, t1); else hi = fminf(hi, t1);
          tn = t1 - f1 * (t1 - te) / (f1 - f);
          shrink_ok = true;
          tp = t1;
          fprev = f1;
        } else {
          if (f >= 0.f) lo = fmaxf(lo, te); else hi = fminf(hi, te);
          tn = te - f * (te - tp) / (f - fprev);
          shrink_ok = fabsf(tn - te) <= 0.5f * fabsf(te - tp);
          tp = te;
          fprev = f;
        }
        done = safeguard_step(tn, te, f, lo, hi, shrink_ok);
        ++nsteps;
        t = tn;
      } else {
        // One solver step per evaluation point. For kappa = 1, 2 and 4, f is
        // a polynomial in t between support changes, so while every member
        // that a step takes out of the support is known (the step stays
        // below the largest of the XK smallest x > 0 kept, or the row has
        // fewer than XK), the sums at the new point follow from those at the
        // old one (binomial expansion of (x - d)^k, less the leaving members'
        // terms), and the next step (the same one another pass would take) is
        // formed without streaming the keys again.
        constexpr bool SHIFT_PM = (PM == PM_K1 || PM == PM_K2 || PM == PM_K4);
        const bool SHIFT = SHIFT_PM && !a.plain;
        float e0 = te, G0 = F0, G1 = F1, G2 = F2, G3 = F3, G4 = F4;
        float xsh[XK];   // the kept x > 0 at e0 (<= 0: left the support)
#pragma unroll
        for (int i = 0; i < XK; ++i) xsh[i] = xs[i];
#pragma unroll 1
        for (int vp = 0; vp < (SHIFT ? 4 : 1); ++vp) {
          const float f = G0 - 1.f;
          if (f >= 0.f) lo = fmaxf(lo, e0); else hi = fminf(hi, e0);
          const float d1 = -kappa * G1;
          float tn;
          if constexpr (SV == SV_HALLEY) {
            const float d2 = kappa * (kappa - 1.f) * G2;
            tn = e0 - 2.f * f * d1 / (2.f * d1 * d1 - f * d2);
          } else {
            tn = e0 - f / d1;
          }
          done = safeguard_step(tn, e0, f, lo, hi, true);
          ++nsteps;
          if constexpr (PM == PM_K4) {
            // kappa = 4: f is three times continuously differentiable and,
            // for a step d > 0, its third derivative -24 sum [x - s]+ stays
            // in [-24 G3, 0] over the step (support changes included), so
            // f(e0 + d) lies between the quadratic Taylor value q and
            // q - 4 G3 d^3. f is convex and decreasing, and wherever
            // sum p <= 1 every x <= 1, so |f'| >= kappa (1 - |f|) there:
            // |tau - tn| <= |f(tn)| / (4 (1 - |f(tn)|)). When that bound
            // meets the step tolerance, tn stands without another pass.
            const float d = tn - e0;
            if (!done && d > 0.f && SHIFT) {
              const float q = fmaf(d, fmaf(6.f * G2, d, -4.f * G1), f);
              const float fb = fmaxf(fabsf(q), fabsf(fmaf(-4.f * G3 * d, d * d, q)));
              done = fb < 0.5f && fb <= 4.f * (1.f - fb) * STEP_TOL * fmaxf(1.f, fabsf(tn));
            }
          }
          t = tn;
          if (done || !SHIFT) break;
          const float d = tn - e0;
          // members with x <= d leave; all of them are kept ones while d
          // stays below the last kept x (every other x > 0 is at least that)
          if (!(d > 0.f && (d < xsh[XK - 1] || xsh[XK - 1] == INFINITY))) break;   // else stream again
          if constexpr (PM == PM_K4) {       // G0..G4 = sum x^4, x^3, x^2, x, count
            const float d2 = d * d, d3 = d2 * d;
            G0 = G0 - 4.f * d * G1 + 6.f * d2 * G2 - 4.f * d3 * G3 + d2 * d2 * G4;
            G1 = G1 - 3.f * d * G2 + 3.f * d2 * G3 - d3 * G4;
            G2 = G2 - 2.f * d * G3 + d2 * G4;
            G3 = fmaf(-d, G4, G3);
#pragma unroll
            for (int i = 0; i < XK; ++i)
              if (xsh[i] > 0.f && xsh[i] <= d) {
                const float r = xsh[i] - d, r2 = r * r;
                G0 -= r2 * r2;
                G1 -= r2 * r;
                G2 -= r2;
                G3 -= r;
                G4 -= 1.f;
              }
          } else if constexpr (PM == PM_K2) {  // G0 = sum x^2, G1 = sum x, G2 = count
            G0 = fmaf(d * d, G2, fmaf(-2.f * d, G1, G0));
            G1 = fmaf(-d, G2, G1);
#pragma unroll
            for (int i = 0; i < XK; ++i)
              if (xsh[i] > 0.f && xsh[i] <= d) {
                const float r = xsh[i] - d;
                G0 -= r * r;
                G1 -= r;
                G2 -= 1.f;
              }
          } else {                           // G0 = sum x, G1 = count
            G0 = fmaf(-d, G1, G0);
#pragma unroll
            for (int i = 0; i < XK; ++i)
              if (xsh[i] > 0.f && xsh[i] <= d) {
                G0 -= xsh[i] - d;
                G1 -= 1.f;
              }
          }
#pragma unroll
          for (int i = 0; i < XK; ++i) xsh[i] -= d;
          e0 = tn;
        }
      }
      if constexpr (PM == PM_GEN) {
        // Other kappa: when the row has at most TOPK scores above te and the
        // root is not below te (f(te) >= 0, so lo >= te), those scores are the
        // whole support anywhere in [lo, hi]: f and its derivatives there
        // follow from them exactly, and the solver's further steps (the ones
        // later passes would take) run on them without streaming the keys.
        if (!done && pass == 1 && npos <= TOPK && lo >= te && !a.plain) {
          auto sums = [&](float e, float& g0, float& g1, float& g2) {
            g0 = g1 = g2 = 0.f;
#pragma unroll
            for (int i = 0; i < TOPK; ++i) {
              const float x = L[i] - (e - te);
              if (i < npos && x > 0.f) {
                const float lx = __builtin_amdgcn_logf(x);
                g0 += __builtin_amdgcn_exp2f(kappa * lx);
                g1 += __builtin_amdgcn_exp2f((kappa - 1.f) * lx);
                g2 += __builtin_amdgcn_exp2f((kappa - 2.f) * lx);
              }
            }
          };
#pragma unroll 1
          for (int vs = 0; vs < MAX_VSTEPS && !done; ++vs) {
            const float e = t;
            float g0, g1, g2;
            sums(e, g0, g1, g2);
            const float f = g0 - 1.f;
            if (f >= 0.f) lo = fmaxf(lo, e); else hi = fminf(hi, e);
            float tn;
            bool ok = true;
            if constexpr (SV == SV_SECANT) {
              tn = e - f * (e - tp) / (f - fprev);
              ok = fabsf(tn - e) <= 0.5f * fabsf(e - tp);
              tp = e;
              fprev = f;
            } else if constexpr (SV == SV_HALLEY) {
              const float d1 = -kappa * g1, d2 = kappa * (kappa - 1.f) * g2;
              tn = e - 2.f * f * d1 / (2.f * d1 * d1 - f * d2);
            } else {
              tn = e + f / (kappa * g1);
            }
            done = safeguard_step(tn, e, f, lo, hi, ok);
            if constexpr (SV == SV_SECANT) {
              // as for the listed rows: a small secant step stands only where
              // f changes sign within the tolerance of the new point
              if (done && !(fabsf(f) <= F_TOL)) {
                const float eps = STEP_TOL * fmaxf(1.f, fabsf(tn));
                float m0, m1, m2, p0, p1, p2;
                sums(tn - eps, m0, m1, m2);
                sums(tn + eps, p0, p1, p2);
                if (!(m0 >= 1.f && p0 <= 1.f)) {
                  if (m0 >= 1.f) lo = fmaxf(lo, tn - eps); else hi = fminf(hi, tn - eps);
                  if (p0 >= 1.f) lo = fmaxf(lo, tn + eps); else hi = fminf(hi, tn + eps);
                  done = false;
                }
              }
            }
            ++nsteps;
            t = tn;
          }
          if (!done) {   // the bracket has shrunk around the root meanwhile
            done = true;
            t = 0.5f * (lo + hi);
          }
        }
      }
      if (!done && pass == cap) {
        // pass cap reached: the root lies in [lo, hi]; take its midpoint
        done = true;
        t = 0.5f * (lo + hi);
        if (a.unconverged && h == 0) atomicAdd(a.unconverged, 1u);
      }
    }
    // workgroup-wide: which blocks still have unconverged rows
    const bool busy = __ballot(!done) != 0;
    my_busy = busy;
    if (lane == 0) wave_busy[wave] = busy ? 1 : 0;
    __syncthreads();
    act0 = wave_busy[0] || wave_busy[1];
    act1 = wave_busy[2] || wave_busy[3];
    __syncthreads();
    if (!act0 && !act1) break;
  }

  // ---------------- write tau, passes and the mask at tau_h ---------------
  if (qvalid && h == 0) {
    a.tau[(size_t)bh * a.N + qrow] = t;
    if (a.passes_out) a.passes_out[(size_t)bh * a.N + qrow] = (uint8_t)npass;
    if (a.iters_out) a.iters_out[(size_t)bh * a.N + qrow] = (uint8_t)min(nsteps, 255);
  }
  __syncthreads();
  for (int i = tid; i < NBLKS * W; i += NTHR) {
    const int b = i / W, w = i % W;
    if (blk0 + b < a.nb) a.mask[((size_t)bh * a.nb + blk0 + b) * W + w] = m1[b][w];
  }
}

// ---------------------------------------------------------------------------
// fwd_out: P.V over the set bits of the mask at tau_h (a superset of every
// block with p > 0 at the final tau), and the final mask
// ---------------------------------------------------------------------------
// At d = 64 the register budget is held to 3 waves per SIMD with the state (168
// VGPRs) and 4 without (128): measured faster than the unconstrained
// allocation, which lands just above either limit.
template <class E, int D, int PM, int NBUF, bool VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? (VB ? 3 : 4) : 1)))
void fwd_out_kernel(FwdArgs a) {
  using S = typename E::storage;
  constexpr int NTHR = 256, NBLKS = 2;
  constexpr int LDK = Ld<E, D>::value;
  constexpr bool TR = E::TR_READ;
  // V tile: row-major like K when the A operand of P.V is read transposed,
  // else stored transposed [D][64 + pad]
  constexpr int LDV = TR ? LDK : Ld<E, BLK>::value;
  __shared__ __attribute__((aligned(16))) S ktile[NBUF][BLK * LDK];
  __shared__ __attribute__((aligned(16))) S vtile[NBUF][TR ? BLK * LDK : D * LDV];
  __shared__ uint32_t m1[NBLKS][WMAX], mf[NBLKS][WMAX];
  __shared__ uint32_t sub_s[4][LIST_MAX_N / 1024];   // per wave: 32-key sub-tiles with p > 0

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

  const S* Q = reinterpret_cast<const S*>(a.q) + a.lq.head(bh, a.H);
  const S* K = reinterpret_cast<const S*>(a.k) + a.lkv.head(bh / a.G, a.H / a.G);
  const S* V = reinterpret_cast<const S*>(a.v) + a.lkv.head(bh / a.G, a.H / a.G);

  for (int i = tid; i < NBLKS * W; i += NTHR) {
    const int b = i / W, w = i % W;
    m1[b][w] = (blk0 + b < a.nb) ? a.mask[((size_t)bh * a.nb + blk0 + b) * W + w] : 0u;
    mf[b][w] = 0u;
  }
  for (int i = tid; i < 4 * (LIST_MAX_N / 1024); i += NTHR) (&sub_s[0][0])[i] = 0u;
  const float zs = a.zscale;
  const float kappa = a.kappa;
  const float tf = qvalid ? a.tau[(size_t)bh * a.N + qrow] : 0.f;
  // rows the refinement solved on their kept keys (marked in word 0 of
  // their row of o): the output is gathered from the rows of V their
  // support names. The other rows take the tile path below, over the mask
  // at tau_h of those rows alone.
  const uint32_t w0 = (!a.nohist && qvalid) ? *reinterpret_cast<const uint32_t*>(
                          reinterpret_cast<const S*>(a.o) + a.lq.head(bh, a.H) + (size_t)qrow * a.lq.sn) : 0u;
  const bool marked = !a.nohist && a.N <= LIST_MAX_N && qvalid && (w0 & 0xFFFF0000u) == LIST_GATHER &&
                      (w0 & 0xFFFFu) <= (uint32_t)LIST_CAP;
  // (the barrier also makes the mask words visible to every wave)
  const bool any_marked = __syncthreads_or(marked);
  uint32_t halves = 0;   // 32x32 sub-tiles whose products this workgroup runs
  if (any_marked) {
    constexpr int DH = D / 2;   // elements of the row this lane forms
    // the lists, staged in LDS (the tile buffers are free until the tile path)
    static_assert(sizeof(ktile) >= 4 * LIST_LDS * 128, "list staging needs 16.5 KB");
    uint32_t* lds_l = reinterpret_cast<uint32_t*>(&ktile[0][0]) + LIST_LDS * (64 * lb + 32 * (wave & 1) + l32);
    if (marked)
      stage_list(lds_l, reinterpret_cast<const uint32_t*>(reinterpret_cast<const S*>(a.o) + a.lq.head(bh, a.H) +
                                                          (size_t)qrow * a.lq.sn), h);
    __syncthreads();
    float ov[DH];
#pragma unroll
    for (int e = 0; e < DH; ++e) ov[e] = 0.f;
    const int n = marked ? (int)(w0 & 0xFFFFu) : 0;
    const int kmax = a.causal ? qrow : a.N - 1;
    const uint32_t* lkw = lds_l + 2 + LIST_CAP;   // keys, two per word
    const S* Vh = V + DH * h;
    // CH rows of V in flight per step
    constexpr int CH = (D * sizeof(S) <= 128) ? 4 : 2;
#pragma unroll
    for (int i = 0; i < LIST_CAP; i += CH) {
      if (i < n) {
        float x[CH];
        int key[CH];
        RowChunk<E, DH> rc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const float xc = xclamp(__uint_as_float(lds_l[2 + i + c]), zs, tf);
          const int kc = (int)((lkw[(i + c) / 2] >> (16 * ((i + c) & 1))) & 0xFFFFu);
          const bool use = i + c < n && xc > 0.f && kc <= kmax;
          x[c] = use ? xc : 0.f;
          key[c] = use ? kc : 0;   // unused entries read row 0 with weight 0
          rc[c].load(Vh + (size_t)key[c] * a.lkv.sn);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          rc[c].fma(ov, pk01<PM>(x[c], kappa));
          if (h == 0 && x[c] > 0.f) {   // mask and sub-tile bits (atomics only for new ones)
            const int J = key[c] >> 6;
            const uint32_t bj = 1u << (J & 31), bs = 1u << ((key[c] >> 5) & 31);
            if ((mf[lb][J >> 5] & bj) == 0u) atomicOr(&mf[lb][J >> 5], bj);
            if ((sub_s[wave][key[c] >> 10] & bs) == 0u) atomicOr(&sub_s[wave][key[c] >> 10], bs);
          }
        }
      }
    }
    if (marked) {
      S* orow = reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) + (size_t)qrow * a.lq.sn;
      if constexpr (sizeof(S) == 2) {
#pragma unroll
        for (int c = 0; c < DH / 8; ++c) {
          uint32_t ww[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ww[e] = (uint32_t)E::from_f(ov[8 * c + 2 * e]) | ((uint32_t)E::from_f(ov[8 * c + 2 * e + 1]) << 16);
          *reinterpret_cast<uint4*>(orow + DH * h + 8 * c) = make_uint4(ww[0], ww[1], ww[2], ww[3]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < DH / 4; ++c)
          *reinterpret_cast<float4*>(orow + DH * h + 4 * c) = make_float4(ov[4 * c], ov[4 * c + 1], ov[4 * c + 2], ov[4 * c + 3]);
      }
      if constexpr (VB) {
        // the backward's state for this row: its support list (words 0 ..
        // 31, the same as in o; word 0 is a NaN as a float, which vbar
        // never holds) and the mask at tau_h of the rows of its block that
        // take the tile path (words 32 .. 32 + W)
        uint32_t* vrow = reinterpret_cast<uint32_t*>(a.state + ((size_t)bh * a.N + qrow) * D);
        if (h == 0) {
#pragma unroll
          for (int c = 0; c < 8; ++c)
            reinterpret_cast<uint4*>(vrow)[c] = make_uint4(lds_l[4 * c], lds_l[4 * c + 1], lds_l[4 * c + 2], lds_l[4 * c + 3]);
        } else {
          // the mask words (the rest of the record is not read)
          for (int c = 0; c < (W + 3) / 4; ++c) {
            uint32_t q4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) q4[e] = (4 * c + e < W) ? m1[lb][4 * c + e] : 0u;
            reinterpret_cast<uint4*>(vrow + 32)[c] = make_uint4(q4[0], q4[1], q4[2], q4[3]);
          }
        }
      }
    }
    if (a.gathered) {
      const uint32_t rows = __popcll(__ballot(marked && h == 0));
      if (lane == 0 && rows) atomicAdd(a.gathered, rows);
    }
    __syncthreads();   // the staged lists are read before the tile path reuses their buffer
  }
  // the tile path: rows not gathered. Both waves of a block compute when
  // either holds such a row (the tiles are counted per block).
  const bool tile_row = qvalid && !marked;
  const float tft = tile_row ? tf : INFINITY;   // gathered rows take p = 0 here
  __shared__ int tile_w[4];
  const bool wave_rows = __ballot(tile_row) != 0;   // (all lanes take the ballot)
  if (lane == 0) tile_w[wave] = wave_rows ? 1 : 0;
  __syncthreads();
  const bool wave_tile = blk_valid && (tile_w[2 * lb] || tile_w[2 * lb + 1]);

  typename E::frag bq[D / E::KPI];
  load_row_frags<E, D>(bq, Q + (size_t)qrow * a.lq.sn, qvalid, h);
  TileIO<E, D, NTHR> iok, iov;

  floatx16 acc_o[D / 32], acc_u[VB ? D / 32 : 1];
  float usum = 0.f;   // sum of the u values the product used (rounded as its operand)
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc_o[db] = floatx16{};
#pragma unroll
  for (int db = 0; db < (VB ? D / 32 : 1); ++db) acc_u[db] = floatx16{};
  const int tr_off = tr_lane_off(lane, LDV);
  {
    UnionIter itr;
    itr.init(m1[0], m1[1], true, blk0 + 1 < a.nb, W);
    int J = itr.next();
    int buf = 0;
    if (J >= 0) {
      iok.load(K, J * BLK, a.N, tid, a.lkv.sn);
      iov.load(V, J * BLK, a.N, tid, a.lkv.sn);
    }
    wait_vmem();
    if (J >= 0) {
      iok.template store_rows<LDK>(ktile[0], tid);
      if constexpr (TR) iov.template store_rows<LDV>(vtile[0], tid);
      else iov.template store_trans<LDV>(vtile[0], tid);
    }
    __syncthreads();
    uint32_t tiles_out = 0;
    while (J >= 0) {
      const int Jn = itr.next();
      if (Jn >= 0) {
        iok.load(K, Jn * BLK, a.N, tid, a.lkv.sn);
        iov.load(V, Jn * BLK, a.N, tid, a.lkv.sn);
      }
      if (wave_tile && ((m1[lb][J >> 5] >> (J & 31)) & 1u)) {
        floatx16 acc[2];
        tile_x_frags<E, D, LDK>(acc, ktile[buf], bq, l32, h);
        if (J * BLK + BLK > a.N || (a.causal && J == myblk)) mask_keys(acc, J * BLK, a.N, a.causal, qrow, h);
        // the products of a 32-key half run only where some row of the wave
        // has a score above tau in it
        bool act[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          float hm = acc[kh][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) hm = fmaxf(hm, acc[kh][r]);
          act[kh] = __ballot(tile_row && hm * zs - tft > 0.f) != 0;
        }
        if (act[0] || act[1]) {
          if (lane == 0) atomicOr(&mf[lb][J >> 5], 1u << (J & 31));
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            if (!act[kh]) continue;
            halves++;
            if (lane == 0 && a.N <= LIST_MAX_N) atomicOr(&sub_s[wave][(2 * J + kh) >> 5], 1u << ((2 * J + kh) & 31));
            floatx16 pv, uv;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float x = xclamp(acc[kh][r], zs, tft);
              pv[r] = pk01<PM>(x, kappa);
              if constexpr (VB) uv[r] = uk01<PM>(x, kappa);
            }
#pragma unroll
            for (int st = 0; st < E::ACC_KSTEPS; ++st) {
              const typename E::frag bp = E::from_acc(pv, st);
              typename E::frag bu{};
              if constexpr (VB) {
                bu = E::from_acc(uv, st);
                usum += frag_sum<E>(bu);
              }
#pragma unroll
              for (int db = 0; db < D / 32; ++db) {
                typename E::frag av;
                if constexpr (TR) av = E::ld_tr(vtile[buf] + tr_off + (32 * kh + 16 * st) * LDV + 32 * db, LDV);
                else av = E::ld_kacc(vtile[buf] + (32 * db + sigma32(l32)) * LDV + 32 * kh, st, h);
                acc_o[db] = E::mma(av, bp, acc_o[db]);
                if constexpr (VB) acc_u[db] = E::mma(av, bu, acc_u[db]);
              }
            }
          }
        }
        if ((wave & 1) == 0) tiles_out++;
      }
      wait_vmem();
      if (Jn >= 0) {
        if (NBUF == 1) __syncthreads();
        iok.template store_rows<LDK>(ktile[NBUF - 1 - buf], tid);
        if constexpr (TR) iov.template store_rows<LDV>(vtile[NBUF - 1 - buf], tid);
        else iov.template store_trans<LDV>(vtile[NBUF - 1 - buf], tid);
      }
      __syncthreads();
      buf = NBUF - 1 - buf;
      J = Jn;
    }
    if (a.tiles_per_pass && lane == 0 && (wave & 1) == 0 && tiles_out)
      atomicAdd(a.tiles_per_pass + MAX_PASSES + 1, tiles_out);
  }

  // ---------------- write O, the state and the final mask ---------------
  if constexpr (VB) {
    usum += __shfl_xor(usum, 32);
    const float rinv = usum > 0.f ? 1.f / usum : 0.f;
    if (tile_row) {
      float* vrow = a.state + ((size_t)bh * a.N + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float* dst = vrow + 32 * db + 16 * half + 8 * h;
          const floatx16& u = acc_u[db];
          *reinterpret_cast<float4*>(dst) = make_float4(u[8 * half + 0] * rinv, u[8 * half + 1] * rinv,
                                                        u[8 * half + 2] * rinv, u[8 * half + 3] * rinv);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(u[8 * half + 4] * rinv, u[8 * half + 5] * rinv,
                                                            u[8 * half + 6] * rinv, u[8 * half + 7] * rinv);
        }
    }
  }
  if (tile_row) {
    S* orow = reinterpret_cast<S*>(a.o) + a.lq.head(bh, a.H) + (size_t)qrow * a.lq.sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        S* dst = orow + 32 * db + 16 * half + 8 * h;
        if constexpr (sizeof(S) == 2) {
          uint32_t wv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            wv[e] = (uint32_t)E::from_f(acc_o[db][8 * half + 2 * e]) |
                    ((uint32_t)E::from_f(acc_o[db][8 * half + 2 * e + 1]) << 16);
          *reinterpret_cast<uint4*>(dst) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(acc_o[db][8 * half + 0], acc_o[db][8 * half + 1],
                                                        acc_o[db][8 * half + 2], acc_o[db][8 * half + 3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(acc_o[db][8 * half + 4], acc_o[db][8 * half + 5],
                                                            acc_o[db][8 * half + 6], acc_o[db][8 * half + 7]);
        }
      }
  }
  __syncthreads();
  for (int i = tid; i < NBLKS * W; i += NTHR) {
    const int b = i / W, w = i % W;
    if (blk0 + b < a.nb) a.mask[((size_t)bh * a.nb + blk0 + b) * W + w] = mf[b][w];
  }
  // sub-tiles holding some p > 0: the bits both paths set (one 32-row wave
  // by 32 keys each), or, past 16-bit key indices, the products run
  if (a.halves_out) {
    uint32_t c = halves;
    if (a.N <= LIST_MAX_N) {
      c = 0;
      for (int i = lane; i < LIST_MAX_N / 1024; i += 64) c += __popc(sub_s[wave][i]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    }
    if (lane == 0 && c) atomicAdd(a.halves_out, c);
  }
  if (a.gathered && lane == 0 && halves) atomicAdd(a.gathered + 1, halves);
}

}  // namespace ea
