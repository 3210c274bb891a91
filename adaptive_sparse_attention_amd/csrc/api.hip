// C ABI of the alpha-entmax attention library (declared in include/entmax_attn.h).
//
// Every entry point checks its arguments before touching the device and
// enqueues work only on the caller's stream. The library allocates nothing.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/entmax_attn.h"
#include "ea_launch.hpp"

namespace {

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

int nblocks(int N) { return (N + EA_BLOCK - 1) / EA_BLOCK; }
int nwords(int N) { return (nblocks(N) + 31) / 32; }

bool aligned4(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// ptrs: tensors read or written a row at a time (16-byte aligned); rowp: the
// per-row tau / lse2 and the mask words (4-byte aligned)
ea_status check_common(const void* const* ptrs, int nptrs, const void* const* rowp, int nrowp, float alpha, int B,
                       int H, int N, int d, int dtype) {
  for (int i = 0; i < nptrs; ++i)
    if (!aligned16(ptrs[i])) return EA_ERR_INVALID_ARG;
  for (int i = 0; i < nrowp; ++i)
    if (!aligned4(rowp[i])) return EA_ERR_INVALID_ARG;
  if (!(alpha > 1.0f) || !isfinite(alpha)) return EA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return EA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return EA_ERR_UNSUPPORTED;
  if (dtype != EA_BF16 && dtype != EA_F32) return EA_ERR_UNSUPPORTED;
  if (N > EA_MAX_N) return EA_ERR_UNSUPPORTED;
  // workgroup count must fit the grid: at most one per 64-row block, and for
  // the row-max pass one per pair of query blocks and chunk of 32 key blocks
  const long long nb = nblocks(N);
  if ((long long)B * H * nb > 0x7fffffffLL) return EA_ERR_UNSUPPORTED;
  if ((long long)B * H * ((nb + 1) / 2) * ((nb + 31) / 32) > 0x7fffffffLL) return EA_ERR_UNSUPPORTED;
  return EA_OK;
}

// Strides of a [B, H, N, d] tensor stored contiguously.
ea_strides dense_strides(int H, int N, int d) {
  ea_strides st;
  st.batch = (int64_t)H * N * d;
  st.head = (int64_t)N * d;
  st.row = d;
  return st;
}

// Strides must keep every row 16-byte aligned and not be negative.
bool strides_ok(const ea_strides& st, int esize) {
  if (st.batch < 0 || st.head < 0 || st.row < 1 || st.row > 0x7fffffffLL) return false;
  return ((st.batch * esize) & 15) == 0 && ((st.head * esize) & 15) == 0 && ((st.row * esize) & 15) == 0;
}

// Whether a [B, Hx, N, d] view with these strides (d contiguous) gives every
// element its own address, so that outputs written with them cannot race:
// the dimensions of size > 1, in increasing stride, each step over the whole
// extent of the previous ones (the innermost over the d elements of a row).
bool layout_injective(const ea_strides& st, int B, int Hx, int N, int d) {
  struct Dim { long long stride, size; } dims[3] = {{st.row, N}, {st.head, Hx}, {st.batch, B}};
  // insertion sort by stride (three entries)
  for (int i = 1; i < 3; ++i)
    for (int j = i; j > 0 && dims[j].stride < dims[j - 1].stride; --j) {
      const Dim t = dims[j];
      dims[j] = dims[j - 1];
      dims[j - 1] = t;
    }
  long long extent = d;   // elements spanned by the dimensions placed so far
  for (const Dim& dm : dims) {
    if (dm.size <= 1) continue;
    if (dm.stride < extent) return false;
    extent = dm.stride * (dm.size - 1) + extent;
  }
  return true;
}

ea::Lay lay_of(const ea_strides& st) {
  ea::Lay l;
  l.sb = st.batch;
  l.sh = st.head;
  l.sn = (int)st.row;
  return l;
}

int esize_of(ea_dtype dtype) { return dtype == EA_BF16 ? 2 : 4; }

// Bytes of one row's record in the forward's state: d fp32 words, which hold
// vbar (d floats) for rows formed by tiles and, for rows formed by gathering,
// the 128-byte support list and the ceil(nb / 32) <= 32 mask words that
// follow it (gathered rows exist only for N <= 65536).
size_t state_row_bytes(int d) { return (size_t)d * sizeof(float); }

// With dry set, only the argument checks run (nothing is enqueued): callers
// that launch several problems check all of them first.
ea_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* tau, uint32_t* mask, void* state, size_t state_bytes,
                   float alpha, int causal, int B, int H, int Hkv, int N, int d, const ea_strides* sq,
                   const ea_strides* skv, ea_dtype dtype, ea_fwd_stats* stats, void* stream, unsigned phases,
                   bool dry = false);
ea_status bwd_impl(const void* q, const void* k, const void* v, const void* dout, const float* tau,
                   const uint32_t* mask, const void* state, size_t state_bytes, void* dq, void* dk, void* dv, float alpha, int causal,
                   int B, int H, int Hkv, int N, int d, const ea_strides* sq, const ea_strides* skv, ea_dtype dtype,
                   void* workspace, size_t workspace_bytes, void* stream, unsigned phases, bool dry = false);

}  // namespace

namespace {

// delta and the key-major mask: what every backward uses
size_t ws_base_bytes(int B, int H, int N) {
  const size_t bhn = (size_t)B * H * N;
  const size_t words = (size_t)B * H * ea_mask_words(N);
  return round256(bhn * sizeof(float)) + round256(words * sizeof(uint32_t));
}

// Workspace of the backward's gather path (rows the forward formed from their
// support lists), after the base part: offsets in bytes, 256-byte aligned.
// Sized with H for the key/value heads too (Hkv <= H). None past 16-bit keys.
struct GatherWs {
  size_t tmask, gblk, rown, ent_key, ent_ds, ent_p, ent_rank, kcnt, koff, kpart, bucket, part, bytes;
};
GatherWs ws_gather(int B, int H, int N, int d) {
  GatherWs g{};
  if (N > ea::LIST_MAX_N) return g;
  const size_t bhn = (size_t)B * H * N;
  const size_t slots = bhn * ea::LIST_CAP;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round256(bytes);
    return at;
  };
  g.tmask = take((size_t)B * H * ea_mask_words(N) * sizeof(uint32_t));
  g.gblk = take((size_t)B * H * ((N + 63) / 64) * sizeof(uint32_t));
  g.rown = take(bhn);
  g.ent_key = take(slots * sizeof(uint32_t));
  g.ent_ds = take(slots * sizeof(float));
  g.ent_p = take(slots * sizeof(float));
  g.ent_rank = take(slots * sizeof(uint32_t));
  g.kcnt = take(bhn * sizeof(uint32_t));
  g.koff = take((bhn + 1) * sizeof(uint32_t));
  g.kpart = take(((bhn + 1 + 2047) / 2048) * sizeof(uint32_t));
  g.bucket = take(slots * sizeof(uint32_t));
  g.part = take(bhn * 2 * (size_t)d * sizeof(float));
  g.bytes = o;
  return g;
}

}  // namespace

extern "C" {

size_t ea_mask_words(int N) {
  if (N < 1) return 0;
  return (size_t)nblocks(N) * (size_t)nwords(N);
}

size_t ea_fwd_state_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return (size_t)B * H * N * state_row_bytes(d);
}

size_t ea_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return ws_base_bytes(B, H, N) + ws_gather(B, H, N, d).bytes;
}

const char* ea_status_str(ea_status status) {
  switch (status) {
    case EA_OK: return "ok";
    case EA_ERR_INVALID_ARG: return "invalid argument";
    case EA_ERR_UNSUPPORTED: return "unsupported configuration";
    case EA_ERR_WORKSPACE: return "workspace missing or too small";
    case EA_ERR_LAUNCH: return "kernel launch failed";
    case EA_ERR_SCRATCH_LIMIT: return "problem needs more scratch than the library's static buffer holds";
  }
  return "unknown status";
}

ea_status entmax_attn_fwd(const void* q, const void* k, const void* v, void* o, float* tau, uint32_t* mask,
                          void* state, size_t state_bytes, float alpha, int causal, int B, int H, int N, int d, ea_dtype dtype,
                          ea_fwd_stats* stats, void* stream) {
  return entmax_attn_fwd_phases(q, k, v, o, tau, mask, state, state_bytes, alpha, causal, B, H, N, d, dtype, stats, stream,
                                EA_FWD_ALL);
}

ea_status entmax_attn_bwd(const void* q, const void* k, const void* v, const void* dout, const float* tau,
                          const uint32_t* mask, const void* state, size_t state_bytes, void* dq, void* dk, void* dv, float alpha,
                          int causal, int B, int H, int N, int d, ea_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return entmax_attn_bwd_phases(q, k, v, dout, tau, mask, state, state_bytes, dq, dk, dv, alpha, causal, B, H, N, d, dtype,
                                workspace, workspace_bytes, stream, EA_BWD_ALL);
}

ea_status entmax_attn_fwd_phases(const void* q, const void* k, const void* v, void* o, float* tau, uint32_t* mask,
                                 void* state, size_t state_bytes, float alpha, int causal, int B, int H, int N, int d, ea_dtype dtype,
                                 ea_fwd_stats* stats, void* stream, unsigned phases) {
  return entmax_attn_fwd_gqa(q, k, v, o, tau, mask, state, state_bytes, alpha, causal, B, H, H, N, d, dtype, stats, stream, phases);
}

ea_status entmax_attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* tau, uint32_t* mask,
                              void* state, size_t state_bytes, float alpha, int causal, int B, int H, int Hkv, int N, int d,
                              ea_dtype dtype, ea_fwd_stats* stats, void* stream, unsigned phases) {
  return fwd_impl(q, k, v, o, tau, mask, state, state_bytes, alpha, causal, B, H, Hkv, N, d, nullptr, nullptr, dtype, stats,
                  stream, phases);
}

ea_status entmax_attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* tau,
                                  uint32_t* mask, void* state, size_t state_bytes, float alpha, int causal, int B, int H, int Hkv, int N,
                                  int d, const ea_strides* q_strides, const ea_strides* kv_strides, ea_dtype dtype,
                                  ea_fwd_stats* stats, void* stream, unsigned phases) {
  if (q_strides == nullptr || kv_strides == nullptr) return EA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, o, tau, mask, state, state_bytes, alpha, causal, B, H, Hkv, N, d, q_strides, kv_strides, dtype, stats,
                  stream, phases);
}

}  // extern "C"

namespace {

ea_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* tau, uint32_t* mask, void* state, size_t state_bytes,
                   float alpha, int causal, int B, int H, int Hkv, int N, int d, const ea_strides* sq,
                   const ea_strides* skv, ea_dtype dtype, ea_fwd_stats* stats, void* stream, unsigned phases,
                   bool dry) {
  if (Hkv < 1 || H % Hkv != 0) return EA_ERR_INVALID_ARG;
  const unsigned lb = (phases >> 8) & 15u;   // histogram bins per unit: 2^lb, 0 = 256
  const unsigned pcap = (phases >> 12) & 15u;   // streamed passes per row, 0 = the mode's cap
  phases &= ~(255u << 8);
  if ((phases & EA_FWD_ALL) == 0 || (phases & ~(EA_FWD_ALL | EA_FWD_NO_HIST | EA_FWD_PLAIN_SOLVER)))
    return EA_ERR_INVALID_ARG;
  if (lb != 0 && (lb < 5 || lb > 9)) return EA_ERR_INVALID_ARG;
  if (pcap > EA_MAX_PASSES) return EA_ERR_INVALID_ARG;
  const int bins = lb ? (1 << lb) : EA_HIST_BINS;
  const void* ptrs[] = {q, k, v, o};
  const void* rowp[] = {tau, mask};
  ea_status s = check_common(ptrs, 4, rowp, 2, alpha, B, H, N, d, (int)dtype);
  if (s != EA_OK) return s;
  if (state && (!aligned16(state) || state_bytes < ea_fwd_state_bytes(B, H, N, d))) return EA_ERR_INVALID_ARG;
  if ((sq && !strides_ok(*sq, esize_of(dtype))) || (skv && !strides_ok(*skv, esize_of(dtype))))
    return EA_ERR_INVALID_ARG;
  if (sq && !layout_injective(*sq, B, H, N, d)) return EA_ERR_INVALID_ARG;   // o is written with q's strides
  // other histogram sizes: bf16 inputs with 16-bit counters (N <= 65536)
  if (bins != EA_HIST_BINS && (dtype != EA_BF16 || N > 65536)) return EA_ERR_UNSUPPORTED;
  if (stats) {
    // tau_h needs float alignment, the counters 4-byte alignment
    if (stats->tau_h && (reinterpret_cast<uintptr_t>(stats->tau_h) & 3u)) return EA_ERR_INVALID_ARG;
    if (stats->tiles_per_pass && (reinterpret_cast<uintptr_t>(stats->tiles_per_pass) & 3u)) return EA_ERR_INVALID_ARG;
    if (stats->unconverged && (reinterpret_cast<uintptr_t>(stats->unconverged) & 3u)) return EA_ERR_INVALID_ARG;
    if (stats->halves_out && (reinterpret_cast<uintptr_t>(stats->halves_out) & 3u)) return EA_ERR_INVALID_ARG;
    if (stats->gathered && (reinterpret_cast<uintptr_t>(stats->gathered) & 3u)) return EA_ERR_INVALID_ARG;
  }
  if (dry) return EA_OK;
  ea::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.tau = tau;
  a.mask = mask;
  a.state = static_cast<float*>(state);
  a.tau_h_out = stats ? stats->tau_h : nullptr;
  a.passes_out = stats ? stats->passes : nullptr;
  a.iters_out = stats ? stats->iters : nullptr;
  a.tiles_per_pass = stats ? stats->tiles_per_pass : nullptr;
  a.unconverged = stats ? stats->unconverged : nullptr;
  a.halves_out = stats ? stats->halves_out : nullptr;
  a.gathered = stats ? stats->gathered : nullptr;
  a.B = B;
  a.H = H;
  a.N = N;
  a.nb = nblocks(N);
  a.W = nwords(N);
  a.causal = causal ? 1 : 0;
  a.alpha = alpha;
  const double kap = 1.0 / ((double)alpha - 1.0);
  a.kappa = (float)kap;
  a.pow_mode = ea::host_pow_mode(a.kappa);
  a.G = H / Hkv;
  a.nohist = (phases & EA_FWD_NO_HIST) ? 1 : 0;
  a.plain = (phases & EA_FWD_PLAIN_SOLVER) ? 1 : 0;
  a.pass_cap = (int)pcap;
  a.zscale = (float)(((double)alpha - 1.0) / sqrt((double)d));
  a.bins = bins;
  a.zscaleB = a.zscale * (float)bins;
  a.delta_h = 1.0f / (float)bins;
  a.lq = lay_of(sq ? *sq : dense_strides(H, N, d));
  a.lkv = lay_of(skv ? *skv : dense_strides(Hkv, N, d));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = (dtype == EA_BF16) ? ea::launch_fwd_bf16(a, d, phases, st) : ea::launch_fwd_f32(a, d, phases, st);
  return e == hipSuccess ? EA_OK : EA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

ea_status entmax_attn_bwd_phases(const void* q, const void* k, const void* v, const void* dout, const float* tau,
                                 const uint32_t* mask, const void* state, size_t state_bytes, void* dq, void* dk, void* dv, float alpha, int causal, int B,
                                 int H, int N, int d, ea_dtype dtype, void* workspace, size_t workspace_bytes,
                                 void* stream, unsigned phases) {
  return entmax_attn_bwd_gqa(q, k, v, dout, tau, mask, state, state_bytes, dq, dk, dv, alpha, causal, B, H, H, N, d, dtype,
                             workspace, workspace_bytes, stream, phases);
}

ea_status entmax_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* dout, const float* tau,
                              const uint32_t* mask, const void* state, size_t state_bytes, void* dq, void* dk, void* dv, float alpha,
                              int causal, int B, int H, int Hkv, int N, int d, ea_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream, unsigned phases) {
  return bwd_impl(q, k, v, dout, tau, mask, state, state_bytes, dq, dk, dv, alpha, causal, B, H, Hkv, N, d, nullptr, nullptr,
                  dtype, workspace, workspace_bytes, stream, phases);
}

ea_status entmax_attn_bwd_strided(const void* q, const void* k, const void* v, const void* dout, const float* tau,
                                  const uint32_t* mask, const void* state, size_t state_bytes, void* dq, void* dk, void* dv, float alpha,
                                  int causal, int B, int H, int Hkv, int N, int d, const ea_strides* q_strides,
                                  const ea_strides* kv_strides, ea_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream, unsigned phases) {
  if (q_strides == nullptr || kv_strides == nullptr) return EA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, dout, tau, mask, state, state_bytes, dq, dk, dv, alpha, causal, B, H, Hkv, N, d, q_strides,
                  kv_strides, dtype, workspace, workspace_bytes, stream, phases);
}

}  // extern "C"

namespace {

ea_status bwd_impl(const void* q, const void* k, const void* v, const void* dout, const float* tau,
                   const uint32_t* mask, const void* state, size_t state_bytes, void* dq, void* dk, void* dv, float alpha, int causal,
                   int B, int H, int Hkv, int N, int d, const ea_strides* sq, const ea_strides* skv, ea_dtype dtype,
                   void* workspace, size_t workspace_bytes, void* stream, unsigned phases, bool dry) {
  if (Hkv < 1 || H % Hkv != 0) return EA_ERR_INVALID_ARG;
  if (phases == 0 || (phases & ~EA_BWD_ALL)) return EA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, dout, dq, dk, dv};
  const void* rowp[] = {tau, mask};
  ea_status s = check_common(ptrs, 7, rowp, 2, alpha, B, H, N, d, (int)dtype);
  if (s != EA_OK) return s;
  if (state && (!aligned16(state) || state_bytes < ea_fwd_state_bytes(B, H, N, d))) return EA_ERR_INVALID_ARG;
  if ((sq && !strides_ok(*sq, esize_of(dtype))) || (skv && !strides_ok(*skv, esize_of(dtype))))
    return EA_ERR_INVALID_ARG;
  // dq is written with q's strides, dk and dv with k's
  if ((sq && !layout_injective(*sq, B, H, N, d)) || (skv && !layout_injective(*skv, B, Hkv, N, d)))
    return EA_ERR_INVALID_ARG;
  const size_t need = ea_bwd_workspace_bytes(B, H, N, d);
  if (workspace == nullptr || workspace_bytes < need) return EA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return EA_ERR_INVALID_ARG;
  if (dry) return EA_OK;
  ea::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.tau = tau;
  a.mask = mask;
  a.state = static_cast<const float*>(state);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = reinterpret_cast<float*>(workspace);
  a.colmask = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(workspace) +
                                          round256((size_t)B * H * N * sizeof(float)));
  {
    // the gather path needs the forward's lists (in the state) and 32-bit key ids
    const GatherWs g = ws_gather(B, H, N, d);
    a.gather = (state != nullptr && g.bytes != 0 && (size_t)B * H * N * ea::LIST_CAP < 0xFFFFFFFFull) ? 1 : 0;
    char* w = reinterpret_cast<char*>(workspace) + ws_base_bytes(B, H, N);
    a.tmask = reinterpret_cast<uint32_t*>(w + g.tmask);
    a.gblk = reinterpret_cast<uint32_t*>(w + g.gblk);
    a.rown = reinterpret_cast<uint8_t*>(w + g.rown);
    a.ent_key = reinterpret_cast<uint32_t*>(w + g.ent_key);
    a.ent_ds = reinterpret_cast<float*>(w + g.ent_ds);
    a.ent_p = reinterpret_cast<float*>(w + g.ent_p);
    a.kcnt = reinterpret_cast<uint32_t*>(w + g.kcnt);
    a.koff = reinterpret_cast<uint32_t*>(w + g.koff);
    a.ent_rank = reinterpret_cast<uint32_t*>(w + g.ent_rank);
    a.kpart = reinterpret_cast<uint32_t*>(w + g.kpart);
    a.bucket = reinterpret_cast<uint32_t*>(w + g.bucket);
    a.part = reinterpret_cast<float*>(w + g.part);
  }
  a.B = B;
  a.H = H;
  a.N = N;
  a.nb = nblocks(N);
  a.W = nwords(N);
  a.causal = causal ? 1 : 0;
  a.kappa = (float)(1.0 / ((double)alpha - 1.0));
  a.zscale = (float)(((double)alpha - 1.0) / sqrt((double)d));
  a.rscale = (float)(1.0 / sqrt((double)d));
  a.G = H / Hkv;
  a.lq = lay_of(sq ? *sq : dense_strides(H, N, d));
  a.lkv = lay_of(skv ? *skv : dense_strides(Hkv, N, d));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = (dtype == EA_BF16) ? ea::launch_bwd_bf16(a, d, phases, st) : ea::launch_bwd_f32(a, d, phases, st);
  return e == hipSuccess ? EA_OK : EA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t ea_softmax_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return ws_base_bytes(B, H, N) + round256((size_t)B * H * ea_mask_words(N) * sizeof(uint32_t));
}

ea_status softmax_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse2, float* o32, int causal,
                           int B, int H, int N, int d, ea_dtype dtype, void* stream) {
  const void* ptrs[] = {q, k, v, o};
  const void* rowp[] = {lse2};
  ea_status s = check_common(ptrs, 4, rowp, 1, 2.0f, B, H, N, d, (int)dtype);
  if (s != EA_OK) return s;
  if (o32 && !aligned16(o32)) return EA_ERR_INVALID_ARG;
  ea::SmArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse2 = lse2;
  a.o32 = o32;
  a.B = B;
  a.H = H;
  a.N = N;
  a.nb = nblocks(N);
  a.causal = causal ? 1 : 0;
  a.G = 1;
  a.lq = lay_of(dense_strides(H, N, d));
  a.lkv = a.lq;
  a.c = (float)(1.4426950408889634 / sqrt((double)d));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = (dtype == EA_BF16) ? ea::launch_sm_fwd_bf16(a, d, st) : ea::launch_sm_fwd_f32(a, d, st);
  return e == hipSuccess ? EA_OK : EA_ERR_LAUNCH;
}

ea_status softmax_attn_bwd(const void* q, const void* k, const void* v, const void* dout, const float* lse2,
                           const float* o32, void* dq, void* dk, void* dv, int causal, int B, int H, int N, int d,
                           ea_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const void* ptrs[] = {q, k, v, dout, dq, dk, dv};
  const void* rowp[] = {lse2};
  ea_status s = check_common(ptrs, 7, rowp, 1, 2.0f, B, H, N, d, (int)dtype);
  if (s != EA_OK) return s;
  if (o32 && !aligned16(o32)) return EA_ERR_INVALID_ARG;
  const size_t need = ea_softmax_bwd_workspace_bytes(B, H, N, d);
  if (workspace == nullptr || workspace_bytes < need) return EA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return EA_ERR_INVALID_ARG;
  char* ws = reinterpret_cast<char*>(workspace);
  const size_t off_col = round256((size_t)B * H * N * sizeof(float));
  const size_t off_row = ws_base_bytes(B, H, N);
  ea::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.tau = lse2;
  a.mask = reinterpret_cast<const uint32_t*>(ws + off_row);
  a.state = o32;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = reinterpret_cast<float*>(ws);
  a.colmask = reinterpret_cast<uint32_t*>(ws + off_col);
  a.B = B;
  a.H = H;
  a.N = N;
  a.nb = nblocks(N);
  a.W = nwords(N);
  a.causal = causal ? 1 : 0;
  a.kappa = 1.0f;
  a.G = 1;
  a.lq = lay_of(dense_strides(H, N, d));
  a.lkv = a.lq;
  a.zscale = (float)(1.4426950408889634 / sqrt((double)d));
  a.rscale = (float)(1.0 / sqrt((double)d));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t* rowmask = reinterpret_cast<uint32_t*>(ws + off_row);
  hipError_t e = (dtype == EA_BF16) ? ea::launch_sm_bwd_bf16(a, rowmask, d, st) : ea::launch_sm_bwd_f32(a, rowmask, d, st);
  return e == hipSuccess ? EA_OK : EA_ERR_LAUNCH;
}


// ---------------------------------------------------------------------------
// Packed variable-length sequences: one call per sequence on the caller's
// stream, each a B = 1 problem on token-major slices of the packed tensors.
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// cu_seqlens: nseq + 1 non-decreasing offsets from 0; every length at most
// EA_MAX_N. Returns the longest length, or -1 when invalid.
int varlen_max(const int* cu, int nseq) {
  if (cu == nullptr || nseq < 1 || cu[0] != 0) return -1;
  int mx = 0;
  for (int b = 0; b < nseq; ++b) {
    const long long n = (long long)cu[b + 1] - cu[b];
    if (n < 0 || n > EA_MAX_N) return -1;
    if (n > mx) mx = (int)n;
  }
  return mx;
}

}  // namespace

extern "C" {

size_t ea_varlen_mask_words(const int* cu_seqlens, int nseq, int H) {
  if (varlen_max(cu_seqlens, nseq) < 0 || H < 1) return 0;
  size_t w = 0;
  for (int b = 0; b < nseq; ++b) w += ea_mask_words(cu_seqlens[b + 1] - cu_seqlens[b]);
  return w * (size_t)H;
}

size_t ea_varlen_fwd_state_bytes(const int* cu_seqlens, int nseq, int H, int d) {
  if (varlen_max(cu_seqlens, nseq) < 0 || H < 1 || (d != 64 && d != 128)) return 0;
  return (size_t)cu_seqlens[nseq] * H * state_row_bytes(d);
}

size_t ea_varlen_bwd_workspace_bytes(const int* cu_seqlens, int nseq, int H, int d) {
  const int mx = varlen_max(cu_seqlens, nseq);
  if (mx < 1) return 0;
  // not monotone in the length (the gather path's buffers stop above
  // 65536), so the largest over the sequences
  size_t need = 0;
  for (int b = 0; b < nseq; ++b) {
    const int n = cu_seqlens[b + 1] - cu_seqlens[b];
    if (n > 0) need = need > ea_bwd_workspace_bytes(1, H, n, d) ? need : ea_bwd_workspace_bytes(1, H, n, d);
  }
  return need;
}

ea_status entmax_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* tau, uint32_t* mask,
                                 void* state, size_t state_bytes, float alpha, int causal, const int* cu_seqlens, int nseq, int H,
                                 int Hkv, int d, ea_dtype dtype, ea_fwd_stats* stats, void* stream,
                                 unsigned phases) {
  const int mx = varlen_max(cu_seqlens, nseq);
  if (mx < 0 || H < 1 || Hkv < 1 || H % Hkv != 0) return EA_ERR_INVALID_ARG;
  if (mx == 0) return EA_OK;
  if (state && state_bytes < ea_varlen_fwd_state_bytes(cu_seqlens, nseq, H, d)) return EA_ERR_INVALID_ARG;
  const int es = esize_of(dtype);
  ea_strides sq, skv;
  sq.batch = 0;
  sq.head = d;
  sq.row = (int64_t)H * d;
  skv.batch = 0;
  skv.head = d;
  skv.row = (int64_t)Hkv * d;
  // every sequence is checked (all of fwd_impl's checks, dry) before any is
  // launched, so a rejected call enqueues nothing
  for (int pass = 0; pass < 2; ++pass) {
    size_t moff = 0;
    for (int b = 0; b < nseq; ++b) {
      const int n = cu_seqlens[b + 1] - cu_seqlens[b];
      if (n == 0) continue;
      const size_t t0 = (size_t)cu_seqlens[b];
      ea_fwd_stats sb;
      ea_fwd_stats* sp = nullptr;
      if (stats) {
        sb = *stats;
        if (sb.tau_h) sb.tau_h += (size_t)H * t0;
        if (sb.passes) sb.passes += (size_t)H * t0;
        if (sb.iters) sb.iters += (size_t)H * t0;
        sp = &sb;
      }
      const ea_status st = fwd_impl(
          static_cast<const char*>(q) + t0 * H * d * es, static_cast<const char*>(k) + t0 * Hkv * d * es,
          static_cast<const char*>(v) + t0 * Hkv * d * es, static_cast<char*>(o) + t0 * H * d * es,
          tau + (size_t)H * t0, mask + moff, state ? static_cast<char*>(state) + state_row_bytes(d) * H * t0 : nullptr,
          state ? ea_fwd_state_bytes(1, H, n, d) : 0, alpha, causal, 1, H, Hkv,
          n, d, &sq, &skv, dtype, sp, stream, phases, pass == 0);
      if (st != EA_OK) return st;
      moff += (size_t)H * ea_mask_words(n);
    }
  }
  return EA_OK;
}

ea_status entmax_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* dout, const float* tau,
                                 const uint32_t* mask, const void* state, size_t state_bytes, void* dq, void* dk, void* dv, float alpha,
                                 int causal, const int* cu_seqlens, int nseq, int H, int Hkv, int d, ea_dtype dtype,
                                 void* workspace, size_t workspace_bytes, void* stream, unsigned phases) {
  const int mx = varlen_max(cu_seqlens, nseq);
  if (mx < 0 || H < 1 || Hkv < 1 || H % Hkv != 0) return EA_ERR_INVALID_ARG;
  if (mx == 0) return EA_OK;
  const int es = esize_of(dtype);
  ea_strides sq, skv;
  sq.batch = 0;
  sq.head = d;
  sq.row = (int64_t)H * d;
  skv.batch = 0;
  skv.head = d;
  skv.row = (int64_t)Hkv * d;
  if (state && state_bytes < ea_varlen_fwd_state_bytes(cu_seqlens, nseq, H, d)) return EA_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < ea_varlen_bwd_workspace_bytes(cu_seqlens, nseq, H, d))
    return EA_ERR_WORKSPACE;
  // every sequence is checked (dry) before any is launched; the sequences
  // then run one after another on the stream and share the workspace
  for (int pass = 0; pass < 2; ++pass) {
    size_t moff = 0;
    for (int b = 0; b < nseq; ++b) {
      const int n = cu_seqlens[b + 1] - cu_seqlens[b];
      if (n == 0) continue;
      const size_t t0 = (size_t)cu_seqlens[b];
      const ea_status st = bwd_impl(
          static_cast<const char*>(q) + t0 * H * d * es, static_cast<const char*>(k) + t0 * Hkv * d * es,
          static_cast<const char*>(v) + t0 * Hkv * d * es, static_cast<const char*>(dout) + t0 * H * d * es,
          tau + (size_t)H * t0, mask + moff,
          state ? static_cast<const char*>(state) + state_row_bytes(d) * H * t0 : nullptr,
          state ? ea_fwd_state_bytes(1, H, n, d) : 0,
          static_cast<char*>(dq) + t0 * H * d * es, static_cast<char*>(dk) + t0 * Hkv * d * es,
          static_cast<char*>(dv) + t0 * Hkv * d * es, alpha, causal, 1, H, Hkv, n, d, &sq, &skv, dtype, workspace,
          workspace_bytes, stream, phases, pass == 0);
      if (st != EA_OK) return st;
      moff += (size_t)H * ea_mask_words(n);
    }
  }
  return EA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward without allocation: the workspace is the library's own static
// device array. In host code `scratch` names a host-side stand-in, not a
// device address: its address on each device comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that pointer is
// passed on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[EA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_DEVICES = 64;
std::once_flag scratch_once[SCRATCH_DEVICES];
void* scratch_dev[SCRATCH_DEVICES];
hipError_t scratch_err[SCRATCH_DEVICES];

// The scratch array's address on the current device.
ea_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_DEVICES) return EA_ERR_LAUNCH;
  std::call_once(scratch_once[dev], [dev]() {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_dev[dev] = p;
  });
  if (scratch_err[dev] != hipSuccess || scratch_dev[dev] == nullptr) return EA_ERR_LAUNCH;
  *out = scratch_dev[dev];
  return EA_OK;
}

}  // namespace

extern "C" {

size_t ea_noalloc_scratch_bytes(void) { return EA_NOALLOC_SCRATCH_BYTES; }

ea_status entmax_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* dout, const float* tau,
                                  const uint32_t* mask, const void* state, size_t state_bytes, void* dq, void* dk,
                                  void* dv, float alpha, int causal, int B, int H, int N, int d, ea_dtype dtype,
                                  void* stream) {
  // the ordinary checks first (with the scratch size standing in for a
  // workspace), so bad arguments report as they do elsewhere
  const ea_status chk = bwd_impl(q, k, v, dout, tau, mask, state, state_bytes, dq, dk, dv, alpha, causal, B, H, H,
                                 N, d, nullptr, nullptr, dtype, reinterpret_cast<void*>(256),
                                 EA_NOALLOC_SCRATCH_BYTES, stream, EA_BWD_ALL, true);
  if (chk == EA_ERR_WORKSPACE) return EA_ERR_SCRATCH_LIMIT;
  if (chk != EA_OK) return chk;
  void* ws = nullptr;
  const ea_status s = scratch_of_current_device(&ws);
  if (s != EA_OK) return s;
  return bwd_impl(q, k, v, dout, tau, mask, state, state_bytes, dq, dk, dv, alpha, causal, B, H, H, N, d, nullptr,
                  nullptr, dtype, ws, EA_NOALLOC_SCRATCH_BYTES, stream, EA_BWD_ALL, false);
}

}  // extern "C"
