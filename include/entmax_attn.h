/*
 * entmax_attn.h -- C ABI of the alpha-entmax attention library for AMD MI355X
 * (gfx950). Link with libentmax_attn.so.
 *
 * What it computes. For every batch b, head h and query row i:
 *   s_ij = q_i . k_j / sqrt(d)      over the visible keys j (all j, or j <= i
 *                                   when causal),
 *   z_ij = (alpha - 1) s_ij,
 *   p_ij = [z_ij - tau_i]_+ ^ (1 / (alpha - 1)),  tau_i such that sum_j p_ij = 1,
 *   o_i  = sum_j p_ij v_j.
 * This is alpha-entmax attention: a sparse replacement of softmax whose
 * normaliser tau has no closed form and is found by root search (AdaSplash-2
 * summary, gist.science German page, section 1 "Problemstellung").
 *
 * How. tau starts from a lower bound tau_h read off a per-row histogram of the
 * scores with 256 left-edge bins held in on-chip memory while key blocks
 * stream through (same page, section 2 "Kernidee", steps 1-3), and is then
 * refined by a safeguarded hybrid solver -- Halley for alpha <= 1.5, Newton
 * for 1.5 < alpha <= 2, secant for alpha > 2, bisection when a step leaves
 * the bracket -- in one or two passes (gist.science Hindi page, section 2,
 * hybrid solver strategy). Key blocks with a non-zero weight are recorded in
 * a bit-packed block mask, 32 blocks per 32-bit word, and the output product
 * and the backward visit only those blocks, found with find-first-set and
 * popcount (German page, section 2 "Bit-Packed Block Mask" and
 * "GPU-Optimierung").
 *
 * Conventions shared by every entry point:
 *  - Tensors are dense row-major [B, H, N, d] in device memory, element type
 *    given by `dtype` (bf16 or fp32; inputs and outputs share it).
 *  - tau is fp32 [B, H, N] in z units (the units of (alpha-1) * s).
 *  - Block size is 64 for queries and keys; nb = ceil(N / 64) blocks and
 *    W = ceil(nb / 32) mask words per query block. The block mask is uint32
 *    [B, H, nb, W]: bit t of word w of query block I is set iff key block
 *    32 w + t holds a key j with p_ij > 0 for some row i of block I. Bits for
 *    key blocks >= nb, and for J > I when causal, are 0.
 *  - Every pointer is caller-owned device memory, 16-byte aligned (tau, lse2
 *    and the mask: 4-byte aligned). The library never allocates or frees
 *    device memory and keeps no pointer after return.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream). Buffers must stay alive until the stream has finished
 *    the work.
 *  - All argument checks run before any launch; on a failed check nothing is
 *    enqueued. Device faults surface on the caller's next synchronisation.
 *  - NaN or Inf inputs give undefined results.
 */
#ifndef ENTMAX_ATTN_H
#define ENTMAX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EA_OK = 0,
  EA_ERR_INVALID_ARG = 1,  /* alpha <= 1 or not finite, B/H/N < 1, NULL or unaligned pointer */
  EA_ERR_UNSUPPORTED = 2,  /* d not in {64, 128}, unknown dtype, N above EA_MAX_N */
  EA_ERR_WORKSPACE = 3,    /* backward workspace missing or smaller than ea_bwd_workspace_bytes */
  EA_ERR_LAUNCH = 4,       /* a kernel launch or the HIP runtime reported an error */
  EA_ERR_SCRATCH_LIMIT = 5 /* entmax_attn_bwd_noalloc: the problem's workspace exceeds
                              EA_NOALLOC_SCRATCH_BYTES */
} ea_status;

typedef enum {
  EA_BF16 = 0,  /* bfloat16 storage, fp32 accumulation */
  EA_F32 = 1    /* fp32 storage and arithmetic */
} ea_dtype;

#define EA_BLOCK 64           /* query / key block size                        */
#define EA_HIST_BINS 256      /* histogram bins per unit of z                  */
#define EA_MAX_PASSES 8       /* cap on refinement passes per row              */
#define EA_MAX_N (1 << 18)    /* longest supported sequence (262144)           */

/* Optional forward diagnostics. Any field may be NULL; the struct pointer
 * itself may be NULL. Buffers are device memory owned by the caller. */
typedef struct {
  float* tau_h;               /* [B,H,N] fp32: histogram lower bound of tau (z units) */
  uint8_t* passes;            /* [B,H,N]: refinement passes the row's solve used       */
  uint32_t* tiles_per_pass;   /* [EA_MAX_PASSES + 2], accumulated with atomics: entry 0
                                 counts 64x64 tiles of the histogram pass, entry k
                                 (1..EA_MAX_PASSES) those of refinement pass k, entry
                                 EA_MAX_PASSES + 1 those of the output pass. The caller
                                 zeroes it. */
  uint32_t* unconverged;      /* [1]: rows that reached EA_MAX_PASSES without meeting
                                 the stop rule (accumulated; caller zeroes it)        */
  uint32_t* halves_out;       /* [1]: 32-row x 32-key sub-tiles holding some p > 0, the
                                 ones whose products the output pass and the backward
                                 run (accumulated; caller zeroes it)                  */
  uint32_t* gathered;         /* [2]: query rows the output pass formed by gathering the
                                 rows of V of their support (no tile products), and
                                 the 32x32 sub-tiles whose products it ran for the
                                 other rows (accumulated; caller zeroes it)           */
  uint8_t* iters;             /* [B,H,N]: safeguarded solver steps the row's solve took
                                 (Halley, Newton, secant or bisection), whether its f
                                 came from a streamed pass, from sums shifted to the
                                 new point, or from its kept scores (capped at 255)  */
} ea_fwd_stats;

/* Mask words per (b, h): ceil(N/64) * ceil(ceil(N/64)/32). 0 when N < 1. */
size_t ea_mask_words(int N);

/* Bytes of the forward's state for the backward (see entmax_attn_fwd):
 * B * H * N records of 4 d bytes. 0 on invalid sizes. */
size_t ea_fwd_state_bytes(int B, int H, int N, int d);

/* Bytes of device workspace entmax_attn_bwd needs: per-row delta (fp32), the
 * key-major copy of the block mask and, for N <= 65536, the buffers of the
 * rows formed by gathering; each part 256-byte aligned. 0 on invalid sizes. */
size_t ea_bwd_workspace_bytes(int B, int H, int N, int d);

/* Static string naming a status code. */
const char* ea_status_str(ea_status status);

/* Forward pass.
 *  q, k, v : [B,H,N,d] inputs.
 *  o       : [B,H,N,d] output.
 *  tau     : [B,H,N] fp32 output, final threshold per row (z units).
 *  mask    : [B,H,nb,W] uint32 output, block mask at the final tau.
 *  state, state_bytes : optional output (NULL to skip; state_bytes is then
 *            ignored), device memory of at least ea_fwd_state_bytes(B,H,N,d)
 *            bytes, 16-byte aligned (EA_ERR_INVALID_ARG otherwise): the
 *            forward's state for the backward, which training callers keep
 *            and pass to entmax_attn_bwd; inference callers pass NULL. Its
 *            contents are private to the library and valid only together
 *            with this call's tau and mask. Each row writes only what its
 *            path needs: rows formed from tiles of the mask the weights
 *            of the entmax Jacobian averaged over V, rows formed by
 *            gathering the rows of V of their support (N <= 65536) that
 *            support list, with which the backward gathers the row too.
 *  alpha   : entmax parameter, alpha > 1.
 *  causal  : nonzero for causal attention (key j visible to row i iff j <= i).
 *  stats   : optional diagnostics (see ea_fwd_stats), may be NULL.
 *  stream  : hipStream_t to enqueue on.
 * Returns EA_OK once the kernels are enqueued. */
ea_status entmax_attn_fwd(const void* q, const void* k, const void* v,
                          void* o, float* tau, uint32_t* mask, void* state, size_t state_bytes,
                          float alpha, int causal, int B, int H, int N, int d,
                          ea_dtype dtype, ea_fwd_stats* stats, void* stream);

/* Backward pass: gradients of sum(o * dout) with respect to q, k and v.
 *  q, k, v, dout : [B,H,N,d] inputs (dout = dL/do).
 *  tau, mask     : the forward's outputs for the same q, k, v, alpha, causal.
 *  state, state_bytes : the forward's state from the same call, or NULL
 *                  (each row's delta is then formed by a sweep over the mask
 *                  and every row takes the tile path; both give the same
 *                  gradients up to rounding). With it, delta = dout . vbar
 *                  for rows formed from tiles, and the rows the forward
 *                  gathered are gathered: dP, delta, dS and dq over their
 *                  support keys, and dk, dv from those entries grouped by
 *                  key (sums independent of the order the entries are
 *                  grouped in); the tile kernels visit only the other rows'
 *                  blocks. A state smaller than ea_fwd_state_bytes or not
 *                  16-byte aligned returns EA_ERR_INVALID_ARG.
 *  dq, dk, dv    : [B,H,N,d] outputs (overwritten, not accumulated).
 *  workspace     : device scratch of at least ea_bwd_workspace_bytes(B,H,N,d)
 *                  bytes, 256-byte aligned; contents on entry are ignored.
 * The gradient of a score is u_j (dP_j - delta) with x_j = z_j - tau,
 * u_j = x_j^(1/(alpha-1) - 1) on the support, dP = dout . v_j and
 * delta = sum_j u_j dP_j / sum_j u_j; only key blocks set in the mask are
 * visited (German page, section 4 "Ergebnisse": gradients only for non-zero
 * blocks). For alpha > 2 the gradient is unbounded as a score approaches tau
 * from above. */
ea_status entmax_attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                          const float* tau, const uint32_t* mask, const void* state, size_t state_bytes,
                          void* dq, void* dk, void* dv,
                          float alpha, int causal, int B, int H, int N, int d,
                          ea_dtype dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Phase-selecting variants. `phases` is a bitmask of the kernels to enqueue;
 * the plain entry points above run all of them. Running a phase alone is
 * meant for profiling and for callers that schedule phases themselves; each
 * phase reads what the earlier ones wrote:
 *   EA_FWD_MAX    maxima of the scores: with the histogram pass to follow,
 *                 those of four classes of each row's keys (its largest
 *                 scores in each half of every 64-key block, split once more
 *                 by key mod 16 below or above 8), as scratch in the row of
 *                 `o`; without it the row max, in `tau` (both as
 *                 order-preserving integer encodings of the floats);
 *   EA_FWD_HIST   histogram pass: reads them, takes the row max and, from
 *                 the four, a lower bound of tau that raises the window's
 *                 lower edge above max z - 1 where it can; writes the lower
 *                 bound tau_h into `tau`, the candidate block mask (the key
 *                 blocks holding a score in the window, for the rows the
 *                 refinement will stream: those without a complete list
 *                 where the row's group of rows was finished from short
 *                 per-row score lists or N <= 16384, else all rows of the
 *                 block) into `mask`, and, as scratch in the row of `o`, the
 *                 row's scores above tau_h - 2^-12 with their key indices
 *                 where it found them all and they are at most 20
 *                 (N <= 65536). With the default 256 bins and N <= 65536,
 *                 rows whose window holds few scores get the same tau_h from
 *                 those scores directly, and only the other rows are binned
 *                 into histograms (gist.science German page, section 2
 *                 "Kernidee", steps 1-2);
 *   EA_FWD_REFINE refinement passes: reads them, writes the final tau into
 *                 `tau`; rows with such scores are solved on them without a
 *                 pass and marked, with their support, in their row of `o`;
 *                 `mask` receives the block mask at tau_h of the other rows;
 *   EA_FWD_OUT    output: reads tau, that mask and the marks, writes o,
 *                 the state (if given) and the final mask. Marked rows are formed
 *                 from the rows of v their support names, the others from
 *                 the tiles of that mask.
 *   EA_BWD_MASK  key-major copy of `mask` into the workspace;
 *   EA_BWD_ROWS  delta (workspace) and dq;
 *   EA_BWD_COLS  dk and dv (reads delta and the key-major mask).
 * Added to the forward's bits, EA_FWD_NO_HIST selects the solver mode
 * without the histogram: EA_FWD_HIST is then skipped, and the refinement
 * starts from the bracket [max z - 1, max z - n^(1-alpha)] of each row (n
 * visible keys) over all visible key blocks, so the passes it needs can be
 * set against those of the histogram start (gist.science German page,
 * section 1 "Problemstellung": without a good start the root search takes
 * many passes). stats->tau_h then receives max z - 1; the pass cap is 40,
 * and stats->tiles_per_pass[EA_MAX_PASSES] also counts passes past 8.
 * Added to the forward's bits, EA_FWD_PLAIN_SOLVER makes every solver step
 * take a streamed pass: no row is solved on the scores the histogram pass
 * kept, and no step is formed from sums shifted to a new point or from a
 * row's few largest scores, so passes equal solver steps (with
 * EA_FWD_NO_HIST this is a Halley-bisection root search from the bracket
 * alone, as the predecessor method does: fugumt.com / openreview.net
 * AdaSplash abstract). Results are the same up to rounding; the pass cap
 * is then 40, as without the histogram.
 * EA_FWD_PASS_CAP(n), n = 1 .. EA_MAX_PASSES, lowers the cap on streamed
 * passes to n: rows still unconverged take the midpoint of their bracket
 * (which holds the root) and are counted in stats->unconverged. Meant for
 * testing that fallback.
 * An empty or unknown bit set returns EA_ERR_INVALID_ARG. */
#define EA_FWD_MAX 1u
#define EA_FWD_HIST 2u
#define EA_FWD_REFINE 4u
#define EA_FWD_OUT 8u
#define EA_FWD_ALL 15u
#define EA_FWD_NO_HIST 16u
#define EA_FWD_PLAIN_SOLVER 32u
#define EA_FWD_PASS_CAP(n) ((unsigned)(n) << 12)
/* Histogram size, added to the forward's bits: 2^l bins per unit of z,
 * l = 5 .. 9 (32 .. 512). The bin count trades on-chip memory against the
 * quality of the start and so the solver's iterations (euno.news page,
 * section "限制与未来工作", limitations and future work). Without it the
 * histogram has EA_HIST_BINS = 256.
 * Sizes other than 256 need bf16 inputs and N <= 65536 (EA_ERR_UNSUPPORTED
 * otherwise). */
#define EA_FWD_HIST_BINS_LOG2(l) ((unsigned)(l) << 8)
#define EA_BWD_MASK 1u
#define EA_BWD_ROWS 2u
#define EA_BWD_COLS 4u
#define EA_BWD_ALL 7u

ea_status entmax_attn_fwd_phases(const void* q, const void* k, const void* v,
                                 void* o, float* tau, uint32_t* mask, void* state, size_t state_bytes,
                                 float alpha, int causal, int B, int H, int N, int d,
                                 ea_dtype dtype, ea_fwd_stats* stats, void* stream,
                                 unsigned phases);

ea_status entmax_attn_bwd_phases(const void* q, const void* k, const void* v, const void* dout,
                                 const float* tau, const uint32_t* mask, const void* state, size_t state_bytes,
                                 void* dq, void* dk, void* dv,
                                 float alpha, int causal, int B, int H, int N, int d,
                                 ea_dtype dtype, void* workspace, size_t workspace_bytes,
                                 void* stream, unsigned phases);

/* Grouped-query attention: q, o, tau, mask, state, dout, dq have H heads; k, v,
 * dk, dv have Hkv heads, H a multiple of Hkv, and query head h reads key /
 * value head h / (H / Hkv) (euno.news page, section "限制与未来工作" names
 * multi-query settings as the next step). dk and dv sum over the query heads
 * that share a key/value head. The _phases entry points above are these with
 * Hkv = H. Hkv < 1 or H not a multiple of Hkv returns EA_ERR_INVALID_ARG. */
ea_status entmax_attn_fwd_gqa(const void* q, const void* k, const void* v,
                              void* o, float* tau, uint32_t* mask, void* state, size_t state_bytes,
                              float alpha, int causal, int B, int H, int Hkv, int N, int d,
                              ea_dtype dtype, ea_fwd_stats* stats, void* stream,
                              unsigned phases);

ea_status entmax_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* dout,
                              const float* tau, const uint32_t* mask, const void* state, size_t state_bytes,
                              void* dq, void* dk, void* dv,
                              float alpha, int causal, int B, int H, int Hkv, int N, int d,
                              ea_dtype dtype, void* workspace, size_t workspace_bytes,
                              void* stream, unsigned phases);

/* ------------------------------------------------------------------------
 * Strided layouts, for drop-in use inside existing attention modules, whose
 * tensors are mostly token-major [B, N, H, d] (euno.news page, section
 * "Practical Implications": same API as nn.MultiheadAttention; section
 * "方法论" point 5: embedded in standard Transformer code). The
 * [B, H, N, d]-shaped tensors may be any view
 * whose last dimension is contiguous: element (b, h, n, e) of q, o, dout and
 * dq sits at b*batch + h*head + n*row + e with q_strides, and of k, v, dk, dv
 * with kv_strides. Strides are in elements, not negative, row >= 1, and
 * every stride times the element size a multiple of 16 bytes
 * (EA_ERR_INVALID_ARG otherwise). o, dout and dq share q's strides, dk and
 * dv share k's. tau, mask and the state keep their dense [B, H, ...] layouts.
 * Output layouts must give every element its own address (the dimensions of
 * size > 1, taken in increasing stride, each stepping over the extent of the
 * previous ones; rows at least d elements apart): EA_ERR_INVALID_ARG
 * otherwise.
 * Outputs must not overlap each other or the inputs.
 * [B, H, N, d] storage: {H*N*d, N*d, d}; [B, N, H, d] storage: {N*H*d, d, H*d}.
 * The _gqa entry points are these with dense strides.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t batch, head, row;
} ea_strides;

ea_status entmax_attn_fwd_strided(const void* q, const void* k, const void* v,
                                  void* o, float* tau, uint32_t* mask, void* state, size_t state_bytes,
                                  float alpha, int causal, int B, int H, int Hkv, int N, int d,
                                  const ea_strides* q_strides, const ea_strides* kv_strides,
                                  ea_dtype dtype, ea_fwd_stats* stats, void* stream,
                                  unsigned phases);

ea_status entmax_attn_bwd_strided(const void* q, const void* k, const void* v, const void* dout,
                                  const float* tau, const uint32_t* mask, const void* state, size_t state_bytes,
                                  void* dq, void* dk, void* dv,
                                  float alpha, int causal, int B, int H, int Hkv, int N, int d,
                                  const ea_strides* q_strides, const ea_strides* kv_strides,
                                  ea_dtype dtype, void* workspace, size_t workspace_bytes,
                                  void* stream, unsigned phases);

/* ------------------------------------------------------------------------
 * Packed variable-length sequences, the batch form of Transformer training
 * code that the method is embedded in (euno.news page, section "方法论"
 * point 5, and "Practical Implications"). nseq sequences of
 * lengths n_b = cu_seqlens[b+1] - cu_seqlens[b] are packed token-major:
 *   q, o, dout, dq : [total, H, d], sequence b at tokens cu_seqlens[b] ..;
 *   k, v, dk, dv   : [total, Hkv, d];
 *   tau (and stats->tau_h, stats->passes) : sequence b's [H, n_b] block at
 *                    element H * cu_seqlens[b];
 *   state          : sequence b's records from byte 4 d H cu_seqlens[b],
 *                    ea_varlen_fwd_state_bytes(cu_seqlens, nseq, H, d) in all;
 *   mask           : the sequences' [H, nb_b, W_b] blocks one after another,
 *                    ea_varlen_mask_words(cu_seqlens, nseq, H) words in all.
 * cu_seqlens is HOST memory: nseq + 1 non-decreasing offsets starting at 0,
 * every length at most EA_MAX_N (EA_ERR_INVALID_ARG otherwise); empty
 * sequences are skipped. Each sequence is its own problem (attention never
 * crosses sequences); causal is within a sequence. The sequences are
 * enqueued one after another on `stream`, so the backward's workspace, of
 * ea_varlen_bwd_workspace_bytes bytes (the most any one sequence needs), is
 * reused by each. Every sequence's arguments are checked, with every check
 * of the single-problem entry points, before the first is enqueued: a
 * rejected call enqueues nothing. The size helpers return 0 for invalid
 * offsets.
 * ------------------------------------------------------------------------ */
size_t ea_varlen_mask_words(const int* cu_seqlens, int nseq, int H);
size_t ea_varlen_fwd_state_bytes(const int* cu_seqlens, int nseq, int H, int d);
size_t ea_varlen_bwd_workspace_bytes(const int* cu_seqlens, int nseq, int H, int d);

ea_status entmax_attn_fwd_varlen(const void* q, const void* k, const void* v,
                                 void* o, float* tau, uint32_t* mask, void* state, size_t state_bytes,
                                 float alpha, int causal, const int* cu_seqlens, int nseq,
                                 int H, int Hkv, int d, ea_dtype dtype, ea_fwd_stats* stats,
                                 void* stream, unsigned phases);

ea_status entmax_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* dout,
                                 const float* tau, const uint32_t* mask, const void* state, size_t state_bytes,
                                 void* dq, void* dk, void* dv,
                                 float alpha, int causal, const int* cu_seqlens, int nseq,
                                 int H, int Hkv, int d, ea_dtype dtype, void* workspace,
                                 size_t workspace_bytes, void* stream, unsigned phases);

/* ------------------------------------------------------------------------
 * Dense softmax attention on the same tile pipeline: the comparator the
 * entmax path is timed against (the pages measure alpha-entmax against
 * FlashAttention-style softmax kernels: gist.science German page, section 1
 * "Problemstellung" and section 4 "Ergebnisse"). O = softmax(Q K^T / sqrt(d)) V
 * over every visible key (causal: j <= i).
 *  softmax_attn_fwd: o [B,H,N,d] output; lse2 [B,H,N] fp32 output, the
 *    base-2 log-sum-exp of the row's scores x = q.k log2(e)/sqrt(d);
 *    o32: optional [B,H,N,d] fp32 copy of O (16-byte aligned, NULL to skip),
 *    the backward's delta = dout . O.
 *  softmax_attn_bwd: gradients of sum(o * dout); lse2 and o32 from the
 *    forward (o32 may be NULL: delta then takes a sweep of its own);
 *    workspace of ea_softmax_bwd_workspace_bytes bytes, 256-byte aligned.
 * Same argument checks and status codes as the entmax entry points.
 * ------------------------------------------------------------------------ */
size_t ea_softmax_bwd_workspace_bytes(int B, int H, int N, int d);

ea_status softmax_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse2, float* o32,
                           int causal, int B, int H, int N, int d, ea_dtype dtype, void* stream);

ea_status softmax_attn_bwd(const void* q, const void* k, const void* v, const void* dout, const float* lse2,
                           const float* o32, void* dq, void* dk, void* dv, int causal, int B, int H, int N,
                           int d, ea_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). The same computation and arguments as entmax_attn_bwd
 * (all phases, dense layouts, H query and key/value heads), without the
 * workspace: its scratch is a static device array of the library,
 * EA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the library's first
 * use on a GPU until the process ends; the call itself allocates nothing.
 * A problem whose ea_bwd_workspace_bytes exceeds it returns
 * EA_ERR_SCRATCH_LIMIT before any launch (for example B H N up to about
 * 65 thousand query rows at d = 64 with the forward's state). Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and give undefined results; calls in
 * one stream's order are safe. The first call on a GPU looks up the array's
 * address on it (hipGetSymbolAddress, no allocation).
 * ------------------------------------------------------------------------ */
#define EA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

size_t ea_noalloc_scratch_bytes(void);

ea_status entmax_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* dout,
                                  const float* tau, const uint32_t* mask, const void* state,
                                  size_t state_bytes, void* dq, void* dk, void* dv,
                                  float alpha, int causal, int B, int H, int N, int d,
                                  ea_dtype dtype, void* stream);

/* Measurement aid: the achievable dense bf16 MFMA rate of the device, the
 * rate the kernels' matrix work is compared with beside the published peak.
 * `workgroups` workgroups of 256 threads each issue `iters` rounds of 8
 * independent 32x32x16 bf16 MFMAs per wave on register operands (no memory
 * traffic); `out` receives one float per workgroup (device memory, caller
 * owned, at least `workgroups` floats). ea_mfma_peak_flop gives the FLOP of
 * one launch; time the launch on `stream`. EA_ERR_INVALID_ARG for a NULL
 * `out` or sizes below 1. */
double ea_mfma_peak_flop(int workgroups, int iters);
ea_status ea_mfma_peak(float* out, int workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ENTMAX_ATTN_H */
