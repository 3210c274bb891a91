#!/usr/bin/env python3
"""Benchmark of alpha-entmax attention forward + backward on one MI355X.

Metric: forward+backward time and dense-equivalent TFLOP/s at N=16k,
alpha=1.5 (B=1, H=16, d=64, causal, bf16, Q and K scaled by a gain g), as a
function of block sparsity, with the executed-FLOP fraction of the bf16 MFMA
peak. One step = one forward and one backward over the whole batch, inputs
already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--gain G]
                    [--no-sweep] [--no-cpu-baseline]
    python bench.py --profile [--workload s16k|train8k|long64k] [--gain G] [--softmax] [--steps K]

Prints one JSON line. Only one GPU is used; --gpus above 1 exits with a
message.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "entmax-attn fwd+bwd dense-equivalent TFLOP/s at N=16k, alpha=1.5"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CPU_HEADS = 4                  # heads of the workload the oracle baseline runs
COPY_BYTES = 1 << 30           # calibration copy of the profiling mode


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def popcount_mask(mask) -> int:
    import numpy as np
    m = mask.cpu().numpy().view(np.uint32)
    return int(np.unpackbits(m.view(np.uint8)).sum())


class Runner:
    """Holds the device tensors of one workload and launches the library."""

    def __init__(self, w, ea, torch):
        from adaptive_sparse_attention_amd import synth
        self.w, self.ea, self.torch = w, ea, torch
        inp = synth.make(w)
        self.q, self.k, self.v, self.do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
        B, H, N, d = self.q.shape
        self.o = torch.empty_like(self.q)
        self.tau = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        self.mask = torch.empty(ea.mask_shape(B, H, N), dtype=torch.int32, device="cuda")
        self.state = torch.empty(ea.fwd_state_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
        self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
        self.ws = torch.empty(ea.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")

    def fwd(self, phases=None):
        ea = self.ea
        self.ea.fwd(self.q, self.k, self.v, self.w.alpha, self.w.causal,
                    out=(self.o, self.tau, self.mask, self.state),
                    phases=ea.FWD_ALL if phases is None else phases)

    def bwd(self, phases=None):
        ea = self.ea
        self.ea.bwd(self.q, self.k, self.v, self.do, self.tau, self.mask, self.w.alpha, self.w.causal,
                    workspace=self.ws, out=(self.dq, self.dk, self.dv), state=self.state,
                    phases=ea.BWD_ALL if phases is None else phases)

    def step(self):
        self.fwd()
        self.bwd()

    def timed(self, fn, k: int) -> float:
        """ms per call of fn over k back-to-back calls (HIP events on the stream)."""
        torch = self.torch
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(k):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / k

    def fwd_bins(self, bins):
        ea = self.ea
        self.ea.fwd(self.q, self.k, self.v, self.w.alpha, self.w.causal,
                    out=(self.o, self.tau, self.mask, self.state), hist_bins=bins)

    def fwd_nohist(self):
        ea = self.ea
        self.ea.fwd(self.q, self.k, self.v, self.w.alpha, self.w.causal,
                    out=(self.o, self.tau, self.mask, self.state), phases=ea.FWD_ALL | ea.FWD_NO_HIST)

    def stats(self, phases=None, bins=None):
        """Work counters of one (untimed) forward with diagnostics."""
        ea, w = self.ea, self.w
        o, tau, mask, st = ea.fwd(self.q, self.k, self.v, w.alpha, w.causal, stats=True,
                                  phases=ea.FWD_ALL if phases is None else phases,
                                  hist_bins=ea.HIST_BINS if bins is None else bins)
        self.torch.cuda.synchronize()
        tiles = [int(x) for x in st["tiles_per_pass"].cpu().numpy()]
        passes = st["passes"].float()
        iters = st["iters"].float()
        B, H, N, d = self.q.shape
        nb = ea.num_blocks(N)
        valid = B * H * (nb * (nb + 1) // 2 if w.causal else nb * nb)
        nz = popcount_mask(mask)
        return {
            "tiles_hist": tiles[0],
            "tiles_refine": tiles[1:ea.MAX_PASSES + 1],
            "tiles_out": tiles[ea.MAX_PASSES + 1],
            "tiles_valid": valid,
            "tiles_nonzero": nz,
            "block_sparsity": 1.0 - nz / valid,
            "passes_max": int(passes.max().item()),
            "passes_mean": float(passes.mean().item()),
            "iters_max": int(iters.max().item()),
            "iters_mean": float(iters.mean().item()),
            "unconverged": int(st["unconverged"].item()),
            "halves_nonzero": int(st["halves_out"].item()),
            "subtile_sparsity": 1.0 - int(st["halves_out"].item()) / (4 * valid),
            "rows_gathered": int(st["gathered"][0].item()),
            "halves_out_products": int(st["gathered"][1].item()),
        }


class SoftmaxRunner:
    """The dense softmax comparator on the same inputs (its cost does not
    depend on the gain)."""

    def __init__(self, r):
        self.r, ea, torch = r, r.ea, r.torch
        B, H, N, d = r.q.shape
        self.o = torch.empty_like(r.q)
        self.lse2 = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        self.o32 = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
        self.dq, self.dk, self.dv = (torch.empty_like(r.q) for _ in range(3))
        self.ws = torch.empty(int(ea.load_library().ea_softmax_bwd_workspace_bytes(B, H, N, d)),
                              dtype=torch.uint8, device="cuda")

    def fwd(self):
        r = self.r
        r.ea.softmax_fwd(r.q, r.k, r.v, r.w.causal, out=(self.o, self.lse2, self.o32))

    def bwd(self):
        r = self.r
        r.ea.softmax_bwd(r.q, r.k, r.v, r.do, self.lse2, r.w.causal, o32=self.o32, workspace=self.ws,
                         out=(self.dq, self.dk, self.dv))

    def step(self):
        self.fwd()
        self.bwd()


def softmax_point(r, steps: int):
    """Timing of the dense softmax comparator on the runner's workload."""
    import adaptive_sparse_attention_amd as ea
    sm = SoftmaxRunner(r)
    for _ in range(2):
        sm.step()
    torch = r.torch
    ms = median_ms(torch, sm.step, steps)[0]
    msf = median_ms(torch, sm.fwd, steps)[0]
    sm.fwd()
    msb = median_ms(torch, sm.bwd, steps)[0]
    w = r.w
    B, H, N, d = r.q.shape
    nb = ea.num_blocks(N)
    tiles = B * H * (nb * (nb + 1) // 2 if w.causal else nb * nb)
    ex = ea.tile_flops(d) * tiles * (2 + 7)   # S, P.V; S, dP, dQ; S, dP, dV, dK
    return {"ms_fwd_bwd": round(ms, 4), "ms_fwd": round(msf, 4), "ms_bwd": round(msb, 4),
            "executed_tflops": round(ex / (ms * 1e-3) / 1e12, 2),
            "mfma_frac_executed": round(ex / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def mfma_peak_point(ea, torch):
    """Achievable dense bf16 MFMA rate of this device: the median of 7
    launches of the register-only MFMA kernel (1024 workgroups of 4 waves,
    each wave 8 independent 32x32x16 chains), each between HIP events on the
    current stream, the stream the kernel is launched on."""
    out = torch.empty(1024, dtype=torch.float32, device="cuda")
    flop = ea.mfma_peak(out, 1024, 4000)
    torch.cuda.synchronize()
    ms = median_ms(torch, lambda: ea.mfma_peak(out, 1024, 4000), 7)[0]
    tf = flop / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "frac_of_published": round(tf / PEAK_BF16_TFLOPS, 4), "ms": round(ms, 4),
            "flop": flop, "shape": "1024 workgroups x 4 waves x 8 chains x 4000 rounds of 32x32x16 bf16"}


def flops(w, st, d):
    """Dense-equivalent and executed FLOPs of one forward and one backward.

    Executed work counts 64x64 tile products, G = 2*64*64*d FLOP each, and
    32x32 sub-tile products, G/4 each, over the H sub-tiles (32 query rows x
    32 keys) that hold some p > 0 ("halves_nonzero"):
    forward = G (2 x histogram tiles (row-max kernel and histogram kernel) +
    refinement tiles + output tiles (S)) + G/4 * 2H' (P.V, and U.V for the
    backward's state),
    H' = the sub-tiles whose products the output pass runs
    ("halves_out_products"; rows it gathers run none);
    backward = G * 2 T' (S in the rows and the column kernel) + G/4 * 5H'
    (dP, dQ; dP, dV, dK) over the rows that take the tile path, whose tiles
    and quadrants are those of the output pass's tile path (T' =
    "tiles_out"); the gathered rows' work (row reads and dot products on
    the vector units) is not counted."""
    import adaptive_sparse_attention_amd as ea
    G = ea.tile_flops(d)
    dense_f, dense_b = ea.dense_equiv_flops(w.B, w.H, w.N, d, w.causal)
    H = st["halves_nonzero"]
    exec_f = (G * (2 * st["tiles_hist"] + sum(st["tiles_refine"]) + st["tiles_out"])
              + G / 4 * 2 * st["halves_out_products"])
    exec_b = G * 2 * st["tiles_out"] + G / 4 * 5 * st["halves_out_products"]
    return dense_f, dense_b, exec_f, exec_b


def kernel_times(r, k: int):
    """Median duration of each phase inside full steps: k steps are run, each
    enqueued behind a GPU spin of about a millisecond so that the host is
    ahead of the GPU, with HIP events recorded on the library's stream (torch's
    current one) between the phases. Each phase's time is then GPU time from
    the end of the previous phase to its own end: its kernels and the gaps
    between them, no host enqueue latency."""
    torch, ea = r.torch, r.ea
    phases = [("fwd_max", lambda: r.fwd(ea.FWD_MAX)), ("fwd_hist", lambda: r.fwd(ea.FWD_HIST)),
              ("fwd_refine", lambda: r.fwd(ea.FWD_REFINE)), ("fwd_out", lambda: r.fwd(ea.FWD_OUT)),
              ("bwd_mask", lambda: r.bwd(ea.BWD_MASK)), ("bwd_rows", lambda: r.bwd(ea.BWD_ROWS)),
              ("bwd_cols", lambda: r.bwd(ea.BWD_COLS))]
    times = {n: [] for n, _ in phases}
    for _ in range(k):
        torch.cuda.synchronize()
        gpu_spin(torch)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
        ev[0].record()
        for i, (_, fn) in enumerate(phases):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        for i, (n, _) in enumerate(phases):
            times[n].append(ev[i].elapsed_time(ev[i + 1]))
    return {n: sorted(v)[len(v) // 2] for n, v in times.items()}


_SPIN = {}


def gpu_spin(torch, ms: float = 1.0):
    """Keep the GPU busy for about ms milliseconds (elementwise passes over
    a 256 MiB buffer), so work enqueued after it waits for the GPU, not the
    host."""
    x = _SPIN.get("x")
    if x is None:
        x = _SPIN["x"] = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    for _ in range(max(1, int(ms / 0.07))):
        x.neg_()


def median_ms(torch, fn, k: int):
    """(median, mean) ms of k calls of fn, each between its own pair of HIP
    events on the current stream."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
    torch.cuda.synchronize()
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    t = sorted(s.elapsed_time(e) for s, e in ev)
    return t[len(t) // 2] if k % 2 else 0.5 * (t[k // 2 - 1] + t[k // 2]), sum(t) / k


def memory_report(ea, w):
    """Bytes the training step keeps between the forward and the backward
    (beyond q, k, v and o), and the backward's workspace."""
    B, H, N, d = w.B, w.H, w.N, w.d
    tau = 4 * B * H * N
    mask = 4 * B * H * ea.mask_words(N)
    state = ea.fwd_state_bytes(B, H, N, d)
    return {"saved_state_bytes": tau + mask + state, "tau_bytes": tau, "mask_bytes": mask, "state_bytes": state,
            "workspace_bytes": ea.bwd_workspace_bytes(B, H, N, d),
            "softmax_comparator_saved_bytes": 4 * B * H * N * (1 + d),   # lse2 and the fp32 copy of O
            "o_bytes": B * H * N * d * (2 if w.dtype == "bf16" else 4)}


def solver_iterations(ea, torch, synth):
    """Solver steps (and streamed passes) per row on the 16k solver workload
    at each alpha: the default solver (histogram start, steps on kept scores
    and shifted sums), the plain solver (every step a pass) from the
    histogram start, and the plain solver from the bracket alone."""
    modes = {"histogram": 0, "histogram_plain": ea.FWD_PLAIN_SOLVER,
             "no_histogram_plain": ea.FWD_PLAIN_SOLVER | ea.FWD_NO_HIST}
    res = {}
    for alpha in synth.SWEEP_ALPHAS:
        w = synth.sweep16k(alpha)
        inp = synth.make(w, with_grad=False)
        q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
        pt = {}
        for name, bits in modes.items():
            _, _, _, st = ea.fwd(q, k, v, alpha, True, stats=True, phases=ea.FWD_ALL | bits)
            torch.cuda.synchronize()
            it, ps = st["iters"].float(), st["passes"].float()
            pt[name] = {"iters_mean": round(float(it.mean()), 4), "iters_max": int(it.max()),
                        "passes_mean": round(float(ps.mean()), 4), "passes_max": int(ps.max()),
                        "unconverged": int(st["unconverged"].item())}
            if alpha == 1.5:
                pt[name]["ms_fwd"] = round(median_ms(torch, lambda: ea.fwd(q, k, v, alpha, True,
                                                                           phases=ea.FWD_ALL | bits), 10)[0], 4)
        res[str(alpha)] = pt
        log(f"[bench] solver steps alpha={alpha}: {pt}")
        del q, k, v
    return res


def workload_point(ea, torch, w, steps: int):
    """fwd, bwd and fwd+bwd medians and the work counters of a workload."""
    r = Runner(w, ea, torch)
    for _ in range(2):
        r.step()
    ms, ms_mean = median_ms(torch, r.step, steps)
    msf = median_ms(torch, r.fwd, steps)[0]
    r.fwd()
    msb = median_ms(torch, r.bwd, steps)[0]
    st = r.stats()
    df, db, ef, eb = flops(w, st, w.d)
    pt = {"ms_fwd_bwd": round(ms, 4), "ms_fwd_bwd_mean": round(ms_mean, 4), "ms_fwd": round(msf, 4),
          "ms_bwd": round(msb, 4), "block_sparsity": round(st["block_sparsity"], 4),
          "dense_equiv_tflops": round((df + db) / (ms * 1e-3) / 1e12, 2),
          "executed_tflops": round((ef + eb) / (ms * 1e-3) / 1e12, 2),
          "mfma_frac_executed": round((ef + eb) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
          "passes_max": st["passes_max"], "passes_mean": round(st["passes_mean"], 4),
          "rows_gathered_frac": round(st["rows_gathered"] / (w.B * w.H * w.N), 4)}
    del r
    torch.cuda.empty_cache()
    return pt


def cpu_baseline(w, torch):
    """The oracle (float64 NumPy) on CPU_HEADS heads of the workload, all
    rows, forward and backward; reported in the metric's unit."""
    import numpy as np
    import oracle
    from adaptive_sparse_attention_amd import synth
    import adaptive_sparse_attention_amd as ea
    inp = synth.make(w)
    sel = {n: inp[n][:1, :CPU_HEADS] for n in ("q", "k", "v", "do")}
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=None)
    except Exception:
        pass
    t0 = time.perf_counter()
    oracle.attn_fwd(sel["q"], sel["k"], sel["v"], w.alpha, w.causal, want_mask=False)
    oracle.attn_bwd(sel["q"], sel["k"], sel["v"], sel["do"], w.alpha, w.causal)
    dt = time.perf_counter() - t0
    f, b = ea.dense_equiv_flops(1, CPU_HEADS, w.N, w.d, w.causal)
    return {
        "value": (f + b) / dt / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": int(threads or len(os.sched_getaffinity(0))),
        "kind": "oracle",
        "sample": f"{CPU_HEADS} of {w.B * w.H} heads (b=0, h=0..{CPU_HEADS - 1}), all {w.N} rows: "
                  f"float64 forward (tau by bisection, O) "
                  f"and backward (full-head Jacobian); {dt:.1f} s",
        "seconds": dt,
    }


def read_traffic(kernels, sha: str):
    """HBM bytes per launch of the named kernels (summed), from the counter
    record, or None unless every one was measured for the current sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    total = 0.0
    for kernel in ([kernels] if isinstance(kernels, str) else kernels):
        ent = rec.get(kernel)
        if not ent or ent.get("source_sha") != sha:
            return None
        total += ent.get("traffic_bytes_per_launch")
    return total


def profile_run(r, steps: int, torch, softmax: bool = False) -> int:
    """Steps for a profiler to record (of the dense softmax comparator on the
    same inputs when softmax is set), then a plain copy of COPY_BYTES (one
    read and one write per element) that calibrates the HBM byte counters."""
    step = SoftmaxRunner(r).step if softmax else r.step
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    log(f"[bench] profile run: {steps} steps, calibration copy of {COPY_BYTES} bytes x 3")
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--gain", type=float, default=2.0)
    ap.add_argument("--sweep-steps", type=int, default=21)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3: run --steps plain steps and a calibration copy, print no metric")
    ap.add_argument("--workload", default="s16k", choices=("s16k", "train8k", "long64k"),
                    help="workload of --profile (the metric is always the 16k one)")
    ap.add_argument("--softmax", action="store_true",
                    help="with --profile: run the dense softmax comparator's steps instead")
    args = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the hot path is a single-GPU kernel set; "
              "use --gpus 1 (multi-GPU sharding is design-only here)", file=sys.stderr)
        return 2

    import torch
    import adaptive_sparse_attention_amd as ea
    from adaptive_sparse_attention_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        return 2
    ea.load_library()
    if args.profile:
        wp = {"s16k": synth.s16k(gain=args.gain, causal=True), "train8k": synth.train8k(),
              "long64k": synth.long64k()}[args.workload]
        log(f"[bench] profile workload {wp}")
        return profile_run(Runner(wp, ea, torch), args.steps, torch, softmax=args.softmax)
    w = synth.s16k(gain=args.gain, causal=True)
    log(f"[bench] workload {w}")
    r = Runner(w, ea, torch)
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()
    ms_step = r.timed(r.step, args.steps)
    ms_med, ms_mean = median_ms(torch, r.step, max(21, args.steps))
    ms_fwd = median_ms(torch, r.fwd, max(21, args.steps))[0]
    r.fwd()
    ms_bwd = median_ms(torch, r.bwd, max(21, args.steps))[0]
    st = r.stats()
    dense_f, dense_b, exec_f, exec_b = flops(w, st, w.d)
    value = (dense_f + dense_b) / (ms_step * 1e-3) / 1e12
    log(f"[bench] fwd+bwd {ms_step:.3f} ms (median {ms_med:.3f})  fwd {ms_fwd:.3f}  bwd {ms_bwd:.3f}  "
        f"sparsity {st['block_sparsity']:.3f}  dense-eq {value:.1f} TFLOP/s")

    kt = kernel_times(r, max(10, args.steps))
    G = ea.tile_flops(w.d)
    units = {
        "fwd_max": G * st["tiles_hist"],
        "fwd_hist": G * st["tiles_hist"],
        "fwd_refine": G * sum(st["tiles_refine"]),
        "fwd_out": G * st["tiles_out"] + G / 4 * 2 * st["halves_out_products"],
        "bwd_rows": G * st["tiles_out"] + G / 4 * 2 * st["halves_out_products"],
        "bwd_cols": G * st["tiles_out"] + G / 4 * 3 * st["halves_out_products"],
    }
    # the backward phases launch several kernels (gathered rows, then the
    # tile rows); they are named for their tile kernel. The histogram stage is
    # the list pass (every row group), the one-row histogram (rows it flags)
    # and the histogram kernel (the groups it leaves; the others exit at once):
    # named for the first, its traffic the sum of the three
    names = {"fwd_max": "fwd_max_kernel", "fwd_hist": "fwd_list_kernel", "fwd_refine": "fwd_refine_kernel",
             "fwd_out": "fwd_out_kernel",
             "bwd_rows": "bwd_rows_kernel", "bwd_cols": "bwd_dkdv_kernel"}
    dom = max(units, key=lambda n: kt[n])
    achieved = units[dom] / (kt[dom] * 1e-3) / 1e12
    from adaptive_sparse_attention_amd.profiling import kernel_source_sha
    sha = kernel_source_sha()
    roofline = {
        "bound": "mfma",
        "kernel": names[dom],
        "achieved": achieved,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved / PEAK_BF16_TFLOPS,
        "traffic": read_traffic(["fwd_list_kernel", "fwd_rowhist_kernel", "fwd_init_kernel"] if dom == "fwd_hist" else names[dom],
                                sha),
        "ms_per_launch": kt[dom],
        "flop_per_launch": units[dom],
        "timing": "median over full steps of HIP events between the phases, host kept ahead of the GPU",
        "stage": ("histogram stage: fwd_list_kernel over every row group, fwd_rowhist_kernel over the rows it "
                  "flags, fwd_init_kernel over the groups it leaves; flop_per_launch counts the score tiles of the "
                  "first and last" if dom == "fwd_hist" else names[dom]),
    }
    per_kernel = {names.get(n, n): {"ms": kt[n],
                                    "tflops_executed": (units[n] / (kt[n] * 1e-3) / 1e12) if n in units else None}
                  for n in kt}
    log(f"[bench] kernels: " + ", ".join(f"{k} {v['ms']:.4f} ms" for k, v in per_kernel.items()))
    mem = memory_report(ea, w)
    log(f"[bench] memory: {mem}")
    peak = mfma_peak_point(ea, torch)
    roofline["frac_of_achievable_mfma"] = achieved / peak["tflops"]
    log(f"[bench] achievable MFMA rate: {peak}")

    # the solver without the histogram start, for the pass counts it needs
    ms_fwd_nh = median_ms(torch, r.fwd_nohist, 11)[0]
    st_nh = r.stats(ea.FWD_ALL | ea.FWD_NO_HIST)
    no_hist = {"ms_fwd": ms_fwd_nh, "passes_mean": st_nh["passes_mean"], "passes_max": st_nh["passes_max"],
               "iters_mean": st_nh["iters_mean"], "iters_max": st_nh["iters_max"],
               "unconverged": st_nh["unconverged"], "tiles_refine": st_nh["tiles_refine"]}
    log(f"[bench] without histogram: fwd {ms_fwd_nh:.3f} ms, passes mean {st_nh['passes_mean']:.3f} "
        f"max {st_nh['passes_max']} (with: mean {st['passes_mean']:.3f} max {st['passes_max']})")
    r.fwd()

    # histogram size: forward time and passes per bin count
    bins_sweep = []
    for bins in (32, 64, 128, 256, 512):
        msb = median_ms(torch, lambda: r.fwd_bins(bins), 11)[0]
        sb = r.stats(bins=bins)
        bins_sweep.append({"bins": bins, "ms_fwd": round(msb, 4), "passes_mean": round(sb["passes_mean"], 4),
                           "passes_max": sb["passes_max"], "iters_mean": round(sb["iters_mean"], 4),
                           "tiles_refine": sb["tiles_refine"][:3]})
        log(f"[bench] histogram bins {bins}: {bins_sweep[-1]}")
    r.fwd()

    softmax = {"causal": softmax_point(r, 21)}
    log(f"[bench] dense softmax comparator (causal): {softmax['causal']}")
    del r
    torch.cuda.empty_cache()

    iters = solver_iterations(ea, torch, synth)

    workloads = {}
    for wl in (synth.train8k(), synth.long64k()):
        workloads[wl.name] = workload_point(ea, torch, wl, 11)
        workloads[wl.name]["memory"] = memory_report(ea, wl)
        log(f"[bench] {wl.name}: {workloads[wl.name]}")

    sweep = []
    if not args.no_sweep:
        points = [(g, True) for g in synth.S16K_GAINS] + [(g, False) for g in synth.S16K_NONCAUSAL_GAINS]
        for g, causal in points:
            ws = synth.s16k(gain=g, causal=causal)
            pt = {"gain": g, "causal": causal}
            pt.update(workload_point(ea, torch, ws, args.sweep_steps))
            key = "causal" if causal else "noncausal"
            if key not in softmax:
                rs = Runner(ws, ea, torch)
                softmax[key] = softmax_point(rs, 21)
                log(f"[bench] dense softmax comparator ({key}): {softmax[key]}")
                del rs
                torch.cuda.empty_cache()
            pt["speedup_vs_softmax"] = round(softmax[key]["ms_fwd_bwd"] / pt["ms_fwd_bwd"], 3)
            sweep.append(pt)
            log(f"[bench] sweep {pt}")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(w, torch)
        log(f"[bench] cpu baseline {cpu['value']:.6f} TFLOP/s on {cpu['cores']} threads ({cpu['seconds']:.1f} s)")

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s (dense-equivalent, fwd+bwd)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q, K, V, dO; Q and K x gain; bf16)",
        "config": {"workload": f"s16k: B=1 H=16 N=16384 d=64 causal alpha=1.5 gain={w.gain}",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal, "alpha": w.alpha,
                   "gain": w.gain},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": {
            "ms_step_median": ms_med, "ms_step_mean": ms_mean, "ms_fwd": ms_fwd, "ms_bwd": ms_bwd,
            "block_sparsity": st["block_sparsity"],
            "executed_tflops": (exec_f + exec_b) / (ms_step * 1e-3) / 1e12,
            "mfma_frac_executed": (exec_f + exec_b) / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "passes_max": st["passes_max"], "passes_mean": st["passes_mean"],
            "iters_max": st["iters_max"], "iters_mean": st["iters_mean"],
            "unconverged": st["unconverged"],
            "memory": mem,
            "tiles": {k: st[k] for k in ("tiles_hist", "tiles_refine", "tiles_out", "tiles_valid",
                                         "tiles_nonzero", "halves_nonzero", "rows_gathered",
                                         "halves_out_products")},
            "subtile_sparsity": st["subtile_sparsity"],
            "kernels": per_kernel,
            "mfma_peak": peak,
            "kernel_source_sha": sha,
            "no_histogram": no_hist,
            "solver_iterations": iters,
            "softmax_comparator": softmax,
            "histogram_bins": bins_sweep,
            "workloads": workloads,
            "sweep": sweep,
        },
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
