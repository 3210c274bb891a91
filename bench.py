#!/usr/bin/env python3
"""Benchmark of alpha-entmax attention forward + backward on one MI355X.

Metric: forward+backward time and dense-equivalent TFLOP/s at N=16k,
alpha=1.5 (B=1, H=16, d=64, causal, bf16, Q and K scaled by a gain g), as a
function of block sparsity, with the executed-FLOP fraction of the bf16 MFMA
peak. One step = one forward and one backward over the whole batch, inputs
already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--gain G]
                    [--no-sweep] [--no-cpu-baseline]

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
    ms = r.timed(sm.step, steps)
    msf = r.timed(sm.fwd, steps)
    sm.fwd()
    msb = r.timed(sm.bwd, steps)
    w = r.w
    B, H, N, d = r.q.shape
    nb = ea.num_blocks(N)
    tiles = B * H * (nb * (nb + 1) // 2 if w.causal else nb * nb)
    ex = ea.tile_flops(d) * tiles * (2 + 7)   # S, P.V; S, dP, dQ; S, dP, dV, dK
    return {"ms_fwd_bwd": round(ms, 4), "ms_fwd": round(msf, 4), "ms_bwd": round(msb, 4),
            "executed_tflops": round(ex / (ms * 1e-3) / 1e12, 2),
            "mfma_frac_executed": round(ex / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


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
    """Average duration of each kernel launched alone, with HIP events around
    each launch on the stream the library launches on (torch's current one).
    The refinement and output kernels overwrite their inputs (tau_h, the
    candidate mask and the lists of kept scores in o; the mask at tau_h and
    o), so those are restored between launches, outside the timed interval."""
    torch, ea = r.torch, r.ea
    torch.cuda.synchronize()
    out = {}

    def per_launch(fn, prep=None):
        tot = 0.0
        for _ in range(k):
            if prep:
                prep()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            e.synchronize()
            tot += s.elapsed_time(e)
        return tot / k

    out["fwd_max"] = per_launch(lambda: r.fwd(ea.FWD_MAX))
    m_row = r.tau.clone()
    out["fwd_hist"] = per_launch(lambda: r.fwd(ea.FWD_HIST), lambda: r.tau.copy_(m_row))
    tau_h, cand, o_hist = r.tau.clone(), r.mask.clone(), r.o.clone()

    def restore():
        r.tau.copy_(tau_h)
        r.mask.copy_(cand)
        r.o.copy_(o_hist)

    out["fwd_refine"] = per_launch(lambda: r.fwd(ea.FWD_REFINE), restore)
    restore()
    r.fwd(ea.FWD_REFINE)
    m_ref, o_ref = r.mask.clone(), r.o.clone()

    def restore_out():
        r.mask.copy_(m_ref)
        r.o.copy_(o_ref)

    out["fwd_out"] = per_launch(lambda: r.fwd(ea.FWD_OUT), restore_out)
    r.fwd()
    torch.cuda.synchronize()
    out["bwd_mask"] = per_launch(lambda: r.bwd(ea.BWD_MASK))
    out["bwd_rows"] = per_launch(lambda: r.bwd(ea.BWD_ROWS))
    out["bwd_cols"] = per_launch(lambda: r.bwd(ea.BWD_COLS))
    return out


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


def read_traffic(kernel: str, sha: str):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_sha") != sha:
        return None
    return ent.get("traffic_bytes_per_launch")


def profile_run(r, steps: int, torch) -> int:
    """Steps for a profiler to record, then a plain copy of COPY_BYTES (one
    read and one write per element) that calibrates the HBM byte counters."""
    for _ in range(steps):
        r.step()
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
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3: run --steps plain steps and a calibration copy, print no metric")
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
    w = synth.s16k(gain=args.gain, causal=True)
    log(f"[bench] workload {w}")
    r = Runner(w, ea, torch)
    if args.profile:
        return profile_run(r, args.steps, torch)
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()
    ms_step = r.timed(r.step, args.steps)
    ms_fwd = r.timed(r.fwd, args.steps)
    r.fwd()
    ms_bwd = r.timed(r.bwd, args.steps)
    st = r.stats()
    dense_f, dense_b, exec_f, exec_b = flops(w, st, w.d)
    value = (dense_f + dense_b) / (ms_step * 1e-3) / 1e12
    log(f"[bench] fwd+bwd {ms_step:.3f} ms  fwd {ms_fwd:.3f}  bwd {ms_bwd:.3f}  "
        f"sparsity {st['block_sparsity']:.3f}  dense-eq {value:.1f} TFLOP/s")

    kt = kernel_times(r, max(5, args.steps // 2))
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
    # tile rows); they are named for their tile kernel
    names = {"fwd_max": "fwd_max_kernel", "fwd_hist": "fwd_init_kernel", "fwd_refine": "fwd_refine_kernel",
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
        "traffic": read_traffic(names[dom], sha),
        "ms_per_launch": kt[dom],
        "flop_per_launch": units[dom],
    }
    per_kernel = {names.get(n, n): {"ms": kt[n],
                                    "tflops_executed": (units[n] / (kt[n] * 1e-3) / 1e12) if n in units else None}
                  for n in kt}
    log(f"[bench] kernels: " + ", ".join(f"{k} {v['ms']:.3f} ms" for k, v in per_kernel.items()))

    # the solver without the histogram start, for the pass counts it needs
    ms_fwd_nh = r.timed(r.fwd_nohist, max(3, args.steps // 2))
    st_nh = r.stats(ea.FWD_ALL | ea.FWD_NO_HIST)
    no_hist = {"ms_fwd": ms_fwd_nh, "passes_mean": st_nh["passes_mean"], "passes_max": st_nh["passes_max"],
               "unconverged": st_nh["unconverged"], "tiles_refine": st_nh["tiles_refine"]}
    log(f"[bench] without histogram: fwd {ms_fwd_nh:.3f} ms, passes mean {st_nh['passes_mean']:.3f} "
        f"max {st_nh['passes_max']} (with: mean {st['passes_mean']:.3f} max {st['passes_max']})")
    r.fwd()

    # histogram size: forward time and passes per bin count
    bins_sweep = []
    for bins in (32, 64, 128, 256, 512):
        msb = r.timed(lambda: r.fwd_bins(bins), max(3, args.steps // 2))
        sb = r.stats(bins=bins)
        bins_sweep.append({"bins": bins, "ms_fwd": round(msb, 4), "passes_mean": round(sb["passes_mean"], 4),
                           "passes_max": sb["passes_max"], "tiles_refine": sb["tiles_refine"][:3]})
        log(f"[bench] histogram bins {bins}: {bins_sweep[-1]}")
    r.fwd()

    softmax = {"causal": softmax_point(r, max(5, args.steps // 2))}
    log(f"[bench] dense softmax comparator (causal): {softmax['causal']}")

    sweep = []
    if not args.no_sweep:
        points = [(g, True) for g in synth.S16K_GAINS] + [(g, False) for g in synth.S16K_NONCAUSAL_GAINS]
        for g, causal in points:
            ws = synth.s16k(gain=g, causal=causal)
            rs = Runner(ws, ea, torch)
            for _ in range(2):
                rs.step()
            ms = rs.timed(rs.step, args.sweep_steps)
            msf = rs.timed(rs.fwd, args.sweep_steps)
            rs.fwd()
            msb = rs.timed(rs.bwd, args.sweep_steps)
            s2 = rs.stats()
            df, db, ef, eb = flops(ws, s2, ws.d)
            pt = {
                "gain": g, "causal": causal, "block_sparsity": round(s2["block_sparsity"], 4),
                "ms_fwd_bwd": round(ms, 4), "ms_fwd": round(msf, 4), "ms_bwd": round(msb, 4),
                "dense_equiv_tflops": round((df + db) / (ms * 1e-3) / 1e12, 2),
                "executed_tflops": round((ef + eb) / (ms * 1e-3) / 1e12, 2),
                "mfma_frac_executed": round((ef + eb) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "passes_max": s2["passes_max"], "passes_mean": round(s2["passes_mean"], 3),
            }
            key = "causal" if causal else "noncausal"
            if key not in softmax:
                softmax[key] = softmax_point(rs, args.sweep_steps)
                log(f"[bench] dense softmax comparator ({key}): {softmax[key]}")
            pt["speedup_vs_softmax"] = round(softmax[key]["ms_fwd_bwd"] / ms, 3)
            sweep.append(pt)
            log(f"[bench] sweep {pt}")
            del rs
            torch.cuda.empty_cache()

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
            "ms_fwd": ms_fwd, "ms_bwd": ms_bwd,
            "block_sparsity": st["block_sparsity"],
            "executed_tflops": (exec_f + exec_b) / (ms_step * 1e-3) / 1e12,
            "mfma_frac_executed": (exec_f + exec_b) / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "passes_max": st["passes_max"], "passes_mean": st["passes_mean"],
            "unconverged": st["unconverged"],
            "tiles": {k: st[k] for k in ("tiles_hist", "tiles_refine", "tiles_out", "tiles_valid",
                                         "tiles_nonzero", "halves_nonzero", "rows_gathered",
                                         "halves_out_products")},
            "subtile_sparsity": st["subtile_sparsity"],
            "kernels": per_kernel,
            "kernel_source_sha": sha,
            "no_histogram": no_hist,
            "softmax_comparator": softmax,
            "histogram_bins": bins_sweep,
            "sweep": sweep,
        },
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
