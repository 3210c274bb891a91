"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding and compare it with the float64 oracle on the same seeded inputs."""
from __future__ import annotations

import concurrent.futures as cf
import math
import multiprocessing as mp
import os
import sys

import numpy as np
import torch

import adaptive_sparse_attention_amd as ea
import oracle
import oracle_jobs

TAU_TOL = 1e-4          # absolute, z units
REL_L2_TOL = 2e-2       # O, dQ, dK, dV for bf16 inputs with fp32 accumulation
MARGIN_TOL = 1e-4       # mask bits compared only where |margin| > this
GRAD_FLOOR = 1e-4       # gradient norms below this scale count as zero (see check_backward)
# Per-row bound, beside the per-head relative L2: every checked row's error
# ||a_i - b_i|| stays within ROW_TOL of max(||b_i||, ROW_FLOOR * the head's
# RMS row norm). bf16 rounding of P and dS (2^-9 relative per term) and of
# the output gives ~4e-3 per row; the floor keeps rows whose exact value is
# almost zero (a one-key support has dS = 0, so dQ_i = 0) from dividing by it,
# while a row formed from wrong keys or weights still errs by ~||b_i||.
ROW_TOL = 5e-2
ROW_FLOOR = 0.1
# Gradient rows are sums of products that bf16 operands round by up to 2^-9
# each, so a row's rounding error scales with the L2 norm of its summands
# (the oracle's *_scale), not with the exact sum, which can cancel to zero
# (all keys equal: dQ = 0). Gradient denominators, per row and per head, are
# floored at TERM_FRAC times that norm: 1.25e-2 (per row) and 5e-3 (per head)
# of it, several times the ~2e-3 that rounding alone gives.
TERM_FRAC = 0.25
# Gradient rows with a score within COND_EPS of the row threshold are the
# ill-conditioned ones for alpha > 2 (see check_backward).
COND_EPS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def same_bits(x, y):
    """Bit-identical tensors (float NaNs, which torch.equal never finds equal,
    included: the state records of gathered rows start with one)."""
    if x.shape != y.shape or x.dtype != y.dtype:
        return False
    if x.dtype.is_floating_point:
        it = {2: torch.int16, 4: torch.int32, 8: torch.int64}[x.element_size()]
        return torch.equal(x.contiguous().view(it), y.contiguous().view(it))
    return torch.equal(x, y)


def same_state(x: torch.Tensor, y: torch.Tensor, d: int, N: int) -> bool:
    """Two forward states (uint8, records of 4 d bytes per row) are equal in
    every word a row's path writes: all d words of a row formed from tiles;
    the 32-word support list and the ceil(ceil(N/64)/32) mask words after it
    of a row formed by gathering (word 0 = 0xFFFF0000 | count <= 20). The
    rest of a gathered row's record is left unwritten."""
    if x.shape != y.shape:
        return False
    a = x.contiguous().view(torch.int32).reshape(-1, d).cpu()
    b = y.contiguous().view(torch.int32).reshape(-1, d).cpu()
    w0 = a[:, 0].to(torch.int64) & 0xFFFFFFFF
    gathered = ((w0 & 0xFFFF0000) == 0xFFFF0000) & ((w0 & 0xFFFF) <= 20)
    W = ((N + 63) // 64 + 31) // 32
    cols = torch.arange(d)
    used = torch.where(gathered[:, None], cols[None, :] < 32 + W, torch.ones_like(cols[None, :], dtype=torch.bool))
    return bool(torch.equal(torch.where(used, a, 0), torch.where(used, b, 0)))


def bits_of(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a CPU tensor for the oracle workers (uint16 for
    bfloat16, float32 otherwise)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float32).numpy()


def run_jobs(fn, jobs, pool=None):
    """fn over the jobs: in worker processes (CPU only, spawned, no GPU use)
    when there are more than two or pool=True, else here."""
    if pool is None:
        pool = len(jobs) > 2
    if not pool or len(jobs) < 2:
        return [fn(j) for j in jobs]
    ncpu = max(1, min(16, len(os.sched_getaffinity(0))))
    workers = max(1, min(len(jobs), max(1, ncpu // 2)))
    threads = max(1, ncpu // workers)
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=oracle_jobs.init_worker,
                                initargs=(threads,)) as ex:
        return list(ex.map(fn, jobs))


def check_rows(g: np.ndarray, r: np.ndarray, label: str, abs_floor=0.0, tol: float = ROW_TOL,
               rms_floor: bool = True):
    """Worst per-row relative L2 of g against r (rows along axis 0), with
    denominators floored at ROW_FLOOR times the RMS row norm of r (when
    rms_floor) and at abs_floor (a number or one per row). Returns the worst
    value."""
    norms = np.sqrt((np.asarray(r, dtype=np.float64) ** 2).sum(axis=-1))
    rms = float(np.sqrt((norms ** 2).mean())) if norms.size else 0.0
    floor = np.maximum(np.maximum(ROW_FLOOR * rms if rms_floor else 0.0, abs_floor), 1e-300)
    e = oracle.rel_l2_rows(g, r, floor)
    worst = float(e.max()) if e.size else 0.0
    assert worst <= tol, f"{label}: worst row rel-L2 {worst:.3e} > {tol} (row {int(np.argmax(e))})"
    return worst


def require_gpu():
    assert torch.cuda.is_available(), "GPU test needs a ROCm GPU"
    ea.load_library()


def to_dev(inp: dict) -> dict:
    return {k: v.to("cuda").contiguous() for k, v in inp.items()}


def mask_bits(mask: torch.Tensor, nb: int) -> np.ndarray:
    """int32 words [B,H,nb,W] -> bool [B,H,nb,nb] (bit (I, J))."""
    m = mask.detach().cpu().numpy().view(np.uint32)
    B, H, nbq, W = m.shape
    bits = ((m[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(bool)
    bits = bits.reshape(B, H, nbq, W * 32)[..., :nb]
    return bits


def rel_l2_per_head(a: np.ndarray, b: np.ndarray, floor: float = 1e-300) -> np.ndarray:
    """relative L2 over the last two axes, per (b, h); the reference norm is
    taken as at least `floor`."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    num = np.sqrt(((a - b) ** 2).sum(axis=(-1, -2)))
    den = np.sqrt((b ** 2).sum(axis=(-1, -2)))
    return num / np.maximum(den, floor)


def check_mask(gpu_bits: np.ndarray, margin: np.ndarray, label=""):
    """GPU bits [Rb, nb] equal the oracle's wherever |margin| > MARGIN_TOL."""
    if margin.size == 0:
        return 0
    decided = np.abs(margin) > MARGIN_TOL
    want = margin > 0
    bad = decided & (gpu_bits != want)
    nbad = int(bad.sum())
    assert nbad == 0, f"{label}: {nbad} mask bits differ outside the {MARGIN_TOL} margin"
    return int(decided.sum())


def check_forward(w, inp_dev, inp_cpu, rows=None, heads=None, o_tol=REL_L2_TOL, tau_tol=TAU_TOL,
                  label="", want_stats=True, want_state=False, phases=None, pool=None):
    """Run the GPU forward on the whole workload; compare sampled rows of the
    selected heads with the oracle (per head: tau, O rel-L2, worst row, mask
    bits). Returns (gpu outputs, per-head oracle outputs). want_state runs the
    training forward (which also writes the backward's state)."""
    B, H, N, d = inp_cpu["q"].shape
    res = ea.fwd(inp_dev["q"], inp_dev["k"], inp_dev["v"], w.alpha, w.causal, stats=want_stats,
                 want_state=want_state, phases=ea.FWD_ALL if phases is None else phases)
    o, tau, mask = res[:3]
    state = res[3] if want_state else None
    st = res[-1] if want_stats else None
    torch.cuda.synchronize()
    rows = np.arange(N) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    G = inp_cpu["q"].shape[1] // inp_cpu["k"].shape[1]
    jobs = [{"q": bits_of(inp_cpu["q"][b, h]), "k": bits_of(inp_cpu["k"][b, h // G]),
             "v": bits_of(inp_cpu["v"][b, h // G]), "alpha": w.alpha, "causal": w.causal, "rows": rows}
            for (b, h) in heads]
    refs = run_jobs(oracle_jobs.fwd_head, jobs, pool)
    o_g = o.float().cpu().numpy()
    tau_g = tau.cpu().numpy()
    nb = ea.num_blocks(N)
    bits = mask_bits(mask, nb)
    terr_max, rl2_max, row_max, ndec = 0.0, 0.0, 0.0, 0
    for (b, h), ref in zip(heads, refs):
        o_sel = o_g[b, h][rows]
        tau_sel = tau_g[b, h][rows]
        assert np.all(np.isfinite(tau_sel)), f"{label}: non-finite tau (head {b},{h})"
        assert np.all(np.isfinite(o_sel)), f"{label}: non-finite O (head {b},{h})"
        terr = float(np.abs(tau_sel - ref["tau"]).max())
        rl2 = oracle.rel_l2(o_sel, ref["o"])
        assert terr <= tau_tol, f"{label}: tau error {terr:.3e} > {tau_tol} (head {b},{h})"
        assert rl2 <= o_tol, f"{label}: O rel-L2 {rl2:.3e} > {o_tol} (head {b},{h})"
        row_max = max(row_max, check_rows(o_sel, ref["o"], f"{label} O head {b},{h}"))
        ndec += check_mask(bits[b, h][ref["mask_blocks"]], ref["margin"], label=f"{label} head {b},{h}")
        terr_max, rl2_max = max(terr_max, terr), max(rl2_max, rl2)
    say(f"[{label}] {len(heads)} heads: tau max err {terr_max:.3e}  O rel-L2 max {rl2_max:.3e}  "
        f"worst row {row_max:.3e}")
    # structural: no bits beyond nb, none above the diagonal when causal
    words = mask.cpu().numpy().view(np.uint32)
    W = words.shape[-1]
    allbits = ((words[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(B, H, nb, W * 32)
    assert not allbits[..., nb:].any(), f"{label}: bits set beyond the last key block"
    if w.causal:
        upper = np.triu(np.ones((nb, nb), dtype=bool), 1)
        assert not (allbits[..., :nb].astype(bool) & upper).any(), f"{label}: bits above the diagonal"
    return {"o": o, "tau": tau, "mask": mask, "state": state, "stats": st, "bits": bits, "decided": ndec}, refs


def check_backward(w, inp_dev, inp_cpu, fwd_out, dq_rows, dkv_rows, heads, tol=REL_L2_TOL, label="",
                   paths=("state", "sweep"), pool=None, row_lo=0):
    """GPU gradients against the oracle's, per head: relative L2 and the
    worst row (check_rows), for each way of forming delta in `paths`:
    "state" (from the forward's state, when the forward wrote it) and "sweep"
    (the backward's own sweep).

    For alpha > 2 the gradient u (dP - delta), u = x^(kappa-1), is unbounded
    as x -> 0+, so a threshold error inside the tau tolerance can move the
    gradient rows that hold a score near the threshold far. The oracle alone
    decides which rows those are (a valid score within COND_EPS of tau; for
    dK, dV rows: a key that such a row has in or near its support). The other
    rows are held to tol and the per-row bound; the near rows to tol plus
    the oracle's own change when its threshold moves by +-TAU_TOL.

    row_lo > 0 (causal only) checks dq on rows >= row_lo and dk, dv on keys
    >= row_lo, which the oracle forms from rows >= row_lo alone.
    """
    grads = {}
    for path in paths:
        state = fwd_out.get("state") if path == "state" else None
        if path == "state" and state is None:
            continue
        grads[path] = ea.bwd(inp_dev["q"], inp_dev["k"], inp_dev["v"], inp_dev["do"], fwd_out["tau"],
                             fwd_out["mask"], w.alpha, w.causal, state=state)
    assert grads, f"{label}: no backward path ran"
    torch.cuda.synchronize()
    dq_rows = np.asarray(dq_rows)
    dkv_rows = np.asarray(dkv_rows)
    if row_lo:
        dq_rows = dq_rows[dq_rows >= row_lo]
        dkv_rows = dkv_rows[dkv_rows >= row_lo]
    B, H, N, d = inp_cpu["q"].shape
    assert inp_cpu["k"].shape[1] == H, "grouped-query gradients are checked as sums by their own tests"
    ill = w.alpha > 2.0
    jobs = [{"q": bits_of(inp_cpu["q"][b, h]), "k": bits_of(inp_cpu["k"][b, h]),
             "v": bits_of(inp_cpu["v"][b, h]), "do": bits_of(inp_cpu["do"][b, h]), "alpha": w.alpha,
             "causal": w.causal, "dq_rows": dq_rows, "dkv_rows": dkv_rows, "row_lo": row_lo,
             "cond_eps": COND_EPS if ill else None, "tau_offsets": (TAU_TOL, -TAU_TOL) if ill else ()}
            for (b, h) in heads]
    refs = run_jobs(oracle_jobs.bwd_head, jobs, pool)
    host = {path: tuple(g.float().cpu().numpy() for g in gs) for path, gs in grads.items()}
    out = {}
    for (b, h), ref in zip(heads, refs):
        # Where the exact gradient vanishes (every sampled row has a one-element
        # support, e.g. N = 1) a relative error is undefined; there the error is
        # measured against an absolute floor of GRAD_FLOOR times the scale of the
        # gradient's factors: |dO| |v| |k| / sqrt(d) for dQ (|q| for dK), |dO| for dV.
        qf, kf, vf, dof = (oracle_jobs.f64(bits_of(inp_cpu[n][b, h])) for n in ("q", "k", "v", "do"))
        rn = lambda t: float(np.sqrt((t ** 2).sum(-1)).max())
        do_n = float(np.linalg.norm(dof))
        floor = {"dq": GRAD_FLOOR * do_n * rn(vf) * rn(kf) / np.sqrt(d),
                 "dk": GRAD_FLOOR * do_n * rn(vf) * rn(qf) / np.sqrt(d), "dv": GRAD_FLOOR * do_n}
        near = {"dq": ref.get("row_near"), "dk": ref.get("key_near"), "dv": ref.get("key_near")}
        for path, (dq, dk, dv) in host.items():
            for name, g, rws in (("dq", dq, dq_rows), ("dk", dk, dkv_rows), ("dv", dv, dkv_rows)):
                gs = g[b, h][rws]
                r = ref[name]
                assert np.all(np.isfinite(gs)), f"{label} [{path}]: non-finite {name} (head {b},{h})"
                nr = near[name] if ill else np.zeros(len(rws), dtype=bool)
                well = ~nr
                hl = f"{label} [{path}] {name} head {b},{h}"

                sc = ref[name + "_scale"]

                def rel(mask_):
                    num = np.linalg.norm(gs[mask_] - r[mask_])
                    den = max(np.linalg.norm(r[mask_]), TERM_FRAC * np.linalg.norm(sc[mask_]), floor[name])
                    return float(num / den)

                e_well = rel(well) if well.any() else 0.0
                assert e_well <= tol, f"{hl}: rel-L2 {e_well:.3e} > {tol} over {int(well.sum())} rows"
                rfloor = np.maximum(TERM_FRAC * sc[well], floor[name] / math.sqrt(max(1, len(rws))))
                worst = check_rows(gs[well], r[well], hl, abs_floor=rfloor, rms_floor=False)
                e_near, b_near = 0.0, 0.0
                if nr.any():
                    den_n = max(np.linalg.norm(r[nr]), TERM_FRAC * np.linalg.norm(sc[nr]), floor[name])
                    b_near = tol + max(float(np.linalg.norm(a[name][nr] - r[nr]) / den_n) for a in ref["alts"])
                    e_near = rel(nr)
                    assert e_near <= b_near, f"{hl}: near-edge rows rel-L2 {e_near:.3e} > {b_near:.3e}"
                key = (path, name)
                prev = out.get(key, (0.0, 0.0, 0.0, 0))
                out[key] = (max(prev[0], e_well), max(prev[1], worst), max(prev[2], e_near),
                            prev[3] + int(nr.sum()))
    for (path, name), (e, wr, en, nn) in sorted(out.items()):
        say(f"[{label} {path}] {name}: rel-L2 max {e:.3e}, worst row {wr:.3e}"
            + (f"; {nn} near-edge rows rel-L2 max {en:.3e}" if nn else ""))
    return {k: v[0] for k, v in out.items()}
