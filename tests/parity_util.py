"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding and compare it with the float64 oracle on the same seeded inputs."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import adaptive_sparse_attention_amd as ea
import oracle

TAU_TOL = 1e-4          # absolute, z units
REL_L2_TOL = 2e-2       # O, dQ, dK, dV for bf16 inputs with fp32 accumulation
MARGIN_TOL = 1e-4       # mask bits compared only where |margin| > this
GRAD_FLOOR = 1e-4       # gradient norms below this scale count as zero (see check_backward)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def same_bits(x, y):
    """Bit-identical tensors (float NaNs, which torch.equal never finds equal,
    included: the forward's vbar rows of gathered rows start with one)."""
    if x.shape != y.shape or x.dtype != y.dtype:
        return False
    if x.dtype.is_floating_point:
        it = {2: torch.int16, 4: torch.int32, 8: torch.int64}[x.element_size()]
        return torch.equal(x.contiguous().view(it), y.contiguous().view(it))
    return torch.equal(x, y)


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


def check_mask(gpu_bits: np.ndarray, ref: dict, heads=None, label=""):
    """GPU bits equal the oracle's wherever |margin| > MARGIN_TOL."""
    blocks = ref["mask_blocks"]
    if blocks.size == 0:
        return 0
    g = gpu_bits[:, :, blocks, :]
    if heads is not None:
        g = np.stack([g[b, h] for (b, h) in heads])[None]
    margin = ref["margin"]
    decided = np.abs(margin) > MARGIN_TOL
    want = margin > 0
    bad = decided & (g != want)
    nbad = int(bad.sum())
    assert nbad == 0, f"{label}: {nbad} mask bits differ outside the {MARGIN_TOL} margin"
    return int(decided.sum())


def check_forward(w, inp_dev, inp_cpu, rows=None, heads=None, o_tol=REL_L2_TOL, tau_tol=TAU_TOL,
                  label="", want_stats=True, want_vbar=False, phases=None):
    """Run the GPU forward on the whole workload; compare sampled rows of the
    selected heads with the oracle. Returns (gpu outputs, oracle outputs).
    want_vbar runs the training forward (which also writes vbar)."""
    B, H, N, d = inp_cpu["q"].shape
    res = ea.fwd(inp_dev["q"], inp_dev["k"], inp_dev["v"], w.alpha, w.causal, stats=want_stats,
                 want_vbar=want_vbar, phases=ea.FWD_ALL if phases is None else phases)
    o, tau, mask = res[:3]
    vbar = res[3] if want_vbar else None
    st = res[-1] if want_stats else None
    torch.cuda.synchronize()
    rows = np.arange(N) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    q = torch.stack([inp_cpu["q"][b, h] for b, h in heads])[None]
    k = torch.stack([inp_cpu["k"][b, h] for b, h in heads])[None]
    v = torch.stack([inp_cpu["v"][b, h] for b, h in heads])[None]
    ref = oracle.attn_fwd(q, k, v, w.alpha, w.causal, rows=rows)
    o_g = o.float().cpu().numpy()
    tau_g = tau.cpu().numpy()
    o_sel = np.stack([o_g[b, h][rows] for b, h in heads])[None]
    tau_sel = np.stack([tau_g[b, h][rows] for b, h in heads])[None]
    assert np.all(np.isfinite(tau_sel)), f"{label}: non-finite tau"
    assert np.all(np.isfinite(o_sel)), f"{label}: non-finite O"
    terr = np.abs(tau_sel - ref["tau"])
    rl2 = rel_l2_per_head(o_sel, ref["o"])
    say(f"[{label}] tau max err {terr.max():.3e}  O rel-L2 max {rl2.max():.3e}")
    assert terr.max() <= tau_tol, f"{label}: tau error {terr.max():.3e} > {tau_tol}"
    assert rl2.max() <= o_tol, f"{label}: O rel-L2 {rl2.max():.3e} > {o_tol}"
    bits = mask_bits(mask, ea.num_blocks(N))
    ndec = check_mask(bits, ref, heads=heads, label=label)
    # structural: no bits beyond nb, none above the diagonal when causal
    words = mask.cpu().numpy().view(np.uint32)
    nb = ea.num_blocks(N)
    W = words.shape[-1]
    allbits = ((words[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(B, H, nb, W * 32)
    assert not allbits[..., nb:].any(), f"{label}: bits set beyond the last key block"
    if w.causal:
        upper = np.triu(np.ones((nb, nb), dtype=bool), 1)
        assert not (allbits[..., :nb].astype(bool) & upper).any(), f"{label}: bits above the diagonal"
    return {"o": o, "tau": tau, "mask": mask, "vbar": vbar, "stats": st, "bits": bits, "decided": ndec}, ref


def check_backward(w, inp_dev, inp_cpu, fwd_out, dq_rows, dkv_rows, heads, tol=REL_L2_TOL, label="",
                   paths=("vbar", "sweep")):
    """GPU gradients against the oracle's, relative L2 per head, for each
    way of forming delta in `paths`: "vbar" (from the forward's vbar, when
    the forward wrote it) and "sweep" (the backward's own sweep).

    For alpha > 2 the gradient u (dP - delta), u = x^(kappa-1), is unbounded
    as x -> 0+, so any threshold inside the tau tolerance can move it far. The
    bound there is tol plus the oracle's own change when its threshold moves
    by +-TAU_TOL (computed from the oracle alone).
    """
    grads = {}
    for path in paths:
        vbar = fwd_out.get("vbar") if path == "vbar" else None
        if path == "vbar" and vbar is None:
            continue
        grads[path] = ea.bwd(inp_dev["q"], inp_dev["k"], inp_dev["v"], inp_dev["do"], fwd_out["tau"],
                             fwd_out["mask"], w.alpha, w.causal, vbar=vbar)
    assert grads, f"{label}: no backward path ran"
    torch.cuda.synchronize()
    B, H, N, d = inp_cpu["q"].shape
    sel = lambda t: torch.stack([t[b, h] for b, h in heads])[None]
    args = (sel(inp_cpu["q"]), sel(inp_cpu["k"]), sel(inp_cpu["v"]), sel(inp_cpu["do"]), w.alpha, w.causal)
    ref = oracle.attn_bwd(*args, dq_rows=dq_rows, dkv_rows=dkv_rows)
    tols = {"dq": tol, "dk": tol, "dv": tol}
    if w.alpha > 2.0:
        for off in (TAU_TOL, -TAU_TOL):
            alt = oracle.attn_bwd(*args, dq_rows=dq_rows, dkv_rows=dkv_rows, tau_offset=off)
            for name in tols:
                tols[name] = max(tols[name], tol + float(rel_l2_per_head(alt[name], ref[name]).max()))
    # Where the exact gradient vanishes (every sampled row has a one-element
    # support, e.g. N = 1) a relative error is undefined; there the error is
    # measured against an absolute floor of GRAD_FLOOR times the scale of the
    # gradient's factors: |dO| |v| |k| / sqrt(d) for dQ (|q| for dK), |dO| for dV.
    def rownorm_max(t):
        return float(np.sqrt((t.double().numpy() ** 2).sum(-1)).max())
    do_n = float(np.linalg.norm(args[3].double().numpy()))
    q_n, k_n, v_n = rownorm_max(args[0]), rownorm_max(args[1]), rownorm_max(args[2])
    floor = {"dq": GRAD_FLOOR * do_n * v_n * k_n / np.sqrt(d), "dk": GRAD_FLOOR * do_n * v_n * q_n / np.sqrt(d),
             "dv": GRAD_FLOOR * do_n}
    out = {}
    for path, (dq, dk, dv) in grads.items():
        for name, g, r, rws in (("dq", dq, ref["dq"], dq_rows), ("dk", dk, ref["dk"], dkv_rows),
                                ("dv", dv, ref["dv"], dkv_rows)):
            gn = g.float().cpu().numpy()
            gs = np.stack([gn[b, h][rws] for b, h in heads])[None]
            assert np.all(np.isfinite(gs)), f"{label} [{path}]: non-finite {name}"
            rl2 = rel_l2_per_head(gs, r, floor[name])
            out[(path, name)] = float(rl2.max())
            say(f"[{label} {path}] {name} rel-L2 max {rl2.max():.3e} (bound {tols[name]:.3e})")
            assert rl2.max() <= tols[name], f"{label} [{path}]: {name} rel-L2 {rl2.max():.3e} > {tols[name]:.3e}"
    return out
