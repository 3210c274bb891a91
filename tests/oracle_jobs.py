"""Oracle calls that the GPU parity tests run in worker processes, one
attention head per job.

CPU only: this module imports numpy and the oracle alone (no torch, no GPU).
Inputs arrive as the raw element bits of one head ([N, d] uint16 for
bfloat16, float32 otherwise) and are upcast here exactly to float64; results
return as float64 arrays of the sampled rows.
"""
from __future__ import annotations

import os

import numpy as np

import oracle


def f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bits (uint16) or float32 values."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _head(job, name):
    return f64(job[name])[None, None]


def init_worker(threads: int) -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(threads)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))


def fwd_head(job: dict) -> dict:
    """Forward oracle of one head on job["rows"]: tau, o, margin, mask_blocks."""
    r = oracle.attn_fwd(_head(job, "q"), _head(job, "k"), _head(job, "v"), job["alpha"], job["causal"],
                        rows=job["rows"])
    return {"tau": r["tau"][0, 0], "o": r["o"][0, 0], "margin": r["margin"][0, 0],
            "mask_blocks": r["mask_blocks"]}


def bwd_head(job: dict) -> dict:
    """Backward oracle of one head: dq on job["dq_rows"], dk / dv on
    job["dkv_rows"], with the L2 norms of each row's summands; with
    job["cond_eps"], which of those rows sit near a support edge; with
    job["tau_offsets"], the same gradients at tau shifted by each offset (the
    sensitivity to a threshold error)."""
    args = (_head(job, "q"), _head(job, "k"), _head(job, "v"), _head(job, "do"), job["alpha"], job["causal"])
    kw = dict(dq_rows=job["dq_rows"], dkv_rows=job["dkv_rows"], row_lo=job.get("row_lo", 0))
    r = oracle.attn_bwd(*args, cond_eps=job.get("cond_eps"), want_scale=True, **kw)
    out = {n: r[n][0, 0] for n in ("dq", "dk", "dv", "dq_scale", "dk_scale", "dv_scale")}
    if job.get("cond_eps") is not None:
        out["row_near"] = r["row_near"][0, 0]
        out["key_near"] = r["key_near"][0, 0]
    alts = []
    for off in job.get("tau_offsets", ()):
        a = oracle.attn_bwd(*args, tau_offset=off, **kw)
        alts.append({n: a[n][0, 0] for n in ("dq", "dk", "dv")})
    out["alts"] = alts
    return out
