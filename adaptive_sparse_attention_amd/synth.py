"""Seeded synthetic inputs for the alpha-entmax attention workloads.

This module only draws random numbers and shapes them (gains, the local-mean
construction of the long-context query, rounding to bfloat16). It holds none of
the attention arithmetic, so both the HIP path and the CPU oracle can take
their inputs from here without sharing any of the method.

Workloads (named by what they are):

* ``tiny``      B=1 H=1 N=256 d=64, fp32, non-causal, alpha=1.5.
* ``medium``    B=2 H=12 N=4096 d=64, bf16, non-causal, alpha=1.5, Q and K
                each scaled by a gain g in {1, 2, 4} to sweep sparsity.
* ``sweep16k``  B=1 H=16 N=16384 d=64, bf16, causal, gain 2, alpha in
                {1.25, 1.5, 2.0, 2.5} (one solver branch each).
* ``train8k``   B=4 H=12 N=8192 d=64, bf16, causal, alpha=1.5, gain 3, with dO.
* ``long64k``   B=1 H=8 N=65536 d=128, bf16, causal, alpha=1.5; K, V ~ N(0,1);
                Q_i = eps_i + 2 * mean(K_{i-256} .. K_{i-1}); Q and K each x4.
* ``s16k``      B=1 H=16 N=16384 d=64, bf16, causal, alpha=1.5, gain g in
                {1, 2, 3, 4, 6, 8}; plus non-causal points at g in {4, 8}.
* ``long_rows`` B=1 H=1 causal bf16 rows of 32768 .. 262144 keys (parity
                cases beyond the named workloads).

``equal_keys`` copies the first key of each head over all others (a
degenerate case: every score of a row is the same).

Draws use ``numpy.random.default_rng(seed)`` in float32, in the order
Q, K, V, dO (long64k: K, V, eps, dO). Gains are applied in fp32 before the
single round-to-nearest-even conversion to bfloat16.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    alpha: float
    causal: bool
    dtype: str = "bf16"          # "bf16" or "f32"
    gain: float = 1.0            # Q and K are each multiplied by this
    backward: bool = False
    local_mean: bool = False     # long-context construction of Q
    hubs: int = 0                # keys shared by many rows' supports: 0 none; g > 0 aligns
                                 # query head h with key head (h // g) g (grouped queries)
    equal_keys: bool = False     # every key of a head a copy of its first (all scores of a row equal)
    seed: int = 0
    check_rows: Optional[int] = None   # sampled query rows per head (None = all)
    note: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def tiny() -> Workload:
    return Workload("tiny", 1, 1, 256, 64, 1.5, False, dtype="f32")


def medium(gain: float = 1.0) -> Workload:
    return Workload("medium", 2, 12, 4096, 64, 1.5, False, gain=gain)


def sweep16k(alpha: float = 1.5) -> Workload:
    return Workload("sweep16k", 1, 16, 16384, 64, alpha, True, gain=2.0, check_rows=512)


def train8k() -> Workload:
    return Workload("train8k", 4, 12, 8192, 64, 1.5, True, gain=3.0, backward=True, check_rows=256)


def long64k() -> Workload:
    return Workload("long64k", 1, 8, 65536, 128, 1.5, True, gain=4.0, backward=True,
                    local_mean=True, check_rows=256)


def s16k(gain: float = 2.0, causal: bool = True) -> Workload:
    return Workload("s16k", 1, 16, 16384, 64, 1.5, causal, gain=gain, backward=True, check_rows=512)


def long_rows(N: int, d: int = 64, gain: float = 2.0, H: int = 1) -> Workload:
    return Workload(f"long_rows_N{N}", 1, H, N, d, 1.5, True, gain=gain, backward=True, check_rows=512)


MEDIUM_GAINS = (1.0, 2.0, 4.0)
SWEEP_ALPHAS = (1.25, 1.5, 2.0, 2.5)
S16K_GAINS = (1.0, 2.0, 3.0, 4.0, 6.0, 8.0)
S16K_NONCAUSAL_GAINS = (4.0, 8.0)

LOCAL_WINDOW = 256
LOCAL_WEIGHT = 2.0


def _local_mean_query(k: np.ndarray, eps: np.ndarray) -> np.ndarray:
    """Q_i = eps_i + 2 * mean(K_{max(0,i-256)} .. K_{i-1}); Q_0 = eps_0.

    Computed with a float64 running sum over the sequence axis (axis -2).
    """
    n = k.shape[-2]
    csum = np.zeros(k.shape[:-2] + (n + 1, k.shape[-1]), dtype=np.float64)
    np.cumsum(k, axis=-2, dtype=np.float64, out=csum[..., 1:, :])
    i = np.arange(n)
    lo = np.maximum(i - LOCAL_WINDOW, 0)
    cnt = (i - lo).astype(np.float64)
    window_sum = csum[..., i, :] - csum[..., lo, :]
    mean = np.where(cnt[:, None] > 0, window_sum / np.maximum(cnt, 1.0)[:, None], 0.0)
    return (eps.astype(np.float64) + LOCAL_WEIGHT * mean).astype(np.float32)


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)          # round-to-nearest-even
    if dtype == "f32":
        return t.to(torch.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def make(w: Workload, with_grad: Optional[bool] = None) -> dict:
    """Host (CPU) tensors q, k, v (and do when the workload has a backward).

    Returns a dict of contiguous torch tensors in the workload dtype, layout
    [B, H, N, d]. The same bits go to the GPU and, upcast exactly, to the
    oracle.
    """
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    want_do = w.backward if with_grad is None else with_grad
    if w.local_mean:
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        eps = rng.standard_normal(shape, dtype=np.float32)
        do = rng.standard_normal(shape, dtype=np.float32) if want_do else None
        q = _local_mean_query(k, eps)
    else:
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        do = rng.standard_normal(shape, dtype=np.float32) if want_do else None
    if w.hubs:
        _add_hubs(q, k, rng, int(w.hubs))
    if w.equal_keys:
        k[...] = k[:, :, :1, :]
    g = np.float32(w.gain)
    if g != 1:
        q = q * g
        k = k * g
    out = {"q": _round(q, w.dtype), "k": _round(k, w.dtype), "v": _round(v, w.dtype)}
    if do is not None:
        out["do"] = _round(do, w.dtype)
    return out


# Hub keys: key j (j = 0, 1, 2) gets a near copy at key 8 + j, and the query
# rows i >= 8 + j with i % m == r, for (m, r) = (50, 1), (12, 5), (4, 2),
# are set to half of key j plus a little noise, so that those rows put both
# keys (and little else) in their supports: about N/50, N/12 and N/4 rows per
# head list the same two keys. Query head h takes the keys of head
# (h // group) group, the head that a grouped-query caller keeps as the
# shared key head of its group.
HUB_ROWS = ((50, 1), (12, 5), (4, 2))


def _add_hubs(q: np.ndarray, k: np.ndarray, rng, group: int = 1) -> None:
    B, H, N, d = q.shape
    src = (np.arange(H) // group) * group
    for j, (m, r) in enumerate(HUB_ROWS):
        k[:, :, 8 + j] = k[:, :, j] + np.float32(0.05) * rng.standard_normal((B, H, d), dtype=np.float32)
        rows = np.arange(N)
        rows = rows[(rows % m == r) & (rows >= 8 + j)]
        noise = np.float32(0.05) * rng.standard_normal((B, H, rows.size, d), dtype=np.float32)
        q[:, :, rows] = np.float32(0.5) * k[:, src, j][:, :, None, :] + noise


def sample_query_blocks(w: Workload, block: int = 64, seed: int = 1) -> np.ndarray:
    """Query rows checked per head: whole blocks of `block` rows.

    ``check_rows`` rows per head are taken as check_rows/block distinct query
    blocks drawn with ``default_rng(seed)``; all rows when check_rows is None.
    The same row set is used for every (b, h). Returns sorted row indices.
    """
    n = w.N
    if w.check_rows is None or w.check_rows >= n:
        return np.arange(n)
    nblk = (n + block - 1) // block
    want = max(1, w.check_rows // block)
    rng = np.random.default_rng(seed)
    blocks = np.sort(rng.choice(nblk, size=min(want, nblk), replace=False))
    rows = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return rows[rows < n]


def small(N: int, d: int, alpha: float, causal: bool, B: int = 1, H: int = 2,
          gain: float = 1.0, dtype: str = "bf16", seed: int = 0,
          backward: bool = True) -> Workload:
    """Small seeded shapes for exhaustive parity (ragged tails, edge cases)."""
    return Workload(f"small_N{N}_d{d}", B, H, N, d, alpha, causal, dtype=dtype,
                    gain=gain, backward=backward, seed=seed)
