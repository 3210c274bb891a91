"""Float64 CPU oracle for alpha-entmax attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
kernels.

What it computes (the plain definition, written out in float64):

* alpha-entmax of one row of scores z_j = (alpha-1) * s_j is
  p_j = [z_j - tau]_+ ** (1/(alpha-1)), with the threshold tau chosen so that
  sum_j p_j = 1. This is the standard alpha-entmax definition; the pages
  describe it as the sparse replacement of softmax that yields exact zeros and
  whose normaliser tau needs a root search (AdaSplash-2 summary, gist.science
  German page, section 1 "Problemstellung"; euno.news summary, section
  "Methodology", point 1).
* Attention: s = q k^T / sqrt(d) per query row (all keys, or keys j <= i when
  causal), p = entmax(s), o = p v.
* The histogram lower bound tau_h (AdaSplash-2 summary, gist.science German
  page, section 2 "Kernidee", steps 1-2): scores are binned by their left bin
  edge into B = 256 bins of width 1/B, and tau_h solves the entmax equation on
  the binned scores. It is provided here only to check the bound
  tau* - 1/B <= tau_h <= tau*; it is not part of the parity contract.
* Backward: the Jacobian of entmax. With x_j = z_j - tau on the support,
  u_j = x_j ** (kappa-1) (kappa = 1/(alpha-1)), dL/ds_j = u_j (dP_j - delta)
  with dP = dO v^T and delta = sum_j u_j dP_j / sum_j u_j. Then
  dQ = dS k / sqrt(d), dK = dS^T q / sqrt(d), dV = P^T dO. The pages state
  only that gradients are formed over non-zero blocks (AdaSplash-2 summary,
  gist.science German page, section 4 "Ergebnisse"); the formula follows from
  differentiating the definition and is pinned by finite differences.

tau is reported in z units (the units of (alpha-1)*s). The threshold is found
by bisection on the bracket [m - 1, m - n**(1-alpha)] (m = max z, n = number of
valid keys) until its width is at most 1e-12: f(m-1) >= 0 because the largest
term alone is 1, and every term is at most 1/n at m - n**(1-alpha).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

TAU_TOL = 1e-12
HIST_BINS = 256
BLOCK = 64


def kappa_of(alpha: float) -> float:
    if not (alpha > 1.0):
        raise ValueError("alpha must be > 1")
    return 1.0 / (alpha - 1.0)


# --------------------------------------------------------------------------
# One-dimensional alpha-entmax
# --------------------------------------------------------------------------

def _power_pos(x: np.ndarray, e: float) -> np.ndarray:
    """max(x, 0) ** e, with 0 where x <= 0 (also when e <= 0)."""
    xp = np.maximum(x, 0.0)
    out = np.zeros_like(xp)
    pos = xp > 0
    out[pos] = xp[pos] ** e
    return out


def entmax_tau(z: np.ndarray, alpha: float, n_valid: Optional[np.ndarray] = None,
               tol: float = TAU_TOL) -> np.ndarray:
    """Threshold tau per row of z (2-D, float64) by bisection.

    Entries equal to -inf are invalid keys. ``n_valid`` (per row) may be given
    when z holds only a subset of each row (entries <= max-1 removed); it must
    then be the full count of valid keys of the row, since the upper end of
    the bracket depends on it.
    """
    z = np.asarray(z, dtype=np.float64)
    if z.ndim == 1:
        return entmax_tau(z[None, :], alpha,
                          None if n_valid is None else np.atleast_1d(n_valid), tol)[0]
    kap = kappa_of(alpha)
    m = z.max(axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("every row needs at least one valid (finite) score")
    if n_valid is None:
        n_valid = np.isfinite(z).sum(axis=1)
    n_valid = np.asarray(n_valid, dtype=np.float64)
    lo = m - 1.0
    hi = m - n_valid ** (1.0 - alpha)
    # f(lo) >= 0 >= f(hi); keep the invariant while halving the bracket.
    while True:
        width = hi - lo
        if np.all(width <= tol):
            break
        mid = 0.5 * (lo + hi)
        f = _power_pos(z - mid[:, None], kap).sum(axis=1) - 1.0
        go_up = f >= 0.0
        lo = np.where(go_up, mid, lo)
        hi = np.where(go_up, hi, mid)
    return 0.5 * (lo + hi)


def entmax(z: np.ndarray, alpha: float):
    """(p, tau) for each row of z (float64); -inf entries get p = 0."""
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    tau = entmax_tau(z, alpha)
    p = _power_pos(z - tau[:, None], kappa_of(alpha))
    return p, tau


def histogram_tau(z: np.ndarray, alpha: float, bins: int = HIST_BINS) -> float:
    """Lower bound tau_h of one row from its left-edge score histogram.

    Each valid z falls in bin k = floor(bins * z) with left edge k / bins.
    Bins below k_top - bins (more than 1 below the largest score) are dropped:
    they hold no support member, since tau >= max z - 1. tau_h is the root of
    f_h(t) = sum_k c_k (k/bins - t)_+^kappa - 1, found by bisection on
    [e_top - 1, e_top] (f_h(e_top - 1) >= 0 from the top bin alone,
    f_h(e_top) = -1).
    """
    z = np.asarray(z, dtype=np.float64)
    z = z[np.isfinite(z)]
    kap = kappa_of(alpha)
    k = np.floor(z * bins).astype(np.int64)
    ktop = int(k.max())
    keep = k >= ktop - bins
    ks, counts = np.unique(k[keep], return_counts=True)
    edges = ks.astype(np.float64) / bins
    lo, hi = ktop / bins - 1.0, ktop / bins
    while hi - lo > TAU_TOL:
        mid = 0.5 * (lo + hi)
        f = float((counts * _power_pos(edges - mid, kap)).sum()) - 1.0
        if f >= 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def entmax_row_grad(z: np.ndarray, alpha: float, g: np.ndarray):
    """Vector-Jacobian product of entmax w.r.t. its scores s (not z).

    For one row z = (alpha-1) s with upstream gradient g = dL/dp, returns
    dL/ds = u * (g - delta), u = x_+^(kappa-1) on the support, delta =
    sum(u g) / sum(u).
    """
    z = np.asarray(z, dtype=np.float64)
    tau = entmax_tau(z[None, :], alpha)[0]
    x = z - tau
    sup = x > 0
    u = np.zeros_like(x)
    u[sup] = x[sup] ** (kappa_of(alpha) - 1.0)
    delta = float((u * g).sum() / u.sum())
    return u * (g - delta)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _f64(a) -> np.ndarray:
    """Exact upcast of a torch tensor or array (bf16 / fp32) to float64."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


def _scores_block(qh: np.ndarray, kh: np.ndarray, rows: np.ndarray, causal: bool,
                  alpha: float, ncols: Optional[int] = None) -> np.ndarray:
    """z = (alpha-1) * q_rows k^T / sqrt(d) in float64, invalid keys = -inf."""
    d = qh.shape[-1]
    n = kh.shape[0] if ncols is None else ncols
    s = (qh[rows] @ kh[:n].T) / math.sqrt(d)
    z = (alpha - 1.0) * s
    if causal:
        cols = np.arange(n)
        z[cols[None, :] > rows[:, None]] = -np.inf
    return z


def _candidates(z: np.ndarray, margin: float = 0.0):
    """Row-major (ii, jj, values) of the entries with z > max z - 1 - margin.

    Every threshold satisfies tau >= max z - 1 (the largest term alone is 1
    there), so no entry at or below max z - 1 is in a support: the support
    of each row lies among these candidates. ``margin`` widens the set by
    that much below the bracket, for callers that also look at scores just
    under the threshold.
    """
    m = z.max(axis=1)
    ii, jj = np.nonzero(z > (m - 1.0 - margin)[:, None])
    return ii, jj, z[ii, jj]


def _pack_rows(ii: np.ndarray, vals: np.ndarray, nrows: int) -> np.ndarray:
    """Dense [nrows, c] array of row-major sparse values (ii sorted), padded
    with -inf (an invalid key for entmax_tau)."""
    counts = np.bincount(ii, minlength=nrows)
    c = max(1, int(counts.max()))
    start = np.zeros(nrows, dtype=np.int64)
    start[1:] = np.cumsum(counts)[:-1]
    out = np.full((nrows, c), -np.inf)
    out[ii, np.arange(ii.size) - start[ii]] = vals
    return out


def _tau_rows(z: np.ndarray, alpha: float, n_valid: Optional[np.ndarray] = None, margin: float = 0.0):
    """Row thresholds of a score block by bisection over its candidates.

    Entries with z <= max - 1 lie at or below every admissible tau and add
    nothing to the entmax sum, so removing them leaves tau unchanged; the
    bracket still uses the row's full valid count. Returns (tau, ii, jj, zc)
    with the candidates (see _candidates) for the caller.
    """
    if n_valid is None:
        n_valid = np.isfinite(z).sum(axis=1)
    ii, jj, zc = _candidates(z, margin)
    top = _pack_rows(ii, zc, z.shape[0])
    return entmax_tau(top, alpha, n_valid=n_valid), ii, jj, zc


def attn_fwd(q, k, v, alpha: float, causal: bool, rows: Optional[Sequence[int]] = None,
             want_support: bool = False, want_mask: bool = True, row_block: int = 512):
    """Forward oracle for query rows ``rows`` of every (b, h).

    Returns a dict with
      tau    [B, H, R]      threshold in z units,
      o      [B, H, R, d]   output rows,
      mask   [B, H, Rb, nb] bool block mask for the query blocks fully covered
                            by ``rows`` (bit (I, J) = some p_ij > 0),
      margin [B, H, Rb, nb] max over i in I, j in J (valid) of z_ij - tau_i,
      mask_blocks           the query-block indices of those rows,
      support [B, H, R, N]  bool, only when want_support.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    kap = kappa_of(alpha)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    nb = (N + BLOCK - 1) // BLOCK
    tau = np.zeros((B, H, R))
    o = np.zeros((B, H, R, d))
    sup = np.zeros((B, H, R, N), dtype=bool) if want_support else None
    # query blocks whose 64 rows (or all rows of a ragged last block) are present
    blk_ids = np.unique(rows // BLOCK)
    full = [I for I in blk_ids
            if np.all(np.isin(np.arange(I * BLOCK, min(N, (I + 1) * BLOCK)), rows))]
    full = np.asarray(full, dtype=np.int64)
    margin = np.full((B, H, full.size, nb), -np.inf)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, h], k[b, h], v[b, h]
            for r0 in range(0, R, row_block):
                rr = rows[r0:r0 + row_block]
                z = _scores_block(qh, kh, rr, causal, alpha)
                t = _tau_rows(z, alpha)[0]
                x = z - t[:, None]
                p = _power_pos(x, kap)
                tau[b, h, r0:r0 + rr.size] = t
                o[b, h, r0:r0 + rr.size] = p @ vh
                if want_support:
                    sup[b, h, r0:r0 + rr.size] = x > 0
                if want_mask and full.size:
                    for bi, I in enumerate(full):
                        sel = (rr // BLOCK) == I
                        if not np.any(sel):
                            continue
                        xb = x[sel]
                        pad = nb * BLOCK - N
                        xb = np.concatenate([xb, np.full((xb.shape[0], pad), -np.inf)], axis=1)
                        mb = xb.reshape(xb.shape[0], nb, BLOCK).max(axis=2).max(axis=0)
                        margin[b, h, bi] = np.maximum(margin[b, h, bi], mb)
    out = {"tau": tau, "o": o, "rows": rows}
    if want_mask:
        out["margin"] = margin
        out["mask"] = margin > 0
        out["mask_blocks"] = full
    if want_support:
        out["support"] = sup
    return out


def attn_bwd(q, k, v, do, alpha: float, causal: bool,
             dq_rows: Optional[Sequence[int]] = None,
             dkv_rows: Optional[Sequence[int]] = None,
             heads: Optional[Sequence[tuple]] = None, row_block: int = 512,
             tau_offset: float = 0.0, row_lo: int = 0, cond_eps: Optional[float] = None,
             want_scale: bool = False):
    """Backward oracle via the analytic entmax Jacobian.

    dK_j and dV_j depend on every query row that can see key j, so each
    selected head is processed in full (all N rows, in blocks of row_block):
    scores by a float64 GEMM, tau by bisection, the support as a sparse set,
    then sparse products for dQ, dK, dV.

    Returns a dict with dq [B,H,Rq,d], dk / dv [B,H,Rk,d] (zeros for heads not
    in ``heads``), tau [B,H,N] and delta [B,H,N] for the processed heads, and
    ``heads`` (the (b, h) pairs processed).

    ``tau_offset`` (default 0) evaluates the same formulas at tau + offset
    instead of the exact threshold; tests use it to measure how strongly the
    gradients react to a threshold error (for alpha > 2 they are unbounded at
    the support edge).

    ``row_lo`` (default 0) processes only the query rows i >= row_lo. With
    causal attention key j is seen only by rows i >= j, so dK_j and dV_j are
    then exact for every j >= row_lo, as are dQ_i for i >= row_lo; other
    requested rows are returned as NaN.

    ``cond_eps`` (optional) also returns how close each gradient row sits to
    a support edge: ``row_near`` [B,H,Rq] is True where some valid score of
    the query row lies within cond_eps of its threshold, and ``key_near``
    [B,H,Rk] is True where some row that has the key within cond_eps of its
    threshold or above it is such a row. For alpha > 2 the weights
    u = x^(1/(alpha-1) - 1) of the Jacobian are unbounded as x -> 0+, so
    those are the rows a threshold error can move far; the others are
    well-conditioned.

    ``want_scale`` also returns the L2 norm of the summands of each gradient
    row: dq_scale_i = sqrt(sum_j dS_ij^2 |k_j|^2) / sqrt(d), dk_scale_j =
    sqrt(sum_i dS_ij^2 |q_i|^2) / sqrt(d), dv_scale_j = sqrt(sum_i p_ij^2
    |dO_i|^2). Rounding each summand by a relative e moves a row by about e
    times its scale, however much the exact sum cancels (with every key
    equal, dQ is exactly 0 while its summands are not).
    """
    import scipy.sparse as sp

    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    kap = kappa_of(alpha)
    scale = 1.0 / math.sqrt(d)
    dq_rows = np.arange(N) if dq_rows is None else np.asarray(dq_rows, dtype=np.int64)
    dkv_rows = np.arange(N) if dkv_rows is None else np.asarray(dkv_rows, dtype=np.int64)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    if row_lo and not causal:
        raise ValueError("row_lo needs causal attention")
    out_dq = np.zeros((B, H, dq_rows.size, d))
    out_dk = np.zeros((B, H, dkv_rows.size, d))
    out_dv = np.zeros((B, H, dkv_rows.size, d))
    tau_all = np.zeros((B, H, N))
    delta_all = np.zeros((B, H, N))
    want_cond = cond_eps is not None
    eps = float(cond_eps) if want_cond else 0.0
    row_near = np.zeros((B, H, dq_rows.size), dtype=bool)
    key_near = np.zeros((B, H, dkv_rows.size), dtype=bool)
    sc_q = np.zeros((B, H, dq_rows.size))
    sc_k = np.zeros((B, H, dkv_rows.size))
    sc_v = np.zeros((B, H, dkv_rows.size))
    for (b, h) in heads:
        qh, kh, vh, doh = q[b, h], k[b, h], v[b, h], do[b, h]
        dQ = np.zeros((N, d))
        dK = np.zeros((N, d))
        dV = np.zeros((N, d))
        near_r = np.zeros(N, dtype=bool)
        near_k = np.zeros(N, dtype=bool)
        s2q = np.zeros(N)
        s2k = np.zeros(N)
        s2v = np.zeros(N)
        for r0 in range(row_lo, N, row_block):
            rr = np.arange(r0, min(N, r0 + row_block))
            ncols = min(N, rr[-1] + 1) if causal else N
            z = _scores_block(qh, kh, rr, causal, alpha, ncols=ncols)
            n_valid = np.minimum(rr + 1, ncols) if causal else np.full(rr.size, ncols)
            # candidates (with eps below the bracket when conditioning is asked)
            t, ci, cj, cz = _tau_rows(z, alpha, n_valid=n_valid, margin=2.0 * eps)
            t = t + tau_offset
            xc = cz - t[ci]
            sup = xc > 0
            ii, jj, xs = ci[sup], cj[sup], xc[sup]
            p = xs ** kap
            u = xs ** (kap - 1.0)
            dP = np.einsum("ed,ed->e", doh[rr[ii]], vh[jj])
            su = np.bincount(ii, weights=u, minlength=rr.size)
            sud = np.bincount(ii, weights=u * dP, minlength=rr.size)
            delta = sud / su
            dS = u * (dP - delta[ii])
            DS = sp.csr_matrix((dS, (ii, jj)), shape=(rr.size, ncols))
            Pm = sp.csr_matrix((p, (ii, jj)), shape=(rr.size, ncols))
            dQ[rr] += (DS @ kh[:ncols]) * scale
            dK[:ncols] += (DS.T @ qh[rr]) * scale
            dV[:ncols] += Pm.T @ doh[rr]
            tau_all[b, h, rr] = t
            delta_all[b, h, rr] = delta
            if want_scale:
                kn2 = (kh[jj] ** 2).sum(axis=1)
                qn2 = (qh[rr[ii]] ** 2).sum(axis=1)
                don2 = (doh[rr[ii]] ** 2).sum(axis=1)
                s2q[rr] += np.bincount(ii, weights=dS ** 2 * kn2, minlength=rr.size) * scale ** 2
                s2k[:ncols] += np.bincount(jj, weights=dS ** 2 * qn2, minlength=ncols) * scale ** 2
                s2v[:ncols] += np.bincount(jj, weights=p ** 2 * don2, minlength=ncols)
            if want_cond:
                # |z - tau| >= eps for every entry outside the candidates
                close = np.abs(xc) < eps
                rnear = np.bincount(ci[close], minlength=rr.size) > 0
                near_r[rr] = rnear
                touch = (xc > -eps) & rnear[ci]
                near_k[cj[touch]] = True
        if row_lo:
            dQ[:row_lo] = np.nan
            dK[:row_lo] = np.nan
            dV[:row_lo] = np.nan
        out_dq[b, h] = dQ[dq_rows]
        out_dk[b, h] = dK[dkv_rows]
        out_dv[b, h] = dV[dkv_rows]
        row_near[b, h] = near_r[dq_rows]
        key_near[b, h] = near_k[dkv_rows]
        sc_q[b, h] = np.sqrt(s2q[dq_rows])
        sc_k[b, h] = np.sqrt(s2k[dkv_rows])
        sc_v[b, h] = np.sqrt(s2v[dkv_rows])
    res = {"dq": out_dq, "dk": out_dk, "dv": out_dv, "tau": tau_all,
           "delta": delta_all, "heads": heads, "dq_rows": dq_rows, "dkv_rows": dkv_rows}
    if want_cond:
        res["row_near"] = row_near
        res["key_near"] = key_near
    if want_scale:
        res["dq_scale"], res["dk_scale"], res["dv_scale"] = sc_q, sc_k, sc_v
    return res


def block_sparsity(mask: np.ndarray, causal: bool, query_blocks: np.ndarray, nb: int) -> float:
    """1 - (set bits) / (valid tiles) over the given query blocks.

    Valid tiles: all key blocks, or J <= I when causal.
    """
    mask = np.asarray(mask, dtype=bool)
    qb = np.asarray(query_blocks)
    if causal:
        valid = (np.arange(nb)[None, :] <= qb[:, None])
    else:
        valid = np.ones((qb.size, nb), dtype=bool)
    nvalid = valid.sum() * (mask.size // max(1, valid.size))
    return 1.0 - float(mask.sum()) / float(nvalid)


def rel_l2(a, b) -> float:
    """Relative L2 error ||a - b|| / ||b|| over all elements (||a|| when b = 0)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a))


def rel_l2_rows(a, b, floor) -> np.ndarray:
    """Per-row relative L2 error over the last axis: ||a_i - b_i|| divided by
    max(||b_i||, floor) (floor broadcast against the row norms)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    num = np.sqrt(((a - b) ** 2).sum(axis=-1))
    den = np.maximum(np.sqrt((b ** 2).sum(axis=-1)), floor)
    return num / den
