"""Pins for the float64 oracle, independent of the oracle's own code path.

Each test checks the oracle against something fixed by the mathematics:
closed forms (sparsemax by sort-and-threshold at alpha=2, the quadratic
prefix solution at alpha=1.5), the softmax limit as alpha -> 1, brute-force
support enumeration with a library root finder on tiny rows, special rows
with known answers, invariants, the histogram bound, and central finite
differences of the forward for the backward.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.optimize import brentq

import oracle
from oracle import entmax_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# closed forms (written here, not in the oracle)
# ---------------------------------------------------------------------------

def sparsemax_sort(z):
    """Textbook sparsemax: sort descending, largest k with 1 + k z_(k) > cumsum."""
    zs = np.sort(z)[::-1]
    cs = np.cumsum(zs)
    ks = np.arange(1, zs.size + 1)
    k = ks[1 + ks * zs > cs].max()
    tau = (cs[k - 1] - 1.0) / k
    return np.maximum(z - tau, 0.0), tau


def entmax15_prefix(z):
    """alpha=1.5 in z units: p = (z - tau)_+^2; on a top-k support the
    equation k t^2 - 2 S1 t + S2 - 1 = 0 gives the smaller root; the right
    k satisfies z_(k) > tau >= z_(k+1)."""
    zs = np.sort(z)[::-1]
    found = []
    for k in range(1, zs.size + 1):
        s1 = zs[:k].sum()
        s2 = (zs[:k] ** 2).sum()
        disc = s1 * s1 - k * (s2 - 1.0)
        if disc < 0:
            continue
        tau = (s1 - math.sqrt(disc)) / k
        nxt = zs[k] if k < zs.size else -np.inf
        if zs[k - 1] > tau >= nxt:
            found.append(tau)
    assert len(found) == 1, found
    tau = found[0]
    return np.maximum(z - tau, 0.0) ** 2, tau


def softmax(s):
    e = np.exp(s - s.max())
    return e / e.sum()


RNG = np.random.default_rng(1234)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 50, 1000])
def test_sparsemax_closed_form(n):
    for trial in range(20):
        z = RNG.standard_normal(n) * RNG.uniform(0.1, 5.0)
        p, tau = oracle.entmax(z[None, :], 2.0)
        p_ref, tau_ref = sparsemax_sort(z)
        assert abs(tau[0] - tau_ref) <= 1e-11
        np.testing.assert_allclose(p[0], p_ref, atol=1e-11)


@pytest.mark.parametrize("n", [1, 2, 5, 40, 700])
def test_entmax15_closed_form(n):
    for trial in range(20):
        z = RNG.standard_normal(n) * RNG.uniform(0.1, 4.0)
        p, tau = oracle.entmax(z[None, :], 1.5)
        p_ref, tau_ref = entmax15_prefix(z)
        assert abs(tau[0] - tau_ref) <= 1e-10
        np.testing.assert_allclose(p[0], p_ref, atol=1e-10)


def test_softmax_limit():
    s = RNG.standard_normal(30) * 2.0
    ref = softmax(s)
    errs = []
    for eps in (1e-2, 1e-3, 1e-4):
        a = 1.0 + eps
        p, _ = oracle.entmax(((a - 1.0) * s)[None, :], a)
        errs.append(np.abs(p[0] - ref).sum())
    # error shrinks ~linearly in (alpha-1): one decade per decade
    assert errs[0] < 0.2
    assert 5.0 < errs[0] / errs[1] < 20.0
    assert 5.0 < errs[1] / errs[2] < 20.0


@pytest.mark.parametrize("alpha", [1.1, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0])
def test_bruteforce_support(alpha):
    """Enumerate every support set of tiny rows; exactly one is consistent."""
    kap = 1.0 / (alpha - 1.0)
    for trial in range(15):
        n = int(RNG.integers(1, 8))
        z = RNG.standard_normal(n) * RNG.uniform(0.2, 3.0)
        taus = []
        for r in range(1, n + 1):
            for S in itertools.combinations(range(n), r):
                zs = z[list(S)]
                g = lambda t: np.sum((zs - t) ** kap) - 1.0
                lo, hi = zs.min() - 1.0 - 1e-9, zs.min()
                # g is decreasing on t < min(zs); g(min) = sum - 1 over others
                if g(hi - 1e-15) > 0:
                    continue  # root would not lie below min(zs)
                t = brentq(g, lo, hi - 1e-15, xtol=1e-14, rtol=1e-15, maxiter=500)
                others = np.delete(z, list(S))
                if others.size == 0 or others.max() <= t:
                    taus.append(t)
        assert len(taus) == 1, (z, taus)
        tau = oracle.entmax_tau(z[None, :], alpha)[0]
        assert abs(tau - taus[0]) <= 1e-10


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
def test_special_rows(alpha):
    # equal scores: uniform, tau = z - n^(1-alpha)
    for n in (1, 2, 17, 64, 1000):
        z = np.full(n, 0.37)
        p, tau = oracle.entmax(z[None, :], alpha)
        # a tau error e moves p by kappa * x^(kappa-1) * e, x = n^(1-alpha)
        kap = 1.0 / (alpha - 1.0)
        x = n ** (1.0 - alpha)
        np.testing.assert_allclose(p[0], 1.0 / n, atol=2 * kap * x ** (kap - 1) * 1e-12 + 1e-15)
        assert abs(tau[0] - (0.37 - n ** (1.0 - alpha))) <= 1e-11
    # single key
    p, tau = oracle.entmax(np.array([[2.5]]), alpha)
    assert p[0, 0] == pytest.approx(1.0, abs=1e-12)
    assert tau[0] == pytest.approx(1.5, abs=1e-11)


def test_two_keys_sparsemax():
    for d in (-2.0, -1.0, -0.3, 0.0, 0.6, 1.0, 1.7):
        p, _ = oracle.entmax(np.array([[d, 0.0]]), 2.0)
        if abs(d) >= 1.0:
            exp = np.array([1.0, 0.0]) if d > 0 else np.array([0.0, 1.0])
        else:
            exp = np.array([(1 + d) / 2, (1 - d) / 2])
        np.testing.assert_allclose(p[0], exp, atol=1e-11)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 2.5])
def test_invariants(alpha):
    z = RNG.standard_normal((6, 200)) * 3.0
    p, tau = oracle.entmax(z, alpha)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-10)
    # shift: z + c -> tau + c, p unchanged
    p2, tau2 = oracle.entmax(z + 1.75, alpha)
    np.testing.assert_allclose(tau2, tau + 1.75, atol=1e-10)
    np.testing.assert_allclose(p2, p, atol=1e-9)
    # permutation equivariance
    perm = RNG.permutation(200)
    p3, tau3 = oracle.entmax(z[:, perm], alpha)
    np.testing.assert_allclose(tau3, tau, atol=1e-11)
    np.testing.assert_allclose(p3, p[:, perm], atol=1e-10)
    # support is a top-k set
    for r in range(z.shape[0]):
        sup = p[r] > 0
        if sup.any() and (~sup).any():
            assert z[r][sup].min() > z[r][~sup].max()
    # -inf entries (masked keys) are inert
    zi = np.concatenate([z, np.full((6, 5), -np.inf)], axis=1)
    p4, tau4 = oracle.entmax(zi, alpha)
    np.testing.assert_allclose(tau4, tau, atol=1e-11)
    assert np.all(p4[:, 200:] == 0)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 2.5])
def test_histogram_bound(alpha):
    for trial in range(40):
        n = int(RNG.integers(1, 3000))
        z = RNG.standard_normal(n) * RNG.uniform(0.05, 6.0) + RNG.uniform(-5, 5)
        tau = oracle.entmax_tau(z[None, :], alpha)[0]
        th = oracle.histogram_tau(z, alpha)
        assert th <= tau + 1e-10
        assert tau - th <= 1.0 / oracle.HIST_BINS + 1e-10


def test_histogram_exact_on_lattice():
    # scores already on bin edges: the histogram is exact and tau_h = tau*
    z = np.array([3.0, 3.0 - 5 / 256, 3.0 - 40 / 256, 2.0, 0.5])
    for alpha in (1.5, 2.0, 1.25):
        assert abs(oracle.histogram_tau(z, alpha) - oracle.entmax_tau(z[None], alpha)[0]) < 1e-10


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 2.5])
def test_row_jacobian_finite_differences(alpha):
    # Own generator, so the rows drawn do not depend on which tests ran first.
    # The differenced p come from tau solved to 1e-14 (|tau| < 8 here): with
    # the default 1e-12 the bisection's own error, divided by 2h, reaches the
    # 1e-6 bound by itself.
    rng = np.random.default_rng(int(alpha * 1000))
    h = 1e-6
    kap = oracle.kappa_of(alpha)

    def p_of(s):
        z = (alpha - 1.0) * s
        t = oracle.entmax_tau(z[None, :], alpha, tol=1e-14)[0]
        return np.where(z > t, np.maximum(z - t, 0.0) ** kap, 0.0)

    for trial in range(10):
        n = 12
        s = rng.standard_normal(n) * 2.0
        z = (alpha - 1.0) * s
        tau = oracle.entmax_tau(z[None, :], alpha)[0]
        if np.min(np.abs(z - tau)) < 1e-3:
            continue
        g = rng.standard_normal(n)
        ana = oracle.entmax_row_grad(z, alpha, g)
        num = np.zeros(n)
        for j in range(n):
            sp = s.copy(); sp[j] += h
            sm = s.copy(); sm[j] -= h
            num[j] = (g @ p_of(sp) - g @ p_of(sm)) / (2 * h)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(ana - num).max() <= 1e-6 * scale


# ---------------------------------------------------------------------------
# attention-level pins
# ---------------------------------------------------------------------------

def test_attention_rank_one_sparsemax():
    """q_i = sqrt(d) a_i e_0, k_j = b_j e_0 -> s_ij = a_i b_j exactly; with
    v_j = e_j (N <= d) the output row equals the probability row."""
    N, d = 16, 64
    a = RNG.standard_normal(N)
    b = RNG.standard_normal(N)
    q = np.zeros((1, 1, N, d)); q[0, 0, :, 0] = math.sqrt(d) * a
    k = np.zeros((1, 1, N, d)); k[0, 0, :, 0] = b
    v = np.zeros((1, 1, N, d)); v[0, 0, np.arange(N), np.arange(N)] = 1.0
    out = oracle.attn_fwd(q, k, v, 2.0, causal=False)
    for i in range(N):
        p_ref, tau_ref = sparsemax_sort(a[i] * b)
        assert abs(out["tau"][0, 0, i] - tau_ref) <= 1e-11
        np.testing.assert_allclose(out["o"][0, 0, i, :N], p_ref, atol=1e-11)
        assert np.all(out["o"][0, 0, i, N:] == 0)


def test_attention_rank_one_entmax15_causal():
    N, d = 20, 64
    a = RNG.standard_normal(N) * 2
    b = RNG.standard_normal(N) * 2
    q = np.zeros((1, 1, N, d)); q[0, 0, :, 0] = math.sqrt(d) * a
    k = np.zeros((1, 1, N, d)); k[0, 0, :, 0] = b
    v = np.zeros((1, 1, N, d)); v[0, 0, np.arange(N), np.arange(N)] = 1.0
    out = oracle.attn_fwd(q, k, v, 1.5, causal=True)
    for i in range(N):
        p_ref, tau_ref = entmax15_prefix(0.5 * a[i] * b[: i + 1])
        assert abs(out["tau"][0, 0, i] - tau_ref) <= 1e-10
        np.testing.assert_allclose(out["o"][0, 0, i, : i + 1], p_ref, atol=1e-10)
        assert np.all(np.abs(out["o"][0, 0, i, i + 1:]) <= 1e-15)


def test_attention_causal_first_row_and_equal_keys():
    N, d = 70, 32
    q = RNG.standard_normal((1, 2, N, d))
    k = np.tile(RNG.standard_normal((1, 2, 1, d)), (1, 1, N, 1))  # all keys equal
    v = RNG.standard_normal((1, 2, N, d))
    for alpha in (1.5, 2.0, 1.25):
        out = oracle.attn_fwd(q, k, v, alpha, causal=True)
        for h in range(2):
            # row 0 sees one key: p = [1], tau = z_00 - 1
            z00 = (alpha - 1) * q[0, h, 0] @ k[0, h, 0] / math.sqrt(d)
            assert out["tau"][0, h, 0] == pytest.approx(z00 - 1.0, abs=1e-11)
            np.testing.assert_allclose(out["o"][0, h, 0], v[0, h, 0], atol=1e-12)
            # equal keys: uniform over the i+1 visible keys
            for i in (1, 5, 63, 64, 69):
                np.testing.assert_allclose(out["o"][0, h, i], v[0, h, : i + 1].mean(axis=0),
                                           atol=1e-10)


def test_attention_block_diagonal_mask():
    """q in block I points at e_I, k in block J at e_J: support = own block."""
    N, d, big = 256, 64, 10.0
    blk = np.arange(N) // 64
    q = np.zeros((1, 1, N, d)); q[0, 0, np.arange(N), blk] = big * math.sqrt(d)
    k = np.zeros((1, 1, N, d)); k[0, 0, np.arange(N), blk] = 1.0
    v = RNG.standard_normal((1, 1, N, d))
    out = oracle.attn_fwd(q, k, v, 1.5, causal=False)
    assert out["mask"].shape == (1, 1, 4, 4)
    np.testing.assert_array_equal(out["mask"][0, 0], np.eye(4, dtype=bool))
    # z = 5 on own block (64 equal keys): tau = 5 - 64^-0.5, margin 1/8
    np.testing.assert_allclose(np.diag(out["margin"][0, 0]), 0.125, atol=1e-11)
    off = out["margin"][0, 0][~np.eye(4, dtype=bool)]
    np.testing.assert_allclose(off, -4.875, atol=1e-11)


def test_attention_blocked_path_matches_rowwise():
    """The blocked / prefiltered forward equals plain per-row entmax."""
    B, H, N, d = 1, 2, 150, 16
    q = RNG.standard_normal((B, H, N, d)) * 2
    k = RNG.standard_normal((B, H, N, d)) * 2
    v = RNG.standard_normal((B, H, N, d))
    for alpha, causal in ((1.5, True), (2.0, False), (1.25, True), (2.5, False)):
        out = oracle.attn_fwd(q, k, v, alpha, causal, row_block=37)
        for h in range(H):
            s = q[0, h] @ k[0, h].T / math.sqrt(d)
            z = (alpha - 1) * s
            if causal:
                z[np.triu_indices(N, 1)] = -np.inf
            for i in range(N):
                p, tau = oracle.entmax(z[i][None, :], alpha)
                assert abs(out["tau"][0, h, i] - tau[0]) <= 1e-11
                np.testing.assert_allclose(out["o"][0, h, i], p[0] @ v[0, h], atol=1e-10)


@pytest.mark.parametrize("alpha,causal", [(1.5, True), (2.0, False), (1.25, False), (2.5, True)])
def test_attention_backward_finite_differences(alpha, causal):
    """attn_bwd against central differences of L = sum(o * do) through attn_fwd."""
    B, H, N, d = 1, 1, 24, 8
    rng = np.random.default_rng(7)
    for attempt in range(10):
        q = rng.standard_normal((B, H, N, d)) * 1.5
        k = rng.standard_normal((B, H, N, d)) * 1.5
        v = rng.standard_normal((B, H, N, d))
        do = rng.standard_normal((B, H, N, d))
        # require every score to be 1e-3 away from its row threshold
        fw = oracle.attn_fwd(q, k, v, alpha, causal, want_mask=False)
        s = q[0, 0] @ k[0, 0].T / math.sqrt(d)
        z = (alpha - 1) * s
        gap = np.abs(z - fw["tau"][0, 0][:, None])
        if causal:
            gap[np.triu_indices(N, 1)] = np.inf
        if gap.min() > 1e-3:
            break
    else:
        pytest.skip("no well-separated draw")
    bw = oracle.attn_bwd(q, k, v, do, alpha, causal)
    # h = 1e-4: the 1e-12 bisection tolerance on tau enters the quotient as
    # ~1e-12 / h, and the 1e-3 gap keeps every score on its side of tau.
    h = 1e-4

    def loss(qq, kk, vv):
        return float((oracle.attn_fwd(qq, kk, vv, alpha, causal, want_mask=False)["o"] * do).sum())

    for name, arr, ana in (("q", q, bw["dq"]), ("k", k, bw["dk"]), ("v", v, bw["dv"])):
        idx = [(0, 0, i, j) for i in rng.choice(N, 6, replace=False) for j in rng.choice(d, 2, replace=False)]
        for ix in idx:
            ap = arr.copy(); ap[ix] += h
            am = arr.copy(); am[ix] -= h
            args_p = {"q": (ap, k, v), "k": (q, ap, v), "v": (q, k, ap)}[name]
            args_m = {"q": (am, k, v), "k": (q, am, v), "v": (q, k, am)}[name]
            num = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(ana[ix] - num) <= 1e-6 * max(1.0, abs(num)), (name, ix, ana[ix], num)


def test_backward_sampled_rows_match_full():
    B, H, N, d = 1, 2, 200, 16
    q = RNG.standard_normal((B, H, N, d)) * 2
    k = RNG.standard_normal((B, H, N, d)) * 2
    v = RNG.standard_normal((B, H, N, d))
    do = RNG.standard_normal((B, H, N, d))
    full = oracle.attn_bwd(q, k, v, do, 1.5, True, row_block=64)
    rows = np.array([0, 3, 64, 150, 199])
    part = oracle.attn_bwd(q, k, v, do, 1.5, True, dq_rows=rows, dkv_rows=rows,
                           heads=[(0, 1)], row_block=33)
    np.testing.assert_allclose(part["dq"][0, 1], full["dq"][0, 1, rows], atol=1e-12)
    np.testing.assert_allclose(part["dk"][0, 1], full["dk"][0, 1, rows], atol=1e-12)
    np.testing.assert_allclose(part["dv"][0, 1], full["dv"][0, 1, rows], atol=1e-12)
    assert np.all(part["dq"][0, 0] == 0)


def test_block_sparsity_definition():
    m = np.zeros((1, 1, 2, 4), dtype=bool)
    m[0, 0, 0, 0] = True
    m[0, 0, 1, 1] = True
    # causal, query blocks 2 and 3: valid tiles 3 + 4 = 7, 2 set
    assert oracle.block_sparsity(m, True, np.array([2, 3]), 4) == pytest.approx(1 - 2 / 7)
    assert oracle.block_sparsity(m, False, np.array([2, 3]), 4) == pytest.approx(1 - 2 / 8)


def test_golden_page_constants():
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        facts = json.load(f)
    assert facts["hist_bins"]["value"] == oracle.HIST_BINS
    assert facts["mask_blocks_per_word"]["value"] == 32
    assert all("cite" in v for k, v in facts.items() if not k.startswith("_"))


# ---------------------------------------------------------------------------
# helpers the GPU parity checks use
# ---------------------------------------------------------------------------

def test_rel_l2_hand_computed():
    # ||(3, 5) - (3, 4)|| / ||(3, 4)|| = 1 / 5
    assert oracle.rel_l2(np.array([3.0, 5.0]), np.array([3.0, 4.0])) == pytest.approx(0.2, abs=1e-15)
    # a zero reference: the error's own norm
    assert oracle.rel_l2(np.array([[1.0, 2.0], [2.0, 0.0]]), np.zeros((2, 2))) == pytest.approx(3.0, abs=1e-15)
    # rows: (0, 0) vs (0, 1) -> 1 / 1; (6, 8) vs (3, 4) -> 5 / 5; (1, 0) vs (0, 0) -> 1 / floor 0.5
    a = np.array([[0.0, 0.0], [6.0, 8.0], [1.0, 0.0]])
    b = np.array([[0.0, 1.0], [3.0, 4.0], [0.0, 0.0]])
    np.testing.assert_allclose(oracle.rel_l2_rows(a, b, 0.5), [1.0, 1.0, 2.0], atol=1e-15)
    np.testing.assert_allclose(oracle.rel_l2_rows(a, b, np.array([2.0, 10.0, 4.0])), [0.5, 0.5, 0.25], atol=1e-15)


def _dense_rows(q, k, alpha, causal):
    """Per-row entmax over dense scores, written out row by row."""
    N, d = q.shape
    z = (alpha - 1.0) * (q @ k.T) / math.sqrt(d)
    if causal:
        z[np.triu_indices(N, 1)] = -np.inf
    p, tau = oracle.entmax(z, alpha)
    return z, p, tau


@pytest.mark.parametrize("alpha,causal", [(1.5, True), (2.5, True), (1.25, False), (3.0, False)])
def test_backward_scales_and_conditioning(alpha, causal):
    """The summand norms and near-edge flags of attn_bwd, against dense
    per-row formulas written here."""
    rng = np.random.default_rng(5)
    N, d, eps = 90, 16, 0.05   # wide enough that some rows and keys are near an edge, and some are not
    q = rng.standard_normal((1, 1, N, d)) * 1.5
    k = rng.standard_normal((1, 1, N, d)) * 1.5
    v = rng.standard_normal((1, 1, N, d))
    do = rng.standard_normal((1, 1, N, d))
    bw = oracle.attn_bwd(q, k, v, do, alpha, causal, cond_eps=eps, want_scale=True, row_block=32)
    z, p, tau = _dense_rows(q[0, 0], k[0, 0], alpha, causal)
    kap = 1.0 / (alpha - 1.0)
    x = z - tau[:, None]
    u = np.where(x > 0, np.maximum(x, 1e-300) ** (kap - 1.0), 0.0)
    dP = do[0, 0] @ v[0, 0].T
    delta = (u * dP).sum(1) / u.sum(1)
    dS = u * (dP - delta[:, None])
    kn2 = (k[0, 0] ** 2).sum(1)
    qn2 = (q[0, 0] ** 2).sum(1)
    don2 = (do[0, 0] ** 2).sum(1)
    np.testing.assert_allclose(bw["dq_scale"][0, 0], np.sqrt((dS ** 2 * kn2[None, :]).sum(1) / d), rtol=1e-9)
    np.testing.assert_allclose(bw["dk_scale"][0, 0], np.sqrt((dS ** 2 * qn2[:, None]).sum(0) / d), rtol=1e-9)
    np.testing.assert_allclose(bw["dv_scale"][0, 0], np.sqrt((p ** 2 * don2[:, None]).sum(0)), rtol=1e-9)
    valid = np.isfinite(z)
    row_near = (valid & (np.abs(x) < eps)).any(1)
    key_near = ((x > -eps) & valid & row_near[:, None]).any(0)
    assert row_near.any() and not row_near.all() and key_near.any()
    np.testing.assert_array_equal(bw["row_near"][0, 0], row_near)
    np.testing.assert_array_equal(bw["key_near"][0, 0], key_near)


def test_backward_row_lo_matches_full():
    """row_lo: dq of rows >= row_lo and dk, dv of keys >= row_lo equal the
    full computation (causal); the rest is NaN."""
    rng = np.random.default_rng(9)
    N, d = 300, 16
    q, k, v, do = (rng.standard_normal((1, 1, N, d)) * 2 for _ in range(4))
    full = oracle.attn_bwd(q, k, v, do, 1.5, True, row_block=64)
    part = oracle.attn_bwd(q, k, v, do, 1.5, True, row_block=64, row_lo=200)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(part[n][0, 0, 200:], full[n][0, 0, 200:], atol=1e-12)
        assert np.all(np.isnan(part[n][0, 0, :200]))
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, k, v, do, 1.5, False, row_lo=10)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_backward_equal_keys_closed_form(alpha):
    """Every key equal, causal: row i is uniform over its n = i + 1 keys, so
    x = n^(1-alpha), u = x^(kappa-1) is the same for every key of the row,
    delta_i = mean_j dP_ij, and dQ_i = u k sum_j (dP_ij - delta_i) / sqrt(d)
    = 0; dV_j = sum_{i>=j} dO_i / (i+1); dK_j = sum_{i>=j} u_i (dP_ij -
    delta_i) q_i / sqrt(d)."""
    rng = np.random.default_rng(3)
    N, d = 150, 32
    q = rng.standard_normal((1, 1, N, d))
    k = np.tile(rng.standard_normal((1, 1, 1, d)), (1, 1, N, 1))
    v, do = rng.standard_normal((1, 1, N, d)), rng.standard_normal((1, 1, N, d))
    bw = oracle.attn_bwd(q, k, v, do, alpha, True, row_block=40)
    kap = 1.0 / (alpha - 1.0)
    n = np.arange(1, N + 1, dtype=np.float64)
    u = (n ** (1.0 - alpha)) ** (kap - 1.0)
    dP = do[0, 0] @ v[0, 0].T
    lower = np.tril(np.ones((N, N), dtype=bool))
    delta = np.where(lower, dP, 0.0).sum(1) / n
    dS = np.where(lower, u[:, None] * (dP - delta[:, None]), 0.0)
    dk = dS.T @ q[0, 0] / math.sqrt(d)
    dv = np.where(lower, 1.0 / n[:, None], 0.0).T @ do[0, 0]
    scale = np.abs(dS).sum() * np.abs(q).max() / math.sqrt(d)
    assert np.abs(bw["dq"][0, 0]).max() <= 1e-9 * scale
    np.testing.assert_allclose(bw["dk"][0, 0], dk, atol=1e-9 * scale)
    np.testing.assert_allclose(bw["dv"][0, 0], dv, atol=1e-10)
