"""GPU: strided (token-major) layouts and packed variable-length sequences.

The kernels compute the same sums in the same order whatever the strides,
so a token-major call must reproduce the dense [B, H, N, d] call bit for bit
(outputs, tau, mask, gradients); the dense call is itself parity-tested
against the float64 oracle. Packed sequences must reproduce separate dense
calls per sequence bit for bit, and one sequence of each batch is also
checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

import adaptive_sparse_attention_amd as ea
from adaptive_sparse_attention_amd import synth
import oracle

from parity_util import REL_L2_TOL, TAU_TOL, require_gpu, same_bits, same_state, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield


def _token_major(t: torch.Tensor) -> torch.Tensor:
    """[B, H, N, d] values stored as [B, N, H, d], returned as a [B, H, N, d] view."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("N,d,H,Hkv,alpha,causal,dtype", [(200, 64, 4, 4, 1.5, True, "bf16"),
                                                          (1000, 64, 4, 2, 2.0, False, "bf16"),
                                                          (333, 128, 2, 1, 1.25, True, "bf16"),
                                                          (130, 64, 2, 2, 2.5, True, "f32")])
def test_token_major_layout_matches_dense(N, d, H, Hkv, alpha, causal, dtype):
    label = f"bnhd N={N} d={d} H={H} Hkv={Hkv} a={alpha} causal={causal} {dtype}"
    say(f"case {label}")
    wq = synth.small(N, d, alpha, causal, B=2, H=H, gain=2.0, seed=N + 11, dtype=dtype)
    wk = synth.small(N, d, alpha, causal, B=2, H=Hkv, gain=2.0, seed=N + 12, dtype=dtype)
    iq, ik = synth.make(wq), synth.make(wk)
    q, do = iq["q"].cuda(), iq["do"].cuda()
    k, v = ik["k"].cuda(), ik["v"].cuda()
    o, tau, mask, state = ea.fwd(q, k, v, alpha, causal, want_state=True)
    dq, dk, dv = ea.bwd(q, k, v, do, tau, mask, alpha, causal, state=state)
    qs, ks, vs, dos = (_token_major(t) for t in (q, k, v, do))
    assert not qs.is_contiguous() and qs.stride(2) == H * d
    o2, tau2, mask2, state2 = ea.fwd(qs, ks, vs, alpha, causal, want_state=True)
    assert o2.stride() == qs.stride()
    dq2, dk2, dv2 = ea.bwd(qs, ks, vs, dos, tau2, mask2, alpha, causal, state=state2)
    torch.cuda.synchronize()
    assert same_bits(tau, tau2) and same_bits(mask, mask2) and same_state(state, state2, d, N), label
    for a, b, name in ((o, o2, "o"), (dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
        assert same_bits(a, b.contiguous()), f"{label}: {name} differs"
    say(f"[{label}] token-major results equal the dense ones bit for bit")


def _pack(ts):
    """[1, H, n, d] tensors -> [sum n, H, d]."""
    return torch.cat([t[0].transpose(0, 1) for t in ts], 0).contiguous()


@pytest.mark.parametrize("lens,d,H,Hkv,alpha,causal", [([1, 63, 64, 0, 200, 517], 64, 4, 2, 1.5, True),
                                                       ([130, 77, 1000], 128, 2, 2, 2.0, False),
                                                       ([300, 5], 64, 2, 1, 2.5, True),
                                                       # both sides of 65536: the short sequence takes the
                                                       # gather path and needs the larger workspace
                                                       ([1000, 66000], 64, 2, 2, 1.5, True)])
def test_varlen_matches_per_sequence_calls(lens, d, H, Hkv, alpha, causal):
    label = f"varlen lens={lens} d={d} H={H} Hkv={Hkv} a={alpha} causal={causal}"
    say(f"case {label}")
    qs, ks, vs, dos = [], [], [], []
    for i, n in enumerate(lens):
        m = max(n, 1)
        iq = synth.make(synth.small(m, d, alpha, causal, B=1, H=H, gain=2.0, seed=100 + i))
        ik = synth.make(synth.small(m, d, alpha, causal, B=1, H=Hkv, gain=2.0, seed=200 + i))
        qs.append(iq["q"][:, :, :n].cuda())
        dos.append(iq["do"][:, :, :n].cuda())
        ks.append(ik["k"][:, :, :n].cuda())
        vs.append(ik["v"][:, :, :n].cuda())
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    q, k, v, do = _pack(qs), _pack(ks), _pack(vs), _pack(dos)
    o, tau, mask, state, st = ea.fwd_varlen(q, k, v, cu, alpha, causal, stats=True, want_state=True)
    dq, dk, dv = ea.bwd_varlen(q, k, v, do, tau, mask, cu, alpha, causal, state=state)
    torch.cuda.synchronize()
    moff = 0
    for b, n in enumerate(lens):
        if n == 0:
            continue
        t0, t1 = cu[b], cu[b + 1]
        qb, kb, vb, dob = (x.contiguous() for x in (qs[b], ks[b], vs[b], dos[b]))
        o1, tau1, mask1, state1 = ea.fwd(qb, kb, vb, alpha, causal, want_state=True)
        dq1, dk1, dv1 = ea.bwd(qb, kb, vb, dob, tau1, mask1, alpha, causal, state=state1)
        torch.cuda.synchronize()
        mw = H * ea.mask_words(n)
        assert same_bits(tau[H * t0:H * t1], tau1.reshape(-1)), f"{label}: tau of sequence {b}"
        assert same_bits(mask[moff:moff + mw], mask1.reshape(-1)), f"{label}: mask of sequence {b}"
        # the state records of a sequence: 4 d bytes per row of its [H, n_b] block
        rb = 4 * d
        assert same_state(state[H * t0 * rb:H * t1 * rb], state1, d, n), \
            f"{label}: state of sequence {b}"
        assert same_bits(o[t0:t1], o1[0].transpose(0, 1)), f"{label}: o of sequence {b}"
        assert same_bits(dq[t0:t1], dq1[0].transpose(0, 1)), f"{label}: dq of sequence {b}"
        assert same_bits(dk[t0:t1], dk1[0].transpose(0, 1)), f"{label}: dk of sequence {b}"
        assert same_bits(dv[t0:t1], dv1[0].transpose(0, 1)), f"{label}: dv of sequence {b}"
        moff += mw
    # the longest sequence (up to 5000 tokens) against the oracle
    b = int(np.argmax([n if n <= 5000 else 0 for n in lens]))
    ke = ks[b].cpu().repeat_interleave(H // Hkv, dim=1)
    ve = vs[b].cpu().repeat_interleave(H // Hkv, dim=1)
    ref = oracle.attn_fwd(qs[b].cpu(), ke, ve, alpha, causal, want_mask=False)
    t0, t1 = cu[b], cu[b + 1]
    tau_b = tau[H * t0:H * t1].reshape(1, H, -1).cpu().numpy()
    o_b = o[t0:t1].transpose(0, 1)[None].float().cpu().numpy()
    terr = float(np.abs(tau_b - ref["tau"]).max())
    rl2 = oracle.rel_l2(o_b, ref["o"])
    say(f"[{label}] sequences equal separate calls; sequence {b} vs oracle: tau err {terr:.2e}, O rel-L2 {rl2:.2e}")
    assert terr <= TAU_TOL and rl2 <= REL_L2_TOL
    assert int(st["unconverged"].item()) == 0
