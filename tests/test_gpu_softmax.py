"""The dense softmax comparator against plain PyTorch (CPU, float64) softmax
attention: O within 1e-2 relative L2 for bf16 inputs (1e-4 for fp32), the
gradients within 2e-2, lse2 within 1e-4."""
import math

import numpy as np
import pytest
import torch

import adaptive_sparse_attention_amd as ea
from adaptive_sparse_attention_amd import synth

from parity_util import require_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield


def reference(q, k, v, do, causal):
    """float64 softmax attention and its gradients by autograd (CPU)."""
    q, k, v, do = (t.double().clone().requires_grad_(True) for t in (q, k, v, do))
    d = q.shape[-1]
    s = q @ k.transpose(-1, -2) / math.sqrt(d)
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    o = torch.softmax(s, dim=-1) @ v
    (o * do).sum().backward()
    return o.detach(), lse.detach(), q.grad, k.grad, v.grad


def rel(a, b, floor=1e-300):
    """relative L2; the reference norm is taken as at least `floor` (where
    the exact gradient vanishes, as for dQ and dK of a one-key row)."""
    a = a.double().cpu()
    b = b.double().cpu()
    return float((a - b).norm() / max(float(b.norm()), floor))


@pytest.mark.parametrize("N,d,causal,dtype", [(1, 64, True, "bf16"), (65, 64, False, "bf16"), (200, 64, True, "bf16"),
                                              (333, 128, True, "bf16"), (130, 128, False, "f32"),
                                              (1000, 64, True, "bf16"), (257, 64, True, "f32")])
def test_softmax_comparator(N, d, causal, dtype):
    w = synth.small(N, d, 1.5, causal, B=1, H=2, gain=2.0, dtype=dtype, seed=N + 7)
    inp = synth.make(w)
    dev = to_dev(inp)
    label = f"softmax N={N} d={d} causal={causal} {dtype}"
    say(f"case {label}")
    o_ref, lse_ref, dq_r, dk_r, dv_r = reference(inp["q"], inp["k"], inp["v"], inp["do"], causal)
    o, lse2, o32 = ea.softmax_fwd(dev["q"], dev["k"], dev["v"], causal, want_o32=True)
    torch.cuda.synchronize()
    tol_o = 1e-4 if dtype == "f32" else 1e-2
    lse = lse2.cpu().double() * math.log(2.0)
    assert float((lse - lse_ref).abs().max()) <= 1e-4, label
    assert rel(o, o_ref) <= tol_o, (label, rel(o, o_ref))
    assert rel(o32, o_ref) <= (1e-4 if dtype == "f32" else 1e-2), label
    for vb in (o32, None):
        dq, dk, dv = ea.softmax_bwd(dev["q"], dev["k"], dev["v"], dev["do"], lse2, causal, o32=vb)
        torch.cuda.synchronize()
        floor = 1e-4 * float(inp["do"].double().norm())   # gradient scale: |dO| |v| |k| / sqrt(d) ~ |dO|
        errs = [rel(dq, dq_r, floor), rel(dk, dk_r, floor), rel(dv, dv_r, floor)]
        say(f"[{label} {'o32' if vb is not None else 'sweep'}] O {rel(o, o_ref):.2e} dq/dk/dv "
            + " ".join(f"{e:.2e}" for e in errs))
        for e in errs:
            assert e <= 2e-2, (label, errs)
