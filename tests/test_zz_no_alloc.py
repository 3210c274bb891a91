"""GPU: the allocation-free backward (entmax_attn_bwd_noalloc, through the C
ABI) gives the same gradients as the backward with a caller workspace, bit
for bit, on two calls in a row (the second smaller, so the shared static
scratch holds the first call's contents), with and without the forward's
state, and on hub keys (integer key-side sums)."""
import pytest
import torch

import adaptive_sparse_attention_amd as ea
from adaptive_sparse_attention_amd import synth

from parity_util import require_gpu, same_bits, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield


def _case(N, H, seed, gain=2.0, hubs=False):
    w = synth.small(N, 64, 1.5, True, B=1, H=H, gain=gain, seed=seed)
    if hubs:
        w = w.with_(hubs=True)
    return w, to_dev(synth.make(w))


@pytest.mark.parametrize("with_state", [True, False])
def test_noalloc_backward_matches_workspace_backward(with_state):
    cases = [_case(3000, 4, 1), _case(700, 2, 2, gain=1.0), _case(500, 2, 7, gain=4.0, hubs=True)]
    for w, inp in cases:
        label = f"noalloc N={w.N} H={w.H} g={w.gain} hubs={bool(w.hubs)} state={with_state}"
        say(f"case {label}")
        q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
        o, tau, mask, state = ea.fwd(q, k, v, w.alpha, w.causal, want_state=True)
        st = state if with_state else None
        assert ea.bwd_workspace_bytes(1, w.H, w.N, 64) <= ea.NOALLOC_SCRATCH_BYTES
        ref = ea.bwd(q, k, v, do, tau, mask, w.alpha, w.causal, state=st)
        got = ea.bwd_noalloc(q, k, v, do, tau, mask, w.alpha, w.causal, state=st)
        again = ea.bwd_noalloc(q, k, v, do, tau, mask, w.alpha, w.causal, state=st)
        torch.cuda.synchronize()
        for name, a, b, c in zip(("dq", "dk", "dv"), ref, got, again):
            assert same_bits(a, b), f"{label}: {name} differs from the workspace backward"
            assert same_bits(a, c), f"{label}: {name} differs on a repeated call"
        say(f"[{label}] bit-identical to the workspace backward")


def test_noalloc_rejects_problems_beyond_its_scratch():
    w, inp = _case(64, 1, 3)
    q = inp["q"]
    big = (1, 64, 65536, 128)
    assert ea.bwd_workspace_bytes(*big) > ea.NOALLOC_SCRATCH_BYTES
    lib = ea.load_library()
    # sizes only: the call returns before any pointer is used
    p = [q.data_ptr()] * 6 + [None, 0] + [q.data_ptr()] * 3
    assert lib.entmax_attn_bwd_noalloc(*p, 1.5, 1, *big, 0, None) == ea.EA_ERR_SCRATCH_LIMIT
