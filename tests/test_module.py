"""The nn.MultiheadAttention-shaped module: construction, parameter layout
(an nn.MultiheadAttention state dict loads into it) and argument checks on
the CPU; its output and gradients on the GPU against the float64 oracle
through the same projections."""
import math

import numpy as np
import pytest
import torch
from torch import nn

import adaptive_sparse_attention_amd as ea
from adaptive_sparse_attention_amd import EntmaxMultiheadAttention


def test_parameters_match_multihead_attention():
    ref = nn.MultiheadAttention(256, 4)
    m = EntmaxMultiheadAttention(256, 4)
    assert {n: p.shape for n, p in m.named_parameters()} == {n: p.shape for n, p in ref.named_parameters()}
    m.load_state_dict(ref.state_dict())
    assert torch.equal(m.in_proj_weight, ref.in_proj_weight)
    g = EntmaxMultiheadAttention(512, 8, num_kv_heads=2, bias=False)
    assert g.q_proj_weight.shape == (512, 512) and g.k_proj_weight.shape == (128, 512)
    assert g.in_proj_weight is None and g.in_proj_bias is None


def test_rejects_what_it_does_not_support():
    with pytest.raises(ValueError):
        EntmaxMultiheadAttention(96, 3)            # head size 32
    with pytest.raises(ValueError):
        EntmaxMultiheadAttention(256, 4, alpha=1.0)
    with pytest.raises(ValueError):
        EntmaxMultiheadAttention(512, 8, num_kv_heads=3)
    m = EntmaxMultiheadAttention(128, 2)
    x = torch.zeros(5, 1, 128)
    with pytest.raises(ValueError):
        m(x, x, x, attn_mask=torch.zeros(5, 5))
    with pytest.raises(ValueError):
        m(x, x, x, key_padding_mask=torch.zeros(1, 5, dtype=torch.bool))
    with pytest.raises(ValueError):
        m(x, torch.zeros(6, 1, 128), torch.zeros(6, 1, 128))


def _oracle_module(m, x, causal):
    """The module's output recomputed in float64: projections, then the
    oracle's attention per head (K, V repeated over each group), then the
    output projection."""
    import oracle
    (wq, bq), (wk, bk), (wv, bv) = (tuple(None if t is None else t.detach().double().cpu() for t in p)
                                    for p in m._weights())
    xb = x.detach().double().cpu()
    if not m.batch_first:
        xb = xb.transpose(0, 1)
    B, L, _ = xb.shape
    hd, H, Hkv = m.head_dim, m.num_heads, m.num_kv_heads

    def proj(w, b, nh):
        y = xb @ w.T + (b if b is not None else 0)
        return y.view(B, L, nh, hd).transpose(1, 2)

    # the kernels see the projections rounded to the module's dtype
    q = proj(wq, bq, H).to(x.dtype).double()
    k = proj(wk, bk, Hkv).to(x.dtype).double().repeat_interleave(H // Hkv, dim=1)
    v = proj(wv, bv, Hkv).to(x.dtype).double().repeat_interleave(H // Hkv, dim=1)
    o = oracle.attn_fwd(q, k, v, m.alpha, causal, want_mask=False)["o"]
    o = torch.from_numpy(o).to(x.dtype).double().transpose(1, 2).reshape(B, L, H * hd)
    out = o @ m.out_proj.weight.detach().double().cpu().T
    if m.out_proj.bias is not None:
        out = out + m.out_proj.bias.detach().double().cpu()
    return out if m.batch_first else out.transpose(0, 1)


@pytest.mark.gpu
@pytest.mark.parametrize("E,H,Hkv,batch_first,causal,dtype", [(256, 4, 4, False, True, torch.bfloat16),
                                                             (512, 4, 2, True, False, torch.bfloat16),
                                                             (128, 2, 1, True, True, torch.float32)])
def test_module_matches_oracle(E, H, Hkv, batch_first, causal, dtype):
    assert torch.cuda.is_available()
    ea.load_library()
    torch.manual_seed(0)
    m = EntmaxMultiheadAttention(E, H, alpha=1.5, batch_first=batch_first, num_kv_heads=Hkv, device="cuda",
                                 dtype=dtype)
    with torch.no_grad():
        # scores of order one: the supports hold a few keys, as in the kernels' tests
        for p in m.parameters():
            p.mul_(4.0)
    L, B = 300, 2
    x = torch.randn((B, L, E) if batch_first else (L, B, E), device="cuda", dtype=dtype, requires_grad=True)
    y, w = m(x, x, x, is_causal=causal)
    assert w is None and y.shape == x.shape and y.dtype == dtype
    ref = _oracle_module(m, x, causal)
    err = (y.detach().double().cpu() - ref).norm() / ref.norm()
    print(f"module E={E} H={H} Hkv={Hkv}: output rel-L2 {err:.3e}", flush=True)
    assert err <= 2e-2
    y.float().square().sum().backward()
    grads = [x.grad] + [p.grad for p in m.parameters()]
    assert all(g is not None and torch.isfinite(g).all() for g in grads)
