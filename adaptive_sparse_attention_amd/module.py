"""nn.MultiheadAttention-shaped module over alpha-entmax attention.

The pages present the kernels as a drop-in for the attention of existing
Transformer code, with the interface of PyTorch's nn.MultiheadAttention
(euno.news AdaSplash-2 summary, "Practical Implications"; "方法论", point 5).
This module keeps that call shape and those parameter names, so a state dict
of an nn.MultiheadAttention with the same sizes loads into it; the
projections are ordinary PyTorch linear maps and the attention itself is the
library's forward and backward (``EntmaxAttention``), in the dtype of the
projected tensors (bfloat16 or float32).

Differences from nn.MultiheadAttention, all raising ValueError when asked
for: query, key and value have the same length (self-attention or
same-length cross-attention), no key_padding_mask or attn_mask tensors
(is_causal=True gives the causal mask), no dropout, and the dense attention
weights are never formed (need_weights returns None in their place).
Grouped-query attention is available through ``num_kv_heads``.
"""
from __future__ import annotations

from typing import Optional

import torch
import torch.nn.functional as F
from torch import nn

from . import entmax_attention

__all__ = ["EntmaxMultiheadAttention"]


class EntmaxMultiheadAttention(nn.Module):
    """alpha-entmax multi-head attention with nn.MultiheadAttention's interface.

    Args:
        embed_dim: model dimension E.
        num_heads: query heads H; E / H (the head size) must be 64 or 128.
        alpha: entmax parameter (> 1; 1.5 by default).
        bias: add biases to the input and output projections.
        batch_first: tensors are (batch, seq, E) instead of (seq, batch, E).
        num_kv_heads: key/value heads (grouped-query attention), dividing H;
            H by default. With fewer than H the projections are separate
            (q_proj_weight, k_proj_weight, v_proj_weight), else packed as
            in_proj_weight like nn.MultiheadAttention.
    """

    def __init__(self, embed_dim: int, num_heads: int, alpha: float = 1.5, bias: bool = True,
                 batch_first: bool = False, num_kv_heads: Optional[int] = None, device=None, dtype=None):
        super().__init__()
        if embed_dim % num_heads != 0:
            raise ValueError("embed_dim must be a multiple of num_heads")
        self.head_dim = embed_dim // num_heads
        if self.head_dim not in (64, 128):
            raise ValueError(f"head size {self.head_dim} is not supported (64 or 128)")
        if not alpha > 1.0:
            raise ValueError("alpha must be > 1")
        kv = num_heads if num_kv_heads is None else int(num_kv_heads)
        if kv < 1 or num_heads % kv != 0:
            raise ValueError("num_kv_heads must divide num_heads")
        self.embed_dim, self.num_heads, self.num_kv_heads = embed_dim, num_heads, kv
        self.alpha, self.batch_first = float(alpha), batch_first
        fk = {"device": device, "dtype": dtype}
        kv_dim = kv * self.head_dim
        if kv == num_heads:
            self.in_proj_weight = nn.Parameter(torch.empty(3 * embed_dim, embed_dim, **fk))
            self.register_parameter("q_proj_weight", None)
            self.register_parameter("k_proj_weight", None)
            self.register_parameter("v_proj_weight", None)
        else:
            self.register_parameter("in_proj_weight", None)
            self.q_proj_weight = nn.Parameter(torch.empty(embed_dim, embed_dim, **fk))
            self.k_proj_weight = nn.Parameter(torch.empty(kv_dim, embed_dim, **fk))
            self.v_proj_weight = nn.Parameter(torch.empty(kv_dim, embed_dim, **fk))
        if bias:
            self.in_proj_bias = nn.Parameter(torch.empty(embed_dim + 2 * kv_dim, **fk))
        else:
            self.register_parameter("in_proj_bias", None)
        self.out_proj = nn.Linear(embed_dim, embed_dim, bias=bias, **fk)
        self._reset_parameters()

    def _reset_parameters(self):
        # the initialisation nn.MultiheadAttention uses
        if self.in_proj_weight is not None:
            nn.init.xavier_uniform_(self.in_proj_weight)
        else:
            for w in (self.q_proj_weight, self.k_proj_weight, self.v_proj_weight):
                nn.init.xavier_uniform_(w)
        if self.in_proj_bias is not None:
            nn.init.constant_(self.in_proj_bias, 0.0)
            nn.init.constant_(self.out_proj.bias, 0.0)

    def _weights(self):
        E, kvd = self.embed_dim, self.num_kv_heads * self.head_dim
        if self.in_proj_weight is not None:
            wq, wk, wv = self.in_proj_weight.split([E, kvd, kvd])
        else:
            wq, wk, wv = self.q_proj_weight, self.k_proj_weight, self.v_proj_weight
        if self.in_proj_bias is not None:
            bq, bk, bv = self.in_proj_bias.split([E, kvd, kvd])
        else:
            bq = bk = bv = None
        return (wq, bq), (wk, bk), (wv, bv)

    def forward(self, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                key_padding_mask: Optional[torch.Tensor] = None, need_weights: bool = True,
                attn_mask: Optional[torch.Tensor] = None, average_attn_weights: bool = True,
                is_causal: bool = False):
        """(attn_output, None): attn_output shaped like query."""
        if key_padding_mask is not None or attn_mask is not None:
            raise ValueError("mask tensors are not supported; use is_causal=True for the causal mask")
        if query.dim() != 3 or key.shape[:-1] != query.shape[:-1] or value.shape[:-1] != query.shape[:-1]:
            raise ValueError("query, key and value must be 3-D with the same batch and sequence sizes")
        if not self.batch_first:
            query, key, value = (t.transpose(0, 1) for t in (query, key, value))
        B, L, _ = query.shape
        (wq, bq), (wk, bk), (wv, bv) = self._weights()
        # [B, L, heads, hd] projections, viewed as [B, heads, L, hd]
        q = F.linear(query, wq, bq).view(B, L, self.num_heads, self.head_dim).transpose(1, 2)
        k = F.linear(key, wk, bk).view(B, L, self.num_kv_heads, self.head_dim).transpose(1, 2)
        v = F.linear(value, wv, bv).view(B, L, self.num_kv_heads, self.head_dim).transpose(1, 2)
        o = entmax_attention(q, k, v, self.alpha, bool(is_causal))
        out = self.out_proj(o.transpose(1, 2).reshape(B, L, self.embed_dim))
        if not self.batch_first:
            out = out.transpose(0, 1)
        return out, None
