"""alpha-entmax attention for AMD MI355X (gfx950).

Thin Python binding of ``libentmax_attn.so`` (C ABI in ``include/entmax_attn.h``).
This module only marshals arguments: torch supplies device memory and the
stream, and every step of the computation runs in the library's HIP kernels.
If the library is not built or cannot be loaded the calls raise; there is no
fallback path.

    o, tau, mask = fwd(q, k, v, alpha, causal)
    o, tau, mask, state = fwd(q, k, v, alpha, causal, want_state=True)   # training
    dq, dk, dv = bwd(q, k, v, do, tau, mask, alpha, causal, state=state)
    o = entmax_attention(q, k, v, alpha, causal)     # autograd-aware
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "BLOCK", "HIST_BINS", "MAX_PASSES", "MAX_N", "EntmaxAttnError", "LIB_PATH",
    "load_library", "mask_words", "fwd_state_bytes", "bwd_workspace_bytes", "status_str", "fwd", "bwd",
    "entmax_attention", "EntmaxAttention", "num_blocks", "mask_shape", "softmax_fwd", "softmax_bwd",
    "fwd_varlen", "bwd_varlen", "EntmaxMultiheadAttention", "bwd_noalloc",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libentmax_attn.so")

# mirrors of the header's constants
BLOCK = 64
HIST_BINS = 256
MAX_PASSES = 8
MAX_N = 1 << 18
EA_OK, EA_ERR_INVALID_ARG, EA_ERR_UNSUPPORTED, EA_ERR_WORKSPACE, EA_ERR_LAUNCH, EA_ERR_SCRATCH_LIMIT = range(6)
NOALLOC_SCRATCH_BYTES = 64 << 20
EA_BF16, EA_F32 = 0, 1
EXPORTED = ("ea_mask_words", "ea_fwd_state_bytes", "ea_bwd_workspace_bytes", "ea_status_str",
            "entmax_attn_fwd", "entmax_attn_bwd", "entmax_attn_fwd_phases", "entmax_attn_bwd_phases",
            "ea_softmax_bwd_workspace_bytes", "softmax_attn_fwd", "softmax_attn_bwd",
            "entmax_attn_fwd_gqa", "entmax_attn_bwd_gqa", "entmax_attn_fwd_strided", "entmax_attn_bwd_strided",
            "ea_varlen_mask_words", "ea_varlen_fwd_state_bytes", "ea_varlen_bwd_workspace_bytes",
            "entmax_attn_fwd_varlen",
            "entmax_attn_bwd_varlen", "ea_noalloc_scratch_bytes", "entmax_attn_bwd_noalloc",
            "ea_mfma_peak_flop", "ea_mfma_peak")
FWD_MAX, FWD_HIST, FWD_REFINE, FWD_OUT, FWD_ALL = 1, 2, 4, 8, 15
FWD_NO_HIST = 16    # with FWD_ALL: solver mode without the histogram pass
FWD_PLAIN_SOLVER = 32   # every solver step a streamed pass (no shortcuts)


def FWD_PASS_CAP(n: int) -> int:
    """Phase bits lowering the cap on streamed refinement passes to n (1..8)."""
    return int(n) << 12
BWD_MASK, BWD_ROWS, BWD_COLS, BWD_ALL = 1, 2, 4, 7


class EntmaxAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


class _Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("row", ctypes.c_int64)]


class _Stats(ctypes.Structure):
    _fields_ = [("tau_h", ctypes.c_void_p), ("passes", ctypes.c_void_p),
                ("tiles_per_pass", ctypes.c_void_p), ("unconverged", ctypes.c_void_p),
                ("halves_out", ctypes.c_void_p),
                ("gathered", ctypes.c_void_p), ("iters", ctypes.c_void_p)]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libentmax_attn.so (once). Raises OSError if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} is not built; run `python -m adaptive_sparse_attention_amd.build`")
    lib = ctypes.CDLL(p)
    vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.ea_mask_words.argtypes = [ci]
    lib.ea_mask_words.restype = sz
    lib.ea_fwd_state_bytes.argtypes = [ci, ci, ci, ci]
    lib.ea_fwd_state_bytes.restype = sz
    lib.ea_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.ea_bwd_workspace_bytes.restype = sz
    lib.ea_status_str.argtypes = [ci]
    lib.ea_status_str.restype = ctypes.c_char_p
    lib.entmax_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, cf, ci, ci, ci, ci, ci, ci, vp, vp]
    lib.entmax_attn_fwd.restype = ci
    lib.entmax_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, cf, ci, ci, ci, ci, ci, ci, vp, sz,
                                    vp]
    lib.entmax_attn_bwd.restype = ci
    cu = ctypes.c_uint
    lib.entmax_attn_fwd_phases.argtypes = lib.entmax_attn_fwd.argtypes + [cu]
    lib.entmax_attn_fwd_phases.restype = ci
    lib.entmax_attn_bwd_phases.argtypes = lib.entmax_attn_bwd.argtypes + [cu]
    lib.entmax_attn_bwd_phases.restype = ci
    lib.entmax_attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, cf, ci, ci, ci, ci, ci, ci, ci, vp, vp, cu]
    lib.entmax_attn_fwd_gqa.restype = ci
    lib.entmax_attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, cf, ci, ci, ci, ci, ci, ci, ci, vp,
                                        sz, vp, cu]
    lib.entmax_attn_bwd_gqa.restype = ci
    lib.entmax_attn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, cf, ci, ci, ci, ci, ci, ci, vp, vp, ci,
                                            vp, vp, cu]
    lib.entmax_attn_fwd_strided.restype = ci
    lib.entmax_attn_bwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, cf, ci, ci, ci, ci, ci, ci,
                                            vp, vp, ci, vp, sz, vp, cu]
    lib.entmax_attn_bwd_strided.restype = ci
    lib.ea_varlen_mask_words.argtypes = [vp, ci, ci]
    lib.ea_varlen_mask_words.restype = sz
    lib.ea_varlen_fwd_state_bytes.argtypes = [vp, ci, ci, ci]
    lib.ea_varlen_fwd_state_bytes.restype = sz
    lib.ea_varlen_bwd_workspace_bytes.argtypes = [vp, ci, ci, ci]
    lib.ea_varlen_bwd_workspace_bytes.restype = sz
    lib.entmax_attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, cf, ci, vp, ci, ci, ci, ci, ci, vp, vp,
                                           cu]
    lib.entmax_attn_fwd_varlen.restype = ci
    lib.entmax_attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, cf, ci, vp, ci, ci, ci, ci,
                                           ci, vp, sz, vp, cu]
    lib.entmax_attn_bwd_varlen.restype = ci
    lib.ea_noalloc_scratch_bytes.argtypes = []
    lib.ea_noalloc_scratch_bytes.restype = sz
    lib.entmax_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, cf, ci, ci, ci, ci, ci, ci,
                                            vp]
    lib.entmax_attn_bwd_noalloc.restype = ci
    lib.ea_mfma_peak_flop.argtypes = [ci, ci]
    lib.ea_mfma_peak_flop.restype = ctypes.c_double
    lib.ea_mfma_peak.argtypes = [vp, ci, ci, vp]
    lib.ea_mfma_peak.restype = ci
    lib.ea_softmax_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.ea_softmax_bwd_workspace_bytes.restype = sz
    lib.softmax_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, vp]
    lib.softmax_attn_fwd.restype = ci
    lib.softmax_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, vp, sz, vp]
    lib.softmax_attn_bwd.restype = ci
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    try:
        return load_library().ea_status_str(int(status)).decode()
    except OSError:
        return {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
                3: "workspace missing or too small", 4: "kernel launch failed",
                5: "problem needs more scratch than the library's static buffer holds"}.get(int(status), "unknown")


def num_blocks(N: int) -> int:
    return (N + BLOCK - 1) // BLOCK


def mask_shape(B: int, H: int, N: int):
    nb = num_blocks(N)
    return (B, H, nb, (nb + 31) // 32)


def mask_words(N: int) -> int:
    return int(load_library().ea_mask_words(int(N)))


def fwd_state_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().ea_fwd_state_bytes(int(B), int(H), int(N), int(d)))


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().ea_bwd_workspace_bytes(int(B), int(H), int(N), int(d)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return EA_BF16
    if t.dtype == torch.float32:
        return EA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check(name: str, t: torch.Tensor, like: Optional[torch.Tensor] = None, strided: bool = False):
    """A GPU tensor; contiguous, or with strided=True any [B, H, N, d] view
    whose last dimension is contiguous (e.g. a transposed [B, N, H, d])."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if strided:
        if t.dim() != 4 or t.stride(-1) != 1 or min(t.stride()) < 0:
            raise ValueError(f"{name} must be a [B, H, N, d] view with a contiguous last dimension")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")
    if like is not None and (t.shape != like.shape or t.dtype != like.dtype or t.device != like.device):
        raise ValueError(f"{name} must match q in shape, dtype and device")


def _check_kv(name: str, t: torch.Tensor, q: torch.Tensor, strided: bool = False) -> int:
    """k and v: like q except for the head count, which divides q's; returns it."""
    _check(name, t, strided=strided)
    if (t.dim() != 4 or t.shape[0] != q.shape[0] or t.shape[2:] != q.shape[2:] or t.dtype != q.dtype
            or t.device != q.device or q.shape[1] % t.shape[1] != 0):
        raise ValueError(f"{name} must be [B, Hkv, N, d] like q, with Hkv dividing q's head count")
    return int(t.shape[1])


def _dense(t: torch.Tensor) -> bool:
    """Whether t's elements fill its storage span exactly (any dimension order)."""
    expect = 1
    for i in sorted(range(t.dim()), key=lambda i: t.stride(i)):
        if t.size(i) == 1:
            continue
        if t.stride(i) != expect:
            return False
        expect *= t.size(i)
    return True


def _strides(t: torch.Tensor) -> "_Strides":
    return _Strides(t.stride(0), t.stride(1), t.stride(2))


def _like(t: torch.Tensor, ref: torch.Tensor) -> torch.Tensor:
    """t in ref's memory layout (a copy only when the strides differ)."""
    if t.stride() == ref.stride():
        return t
    return torch.empty_like(ref).copy_(t)


def _check_state(state: Optional[torch.Tensor]):
    if state is not None and (not isinstance(state, torch.Tensor) or state.device.type != "cuda"
                              or not state.is_contiguous()):
        raise ValueError("state must be the forward's contiguous GPU state tensor")


def _state_args(state: Optional[torch.Tensor]):
    """(pointer, bytes) of the forward's state, or (None, 0)."""
    if state is None:
        return None, 0
    return state.data_ptr(), state.numel() * state.element_size()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: float, causal: bool = False,
        stats: bool = False, out: Optional[tuple] = None, phases: int = FWD_ALL, want_state: bool = False,
        hist_bins: int = HIST_BINS):
    """Forward pass. Returns (o, tau, mask), then, when want_state, the
    forward's state for the backward (an opaque uint8 tensor of
    fwd_state_bytes(B, H, N, d) bytes), then, with
    stats=True, a dict of diagnostics: tau_h [B,H,N], passes [B,H,N] and
    iters [B,H,N] (uint8: the row's streamed refinement passes and its
    solver steps), tiles_per_pass [MAX_PASSES+2], unconverged [1] and
    halves_out [1] and gathered [2] (int32 counters; halves_out counts the
    32x32 sub-tiles holding some p > 0, gathered the rows the output pass
    formed from the rows of V of their support and the sub-tiles whose
    products it ran for the other rows).

    ``mask`` is an int32 tensor [B, H, nb, W] holding the uint32 mask words.
    ``out`` may supply preallocated (o, tau, mask[, state]). ``hist_bins``
    (32 .. 512, a power of two) sets the histogram's bins per unit of z.
    """
    if hist_bins != HIST_BINS:
        lb = int(hist_bins).bit_length() - 1
        if hist_bins != 1 << lb or not 5 <= lb <= 9:
            raise ValueError("hist_bins must be a power of two in 32 .. 512")
        phases |= lb << 8
    lib = load_library()
    _check("q", q, strided=True)
    hkv = _check_kv("k", k, q, strided=True)
    if _check_kv("v", v, q, strided=True) != hkv:
        raise ValueError("k and v must have the same head count")
    if not _dense(q):
        q = q.contiguous()
    if not _dense(k):
        k = k.contiguous()
    v = _like(v, k)
    B, H, N, d = q.shape
    state = None
    if out is None:
        o = torch.empty_like(q)   # q's layout
        tau = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        mask = torch.empty(mask_shape(B, H, N), dtype=torch.int32, device=q.device)
    else:
        o, tau, mask = out[:3]
        if len(out) > 3:
            state = out[3]
    if want_state and state is None:
        state = torch.empty(fwd_state_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    _check_state(state)
    st = None
    st_ptr = None
    if stats:
        st = {
            "tau_h": torch.empty((B, H, N), dtype=torch.float32, device=q.device),
            "passes": torch.empty((B, H, N), dtype=torch.uint8, device=q.device),
            "tiles_per_pass": torch.zeros(MAX_PASSES + 2, dtype=torch.int32, device=q.device),
            "unconverged": torch.zeros(1, dtype=torch.int32, device=q.device),
            "halves_out": torch.zeros(1, dtype=torch.int32, device=q.device),
            "gathered": torch.zeros(2, dtype=torch.int32, device=q.device),
            "iters": torch.zeros((B, H, N), dtype=torch.uint8, device=q.device),
        }
        cs = _Stats(st["tau_h"].data_ptr(), st["passes"].data_ptr(),
                    st["tiles_per_pass"].data_ptr(), st["unconverged"].data_ptr(),
                    st["halves_out"].data_ptr(), st["gathered"].data_ptr(), st["iters"].data_ptr())
        st_ptr = ctypes.byref(cs)
    if o.stride() != q.stride():
        raise ValueError("o must have q's layout")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), tau.data_ptr(), mask.data_ptr(),
            *_state_args(state), float(alpha), int(bool(causal)), B, H, hkv, N, d)
    if q.is_contiguous() and k.is_contiguous():
        status = lib.entmax_attn_fwd_gqa(*args, _dtype_code(q), st_ptr, _stream(q), int(phases))
    else:
        sq, skv = _strides(q), _strides(k)
        status = lib.entmax_attn_fwd_strided(*args, ctypes.byref(sq), ctypes.byref(skv), _dtype_code(q), st_ptr,
                                             _stream(q), int(phases))
    if status != EA_OK:
        raise EntmaxAttnError(status, "entmax_attn_fwd")
    res = (o, tau, mask) + ((state,) if state is not None else ())
    if stats:
        return res + (st,)
    return res


def bwd(q, k, v, dout, tau, mask, alpha: float, causal: bool = False,
        workspace: Optional[torch.Tensor] = None, out: Optional[tuple] = None, phases: int = BWD_ALL,
        state: Optional[torch.Tensor] = None):
    """Backward pass: (dq, dk, dv) for the loss sum(o * dout). ``state`` is
    the forward's state output (optional: without it each row's delta takes
    a sweep of its own and no row is gathered)."""
    lib = load_library()
    _check("q", q, strided=True)
    _check("dout", dout, q, strided=True)
    hkv = _check_kv("k", k, q, strided=True)
    if _check_kv("v", v, q, strided=True) != hkv:
        raise ValueError("k and v must have the same head count")
    if not _dense(q):
        q = q.contiguous()
    if not _dense(k):
        k = k.contiguous()
    v = _like(v, k)
    dout = _like(dout, q)
    B, H, N, d = q.shape
    if tau.dtype != torch.float32 or tuple(tau.shape) != (B, H, N) or not tau.is_contiguous():
        raise ValueError("tau must be a contiguous float32 [B, H, N] tensor")
    if tuple(mask.shape) != mask_shape(B, H, N) or mask.dtype != torch.int32 or not mask.is_contiguous():
        raise ValueError("mask must be the forward's int32 [B, H, nb, W] tensor")
    _check_state(state)
    need = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != k.stride():
        raise ValueError("dq must have q's layout, dk and dv k's")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), tau.data_ptr(), mask.data_ptr(),
            *_state_args(state), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            float(alpha), int(bool(causal)), B, H, hkv, N, d)
    ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q), int(phases))
    if q.is_contiguous() and k.is_contiguous():
        status = lib.entmax_attn_bwd_gqa(*args, _dtype_code(q), *ws)
    else:
        sq, skv = _strides(q), _strides(k)
        status = lib.entmax_attn_bwd_strided(*args, ctypes.byref(sq), ctypes.byref(skv), _dtype_code(q), *ws)
    if status != EA_OK:
        raise EntmaxAttnError(status, "entmax_attn_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, dout, tau, mask, alpha: float, causal: bool = False,
                state: Optional[torch.Tensor] = None, out: Optional[tuple] = None):
    """The backward without a workspace argument (entmax_attn_bwd_noalloc):
    the library's static scratch instead, for dense [B, H, N, d] tensors
    with as many key/value heads as query heads. Calls that overlap on one
    GPU race. Raises EntmaxAttnError (EA_ERR_SCRATCH_LIMIT) when the problem
    needs more than NOALLOC_SCRATCH_BYTES of workspace."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check(name, t, q)
    B, H, N, d = q.shape
    if tau.dtype != torch.float32 or tuple(tau.shape) != (B, H, N) or not tau.is_contiguous():
        raise ValueError("tau must be a contiguous float32 [B, H, N] tensor")
    if tuple(mask.shape) != mask_shape(B, H, N) or mask.dtype != torch.int32 or not mask.is_contiguous():
        raise ValueError("mask must be the forward's int32 [B, H, nb, W] tensor")
    _check_state(state)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3)) if out is None else out
    for t in (dq, dk, dv):
        _check("gradient output", t, q)
    status = lib.entmax_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), tau.data_ptr(),
                                         mask.data_ptr(), *_state_args(state), dq.data_ptr(), dk.data_ptr(),
                                         dv.data_ptr(), float(alpha), int(bool(causal)), B, H, N, d, _dtype_code(q),
                                         _stream(q))
    if status != EA_OK:
        raise EntmaxAttnError(status, "entmax_attn_bwd_noalloc")
    return dq, dk, dv


def mfma_peak(out: torch.Tensor, workgroups: int, iters: int) -> float:
    """Enqueue the achievable-MFMA-rate measurement (ea_mfma_peak) on the
    current stream; out: float32 GPU tensor of at least `workgroups` elements.
    Returns the FLOP of the launch."""
    lib = load_library()
    if out.dtype != torch.float32 or out.device.type != "cuda" or out.numel() < workgroups:
        raise ValueError("out must be a float32 GPU tensor of at least `workgroups` elements")
    status = lib.ea_mfma_peak(out.data_ptr(), int(workgroups), int(iters), _stream(out))
    if status != EA_OK:
        raise EntmaxAttnError(status, "ea_mfma_peak")
    return float(lib.ea_mfma_peak_flop(int(workgroups), int(iters)))


def _cu_array(cu_seqlens):
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    if len(cu) < 2 or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must be non-decreasing offsets starting at 0")
    return cu, (ctypes.c_int * len(cu))(*cu)


def _check_packed(name: str, t: torch.Tensor, total: int, q: Optional[torch.Tensor] = None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous() or t.dim() != 3:
        raise ValueError(f"{name} must be a contiguous GPU tensor [total, heads, d]")
    if t.shape[0] != total or (q is not None and (t.shape[2] != q.shape[2] or t.dtype != q.dtype)):
        raise ValueError(f"{name} must be [cu_seqlens[-1], heads, d] like q")
    return int(t.shape[1])


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens, alpha: float, causal: bool = False,
               stats: bool = False, want_state: bool = False, phases: int = FWD_ALL):
    """Forward over packed variable-length sequences: q [total, H, d], k and v
    [total, Hkv, d], sequence b at tokens cu_seqlens[b] .. cu_seqlens[b+1]
    (host offsets: a list, or a CPU tensor). Returns (o [total, H, d], tau,
    mask) with tau fp32 [H * total] (sequence b's [H, n_b] block at
    H * cu_seqlens[b]) and mask int32 words (the sequences' [H, nb, W]
    blocks in order), then the forward's state (uint8) when want_state,
    then the statistics dict when stats."""
    lib = load_library()
    cu, cu_c = _cu_array(cu_seqlens)
    nseq, total = len(cu) - 1, cu[-1]
    H = _check_packed("q", q, total)
    hkv = _check_packed("k", k, total, q)
    if _check_packed("v", v, total, q) != hkv or H % hkv != 0:
        raise ValueError("k and v need the same head count, dividing q's")
    d = int(q.shape[2])
    o = torch.empty_like(q)
    tau = torch.empty(max(1, H * total), dtype=torch.float32, device=q.device)
    mask = torch.empty(max(1, int(lib.ea_varlen_mask_words(cu_c, nseq, H))), dtype=torch.int32, device=q.device)
    state = (torch.empty(max(16, int(lib.ea_varlen_fwd_state_bytes(cu_c, nseq, H, d))), dtype=torch.uint8,
                         device=q.device) if want_state else None)
    st, st_ptr = None, None
    if stats:
        st = {"tau_h": torch.empty(max(1, H * total), dtype=torch.float32, device=q.device),
              "passes": torch.empty(max(1, H * total), dtype=torch.uint8, device=q.device),
              "tiles_per_pass": torch.zeros(MAX_PASSES + 2, dtype=torch.int32, device=q.device),
              "unconverged": torch.zeros(1, dtype=torch.int32, device=q.device),
              "halves_out": torch.zeros(1, dtype=torch.int32, device=q.device),
              "gathered": torch.zeros(2, dtype=torch.int32, device=q.device),
              "iters": torch.zeros(max(1, H * total), dtype=torch.uint8, device=q.device)}
        cs = _Stats(st["tau_h"].data_ptr(), st["passes"].data_ptr(), st["tiles_per_pass"].data_ptr(),
                    st["unconverged"].data_ptr(), st["halves_out"].data_ptr(), st["gathered"].data_ptr(),
                    st["iters"].data_ptr())
        st_ptr = ctypes.byref(cs)
    status = lib.entmax_attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), tau.data_ptr(),
                                        mask.data_ptr(), *_state_args(state),
                                        float(alpha), int(bool(causal)), cu_c, nseq, H, hkv, d, _dtype_code(q),
                                        st_ptr, _stream(q), int(phases))
    if status != EA_OK:
        raise EntmaxAttnError(status, "entmax_attn_fwd_varlen")
    res = (o, tau, mask) + ((state,) if state is not None else ())
    return res + ((st,) if stats else ())


def bwd_varlen(q, k, v, dout, tau, mask, cu_seqlens, alpha: float, causal: bool = False,
               state: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               phases: int = BWD_ALL):
    """Backward over packed variable-length sequences: (dq, dk, dv) in the
    packed layouts of q, k, v; tau, mask and state from fwd_varlen."""
    lib = load_library()
    cu, cu_c = _cu_array(cu_seqlens)
    nseq, total = len(cu) - 1, cu[-1]
    H = _check_packed("q", q, total)
    _check_packed("dout", dout, total, q)
    hkv = _check_packed("k", k, total, q)
    if _check_packed("v", v, total, q) != hkv or H % hkv != 0 or dout.shape != q.shape:
        raise ValueError("k and v need the same head count, dividing q's; dout is shaped like q")
    d = int(q.shape[2])
    need = int(lib.ea_varlen_bwd_workspace_bytes(cu_c, nseq, H, d))
    if workspace is None:
        workspace = torch.empty(max(256, need), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    status = lib.entmax_attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), tau.data_ptr(),
                                        mask.data_ptr(), *_state_args(state),
                                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), float(alpha),
                                        int(bool(causal)), cu_c, nseq, H, hkv, d, _dtype_code(q),
                                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                        _stream(q), int(phases))
    if status != EA_OK:
        raise EntmaxAttnError(status, "entmax_attn_bwd_varlen")
    return dq, dk, dv


def softmax_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                want_o32: bool = False, out: Optional[tuple] = None):
    """Dense softmax attention (the comparator). Returns (o, lse2) and, with
    want_o32, the fp32 copy of o the backward uses for delta. lse2 is the
    base-2 log-sum-exp of q.k log2(e)/sqrt(d)."""
    lib = load_library()
    _check("q", q)
    _check("k", k, q)
    _check("v", v, q)
    B, H, N, d = q.shape
    o32 = None
    if out is None:
        o = torch.empty_like(q)
        lse2 = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse2 = out[:2]
        if len(out) > 2:
            o32 = out[2]
    if want_o32 and o32 is None:
        o32 = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    status = lib.softmax_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse2.data_ptr(),
                                  o32.data_ptr() if o32 is not None else None, int(bool(causal)), B, H, N, d,
                                  _dtype_code(q), _stream(q))
    if status != EA_OK:
        raise EntmaxAttnError(status, "softmax_attn_fwd")
    return (o, lse2) + ((o32,) if o32 is not None else ())


def softmax_bwd(q, k, v, dout, lse2, causal: bool = False, o32: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, out: Optional[tuple] = None):
    """Backward of the dense softmax comparator: (dq, dk, dv)."""
    lib = load_library()
    _check("q", q)
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        _check(name, t, q)
    B, H, N, d = q.shape
    need = int(lib.ea_softmax_bwd_workspace_bytes(B, H, N, d))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = out
    status = lib.softmax_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), lse2.data_ptr(),
                                  o32.data_ptr() if o32 is not None else None, dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), int(bool(causal)), B, H, N, d, _dtype_code(q),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    if status != EA_OK:
        raise EntmaxAttnError(status, "softmax_attn_bwd")
    return dq, dk, dv


class EntmaxAttention(torch.autograd.Function):
    """Autograd wrapper: saves q, k, v, tau, the block mask and the forward's
    state (fwd_state_bytes: 4 d bytes per query row)."""

    @staticmethod
    def forward(ctx, q, k, v, alpha, causal):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, tau, mask, state = fwd(q, k, v, alpha, causal, want_state=True)
        ctx.save_for_backward(q, k, v, tau, mask, state)
        ctx.alpha, ctx.causal = alpha, causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, tau, mask, state = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, do.contiguous(), tau, mask, ctx.alpha, ctx.causal, state=state)
        return dq, dk, dv, None, None


def entmax_attention(q, k, v, alpha: float = 1.5, causal: bool = False):
    return EntmaxAttention.apply(q, k, v, alpha, causal)


def dense_equiv_flops(B: int, H: int, N: int, d: int, causal: bool):
    """FlashAttention convention: forward 4 B H N^2 d (halved when causal),
    backward 2.5x the forward."""
    f = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
    return f, 2.5 * f


def tile_flops(d: int) -> float:
    """FLOPs of one 64x64 tile product over head dim d."""
    return 2.0 * BLOCK * BLOCK * d



from .module import EntmaxMultiheadAttention  # noqa: E402  (uses entmax_attention above)
