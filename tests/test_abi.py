"""Host-side checks of the C ABI: the library loads on a machine without a GPU,
exports every function the header declares, sizes its buffers as documented
and rejects bad arguments before any launch (these calls never reach the
device)."""
import ctypes
import os
import re

import pytest

import adaptive_sparse_attention_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "entmax_attn.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ea.LIB_PATH):
        pytest.fail("libentmax_attn.so is not built (run __graft_entry__.build())")
    return ea.load_library()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(ea.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    src = open(HEADER).read()
    consts = dict(re.findall(r"#define (EA_\w+) \(?([0-9 <]+)\)?", src))
    assert int(consts["EA_BLOCK"]) == ea.BLOCK
    assert int(consts["EA_HIST_BINS"]) == ea.HIST_BINS
    assert int(consts["EA_MAX_PASSES"]) == ea.MAX_PASSES
    assert eval(consts["EA_MAX_N"]) == ea.MAX_N


def test_mask_words(lib):
    for N in (1, 63, 64, 65, 2048, 2049, 4096, 16384, 65536, ea.MAX_N):
        nb = (N + 63) // 64
        assert ea.mask_words(N) == nb * ((nb + 31) // 32)
    assert ea.mask_words(0) == 0
    assert ea.mask_words(-5) == 0


def test_workspace_bytes(lib):
    """delta and the key-major mask, then (N <= 65536: 16-bit keys in the
    forward's lists) the gather path's buffers: the tile rows' mask, a flag
    per 64-row block (it holds gathered rows), a byte per row (its list
    length), four arrays of 20 list entries per row, key counts and offsets (one more),
    scan partials per 2048 keys, entry buckets, and the gathered dK / dV
    sums (2 d floats per key)."""
    for (B, H, N, d) in ((1, 1, 1, 64), (2, 12, 4096, 64), (1, 8, 65536, 128), (3, 5, 1000, 128),
                         (1, 2, 65537, 64)):
        r = lambda x: (x + 255) // 256 * 256
        bhn = B * H * N
        want = r(bhn * 4) + r(B * H * ea.mask_words(N) * 4)
        if N <= 65536:
            want += (r(B * H * ea.mask_words(N) * 4) + r(B * H * ((N + 63) // 64) * 4) + r(bhn)
                     + 4 * r(bhn * 20 * 4) + r(bhn * 4) + r((bhn + 1) * 4)
                     + r((bhn + 1 + 2047) // 2048 * 4) + r(bhn * 20 * 4) + r(bhn * 2 * d * 4))
        assert ea.bwd_workspace_bytes(B, H, N, d) == want
    assert ea.bwd_workspace_bytes(1, 1, 64, 96) == 0
    assert ea.bwd_workspace_bytes(0, 1, 64, 64) == 0


def test_status_strings(lib):
    for code in range(6):
        assert isinstance(ea.status_str(code), str) and ea.status_str(code)
    assert ea.status_str(99) == "unknown status"


def _fwd(lib, alpha=1.5, B=1, H=1, N=64, d=64, dtype=0, ptrs=None, state=None, state_bytes=0):
    p = ptrs or [FAKE] * 6
    return lib.entmax_attn_fwd(*p, state, state_bytes, alpha, 0, B, H, N, d, dtype, None, None)


def _bwd(lib, alpha=1.5, B=1, H=1, N=64, d=64, dtype=0, ptrs=None, ws=FAKE, wsb=None, state=None, state_bytes=0):
    p = ptrs or [FAKE] * 9
    wsb = ea.bwd_workspace_bytes(B, H, N, d) if wsb is None else wsb
    return lib.entmax_attn_bwd(*p[:6], state, state_bytes, *p[6:], alpha, 1, B, H, N, d, dtype, ws, wsb, None)


def test_state_bytes(lib):
    """The forward's state: one record of 4 d bytes per query row (vbar, or a
    gathered row's 128-byte support list and its block's mask words, at most
    32 of them where rows are gathered)."""
    assert ea.fwd_state_bytes(2, 3, 100, 64) == 2 * 3 * 100 * 256
    assert ea.fwd_state_bytes(1, 1, 70000, 128) == 70000 * 512
    for bad in ((0, 1, 64, 64), (1, 0, 64, 64), (1, 1, 0, 64), (1, 1, 64, 96)):
        assert ea.fwd_state_bytes(*bad) == 0
    # a gathered row's list and mask words fit its record (N <= 65536)
    nb = (65536 + 63) // 64
    assert 128 + 4 * ((nb + 31) // 32) <= 4 * 64
    import ctypes
    cu = [0, 5, 5, 300]
    arr = (ctypes.c_int * len(cu))(*cu)
    assert lib.ea_varlen_fwd_state_bytes(arr, 3, 2, 64) == 2 * 300 * 256
    assert lib.ea_varlen_fwd_state_bytes((ctypes.c_int * 2)(1, 5), 1, 2, 64) == 0


def test_fwd_validation(lib):
    assert _fwd(lib, alpha=1.0) == ea.EA_ERR_INVALID_ARG
    assert _fwd(lib, alpha=0.5) == ea.EA_ERR_INVALID_ARG
    assert _fwd(lib, alpha=float("nan")) == ea.EA_ERR_INVALID_ARG
    assert _fwd(lib, alpha=float("inf")) == ea.EA_ERR_INVALID_ARG
    assert _fwd(lib, B=0) == ea.EA_ERR_INVALID_ARG
    assert _fwd(lib, H=-1) == ea.EA_ERR_INVALID_ARG
    assert _fwd(lib, N=0) == ea.EA_ERR_INVALID_ARG
    assert _fwd(lib, d=96) == ea.EA_ERR_UNSUPPORTED
    assert _fwd(lib, d=32) == ea.EA_ERR_UNSUPPORTED
    assert _fwd(lib, dtype=7) == ea.EA_ERR_UNSUPPORTED
    assert _fwd(lib, N=ea.MAX_N + 1) == ea.EA_ERR_UNSUPPORTED
    for i in range(6):
        p = [FAKE] * 6
        p[i] = None
        assert _fwd(lib, ptrs=p) == ea.EA_ERR_INVALID_ARG
        # misaligned: q, k, v, o need 16 bytes; tau and the mask words 4
        p[i] = FAKE + (8 if i < 4 else 2)
        assert _fwd(lib, ptrs=p) == ea.EA_ERR_INVALID_ARG
    # the state, when given, is 16-byte aligned and at least ea_fwd_state_bytes
    need = ea.fwd_state_bytes(1, 1, 64, 64)
    assert _fwd(lib, state=FAKE + 4, state_bytes=need) == ea.EA_ERR_INVALID_ARG
    assert _fwd(lib, state=FAKE, state_bytes=need - 1) == ea.EA_ERR_INVALID_ARG


def test_bwd_validation(lib):
    assert _bwd(lib, alpha=1.0) == ea.EA_ERR_INVALID_ARG
    assert _bwd(lib, d=80) == ea.EA_ERR_UNSUPPORTED
    assert _bwd(lib, ws=None) == ea.EA_ERR_WORKSPACE
    assert _bwd(lib, wsb=16) == ea.EA_ERR_WORKSPACE
    assert _bwd(lib, ws=FAKE + 16) == ea.EA_ERR_INVALID_ARG   # workspace must be 256-aligned
    for i in range(9):
        p = [FAKE] * 9
        p[i] = None
        assert _bwd(lib, ptrs=p) == ea.EA_ERR_INVALID_ARG
    need = ea.fwd_state_bytes(1, 1, 64, 64)
    assert _bwd(lib, state=FAKE + 4, state_bytes=need) == ea.EA_ERR_INVALID_ARG
    assert _bwd(lib, state=FAKE, state_bytes=need - 16) == ea.EA_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.fwd(q, q, q, 1.5)


def test_softmax_entry_points_validate(lib):
    """The comparator's entry points check their arguments before any launch."""
    f = lib.softmax_attn_fwd
    ok = [FAKE] * 5
    assert f(*ok, None, 0, 1, 1, 64, 96, 0, None) == ea.EA_ERR_UNSUPPORTED          # d
    assert f(*ok, None, 0, 0, 1, 64, 64, 0, None) == ea.EA_ERR_INVALID_ARG          # B
    assert f(FAKE, FAKE, FAKE, None, FAKE, None, 0, 1, 1, 64, 64, 0, None) == ea.EA_ERR_INVALID_ARG
    assert f(*ok, FAKE + 4, 0, 1, 1, 64, 64, 0, None) == ea.EA_ERR_INVALID_ARG      # o32 alignment
    b = lib.softmax_attn_bwd
    need = lib.ea_softmax_bwd_workspace_bytes(1, 1, 64, 64)
    r = lambda x: (x + 255) // 256 * 256
    assert need == r(64 * 4) + 2 * r(ea.mask_words(64) * 4)   # delta, key-major and row-major masks
    args = [FAKE] * 5 + [None] + [FAKE] * 3
    assert b(*args, 0, 1, 1, 64, 64, 0, None, need, None) == ea.EA_ERR_WORKSPACE
    assert b(*args, 0, 1, 1, 64, 64, 0, FAKE, need - 1, None) == ea.EA_ERR_WORKSPACE
    assert b(*args, 0, 1, 1, 64, 64, 0, FAKE + 16, need, None) == ea.EA_ERR_INVALID_ARG


def test_strided_entry_points_validate(lib):
    """Stride checks run before any launch."""
    import ctypes
    S = ea._Strides
    ok = S(64 * 64, 64 * 64, 64)
    f = lib.entmax_attn_fwd_strided
    base = [FAKE] * 6 + [None, 0, 1.5, 0, 1, 1, 1, 64, 64]
    assert f(*base, None, ctypes.byref(ok), 0, None, None, 15) == ea.EA_ERR_INVALID_ARG
    assert f(*base, ctypes.byref(ok), None, 0, None, None, 15) == ea.EA_ERR_INVALID_ARG
    bad_row = S(64 * 64, 64 * 64, 65)       # rows 130 bytes apart: not 16-byte aligned
    assert f(*base, ctypes.byref(bad_row), ctypes.byref(ok), 0, None, None, 15) == ea.EA_ERR_INVALID_ARG
    neg = S(64 * 64, -64, 64)
    assert f(*base, ctypes.byref(ok), ctypes.byref(neg), 0, None, None, 15) == ea.EA_ERR_INVALID_ARG
    b = lib.entmax_attn_bwd_strided
    bargs = [FAKE] * 6 + [None, 0] + [FAKE] * 3 + [1.5, 0, 1, 1, 1, 64, 64]
    wsb = ea.bwd_workspace_bytes(1, 1, 64, 64)
    assert b(*bargs, ctypes.byref(bad_row), ctypes.byref(ok), 0, FAKE, wsb, None, 7) == ea.EA_ERR_INVALID_ARG
    assert b(*bargs, ctypes.byref(ok), ctypes.byref(ok), 0, None, wsb, None, 7) == ea.EA_ERR_WORKSPACE
    # layouts whose outputs would overlap: rows closer than d, heads or batches
    # that alias (o, dq share q's strides; dk, dv share k's)
    fb = [FAKE] * 6 + [None, 0, 1.5, 0, 2, 2, 2, 64, 64]
    good = S(2 * 64 * 64, 64 * 64, 64)
    for bad in (S(2 * 64 * 64, 64 * 64, 32), S(2 * 64 * 64, 0, 64), S(0, 64 * 64, 64), S(64 * 64, 64 * 64, 64),
                S(2 * 64 * 64, 64 * 32, 64)):
        assert f(*fb, ctypes.byref(bad), ctypes.byref(good), 0, None, None, 15) == ea.EA_ERR_INVALID_ARG
        bb = [FAKE] * 6 + [None, 0] + [FAKE] * 3 + [1.5, 0, 2, 2, 2, 64, 64]
        wsb2 = ea.bwd_workspace_bytes(2, 2, 64, 64)
        assert b(*bb, ctypes.byref(good), ctypes.byref(bad), 0, FAKE, wsb2, None, 7) == ea.EA_ERR_INVALID_ARG
        assert b(*bb, ctypes.byref(bad), ctypes.byref(good), 0, FAKE, wsb2, None, 7) == ea.EA_ERR_INVALID_ARG


def test_varlen_sizes_and_validation(lib):
    import ctypes
    cu = [0, 1, 64, 64, 300, 1300]
    arr = (ctypes.c_int * len(cu))(*cu)
    H, d = 3, 64
    lens = [b - a for a, b in zip(cu, cu[1:])]
    assert lib.ea_varlen_mask_words(arr, len(cu) - 1, H) == H * sum(ea.mask_words(n) for n in lens if n > 0)
    assert lib.ea_varlen_bwd_workspace_bytes(arr, len(cu) - 1, H, d) == max(
        ea.bwd_workspace_bytes(1, H, n, d) for n in lens if n > 0)
    # lengths on both sides of 65536: the shorter sequence (which keeps the
    # gather path's buffers) needs more workspace than the longer one, and
    # the helper covers it; one byte less is rejected before any launch
    mix = (ctypes.c_int * 3)(0, 1000, 71000)
    need = lib.ea_varlen_bwd_workspace_bytes(mix, 2, 8, 64)
    assert ea.bwd_workspace_bytes(1, 8, 1000, 64) > ea.bwd_workspace_bytes(1, 8, 70000, 64)
    assert need == ea.bwd_workspace_bytes(1, 8, 1000, 64)
    margs = [FAKE] * 6 + [None, 0] + [FAKE] * 3 + [1.5, 1, mix, 2, 8, 8, 64, 0]
    assert lib.entmax_attn_bwd_varlen(*margs, FAKE, need - 1, None, 7) == ea.EA_ERR_WORKSPACE
    bad = (ctypes.c_int * 3)(1, 5, 9)          # does not start at 0
    dec = (ctypes.c_int * 3)(0, 9, 5)          # decreasing
    for c in (bad, dec):
        assert lib.ea_varlen_mask_words(c, 2, H) == 0
        assert lib.entmax_attn_fwd_varlen(*([FAKE] * 6), None, 0, 1.5, 0, c, 2, H, H, d, 0, None, None,
                                          15) == ea.EA_ERR_INVALID_ARG
    # every sequence empty: nothing to do, nothing launched
    empty = (ctypes.c_int * 3)(0, 0, 0)
    assert lib.entmax_attn_fwd_varlen(*([FAKE] * 6), None, 0, 1.5, 0, empty, 2, H, H, d, 0, None, None,
                                      15) == ea.EA_OK
    # head counts, workspace
    assert lib.entmax_attn_fwd_varlen(*([FAKE] * 6), None, 0, 1.5, 0, arr, len(cu) - 1, 3, 2, d, 0, None, None,
                                      15) == ea.EA_ERR_INVALID_ARG
    # a state smaller than ea_varlen_fwd_state_bytes
    sneed = lib.ea_varlen_fwd_state_bytes(arr, len(cu) - 1, H, d)
    assert lib.entmax_attn_fwd_varlen(*([FAKE] * 6), FAKE, sneed - 16, 1.5, 0, arr, len(cu) - 1, H, H, d, 0, None,
                                      None, 15) == ea.EA_ERR_INVALID_ARG
    bargs = [FAKE] * 6 + [None, 0] + [FAKE] * 3 + [1.5, 1, arr, len(cu) - 1, H, H, d, 0]
    assert lib.entmax_attn_bwd_varlen(*bargs, FAKE, 16, None, 7) == ea.EA_ERR_WORKSPACE


def test_noalloc_entry_point_validates(lib):
    """The allocation-free backward rejects, before touching the device, bad
    arguments and problems larger than its static scratch."""
    assert lib.ea_noalloc_scratch_bytes() == ea.NOALLOC_SCRATCH_BYTES == 64 << 20
    f = lib.entmax_attn_bwd_noalloc
    p = [FAKE] * 6 + [None, 0] + [FAKE] * 3
    assert f(*p, 1.0, 1, 1, 1, 64, 64, 0, None) == ea.EA_ERR_INVALID_ARG
    assert f(*p, 1.5, 1, 1, 1, 64, 80, 0, None) == ea.EA_ERR_UNSUPPORTED
    # 64 heads of 65536 rows need far more than 64 MiB of workspace
    assert ea.bwd_workspace_bytes(1, 64, 65536, 128) > ea.NOALLOC_SCRATCH_BYTES
    assert f(*p, 1.5, 1, 1, 64, 65536, 128, 0, None) == ea.EA_ERR_SCRATCH_LIMIT
    assert "static buffer" in ea.status_str(ea.EA_ERR_SCRATCH_LIMIT)


def test_mfma_peak_entry_point_validates(lib):
    """The MFMA-rate diagnostic counts 32x32x16 products (2*32*32*16 FLOP
    each) over 8 chains per wave and 4 waves per workgroup, and rejects bad
    arguments before any launch."""
    assert lib.ea_mfma_peak_flop(1, 1) == 2 * 32 * 32 * 16 * 8 * 4
    assert lib.ea_mfma_peak_flop(1024, 4000) == 2 * 32 * 32 * 16 * 8 * 4 * 1024 * 4000
    assert lib.ea_mfma_peak_flop(0, 10) == 0.0
    assert lib.ea_mfma_peak(None, 1, 1, None) == ea.EA_ERR_INVALID_ARG
    assert lib.ea_mfma_peak(FAKE, 0, 1, None) == ea.EA_ERR_INVALID_ARG
    assert lib.ea_mfma_peak(FAKE, 1, 0, None) == ea.EA_ERR_INVALID_ARG
