"""CPU oracle for alpha-entmax attention: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP path never imports, calls or
links it, and it shares no code with the kernels.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms (sparsemax by sort-and-threshold at alpha=2, the
quadratic prefix solution at alpha=1.5, the softmax limit as alpha->1),
brute-force support enumeration on tiny rows, special rows with known
answers, invariants, and central finite differences for the backward.
"""
from .entmax_ref import (  # noqa: F401
    BLOCK, HIST_BINS, TAU_TOL, attn_bwd, attn_fwd, block_sparsity, entmax,
    entmax_row_grad, entmax_tau, histogram_tau, kappa_of, rel_l2, rel_l2_rows,
)
