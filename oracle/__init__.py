"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the CPU-baseline leg of the
benchmark may import anything from this package.  The GPU product path never
calls it: it shares no code, no constants and no helpers with the HIP
kernels, and it imports nothing from the product package.

What is here
------------
recurrence.py    the token-by-token recurrence (the definition the GPU path
                 must reproduce), for the three gates: none (DeltaNet),
                 scalar (Gated DeltaNet) and per-channel (KDA).
closed_forms.py  independent formulations used only to pin the recurrence:
                 brute-force additive linear attention, the unrolled
                 transition-product sum, and the scalar (d_k = 1) recurrence.
chunked.py       a plain fp64 chunkwise (WY / triangular-solve) evaluation,
                 pinned against the recurrence; it checks the block algebra
                 the GPU kernels are built on, never the kernels themselves.
fused.py         the prologue / epilogue activations (q, k normalisation,
                 sigmoid, softplus, GLA's gate, SiLU output gate).
backward.py      reverse-mode gradients of the token recurrence (dq, dk,
                 dv, dbeta, dlog_alpha, dS0), pinned by finite differences.

Every function works in float64 on numpy arrays.  Inputs that arrive in a
lower precision (bf16, fp32) are upcast exactly before any arithmetic.

Parity status: every public function here is pinned by a ``-m "not gpu"``
test against a property the pages or the mathematics fix (see tests/
test_oracle_*.py).  No function is "parity unpinned".
"""

from .recurrence import gated_delta_recurrence, recurrent_step, GATES
from .closed_forms import (
    additive_closed_form,
    unrolled_transition_sum,
    scalar_recurrence_d1,
)
from .chunked import chunked_gated_delta
from . import fused
from .backward import gated_delta_backward

__all__ = [
    "GATES",
    "gated_delta_recurrence",
    "recurrent_step",
    "additive_closed_form",
    "unrolled_transition_sum",
    "scalar_recurrence_d1",
    "chunked_gated_delta",
    "gated_delta_backward",
]
