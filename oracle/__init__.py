"""Plain, slow CPU oracle for exact attention, in float64.

This package is test infrastructure. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the
HIP library and its Python binding) never calls it and never falls back to it.
It shares no code, table or helper with the HIP path.

What it computes is the plain definition of attention,
O = softmax(scale * Q K^T) V, with the per-row log-sum-exp of the scaled scores
as the saved statistic, and the analytic gradients of O. The definition is
the one on the pranaymahendrakar.com lesson "FlashAttention" (Researcher tier,
"The problem being solved", the equation for O). Every function in
``oracle.attention`` says which passage it follows.

``oracle.dropout`` adds dropout on the probabilities (Philox4x32-10 keep
decisions addressed by batch-head, query and key), used by the forward and
backward functions when a positive rate is given.

Parity pins: every function is checked in ``tests/test_oracle.py`` against values
or facts that do not come from the oracle itself (the lesson's worked example,
brute force with scalar loops, closed forms, invariants, finite differences,
PyTorch's own float64 CPU attention, the generator's published known-answer
vectors and the statistics of its keep decisions). No function here is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    MASK_BLOCK,
    visible,
    candidate_keys,
    head_forward,
    head_probabilities,
    head_backward,
    forward,
    backward,
    forward_varlen,
    backward_varlen,
)
from . import dropout  # noqa: F401
from . import fp8  # noqa: F401
