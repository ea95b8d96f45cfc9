"""fp64 CPU oracle for exact relative-position attention (TEST INFRASTRUCTURE).

This package is the slow, plain reference that the GPU library is checked
against.  Only the test-suite, the smoke check and the CPU-baseline leg of the
bench may import it; the library never does, and it imports nothing from the
library.  It shares no code with the GPU path: only the seeded input module
``synth`` feeds both.

Source of the method: "Fast and Exact Relative-Position Attention via
Structure-Aware Kernels" (arXiv 2611.01182), cited below as [RPA].

Every function here follows the plain definition of the result, not the
tiled algorithm: [RPA] proves the tiled forward and backward exact (App. B.2,
the online-softmax lemma and the two exactness theorems), so the oracle
materialises the full N x N score matrix per (batch, head).

Parity pins: see ``tests/test_oracle_*.py``.  The map functions for the T5
and DeBERTa buckets are named but not defined on the pages ([RPA] §5.1
"Mechanisms"); they follow the standard published definitions and are pinned
by exact integer evaluation and structural properties, but against the pages
themselves they are "parity unpinned".
"""

from .maps import t5_bucket, log_bucket, map_rows, relation_rows  # noqa: F401
from .attention import (forward, backward, forward_backward, slice_forward_backward,  # noqa: F401
                        query_rows)
from .bruteforce import brute_forward_backward  # noqa: F401
