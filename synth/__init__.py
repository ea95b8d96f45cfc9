"""Seeded synthetic inputs for relative-position attention.

This module only draws random numbers and assembles the input tensors of a
problem (queries, keys, values, output gradient, relation tables and biases).
It holds none of the attention arithmetic: both the fp64 oracle and the GPU
library consume what it returns, and neither is imported here.

Every problem is a plain dict ("spec") plus a dict of float64 numpy arrays
("arrays").  Values are drawn in float64 and rounded once, round-to-nearest-
even, to the problem's dtype; the arrays returned hold the rounded values
(still as float64), so the oracle upcasts exactly what the GPU sees.
"""

from .problems import (  # noqa: F401
    CONFIGS,
    BENCH_SHAPES,
    make_problem,
    make_mixed,
    make_config,
    make_bench,
    round_to_dtype,
    scaled_config,
)
