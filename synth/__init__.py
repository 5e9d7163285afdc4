"""Seeded synthetic inputs shared by the tests, ``bench.py`` and ``smoke()``.

This package holds none of the method's arithmetic: it only draws inputs
(GEMM operands, completion orders) and names the workloads.  Both the CPU
oracle and the GPU path receive what it produces as plain inputs.
"""

from .inputs import (BASE_SEED, SENTINEL, gemm_operands, shuffled_order,  # noqa: F401
                     round_seed)
from . import workloads  # noqa: F401
