"""Seeded synthetic inputs for the fused vocabulary cross-entropy.

Shared by the tests, the smoke check and the benchmark; it holds no arithmetic
of the loss itself (no softmax, logsumexp or gradient), only input construction.
"""

from .ce_inputs import (  # noqa: F401
    LMHEAD_WORKLOADS,
    WORKLOADS,
    LmHeadWorkload,
    Workload,
    alg_bytes,
    lmhead_flops,
    make_inputs,
    make_lmhead_inputs,
    workload,
)
