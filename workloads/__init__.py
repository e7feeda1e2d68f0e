"""Seeded synthetic inputs for the fused vocabulary cross-entropy.

Shared by the tests, the smoke check and the benchmark; it holds no arithmetic
of the loss itself (no softmax, logsumexp or gradient), only input construction.
"""

from .ce_inputs import WORKLOADS, Workload, alg_bytes, make_inputs, workload  # noqa: F401
