"""Plain fp64 CPU oracle for the fused vocabulary cross-entropy (test infrastructure).

This package is test infrastructure, not product code. Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import or
call it. The GPU library never imports it, links it or falls back to it, and it
shares no code, tables or helpers with the HIP path.

What it computes is written out from the pages' definitions (torchtitan PR #5661
"fix softmax collapse with improved CE perf": the revised PR description's
Numerics paragraph and the second review's margin-20 example; Fast-LLM PR #552
"Fuse GSPO into the monolithic compiled loss": the PR body's What/Approach
paragraphs for z-loss sharing the softmax and per-segment sums) in float64 numpy. ``lmhead_ce`` composes that loss with a linear LM head
(logits = hidden @ weight.T) and writes the chain rule out.
"""

from .ce_oracle import (  # noqa: F401
    IGNORE_INDEX,
    ce_oracle,
    row_entropy,
    segment_lengths,
    shard_nontarget_lse,
    sigmoid,
    softplus,
)
from .distill_oracle import distill_oracle  # noqa: F401
from .lmhead_oracle import lmhead_ce  # noqa: F401
