"""fp64 reference for the vocabulary loss fed by a linear LM head (test infrastructure).

Test infrastructure only: the test suite, the smoke check and the CPU-baseline
leg of the benchmark call this module; the GPU library never does.

The logits of a language model's last layer are ``z = X W^T`` (hidden states
``X`` [T, H] times the head's weight ``W`` [V, H], one row per vocabulary
entry), and the loss of each row is the collapse-free cross-entropy of
``ce_oracle`` (torchtitan PR #5661, revised PR description, Numerics; z-loss
and scales as there). Fast-LLM PR #552 (PR body, the LM-head layer tests)
places the loss directly after this head. The pages do not describe fusing the
head's matrix product into the loss; this reference is the plain composition,
with the chain rule written out:

* ``G = dL/dz`` is the scaled softmax-minus-onehot (plus the z-loss term) of
  ``ce_oracle``;
* ``dL/dX = G W`` and ``dL/dW = G^T X``.

Every product is a float64 numpy matmul of the inputs as given (bf16 values
are exact in float64), so the only rounding is float64's.
"""

from __future__ import annotations

import numpy as np

from .ce_oracle import IGNORE_INDEX, ce_oracle


def lmhead_ce(hidden, weight, targets, *, mask=None, z_alpha=0.0, grad_scale=1.0,
              ignore_index=IGNORE_INDEX, want_grad=True):
    """Loss of ``z = hidden @ weight.T`` per row, and the gradients of
    ``sum_r scale * loss_r`` with respect to ``hidden`` and ``weight``.

    Returns a dict: ``loss`` [T], ``lse`` [T] (0 for ignored rows, NaN for
    out-of-range targets, like the loss), ``valid`` [T], and with
    ``want_grad``: ``grad_logits`` [T, V], ``dhidden`` [T, H],
    ``dweight`` [V, H].
    """
    X = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(weight, dtype=np.float64)
    T, H = X.shape
    V, H2 = W.shape
    if H != H2:
        raise ValueError("hidden and weight disagree on the hidden size")
    z = X @ W.T
    r = ce_oracle(z, targets, mask=mask, z_alpha=z_alpha, grad_scale=grad_scale,
                  ignore_index=ignore_index, want_grad=want_grad)
    out = {"loss": r["loss"], "lse": r["lse"], "valid": r["valid"]}
    if want_grad:
        G = r["grad"]
        out["grad_logits"] = G
        out["dhidden"] = G @ W
        out["dweight"] = G.T @ X
    return out
