"""fp64 reference for a distillation child sharing the student's softmax (test infrastructure).

Test infrastructure only: the test suite, the smoke check and the CPU-baseline
leg of the benchmark call this module; the GPU library never does.

Fast-LLM PR #552 ("Fuse GSPO into the monolithic compiled loss", PR body,
What) lists distillation among the losses that combine with cross-entropy and
z-loss on one vocabulary softmax and finish their loss and gradient in the
same pass. The pages give no formula; the reading taken here is the plainest
one: per valid row, the forward KL divergence from the teacher's softmax to
the student's,

    KL_r = sum_j pT_j (log pT_j - log pS_j),   (0 log 0 = 0)

weighted by ``kl_beta`` and added to the row's loss (CE + z-loss of
``ce_oracle``); its gradient with respect to the student logits is
``kl_beta * scale * (pS - pT)``.

Written from the definitions in float64, with the target column treated as
torchtitan #5661 (revised PR description, Numerics) treats it for the NLL: on
a confident row ``z_t - logsumexp(z)`` rounds to 0 even in float64, so the
target's log-probability is taken as ``-softplus(LSE_nt - z_t)`` (minus the
row's NLL) and its term is ``pT_t (NLL_S - NLL_T)``; the other columns use
``log p_j = z_j - logsumexp(z)``. Likewise the target column's gradient
difference pS_t - pT_t is written as (the teacher's probability off the
target) - (the student's), the same number without forming 1 - 1.
"""

from __future__ import annotations

import numpy as np

from .ce_oracle import IGNORE_INDEX, ce_oracle, sigmoid, softplus


def _log_softmax(z):
    m = z.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    return z - lse


def _nll_and_pt(z, t):
    """Per row: softplus(LSE_nt - z_t) (the NLL, minus log p_t) and
    p_t = sigmoid(z_t - LSE_nt), with LSE_nt the logsumexp of the other
    columns (-inf when they are all -inf)."""
    R = z.shape[0]
    ar = np.arange(R)
    zt = z[ar, t]
    znt = z.copy()
    znt[ar, t] = -np.inf
    m = znt.max(axis=1) if z.shape[1] > 1 else np.full(R, -np.inf)
    fin = np.isfinite(m)
    ms = np.where(fin, m, 0.0)
    with np.errstate(divide="ignore"):
        lse_nt = np.where(fin, ms + np.log(np.exp(znt - ms[:, None]).sum(axis=1)), -np.inf)
    with np.errstate(invalid="ignore"):
        x = lse_nt - zt
    return softplus(x), sigmoid(-x)


def distill_oracle(logits, teacher, targets, *, mask=None, z_alpha=0.0, kl_beta=0.0,
                   grad_scale=1.0, ignore_index=IGNORE_INDEX, want_grad=True):
    """CE + z-loss (``ce_oracle``) plus ``kl_beta`` times the KL divergence
    from the teacher's softmax to the student's, per row, with the gradient
    of ``sum_r scale * loss_r`` with respect to the student logits.

    Returns a dict: ``loss`` [T] (0 ignored, NaN for out-of-range targets),
    ``kl`` [T] (likewise), ``valid`` [T], ``grad`` [T, V] or None, ``ce``
    (the ``ce_oracle`` result).
    """
    zs = np.asarray(logits, dtype=np.float64)
    zt = np.asarray(teacher, dtype=np.float64)
    if zs.shape != zt.shape:
        raise ValueError("student and teacher logits differ in shape")
    T, V = zs.shape
    r = ce_oracle(zs, targets, mask=mask, z_alpha=z_alpha, grad_scale=grad_scale,
                  ignore_index=ignore_index, want_grad=want_grad)
    t = np.asarray(targets, dtype=np.int64).reshape(T)
    valid = r["valid"]
    live = valid & (t >= 0) & (t < V)
    kl = np.zeros(T)
    kl[valid & ~live] = np.nan
    grad = r["grad"]
    rows = np.nonzero(live)[0]
    if rows.size:
        lps = _log_softmax(zs[rows])
        lpt = _log_softmax(zt[rows])
        ps, pt = np.exp(lps), np.exp(lpt)
        ti = t[rows]
        ar = np.arange(rows.size)
        with np.errstate(invalid="ignore"):
            terms = np.where(pt > 0, pt * (lpt - lps), 0.0)
        terms[ar, ti] = 0.0
        # the target column from the non-target logsumexps: pT_t (NLL_S - NLL_T)
        nll_s, _ = _nll_and_pt(zs[rows], ti)
        nll_t, pt_t = _nll_and_pt(zt[rows], ti)
        with np.errstate(invalid="ignore"):
            tgt = np.where(pt_t > 0, pt_t * (nll_s - nll_t), 0.0)
        kl[rows] = terms.sum(axis=1) + tgt
        if want_grad and kl_beta != 0.0:
            d = ps - pt
            # probability off the target column: the other columns' sum
            ps_nt = np.array([np.delete(ps[i], ti[i]).sum() for i in ar])
            pt_nt = np.array([np.delete(pt[i], ti[i]).sum() for i in ar])
            d[ar, ti] = pt_nt - ps_nt
            grad[rows] += (r["scale"][rows] * kl_beta)[:, None] * d
    loss = r["loss"] + kl_beta * np.where(valid, kl, 0.0)
    return {"loss": loss, "kl": kl, "valid": valid, "grad": grad, "ce": r}
