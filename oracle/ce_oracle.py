"""fp64 reference for the fused vocabulary cross-entropy forward + backward.

Test infrastructure only: the test suite, the smoke check and the CPU-baseline
leg of the benchmark call this module; the GPU library never does.

Sources (the pages this follows):

* torchtitan PR #5661, "fix softmax collapse with improved CE perf".
  - Revised PR description, Numerics paragraph: the loss of a row is
    softplus(logsumexp over the non-target columns minus the target logit); the
    target column is dropped *before* the non-target sum; the target gradient is
    minus the non-target probability; ignored labels yield a finite loss and a
    gradient that the label mask zeroes.
  - Second review, "Example": a row whose target margin over the non-target
    logsumexp is 20 has NLL = softplus(-20), about 2.06e-9, a target gradient of
    about -2.06e-9, and a gradient row that sums to zero.
  - Approving review, "What this PR does": backward rebuilds the softmax, puts
    the target gradient in the target slot and scales the result by the
    incoming gradient.
* Fast-LLM PR #552, "Fuse GSPO into the monolithic compiled loss", PR body
  (What / Approach): z-loss shares the vocabulary softmax with the CE; GSPO's
  seam sums per-token quantities per segment with an index_add over a per-batch
  number of segments.
* xtuner PR #1963, "[FSDP][Loss] Switch gradient reduction to SUM", PR body:
  the z-loss term is scaled by a caller factor (alpha over the batch size), so
  the global token mean is a scale handed in, not a reduction inside the loss.

Readings where the pages are silent (each is listed with its basis in the
design notes of this repository):

* z-loss is ``alpha * lse**2`` per valid row, with ``lse`` the full
  logsumexp (target included); its gradient ``2 * alpha * lse * p_j`` lands on
  every column, the target column included.
* The per-row gradient scale is ``grad_scale``, or ``grad_scale / len(segment)``
  when ``segment_mean`` is set; a segment's length counts every row carrying
  its id, masked rows included.
* The per-segment output is the sum of the NLL (z-loss excluded) over the valid
  rows of the segment. The sum of full token losses is also returned.
* A row is invalid when its target equals ``ignore_index`` or its mask byte is
  0; its loss and whole gradient row are +0.0 and it is left out of segment
  sums. A valid row whose target lies outside ``[0, V)`` is NaN (loss and
  gradient row).

Every quantity is float64; bf16 / fp32 inputs are widened exactly before any
arithmetic.
"""

from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100

_NEG_INF = -np.inf


def softplus(x):
    """softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^-|x|).

    The second form never overflows and keeps full relative accuracy for very
    negative x, where softplus(x) ~ e^x (the collapse regime of the pages'
    margin-20 example).
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """Logistic function 1 / (1 + e^-x), in the branch form that never overflows."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    with np.errstate(over="ignore", invalid="ignore"):
        out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
        ex = np.exp(x[~pos])
        out[~pos] = ex / (1.0 + ex)
    return out


def segment_lengths(segment_ids, num_segments):
    """Number of rows carrying each segment id (masked rows included)."""
    ids = np.asarray(segment_ids, dtype=np.int64)
    return np.bincount(ids, minlength=num_segments)[:num_segments].astype(np.int64)


def _row_block(z, t, valid, z_alpha, scale, want_grad, weight=None):
    """Loss pieces and gradient for one block of rows, all in float64.

    z: [R, V] float64 logits; t: [R] int64 targets; valid: [R] bool;
    scale: [R] float64 per-row gradient scale; weight: [R] weights of the
    NLL term's gradient (None: the scale).
    """
    R, V = z.shape
    in_range = (t >= 0) & (t < V)
    live = valid & in_range          # rows that carry a finite definition
    bad = valid & ~in_range          # rows poisoned with NaN

    rows = np.nonzero(live)[0]
    tl = t[rows]
    zl = z[rows]                     # copy (fancy indexing)
    z_t = zl[np.arange(rows.size), tl]

    # Non-target logsumexp: the target column is removed before the sum
    # (torchtitan #5661, Numerics), so none of the small terms is lost
    # against the target's contribution.
    z_nt = zl.copy()
    z_nt[np.arange(rows.size), tl] = _NEG_INF
    m_nt = z_nt.max(axis=1) if V > 1 else np.full(rows.size, _NEG_INF)
    empty = ~np.isfinite(m_nt) & (m_nt < 0)          # every non-target is -inf
    m_safe = np.where(empty, 0.0, m_nt)
    with np.errstate(divide="ignore"):
        s_nt = np.exp(z_nt - m_safe[:, None]).sum(axis=1)
        lse_nt = np.where(empty, _NEG_INF, m_safe + np.log(s_nt))

    # NLL = softplus(LSE_nt - z_t)  (torchtitan #5661, Numerics).
    x = lse_nt - z_t
    nll = softplus(x)
    # Full logsumexp as the log-add of its two parts; equals z_t + NLL in exact
    # arithmetic but stays defined when z_t = -inf.
    with np.errstate(invalid="ignore"):
        lse = np.maximum(lse_nt, z_t) + np.log1p(np.exp(-np.abs(x)))
    p_nt = sigmoid(x)                # total probability off the target
    p_t = sigmoid(-x)                # target probability

    loss = np.zeros(R, dtype=np.float64)
    nll_all = np.zeros(R, dtype=np.float64)
    lse_all = np.zeros(R, dtype=np.float64)
    loss[rows] = nll + z_alpha * lse * lse
    nll_all[rows] = nll
    lse_all[rows] = lse
    loss[bad] = np.nan
    nll_all[bad] = np.nan
    lse_all[bad] = np.nan

    grad = None
    if want_grad:
        grad = np.zeros((R, V), dtype=np.float64)
        sc = scale[rows]
        w = sc if weight is None else weight[rows]   # weight of the NLL gradient
        zl = sc * 2.0 * z_alpha * lse                # weight of the softmax in the z-loss gradient
        # Non-target columns: softmax probability times the NLL weight plus
        # the z-loss factor.
        with np.errstate(invalid="ignore", over="ignore"):
            p = np.exp(z_nt - lse[:, None])
        g = (w + zl)[:, None] * p
        # Target column: the NLL part is p_t - 1 = -p_nt exactly (torchtitan
        # #5661, Numerics, "target gradient"); the z-loss part is 2 alpha lse p_t.
        g[np.arange(rows.size), tl] = -w * p_nt + zl * p_t
        grad[rows] = g
        grad[bad] = np.nan
    return loss, nll_all, lse_all, grad


def ce_oracle(logits, targets, *, mask=None, segment_ids=None, num_segments=0,
              z_alpha=0.0, grad_scale=1.0, segment_mean=False, row_weight=None,
              ignore_index=IGNORE_INDEX, want_grad=True, block_rows=256):
    """Fused CE (+ z-loss) forward and backward over a [T, V] logit matrix.

    Arguments
    ---------
    logits : array [T, V] (any real dtype; widened to float64 exactly)
    targets : int array [T]; ``ignore_index`` marks an ignored row
    mask : optional uint8/bool array [T]; 0 marks an ignored row
    segment_ids : optional non-decreasing int array [T] with values in
        ``[0, num_segments)``
    z_alpha : z-loss weight alpha
    grad_scale : gamma, the upstream gradient factor (e.g. 1 / n_valid)
    segment_mean : divide row r's gradient scale by the length of its segment
    row_weight : optional [T] weights of each row's NLL gradient, chosen after
        the forward (a GSPO/GRPO-style child sharing the softmax: Fast-LLM
        #552, PR body, Approach); the z-loss gradient keeps the row's scale.
        The loss values do not depend on it.

    Returns a dict with float64 arrays
    ``loss[T]`` (NLL + alpha lse^2, 0 for ignored rows), ``nll[T]``, ``lse[T]``,
    ``valid[T]`` (bool), ``scale[T]``, ``grad[T, V]`` (or None),
    ``seg_nll[S]`` (per-segment NLL sums over valid rows), ``seg_loss[S]``
    (the same with the z-loss term), ``mean`` (sum of valid losses / n_valid,
    0 if none) and ``n_valid``.
    """
    z_all = np.asarray(logits)
    T, V = z_all.shape
    t_all = np.asarray(targets, dtype=np.int64).reshape(T)
    valid = t_all != ignore_index
    if mask is not None:
        valid &= np.asarray(mask).reshape(T) != 0

    scale = np.full(T, float(grad_scale), dtype=np.float64)
    seg = None
    if segment_ids is not None:
        seg = np.asarray(segment_ids, dtype=np.int64).reshape(T)
        if segment_mean:
            lens = segment_lengths(seg, num_segments)
            scale = float(grad_scale) / lens[seg].astype(np.float64)

    loss = np.zeros(T, dtype=np.float64)
    nll = np.zeros(T, dtype=np.float64)
    lse = np.zeros(T, dtype=np.float64)
    grad = np.zeros((T, V), dtype=np.float64) if want_grad else None
    for r0 in range(0, T, block_rows):
        r1 = min(T, r0 + block_rows)
        zb = z_all[r0:r1].astype(np.float64)
        wb = None if row_weight is None else np.asarray(row_weight, dtype=np.float64)[r0:r1]
        lb, nb, eb, gb = _row_block(zb, t_all[r0:r1], valid[r0:r1],
                                    float(z_alpha), scale[r0:r1], want_grad, wb)
        loss[r0:r1] = lb
        nll[r0:r1] = nb
        lse[r0:r1] = eb
        if want_grad:
            grad[r0:r1] = gb

    seg_nll = seg_loss = None
    if seg is not None:
        # index_add over the segment ids (Fast-LLM #552, GSPO seam); invalid
        # rows contribute nothing.
        seg_nll = np.zeros(num_segments, dtype=np.float64)
        seg_loss = np.zeros(num_segments, dtype=np.float64)
        np.add.at(seg_nll, seg[valid], nll[valid])
        np.add.at(seg_loss, seg[valid], loss[valid])

    n_valid = int(valid.sum())
    mean = float(loss[valid].sum() / n_valid) if n_valid else 0.0
    return {
        "loss": loss, "nll": nll, "lse": lse, "valid": valid, "scale": scale,
        "grad": grad, "seg_nll": seg_nll, "seg_loss": seg_loss,
        "mean": mean, "n_valid": n_valid,
    }


def shard_nontarget_lse(z_shard, targets, v0, *, mask=None, ignore_index=IGNORE_INDEX):
    """Per-row statistics of one column shard, in float64.

    A shard holds columns [v0, v0 + V_k) of the vocabulary (torchtitan PR
    #5661, third review, inline diff: each rank reduces over its own columns;
    the rank that owns the target column supplies the target logit).
    Returns ``(lse, zt)``: ``lse[r]`` = log sum of exp over the shard's
    columns other than the row's target (-inf when none is left or the row is
    ignored) and ``zt[r]`` = the target logit if the shard holds the target
    column, else -inf.
    """
    z = np.asarray(z_shard, dtype=np.float64)
    T, Vk = z.shape
    t = np.asarray(targets, dtype=np.int64).reshape(T)
    valid = t != ignore_index
    if mask is not None:
        valid &= np.asarray(mask).reshape(T) != 0
    lse = np.full(T, _NEG_INF)
    zt = np.full(T, _NEG_INF)
    for r in range(T):
        if not valid[r]:
            continue
        row = z[r].copy()
        tl = t[r] - v0
        if 0 <= tl < Vk:
            zt[r] = row[tl]
            row[tl] = _NEG_INF
        m = row.max()
        if np.isfinite(m) or m > 0:
            lse[r] = m + np.log(np.exp(row - m).sum())
    return lse, zt


def row_entropy(logits, targets, *, mask=None, ignore_index=IGNORE_INDEX):
    """Entropy of each row's softmax, H = -sum_j p_j log p_j (0 log 0 = 0), in
    float64; 0 for ignored rows, NaN for valid rows whose target is outside
    [0, V). Callers reuse the logits for such quantities (torchtitan #5661,
    fourth review, inline diff: the input logits are never modified, e.g. for
    entropy). Also returns the full logsumexp per row (0 / NaN likewise).

    The target's term -p_t log p_t = p_t softplus(LSE_nt - z_t) is formed from
    the non-target logsumexp, as the NLL is (revised PR description,
    Numerics): written as p_t (lse - z_t) it rounds to 0 once the target
    dominates, even in float64. The other terms p_j (lse - z_j) are all >= 0.
    """
    z = np.asarray(logits, dtype=np.float64)
    T, V = z.shape
    t = np.asarray(targets, dtype=np.int64).reshape(T)
    valid = t != ignore_index
    if mask is not None:
        valid &= np.asarray(mask).reshape(T) != 0
    H = np.zeros(T)
    lse = np.zeros(T)
    for r in range(T):
        if not valid[r]:
            continue
        if not (0 <= t[r] < V):
            H[r] = lse[r] = np.nan
            continue
        zt = z[r, t[r]]
        z_nt = np.delete(z[r], t[r])
        m = z_nt.max() if z_nt.size else _NEG_INF
        lse_nt = m + np.log(np.exp(z_nt - m).sum()) if np.isfinite(m) else _NEG_INF
        x = lse_nt - zt
        nll = float(softplus(x))
        lse[r] = max(lse_nt, zt) + np.log1p(np.exp(-abs(x)))
        p_t = float(sigmoid(np.array([-x]))[0])
        p = np.exp(z_nt - lse[r])
        with np.errstate(invalid="ignore"):
            terms = np.where(p > 0, p * (lse[r] - z_nt), 0.0)
        H[r] = (p_t * nll if p_t > 0 else 0.0) + terms.sum()
    return H, lse
