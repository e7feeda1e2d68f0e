"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
the same inputs, compare to the stated tolerances.

Tolerances (fixed by the statement of this path):
* fp32 losses (per row, means, segment sums): relative 1e-5;
* fp32 gradients: absolute 1e-6, and absolute 1e-6 on grad / s_r as well,
  s_r the row's gradient scale (grad_scale, divided by the segment length
  under the segment mean). With s_r = 1/n the raw bar alone would hold
  anything below 1e-6 -- every non-target element of a 32768-row mean -- so
  the second bar holds the softmax-scale values to 1e-6, the unit scale at
  which the pages quote their gradient agreement (torchtitan PR #5661,
  revised PR description: eager and compiled gradients agree to ~1e-6).
  Rows far in the collapse regime (target margin above ~15) have every
  non-target softmax value below 1e-6 even at unit scale, so a third bar,
  derived from the arithmetic, holds each element to relative 2^-16 (plus
  2^-126 for the subnormal range): an element is c_r 2^(z log2 e - k_r),
  whose float exponent argument (|.| < 128) rounds to 2^-18 and whose row
  statistics carry a relative error of a few 1e-6 at most, well inside
  2^-16 = 1.5e-5. It applies to elements formed as one product, not to the
  target column given by ``targets``: with z-loss its value s (-p_nt + 2 alpha
  lse p_t) is a difference whose terms can nearly cancel on confident rows,
  which magnifies the statistics' relative error (the absolute bars still
  hold it), nor where the caller says ``rel=False``;
* bf16 gradients: 2 bf16 ulp of the fp64 reference, where
  ulp_bf16(x) = 2^(max(floor(log2|x|), -126) - 7); below 2^-126 an absolute
  2^-126 is also accepted (fp32/bf16 subnormal range, flush to zero allowed),
  so an exact-0 reference accepts |g| <= 2^-126 and nothing more;
* infinities: equal to the reference (an infinite reference takes no bound);
* ignored rows and segment indexing: bit-exact (+0.0 everywhere).
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import ce_oracle

LOSS_REL = 1e-5
GRAD_F32_ABS = 1e-6
GRAD_F32_REL = 2.0 ** -16
BF16_ULPS = 2.0


def bf16_ulp(x):
    """2^(max(floor(log2|x|), -126) - 7); a zero x takes the floor exponent
    -126 (its ulp is 2^-133), never that of 1."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -126)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def bf16_bound(ref):
    """The bf16 gradient bar: 2 ulp of the reference, at least 2^-126."""
    ref = np.asarray(ref, dtype=np.float64)
    bound = BF16_ULPS * bf16_ulp(ref)
    return np.where(np.abs(ref) < 2.0 ** -126, np.maximum(bound, 2.0 ** -126), bound)


def f32_bound(ref, scale):
    """The fp32 gradient bar: absolute 1e-6 on the value and on value / s_r,
    i.e. 1e-6 * min(1, |s_r|). ``scale``: a scalar or one s_r per row
    (broadcast along the row)."""
    ref = np.asarray(ref, dtype=np.float64)
    sc = np.abs(np.asarray(scale, dtype=np.float64))
    if sc.ndim == 1 and ref.ndim == 2:
        sc = sc[:, None]
    return np.broadcast_to(GRAD_F32_ABS * np.minimum(1.0, sc), ref.shape)


def to_np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_loss(got, ref, what="loss", rel=LOSS_REL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nan_ok = np.isnan(got) == np.isnan(ref)
    assert nan_ok.all(), f"{what}: NaN pattern differs at {np.argwhere(~nan_ok)[:5].ravel()}"
    fin = ~np.isnan(ref)
    inf_ref = np.isinf(ref) & fin
    assert np.array_equal(got[inf_ref], ref[inf_ref]), f"{what}: inf mismatch"
    m = fin & ~inf_ref
    err = np.abs(got[m] - ref[m])
    bound = rel * np.abs(ref[m])
    bad = err > bound
    if bad.any():
        i = np.argmax(err / np.maximum(bound, 1e-300))
        raise AssertionError(f"{what}: {bad.sum()} values off; worst got {got[m][i]!r} "
                             f"ref {ref[m][i]!r} rel {err[i] / max(abs(ref[m][i]), 1e-300):.3e}")


def f32_rel_bound(ref, targets=None):
    """The fp32 relative bar 2^-16 |ref| + 2^-126 (inf where it does not
    apply: the target column of each row when ``targets`` is given)."""
    ref = np.asarray(ref, dtype=np.float64)
    b = GRAD_F32_REL * np.abs(ref) + 2.0 ** -126
    if targets is not None and ref.ndim == 2:
        t = np.asarray(targets).astype(np.int64)
        rows = np.nonzero((t >= 0) & (t < ref.shape[1]))[0]
        b = b.copy()
        b[rows, t[rows]] = np.inf
    return b


def check_grad(got, ref, dtype, what="grad", scale=None, targets=None, rel=True):
    """got: float64 array of the GPU's values; ref: float64 oracle values.
    ``scale`` (required for fp32): each row's gradient scale s_r, a scalar or
    one per row, for the bar on grad / s_r; ``targets`` / ``rel``: where the
    fp32 relative bar applies (see the module notes)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nan_ok = np.isnan(got) == np.isnan(ref)
    assert nan_ok.all(), f"{what}: NaN pattern differs"
    inf_ref = np.isinf(ref)
    assert np.array_equal(got[inf_ref], ref[inf_ref]), f"{what}: infinity mismatch"
    if dtype == torch.float32:
        if scale is None:
            raise ValueError("fp32 gradients need the row scales for the grad / s_r bar")
        full = f32_bound(ref, scale)
        if rel:
            full = np.minimum(full, f32_rel_bound(ref, targets))
    else:
        full = None
    m = ~np.isnan(ref) & ~inf_ref
    assert np.isfinite(got[m]).all(), f"{what}: non-finite value where the reference is finite"
    err = np.abs(got[m] - ref[m])
    bound = full[m] if full is not None else bf16_bound(ref[m])
    bad = err > bound
    if bad.any():
        i = np.argmax(err / np.maximum(bound, 1e-300))
        idx = np.argwhere(m)[i]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} off; worst at {tuple(idx)} "
                             f"got {got[m][i]!r} ref {ref[m][i]!r} bound {bound[i]:.3e}")


def row_scales(T, grad_scale, segment_ids=None, num_segments=0, segment_mean=False):
    """Each row's gradient scale s_r: grad_scale, divided by the number of
    rows that carry the row's segment id under the segment mean."""
    s = np.full(T, float(grad_scale))
    if segment_mean and segment_ids is not None:
        ids = np.asarray(segment_ids).astype(np.int64)
        lens = np.bincount(ids, minlength=num_segments)
        s = s / lens[ids]
    return s


def check_zero_rows(loss_rows, grad_rows):
    """Ignored rows are +0.0 bit for bit."""
    if loss_rows is not None:
        lb = loss_rows.detach().cpu().contiguous().view(torch.int32)
        assert int(lb.abs().max()) == 0 if lb.numel() else True, "ignored loss not +0.0"
    if grad_rows is not None and grad_rows.numel():
        g = grad_rows.detach()
        bits = g.view(torch.int16) if g.dtype == torch.bfloat16 else g.view(torch.int32)
        assert int((bits != 0).sum()) == 0, "ignored gradient row not +0.0"


ROW_ALIGN = 8      # elements: 16 bytes of bf16, 32 of fp32
PAD_GRAD = 5.0     # what the padding columns of a padded gradient must keep


def padded_rows(z, fill=float("nan")):
    """A copy of z as the first V columns of a buffer whose rows are
    ROW_ALIGN elements longer than V rounded up (16-byte aligned rows, so the
    16-byte chunk kernels run even for a ragged V), padding set to ``fill``
    (NaN: a read of the padding would poison the row)."""
    T, V = z.shape
    ld = -(-V // ROW_ALIGN) * ROW_ALIGN + ROW_ALIGN
    big = torch.full((T, ld), fill, dtype=z.dtype, device=z.device)
    big[:, :V] = z
    return big[:, :V]


def run_hip(inp, grad_dtype=None, in_place=False, want_grad=True, mask=None, pad=False):
    """One fused call. ``pad``: logits and gradient as padded rows (the
    logits padding NaN, the gradient padding PAD_GRAD, checked untouched)."""
    import loss_vocab_amd as L
    if not pad:
        return L.ce_fused(inp["logits"], inp["targets"], mask=mask,
                          segment_ids=inp.get("segment_ids"), num_segments=inp.get("num_segments", 0),
                          z_alpha=inp["z_alpha"], grad_scale=inp["grad_scale"],
                          segment_mean=inp.get("segment_mean", False), grad_dtype=grad_dtype,
                          in_place=in_place, want_grad=want_grad)
    z = padded_rows(inp["logits"])
    T, V = z.shape
    S = inp.get("num_segments", 0)
    ids = inp.get("segment_ids")
    loss = torch.empty(T, dtype=torch.float32, device=z.device)
    seg = torch.empty(S, dtype=torch.float32, device=z.device) if ids is not None else None
    if not want_grad:
        grad = None
    elif in_place:
        grad = z
    else:
        grad = padded_rows(torch.empty((T, V), dtype=grad_dtype or z.dtype, device=z.device),
                           fill=PAD_GRAD)
    L.ce_fused_fwd_bwd(z, inp["targets"], mask, ids, inp["z_alpha"], inp["grad_scale"], loss, seg,
                       grad, num_segments=S, segment_mean=inp.get("segment_mean", False))
    if grad is not None:
        rest = grad.as_strided((T, grad.stride(0) - V), (grad.stride(0), 1), grad.storage_offset() + V)
        want = float("nan") if in_place else PAD_GRAD
        assert bool(torch.all(rest.isnan() if in_place else rest == want)), \
            "padding columns of the gradient were written"
    return loss, grad, seg


def run_oracle(logits_cpu64, targets, *, mask=None, segment_ids=None, num_segments=0,
               z_alpha=0.0, grad_scale=1.0, segment_mean=False, want_grad=True):
    return ce_oracle(logits_cpu64, targets, mask=mask, segment_ids=segment_ids,
                     num_segments=num_segments, z_alpha=z_alpha, grad_scale=grad_scale,
                     segment_mean=segment_mean, want_grad=want_grad)


def check_entropy(got, H, z64, t, lse, what):
    """Softmax entropy bar: relative 1e-5 plus 2^-18 p_nt (1 + |lse -
    max_{j != t} z_j|) absolute, the error that the fp32 pass-1 partials
    (relative error below 64 roundings of 2^-24 along a row's accumulation)
    carry into H_nt = ln2 2^(M - L2) ((L2 - M) S - U). It matters only where
    one non-target column holds nearly all the mass; on confident rows
    (H ~ p_nt margin) it is about 2^-18 H."""
    got = np.asarray(got, dtype=np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(H)), f"{what}: NaN pattern differs"
    fin = np.isfinite(H) & np.isfinite(lse)
    assert np.array_equal(got[~fin & ~np.isnan(H)], H[~fin & ~np.isnan(H)]), f"{what}: inf mismatch"
    rows = np.nonzero(fin)[0]
    tt = np.asarray(t).astype(np.int64)[rows]
    zr = z64[rows]
    inr = (tt >= 0) & (tt < z64.shape[1])
    zt = np.where(inr, zr[np.arange(len(rows)), np.clip(tt, 0, z64.shape[1] - 1)], -np.inf)
    znt = zr.copy()
    znt[np.arange(len(rows))[inr], tt[inr]] = -np.inf
    zmax = znt.max(axis=1) if z64.shape[1] > 1 else np.full(len(rows), -np.inf)
    with np.errstate(over="ignore", invalid="ignore"):
        p_nt = np.clip(np.where(np.isfinite(zt), -np.expm1(zt - lse[rows]), 1.0), 0.0, 1.0)
        span = np.where(np.isfinite(zmax), np.abs(lse[rows] - zmax), 0.0)
    tol = 1e-5 * np.abs(H[rows]) + 2.0 ** -18 * p_nt * (1.0 + span)
    err = np.abs(got[rows] - H[rows])
    bad = err > tol
    if bad.any():
        i = np.argmax(err / np.maximum(tol, 1e-300))
        raise AssertionError(f"{what}: {bad.sum()} values off; worst row {rows[i]} got {got[rows][i]!r} "
                             f"ref {H[rows][i]!r} tol {tol[i]:.3e}")
