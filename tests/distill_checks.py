"""Row checks of the distillation child against its fp64 oracle, shared by
the GPU parity tests and the CPU tests of the checkers themselves.

Tolerances (derived from the arithmetic):
* the CE part of the loss and of the gradient keeps the fused path's bars
  (loss relative 1e-5; fp32 gradient absolute 1e-6 on the value and on
  value / grad_scale; bf16 gradient 2 ulp);
* KL is assembled from fp32 row statistics whose relative error is ~1e-6, in
  pieces of size up to pT_nt (|lse_z| + |lse_y| + max|y - z|) + |pT_t (NLL_z -
  NLL_y)|; its error is held to 1e-5 |KL| + 4e-6 times that size;
* each gradient element s ((1 + 2 alpha lse + beta) pS - beta pT) carries
  relative error ~1e-6 in each of its two terms: 4e-6 s ((1 + 2 alpha lse +
  beta) pS + beta pT) is added to the element's bar;
* an infinite reference (a -inf student column under a live teacher column
  makes KL +inf) takes no bound: the value must be that same infinity.
"""

from __future__ import annotations

import numpy as np
import torch

from parity_utils import bf16_bound, f32_bound


def _lse(z):
    m = z.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        return (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]


def kl_bound(zs64, zt64, ref):
    """1e-5 |KL| + 4e-6 (|lse_z| + |lse_y| + max|y - z| + NLL) per row, and
    the two logsumexps."""
    ls, lt = _lse(zs64), _lse(zt64)
    with np.errstate(invalid="ignore"):
        w = np.where(np.isfinite(zt64) & np.isfinite(zs64), np.abs(zt64 - zs64), 0.0)
    size = np.abs(ls) + np.abs(lt) + w.max(axis=1) + np.abs(ref["ce"]["nll"])
    return 1e-5 * np.abs(ref["kl"]) + 4e-6 * size, ls, lt


def check_rows(zs64, zt64, t_np, got_loss, got_kl, g, ref, *, alpha, beta, gamma, gdt, what):
    """The tolerances above, row by row, on host copies of the outputs."""
    valid = ref["valid"]
    V = zs64.shape[1]
    live = valid & (t_np >= 0) & (t_np < V)
    kb, ls, lt = kl_bound(zs64, zt64, ref)
    with np.errstate(invalid="ignore", over="ignore"):
        pt = np.exp(zt64 - lt[:, None])
    got_kl, got_loss = got_kl.astype(np.float64), got_loss.astype(np.float64)
    assert np.array_equal(np.isnan(got_kl), np.isnan(ref["kl"])), what + " kl NaN pattern"
    assert np.array_equal(np.isnan(got_loss), np.isnan(ref["loss"])), what + " loss NaN pattern"
    # infinite references: equal, before any bound (an infinite bound holds anything)
    for name, got, rv in (("kl", got_kl, ref["kl"]), ("loss", got_loss, ref["loss"])):
        inf = live & np.isinf(rv)
        assert np.array_equal(got[inf], rv[inf]), (what + f" {name} infinity", got[inf], rv[inf])
        fin = live & np.isfinite(rv)
        assert np.isfinite(got[fin]).all(), what + f" {name}: non-finite where the reference is finite"
    m = live & np.isfinite(ref["kl"]) & np.isfinite(ref["loss"])
    assert np.isfinite(kb[m]).all(), what + " kl bound not finite on a finite row"
    bad = np.abs(got_kl[m] - ref["kl"][m]) > kb[m]
    assert not bad.any(), (what + " kl", got_kl[m][bad][:3], ref["kl"][m][bad][:3])
    lb = 1e-5 * np.abs(ref["loss"][m]) + beta * kb[m]
    bad = np.abs(got_loss[m] - ref["loss"][m]) > lb
    assert not bad.any(), (what + " loss", got_loss[m][bad][:3], ref["loss"][m][bad][:3])
    # ignored rows +0.0 bit for bit
    for x in (got_loss, got_kl):
        assert np.all(x[~valid].astype(np.float32).view(np.int32) == 0), what + " ignored row"
    # gradient
    r = ref["grad"]
    with np.errstate(invalid="ignore", over="ignore"):
        ps = np.exp(zs64 - ls[:, None])
    fac = gamma * ((1 + 2 * alpha * np.abs(ls)[:, None] + beta) * ps + beta * pt)
    fac = np.where(live[:, None], fac, 0.0)
    if gdt == torch.float32:
        gb = f32_bound(r, gamma) + 4e-6 * fac
    else:
        gb = bf16_bound(r) + 4e-6 * fac
    assert np.array_equal(np.isnan(g), np.isnan(r)), what + " grad NaN pattern"
    ginf = np.isinf(r)
    assert np.array_equal(g[ginf], r[ginf]), what + " grad infinity"
    mm = ~np.isnan(r) & ~ginf
    err = np.abs(g[mm] - r[mm])
    bad = err > gb[mm]
    if bad.any():
        i = np.argmax(err / gb[mm])
        raise AssertionError(f"{what} grad: {bad.sum()} off; got {g[mm][i]!r} ref {r[mm][i]!r} "
                             f"bound {gb[mm][i]:.3e}")
