"""The parity checkers themselves, on the CPU: each bar must accept the
oracle's own values rounded to the output dtype and must reject the planted
mistakes it exists to catch. A checker that cannot fail proves nothing.

* fp32 gradients at the scale of a 32768-row token mean (the peaked fp32
  workload, grad_scale 1/32768): every non-target element is below 1e-6, so
  the raw absolute 1e-6 bar alone accepts a gradient whose non-target columns
  are all zero; the bars on grad / s_r and on each element's relative error
  must reject it, and a permutation of the columns too. Rows with a margin
  past ~15 have every non-target element below 1e-6 even at unit scale:
  there only the relative bar sees them.
* bf16 gradients: a reference of exactly 0 accepts |g| <= 2^-126, not 0.01.
* distillation: a row whose KL is +inf (a -inf student column under a live
  teacher column) accepts only +inf.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from distill_checks import check_rows
from oracle import ce_oracle, distill_oracle
from parity_utils import GRAD_F32_ABS, bf16_bound, bf16_ulp, check_grad, row_scales
from workloads import WORKLOADS, make_inputs


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


@pytest.fixture(scope="module")
def peaked_rows():
    """Four rows of the peaked fp32 recipe at full width (V = 151936), the
    workload's own grad_scale 1/32768 and z-loss."""
    wl = WORKLOADS["cez_f32_T32768_V151936_peaked"]
    inp = make_inputs(wl.scaled(T=4), device="cpu")
    z = inp["logits"].double().numpy()
    t = inp["targets"].numpy()
    gamma = 1.0 / wl.T
    ref = ce_oracle(z, t, z_alpha=wl.z_alpha, grad_scale=gamma)
    return z, t, gamma, ref


def test_fp32_bar_accepts_rounded_reference(peaked_rows):
    _, _, gamma, ref = peaked_rows
    check_grad(_f32(ref["grad"]), ref["grad"], torch.float32, scale=gamma)


def test_fp32_bar_rejects_zeroed_non_targets(peaked_rows):
    _, t, gamma, ref = peaked_rows
    g = _f32(ref["grad"])
    keep = np.zeros_like(g, dtype=bool)
    keep[np.arange(len(t)), t] = True
    bad = np.where(keep, g, 0.0)
    # the raw bar alone cannot see it: every non-target element is < 1e-6
    assert np.abs(bad - ref["grad"]).max() <= GRAD_F32_ABS
    with pytest.raises(AssertionError):
        check_grad(bad, ref["grad"], torch.float32, scale=gamma)


def test_fp32_scaled_and_relative_bars_each_needed():
    """Two rows of the peaked recipe's width with planted margins 2 and 25:
    zeroing the first row's non-targets fails the grad / s_r bar alone; the
    second row's non-target values are all below 1e-6 even at unit scale, so
    only the relative bar sees them zeroed."""
    rng = np.random.default_rng(5)
    V, gamma = 151936, 1.0 / 32768
    z = rng.standard_normal((2, V)).astype(np.float32).astype(np.float64)
    t = np.array([10, 20])
    for r, margin in enumerate((2.0, 25.0)):
        z[r, t[r]] = z[r].max() + margin
    ref = ce_oracle(z, t, z_alpha=1e-4, grad_scale=gamma)["grad"]
    nt = np.ones_like(ref, dtype=bool)
    nt[[0, 1], t] = False
    assert np.abs(ref[0][nt[0]]).max() / gamma > 1e-5
    assert np.abs(ref[1][nt[1]]).max() / gamma < 1e-6
    bad = np.where(nt, 0.0, _f32(ref))
    with pytest.raises(AssertionError):
        check_grad(bad[:1], ref[:1], torch.float32, scale=gamma, rel=False)
    check_grad(bad[1:], ref[1:], torch.float32, scale=gamma, rel=False)   # blind
    with pytest.raises(AssertionError):
        check_grad(bad[1:], ref[1:], torch.float32, scale=gamma)


def test_fp32_bar_rejects_permuted_columns(peaked_rows):
    _, _, gamma, ref = peaked_rows
    bad = np.roll(_f32(ref["grad"]), 1, axis=1)
    with pytest.raises(AssertionError):
        check_grad(bad, ref["grad"], torch.float32, scale=gamma)


def test_fp32_bar_needs_the_scale(peaked_rows):
    _, _, _, ref = peaked_rows
    with pytest.raises(ValueError):
        check_grad(ref["grad"], ref["grad"], torch.float32)


def test_fp32_bar_at_unit_scale():
    """At s_r = 1 a relative error of 2e-6 on an element near 0.9 fails."""
    z = np.array([[0.0, 2.5, -1.0]])
    ref = ce_oracle(z, np.array([2]), grad_scale=1.0)["grad"]
    check_grad(_f32(ref), ref, torch.float32, scale=1.0)
    bad = ref.copy()
    bad[0, 1] *= 1 + 2e-6
    with pytest.raises(AssertionError):
        check_grad(bad, ref, torch.float32, scale=1.0)


def test_row_scales_follow_segments():
    ids = np.array([0, 0, 0, 1, 2, 2])
    s = row_scales(6, 0.5, ids, 4, segment_mean=True)
    assert np.allclose(s, [0.5 / 3] * 3 + [0.5] + [0.25, 0.25])
    assert np.all(row_scales(6, 0.5) == 0.5)


def test_bf16_zero_reference():
    assert bf16_ulp(0.0) == 2.0 ** -133
    assert bf16_ulp(1.0) == 2.0 ** -7 and bf16_ulp(3.0) == 2.0 ** -6
    ref = np.zeros((2, 3))
    check_grad(np.zeros((2, 3)), ref, torch.bfloat16)
    tiny = np.zeros((2, 3))
    tiny[0, 0] = 2.0 ** -127
    check_grad(tiny, ref, torch.bfloat16)
    for v in (0.01, 2.0 ** -120):
        bad = np.zeros((2, 3))
        bad[1, 2] = v
        with pytest.raises(AssertionError):
            check_grad(bad, ref, torch.bfloat16)
    assert bf16_bound(np.array([0.0]))[0] == 2.0 ** -126


def test_grad_infinity_must_match():
    ref = np.array([[np.inf, 1.0]])
    with pytest.raises(AssertionError):
        check_grad(np.array([[1e30, 1.0]]), ref, torch.bfloat16)


def _distill_case():
    rng = np.random.default_rng(3)
    T, V = 4, 40
    zs = rng.normal(0, 2, (T, V))
    zt = rng.normal(0, 2, (T, V))
    t = np.array([3, 7, 11, 19])
    zs[0, 5] = -np.inf              # student rules out a column the teacher keeps
    ref = distill_oracle(zs, zt, t, z_alpha=1e-4, kl_beta=0.8, grad_scale=0.3)
    return zs, zt, t, ref


def _run(zs, zt, t, ref, loss, kl, g, gdt=torch.float32):
    check_rows(zs, zt, t, loss, kl, g, ref, alpha=1e-4, beta=0.8, gamma=0.3, gdt=gdt,
               what="checker")


def test_distill_rows_accept_rounded_reference():
    zs, zt, t, ref = _distill_case()
    assert np.isposinf(ref["kl"][0]) and np.isfinite(ref["kl"][1:]).all()
    _run(zs, zt, t, ref, _f32(ref["loss"]), _f32(ref["kl"]), _f32(ref["grad"]))


@pytest.mark.parametrize("val", [1e30, 0.0, -np.inf])
def test_distill_rows_reject_finite_kl_for_infinite_reference(val):
    zs, zt, t, ref = _distill_case()
    kl = _f32(ref["kl"])
    kl[0] = val
    with pytest.raises(AssertionError):
        _run(zs, zt, t, ref, _f32(ref["loss"]), kl, _f32(ref["grad"]))


def test_distill_rows_reject_finite_loss_for_infinite_reference():
    zs, zt, t, ref = _distill_case()
    loss = _f32(ref["loss"])
    loss[0] = 12.0
    with pytest.raises(AssertionError):
        _run(zs, zt, t, ref, loss, _f32(ref["kl"]), _f32(ref["grad"]))


def test_distill_fp32_grad_scaled_bar():
    """grad_scale 0.3 with a planted 2e-6 relative error on the largest
    element of a finite row: the raw 1e-6 bar would hold it, the bar on
    grad / s must not."""
    zs, zt, t, ref = _distill_case()
    g = _f32(ref["grad"])
    i = int(np.argmax(np.abs(ref["grad"][1])))
    g[1, i] += 3e-6 * 0.3 * max(1.0, abs(ref["grad"][1, i]) / 0.3)
    with pytest.raises(AssertionError):
        _run(zs, zt, t, ref, _f32(ref["loss"]), _f32(ref["kl"]), g)


def test_entropy_bar():
    """The entropy bar accepts fp32-sized errors where one non-target column
    holds nearly all the mass (H small, p_nt ~ 1) and still rejects a 3e-5
    relative error on a confident row, 1e-4 on an ordinary row and a term
    lost outright."""
    from oracle import row_entropy
    from parity_utils import check_entropy
    rng = np.random.default_rng(0)
    z = rng.normal(0, 4, (6, 12))
    t = np.array([1, 2, 3, 4, 5, 6])
    z[0, 7] = z[0].max() + 9      # a non-target column dominates
    z[1, 2] = z[1].max() + 30     # confident row
    H, lse = row_entropy(z, t)
    check_entropy(H, H, z, t, lse, "exact")
    g = H.copy()
    g[0] += 1e-7                  # the size of the fp32 partials' error
    check_entropy(g, H, z, t, lse, "non-target-dominated row")
    for r, f in ((1, 1 + 3e-5), (0, 1.5), (4, 1 + 1e-4)):
        g = H.copy()
        g[r] *= f
        with pytest.raises(AssertionError):
            check_entropy(g, H, z, t, lse, "planted")
