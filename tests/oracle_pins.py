"""Checks that pin the fp64 oracle to facts outside itself.

Each ``pin_*`` function takes an oracle callable with the signature of
``oracle.ce_oracle`` and raises AssertionError when it disagrees with:

* the worked example the pages print (torchtitan PR #5661, second review,
  "Example": margin 20 gives NLL about 2.06e-9, target gradient about
  -2.06e-9, and a row that sums to zero);
* closed forms (uniform logits give NLL = ln V; a single-column row);
* a brute-force evaluation of the textbook definition (log-sum-exp minus the
  target logit, softmax minus one-hot) in 120-digit mpmath arithmetic;
* torch's own fp64 cross_entropy / logsumexp with autograd gradients;
* brute-force Python loops (math.fsum) for masking and segment sums.

The mutation test in ``test_oracle.py`` runs all of them against oracles with a
planted mistake and requires each mutant to fail at least one.
"""

from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
IGNORE = -100


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, rel, abs_=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_nan = np.isnan(a) & np.isnan(b)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    ok = both_nan | same_inf | (np.abs(a - b) <= rel * np.abs(b) + abs_)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: mismatch at {tuple(i)}: {a[tuple(i)]!r} vs {b[tuple(i)]!r}")


# ---------------------------------------------------------------------------
# The pages' worked example and the fp32 collapse margin
# ---------------------------------------------------------------------------

def pin_margin20(fn):
    g = _golden("pages_margin20.json")
    z = np.array([g["logits"]], dtype=np.float64)
    t = np.array([g["target"]])
    out = fn(z, t, z_alpha=0.0, grad_scale=1.0)
    nll = out["loss"][0]
    gt = out["grad"][0, g["target"]]
    tol = 0.5 * 10.0 ** (-(g["printed_significant_digits"] - 1))  # half a unit in the last printed digit
    assert abs(nll - g["nll_approx"]) <= tol * 1e-9, nll
    assert abs(gt - g["target_grad_approx"]) <= tol * 1e-9, gt
    # The row sums to zero: the target gradient balances the non-target one
    # to within fp64 rounding of exp(-20.000000002) (about 20 * 2^-53 relative).
    assert abs(out["grad"][0].sum() - g["row_sum"]) <= 1e-14 * np.abs(out["grad"][0]).sum(), out["grad"][0]
    assert out["grad"][0, 0] > 0


def pin_collapse_is_avoided(fn):
    """Margins past the fp32 (~16.6) and fp64 (~36.7) collapse points keep a
    nonzero loss equal to the 60-digit value."""
    for margin in (16.7, 25.0, 37.5, 60.0, 100.0):
        z = np.array([[0.0, margin, -1.0]])
        out = fn(z, np.array([1]), z_alpha=0.0, grad_scale=1.0)
        mpmath.mp.dps = 60
        lse = mpmath.log(mpmath.exp(0) + mpmath.exp(margin) + mpmath.exp(-1))
        ref = float(lse - margin)
        assert out["loss"][0] > 0
        _close(out["loss"][0], ref, 1e-13, what=f"margin {margin}")
        _close(out["grad"][0, 1], float(mpmath.exp(margin - lse) - 1), 1e-12,
               what=f"target grad margin {margin}")


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def pin_uniform(fn):
    """Constant logits c: NLL = ln V, lse = c + ln V, p_j = 1/V."""
    for V in (1, 2, 7, 4096):
        for c in (0.0, 3.5, -7.25):
            for alpha in (0.0, 1e-4, 0.3):
                gamma = 0.125
                z = np.full((3, V), c)
                t = np.array([0, V - 1, V // 2])
                out = fn(z, t, z_alpha=alpha, grad_scale=gamma)
                lnV = math.log(V)
                lse = c + lnV
                _close(out["nll"], np.full(3, lnV), 1e-13, 1e-15, "uniform nll")
                _close(out["lse"], np.full(3, lse), 1e-13, 1e-15, "uniform lse")
                _close(out["loss"], np.full(3, lnV + alpha * lse * lse), 1e-13, 1e-15, "uniform loss")
                g = out["grad"]
                for r in range(3):
                    exp_t = gamma * (1.0 / V - 1.0 + 2.0 * alpha * lse / V)
                    exp_j = gamma * (1.0 + 2.0 * alpha * lse) / V
                    ref = np.full(V, exp_j)
                    ref[t[r]] = exp_t
                    _close(g[r], ref, 1e-12, 1e-17, f"uniform grad V={V} c={c} a={alpha}")


def pin_single_column_and_infinities(fn):
    """V = 1: the non-target set is empty, so NLL = 0, lse = z_t and the only
    gradient is the z-loss term. A -inf target logit: NLL = +inf, target
    gradient -gamma."""
    alpha, gamma = 0.01, 0.5
    z = np.array([[2.5]])
    out = fn(z, np.array([0]), z_alpha=alpha, grad_scale=gamma)
    assert out["nll"][0] == 0.0
    _close(out["lse"][0], 2.5, 0, 0, "V=1 lse")
    _close(out["grad"][0, 0], gamma * 2 * alpha * 2.5, 1e-15, 0, "V=1 grad")
    # Every non-target at -inf behaves like V = 1.
    z = np.array([[-np.inf, 1.0, -np.inf]])
    out = fn(z, np.array([1]), z_alpha=alpha, grad_scale=gamma)
    assert out["nll"][0] == 0.0
    assert out["grad"][0, 0] == 0.0 and out["grad"][0, 2] == 0.0
    _close(out["grad"][0, 1], gamma * 2 * alpha * 1.0, 1e-15, 0, "all -inf grad")
    # -inf target logit.
    z = np.array([[0.0, -np.inf, math.log(3.0)]])
    out = fn(z, np.array([1]), z_alpha=0.0, grad_scale=gamma)
    assert out["nll"][0] == np.inf
    _close(out["lse"][0], math.log(4.0), 1e-15, 0, "-inf target lse")
    _close(out["grad"][0], [gamma * 0.25, -gamma, gamma * 0.75], 1e-14, 0, "-inf target grad")


# ---------------------------------------------------------------------------
# Brute force with the textbook definition in 120-digit arithmetic
# ---------------------------------------------------------------------------

def _mp_row(z, t, alpha, scale):
    mpmath.mp.dps = 120
    zs = [mpmath.mpf(float(v)) if np.isfinite(v) else mpmath.mpf("-inf") for v in z]
    terms = [mpmath.exp(v) for v in zs]
    lse = mpmath.log(mpmath.fsum(terms))
    nll = lse - zs[t]
    loss = nll + alpha * lse * lse
    p = [mpmath.exp(v - lse) for v in zs]
    grad = [scale * ((1 + 2 * alpha * lse) * p[j] - (1 if j == t else 0)) for j in range(len(z))]
    return float(loss), float(nll), float(lse), [float(g) for g in grad]


def pin_mpmath_bruteforce(fn):
    rng = np.random.default_rng(1234)
    for V in (1, 2, 3, 5, 8):
        for case in range(6):
            T = 4
            z = rng.normal(0.0, 3.0, size=(T, V))
            t = rng.integers(0, V, size=T)
            if case >= 2:
                # confident rows: target margins up to 100
                z[np.arange(T), t] = z.max(axis=1) + rng.uniform(0, 100, size=T)
            if case >= 4 and V > 2:
                # -inf entries away from the target
                for r in range(T):
                    j = (t[r] + 1) % V
                    z[r, j] = -np.inf
            alpha = [0.0, 1e-4, 0.05][case % 3]
            gamma = [1.0, 0.25, 1.0 / 3.0][case % 3]
            out = fn(z, t, z_alpha=alpha, grad_scale=gamma)
            for r in range(T):
                loss, nll, lse, grad = _mp_row(z[r], int(t[r]), alpha, gamma)
                # absolute floor 1e-100: the 120-digit reference of lse - z_t
                # carries ~1e-118 of rounding; the smallest NLL here is ~e^-100.
                _close(out["loss"][r], loss, 1e-12, 1e-100, f"mp loss V={V} case={case}")
                _close(out["nll"][r], nll, 1e-12, 1e-100, f"mp nll V={V} case={case}")
                _close(out["lse"][r], lse, 1e-13, 1e-300, f"mp lse V={V} case={case}")
                # Gradients: relative to each element, except where the exact
                # value sits below the cancellation floor of scale * 1e-16.
                _close(out["grad"][r], grad, 1e-11, gamma * 1e-16 * (1 + 2 * alpha * abs(lse)),
                       f"mp grad V={V} case={case}")


# ---------------------------------------------------------------------------
# A library routine: torch fp64 cross_entropy + logsumexp with autograd
# ---------------------------------------------------------------------------

def pin_torch_library(fn):
    g = torch.Generator().manual_seed(7)
    T, V = 24, 50
    z = torch.randn(T, V, generator=g, dtype=torch.float64) * 3.0
    t = torch.randint(0, V, (T,), generator=g)
    t[3] = IGNORE
    t[11] = IGNORE
    valid = t != IGNORE
    alpha = 1e-3
    gamma = 1.0 / int(valid.sum())
    zr = z.clone().requires_grad_(True)
    ce = torch.nn.functional.cross_entropy(zr, t, reduction="none", ignore_index=IGNORE)
    zl = alpha * torch.logsumexp(zr, dim=1) ** 2 * valid
    per_row = ce + zl
    (gamma * per_row.sum()).backward()
    out = fn(z.numpy(), t.numpy(), z_alpha=alpha, grad_scale=gamma)
    _close(out["loss"], per_row.detach().numpy(), 1e-12, 1e-15, "torch loss")
    _close(out["grad"], zr.grad.numpy(), 1e-10, 1e-18, "torch grad")
    _close(out["mean"], float(per_row.detach().sum() / valid.sum()), 1e-12, 0, "torch mean")


def pin_row_weights(fn):
    """Per-row NLL weights chosen after the forward: torch fp64 autograd of
    sum_r w_r CE_r + gamma alpha lse_r^2 (the z-loss keeps the uniform scale)."""
    g = torch.Generator().manual_seed(21)
    T, V = 10, 33
    z = torch.randn(T, V, generator=g, dtype=torch.float64) * 2.0
    t = torch.randint(0, V, (T,), generator=g)
    t[4] = IGNORE
    w = torch.randn(T, generator=g, dtype=torch.float64)
    alpha, gamma = 5e-3, 0.3
    valid = (t != IGNORE).double()
    zr = z.clone().requires_grad_(True)
    ce = torch.nn.functional.cross_entropy(zr, t, reduction="none", ignore_index=IGNORE)
    total = (w * ce).sum() + gamma * (alpha * torch.logsumexp(zr, dim=1) ** 2 * valid).sum()
    total.backward()
    out = fn(z.numpy(), t.numpy(), z_alpha=alpha, grad_scale=gamma, row_weight=w.numpy())
    _close(out["grad"], zr.grad.numpy(), 1e-10, 1e-18, "row-weight grad")
    plain = fn(z.numpy(), t.numpy(), z_alpha=alpha, grad_scale=gamma)
    assert np.array_equal(out["loss"], plain["loss"])


# ---------------------------------------------------------------------------
# Invariants, masking, segments
# ---------------------------------------------------------------------------

def pin_row_sums(fn):
    """Sum_j g_rj = scale * 2 alpha lse (zero without z-loss): torchtitan #5661
    second review, the row sums to zero; with z-loss the softmax sums to one."""
    rng = np.random.default_rng(99)
    T, V = 16, 300
    z = rng.normal(0, 2.0, size=(T, V))
    t = rng.integers(0, V, size=T)
    z[:4, :] += 0.0
    z[np.arange(4), t[:4]] = z[:4].max(axis=1) + 30.0
    for alpha in (0.0, 1e-4, 0.1):
        out = fn(z, t, z_alpha=alpha, grad_scale=0.5)
        s = out["grad"].sum(axis=1)
        bound = 1e-14 * np.abs(out["grad"]).sum(axis=1) + 1e-300
        expect = 0.5 * 2 * alpha * out["lse"]
        assert np.all(np.abs(s - expect) <= bound + 1e-15 * np.abs(expect)), (alpha, s - expect)


def pin_masking(fn):
    rng = np.random.default_rng(5)
    T, V = 12, 40
    z = rng.normal(0, 1.0, size=(T, V))
    t = rng.integers(0, V, size=T)
    t[[1, 7]] = IGNORE
    mask = np.ones(T, dtype=np.uint8)
    mask[[2, 9]] = 0
    # garbage in ignored rows must not matter
    z[1, :] = np.nan
    z[2, :] = -np.inf
    z[9, 5] = np.inf
    out = fn(z, t, mask=mask, z_alpha=1e-3, grad_scale=1.0 / 8)
    bad = [1, 2, 7, 9]
    for r in bad:
        assert out["loss"][r] == 0.0 and not np.signbit(out["loss"][r])
        assert np.all(out["grad"][r] == 0.0) and not np.any(np.signbit(out["grad"][r]))
    assert not out["valid"][bad].any() and out["valid"].sum() == T - 4
    good = [r for r in range(T) if r not in bad]
    assert np.all(np.isfinite(out["loss"][good])) and np.all(np.isfinite(out["grad"][good]))
    # each valid row equals the same row evaluated alone
    for r in good:
        one = fn(z[r:r + 1], t[r:r + 1], z_alpha=1e-3, grad_scale=1.0 / 8)
        assert out["loss"][r] == one["loss"][0]
        assert np.array_equal(out["grad"][r], one["grad"][0])
    _close(out["mean"], math.fsum(out["loss"][good]) / len(good), 1e-14, 0, "mean")


def pin_out_of_range_target(fn):
    z = np.zeros((3, 5))
    out = fn(z, np.array([5, -3, 2]), z_alpha=0.0, grad_scale=1.0)
    assert np.isnan(out["loss"][0]) and np.isnan(out["loss"][1])
    assert np.all(np.isnan(out["grad"][0])) and np.all(np.isnan(out["grad"][1]))
    assert np.isfinite(out["loss"][2])


def pin_segments(fn):
    rng = np.random.default_rng(11)
    T, V, S = 40, 17, 6
    lens = [1, 9, 4, 0, 14, 12]          # segment 3 is empty
    seg = np.repeat(np.arange(S), lens)
    assert seg.size == T
    z = rng.normal(0, 2.0, size=(T, V))
    t = rng.integers(0, V, size=T)
    t[[0, 5, 6, 20]] = IGNORE             # segment 0 is fully ignored
    alpha, gamma = 1e-2, 2.0
    out = fn(z, t, segment_ids=seg, num_segments=S, z_alpha=alpha, grad_scale=gamma,
             segment_mean=True)
    plain = fn(z, t, z_alpha=alpha, grad_scale=1.0)
    # brute force: per-segment sums with math.fsum over valid rows
    for s in range(S):
        rows = [r for r in range(T) if seg[r] == s and t[r] != IGNORE]
        ref_nll = math.fsum(plain["nll"][r] for r in rows)
        ref_loss = math.fsum(plain["loss"][r] for r in rows)
        _close(out["seg_nll"][s], ref_nll, 1e-13, 0, f"seg nll {s}")
        _close(out["seg_loss"][s], ref_loss, 1e-13, 0, f"seg loss {s}")
    assert out["seg_nll"][0] == 0.0 and out["seg_nll"][3] == 0.0
    # gradient scale: gamma / (number of rows carrying the id, ignored ones included)
    for r in range(T):
        n = sum(1 for q in range(T) if seg[q] == seg[r])
        _close(out["grad"][r], plain["grad"][r] * (gamma / n), 1e-15, 0, f"seg scale row {r}")


def pin_shard_nontarget_lse(shard_fn):
    """Per-shard non-target logsumexp against 120-digit brute force, and the
    closed form of a uniform shard."""
    mpmath.mp.dps = 120
    rng = np.random.default_rng(8)
    z = rng.normal(0, 3.0, size=(6, 7))
    z[2, 3] = 60.0
    z[4, :] = -np.inf
    z[4, 5] = 1.0
    t = np.array([10, 13, 13, 5, 15, -100])   # shard holds columns [10, 17)
    lse, zt = shard_fn(z, t, 10)
    for r in range(6):
        if t[r] == -100:
            assert lse[r] == -np.inf and zt[r] == -np.inf
            continue
        tl = t[r] - 10
        cols = [j for j in range(7) if j != tl]
        terms = [mpmath.exp(mpmath.mpf(float(z[r, j]))) for j in cols if np.isfinite(z[r, j])]
        ref = float(mpmath.log(mpmath.fsum(terms))) if terms else -np.inf
        _close(lse[r], ref, 1e-14, 0, f"shard lse row {r}")
        if 0 <= tl < 7:
            assert zt[r] == z[r, tl]
        else:
            assert zt[r] == -np.inf
    # uniform shard of width 9 holding the target: lse = c + ln 8
    lse, zt = shard_fn(np.full((1, 9), 2.5), np.array([4]), 0)
    _close(lse[0], 2.5 + math.log(8.0), 1e-15, 0, "uniform shard")
    assert zt[0] == 2.5


def pin_row_entropy(ent_fn):
    """Entropy: uniform rows give ln V, a single finite column gives 0, and
    random rows match 120-digit brute force of -sum p log p."""
    H, lse = ent_fn(np.full((2, 7), 1.5), np.array([0, 6]))
    _close(H, [math.log(7)] * 2, 1e-14, 0, "uniform entropy")
    _close(lse, [1.5 + math.log(7)] * 2, 1e-14, 0, "uniform lse")
    z = np.full((1, 5), -np.inf)
    z[0, 2] = 3.0
    H, lse = ent_fn(z, np.array([2]))
    assert H[0] == 0.0 and lse[0] == 3.0
    rng = np.random.default_rng(4)
    z = rng.normal(0, 3, size=(4, 6))
    z[1, 2] = 80.0           # confident row: entropy ~ 1e-33
    H, _ = ent_fn(z, np.array([0, 2, 5, 1]))
    mpmath.mp.dps = 120
    for r in range(4):
        zs = [mpmath.mpf(float(v)) for v in z[r]]
        lse_r = mpmath.log(mpmath.fsum([mpmath.exp(v) for v in zs]))
        ref = -mpmath.fsum([mpmath.exp(v - lse_r) * (v - lse_r) for v in zs])
        _close(H[r], float(ref), 1e-10, 1e-300, f"entropy row {r}")
    H, _ = ent_fn(np.zeros((3, 4)), np.array([-100, 9, 1]))
    assert H[0] == 0.0 and np.isnan(H[1]) and H[2] > 0


def pin_lmhead(lm_fn):
    """Loss behind a linear head: torch fp64 autograd of F.linear followed by
    cross-entropy + z-loss gives the loss, dX and dW; a zero weight gives the
    uniform closed form (loss ln V, dX = 0, dW = G^T X with G written out)."""
    g = torch.Generator().manual_seed(33)
    T, H, V = 12, 20, 37
    X = torch.randn(T, H, generator=g, dtype=torch.float64)
    W = torch.randn(V, H, generator=g, dtype=torch.float64) * 0.5
    t = torch.randint(0, V, (T,), generator=g)
    t[5] = IGNORE
    alpha, gamma = 2e-3, 0.125
    valid = (t != IGNORE).double()
    Xr = X.clone().requires_grad_(True)
    Wr = W.clone().requires_grad_(True)
    z = torch.nn.functional.linear(Xr, Wr)
    ce = torch.nn.functional.cross_entropy(z, t, reduction="none", ignore_index=IGNORE)
    lse = torch.logsumexp(z, dim=1)
    per_row = ce + alpha * lse ** 2 * valid
    (gamma * per_row.sum()).backward()
    out = lm_fn(X.numpy(), W.numpy(), t.numpy(), z_alpha=alpha, grad_scale=gamma)
    _close(out["loss"], per_row.detach().numpy(), 1e-12, 1e-15, "lm-head loss")
    _close(out["lse"], (lse * valid).detach().numpy(), 1e-13, 1e-15, "lm-head lse")
    _close(out["dhidden"], Xr.grad.numpy(), 1e-10, 1e-16, "lm-head dX")
    _close(out["dweight"], Wr.grad.numpy(), 1e-10, 1e-16, "lm-head dW")
    # zero head: every logit 0, softmax uniform
    Wz = np.zeros((V, H))
    out = lm_fn(X.numpy(), Wz, t.numpy(), z_alpha=alpha, grad_scale=gamma)
    v = valid.numpy().astype(bool)
    _close(out["loss"][v], np.full(v.sum(), math.log(V) + alpha * math.log(V) ** 2), 1e-13, 0,
           "zero-head loss")
    assert np.all(out["dhidden"] == 0)
    Gz = np.zeros((T, V))
    Gz[v] = gamma * (1.0 + 2 * alpha * math.log(V)) / V
    Gz[np.nonzero(v)[0], t.numpy()[v]] -= gamma
    _close(out["dweight"], Gz.T @ X.numpy(), 1e-12, 1e-15, "zero-head dW")


def pin_distill(fn):
    """Distillation child: teacher = student gives KL 0 and the CE values
    exactly; kl_beta = 0 gives the CE values exactly; torch fp64 autograd of
    CE + z-loss + beta KL (F.kl_div with log targets); 120-digit brute force
    of KL including confident rows and -inf entries; the uniform-teacher
    closed form KL = -log V - mean_j log pS_j; ignored rows 0, out-of-range
    targets NaN."""
    from oracle import ce_oracle
    rng = np.random.default_rng(41)
    T, V = 9, 23
    zs = rng.normal(0, 2.5, size=(T, V))
    zt = rng.normal(0, 2.0, size=(T, V))
    t = rng.integers(0, V, size=T)
    t[4] = IGNORE
    ce = ce_oracle(zs, t, z_alpha=1e-3, grad_scale=0.2)
    same = fn(zs, zs, t, z_alpha=1e-3, kl_beta=0.7, grad_scale=0.2)
    assert np.all(same["kl"] == 0.0)
    assert np.array_equal(same["grad"], ce["grad"]) and np.array_equal(same["loss"], ce["loss"])
    nob = fn(zs, zt, t, z_alpha=1e-3, kl_beta=0.0, grad_scale=0.2)
    assert np.array_equal(nob["grad"], ce["grad"]) and np.array_equal(nob["loss"], ce["loss"])
    # torch fp64 autograd
    alpha, beta, gamma = 2e-3, 0.6, 0.25
    tt = torch.as_tensor(t)
    valid = (tt != IGNORE).double()
    zr = torch.tensor(zs, dtype=torch.float64, requires_grad=True)
    ztt = torch.tensor(zt, dtype=torch.float64)
    cel = torch.nn.functional.cross_entropy(zr, tt, reduction="none", ignore_index=IGNORE)
    klr = torch.nn.functional.kl_div(torch.log_softmax(zr, 1), torch.log_softmax(ztt, 1),
                                     reduction="none", log_target=True).sum(1)
    per_row = cel + (alpha * torch.logsumexp(zr, 1) ** 2 + beta * klr) * valid
    (gamma * per_row.sum()).backward()
    out = fn(zs, zt, t, z_alpha=alpha, kl_beta=beta, grad_scale=gamma)
    _close(out["loss"], per_row.detach().numpy(), 1e-12, 1e-15, "distill loss")
    _close(out["kl"] * valid.numpy(), (klr * valid).detach().numpy(), 1e-12, 1e-15, "distill kl")
    _close(out["grad"], zr.grad.numpy(), 1e-10, 1e-18, "distill grad")
    # 120-digit brute force
    mpmath.mp.dps = 120
    zs2 = rng.normal(0, 3, size=(4, 5))
    zt2 = rng.normal(0, 3, size=(4, 5))
    t2 = np.array([0, 3, 4, 2])
    zs2[1, 3] = 60.0                 # confident student
    zt2[1, 3] = 55.0                 # confident teacher
    zt2[2, 0] = -np.inf              # a column the teacher rules out
    out = fn(zs2, zt2, t2, kl_beta=1.0)
    for r in range(4):
        a = [mpmath.mpf(float(v)) for v in zs2[r]]
        b = [mpmath.mpf(float(v)) if np.isfinite(v) else None for v in zt2[r]]
        la = mpmath.log(mpmath.fsum([mpmath.exp(v) for v in a]))
        lb = mpmath.log(mpmath.fsum([mpmath.exp(v) for v in b if v is not None]))
        ref = mpmath.fsum([mpmath.exp(bj - lb) * ((bj - lb) - (aj - la))
                           for aj, bj in zip(a, b) if bj is not None])
        _close(out["kl"][r], float(ref), 1e-9, 1e-300, f"distill kl row {r}")
    # uniform teacher
    out = fn(zs, np.zeros((T, V)), t, kl_beta=1.0)
    lps = zs - (zs.max(1, keepdims=True) + np.log(np.exp(zs - zs.max(1, keepdims=True)).sum(1,
                                                                                 keepdims=True)))
    ref = -np.log(V) - lps.mean(axis=1)
    v = t != IGNORE
    _close(out["kl"][v], ref[v], 1e-12, 1e-15, "uniform-teacher kl")
    # ignored / out of range
    out = fn(zs[:3], zt[:3], np.array([IGNORE, V + 1, 0]), kl_beta=0.5)
    assert out["kl"][0] == 0.0 and out["loss"][0] == 0.0
    assert np.isnan(out["kl"][1]) and np.isnan(out["loss"][1])
    assert np.all(np.isnan(out["grad"][1])) and np.all(out["grad"][0] == 0.0)


ALL_PINS = [
    pin_margin20,
    pin_collapse_is_avoided,
    pin_uniform,
    pin_single_column_and_infinities,
    pin_mpmath_bruteforce,
    pin_torch_library,
    pin_row_weights,
    pin_row_sums,
    pin_masking,
    pin_out_of_range_target,
    pin_segments,
]
