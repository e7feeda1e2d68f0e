"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ce_oracle

from oracle_pins import ALL_PINS, GOLDEN, pin_row_entropy, pin_shard_nontarget_lse

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ce_oracle)


def test_pin_shard_nontarget_lse():
    pin_shard_nontarget_lse(oracle.shard_nontarget_lse)


def test_pin_row_entropy():
    pin_row_entropy(oracle.row_entropy)


def test_shard_lses_merge_to_the_row():
    """Merging the shards' non-target logsumexps with the owner's target logit
    (log-add) gives the full row's lse of the oracle."""
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2.0, size=(5, 50))
    t = rng.integers(0, 50, size=5)
    full = ce_oracle(z, t)
    parts = [oracle.shard_nontarget_lse(z[:, a:b], t, a) for a, b in [(0, 16), (16, 40), (40, 50)]]
    lse_nt = np.logaddexp.reduce(np.stack([p[0] for p in parts]), axis=0)
    zt = np.max(np.stack([p[1] for p in parts]), axis=0)
    assert np.allclose(np.logaddexp(lse_nt, zt), full["lse"], rtol=1e-14, atol=0)
    assert np.array_equal(zt, z[np.arange(5), t])


def test_naive_fp32_collapses_where_the_pages_say():
    """Negative control for the pages' claim (torchtitan #5661, loss docstring):
    the naive fp32 loss logsumexp(z) - z_t rounds to exactly 0 past a margin of
    about 16.6, and the target gradient p_t - 1 with it, while the oracle keeps
    both nonzero."""
    with open(os.path.join(GOLDEN, "pages_fp32_collapse_margin.json")) as f:
        g = json.load(f)
    def naive(m):
        # the max-shifted fp32 form: shift by the row max, sum the exps, take
        # the log; gradient softmax - onehot
        z = torch.tensor([0.0, m], dtype=torch.float32)
        shifted = z - z.max()
        sumexp = torch.exp(shifted).sum()
        loss = torch.log(sumexp) - shifted[1]
        grad = torch.exp(shifted) / sumexp
        grad[1] -= 1.0
        return float(loss), float(grad[1]), float(grad.sum())
    lo, hi = naive(g["probe_below"]), naive(g["probe_above"])
    assert lo[0] > 0 and lo[1] < 0
    assert hi[0] == 0.0 and hi[1] == 0.0
    # margin-20 example: naive NLL 0, target grad 0, non-target still ~2e-9
    with open(os.path.join(GOLDEN, "pages_margin20.json")) as f:
        m20 = json.load(f)
    n20 = naive(20.0)
    assert n20[0] == m20["naive_fp32"]["nll"] and n20[1] == m20["naive_fp32"]["target_grad"]
    assert abs(n20[2] - m20["naive_fp32"]["nontarget_grad_sum_approx"]) < 0.1e-9
    for m in (g["probe_above"], 20.0, 40.0):
        out = ce_oracle(np.array([[0.0, m]]), np.array([1]))
        assert out["loss"][0] > 0 and out["grad"][0, 1] < 0


# Planted mistakes: each mutant of the oracle must fail at least one pin.
MUTANTS = [
    ("target kept in the non-target sum",
     "z_nt[np.arange(rows.size), tl] = _NEG_INF", "pass"),
    ("softplus argument sign flipped", "x = lse_nt - z_t", "x = z_t - lse_nt"),
    ("log1p term dropped from lse",
     "lse = np.maximum(lse_nt, z_t) + np.log1p(np.exp(-np.abs(x)))",
     "lse = np.maximum(lse_nt, z_t)"),
    ("z-loss dropped from the loss",
     "loss[rows] = nll + z_alpha * lse * lse", "loss[rows] = nll"),
    ("z-loss not squared", "loss[rows] = nll + z_alpha * lse * lse",
     "loss[rows] = nll + z_alpha * lse"),
    ("z-loss gradient factor halved",
     "zl = sc * 2.0 * z_alpha * lse", "zl = sc * z_alpha * lse"),
    ("z-loss gradient on the target loses p_t",
     "-w * p_nt + zl * p_t", "-w * p_nt + zl"),
    ("target gradient sign flipped", "-w * p_nt + zl * p_t", "w * p_nt + zl * p_t"),
    ("target gradient uses p_t instead of -p_nt",
     "-w * p_nt + zl * p_t", "-w * p_t + zl * p_t"),
    ("z-loss gradient weighted by the row weight",
     "zl = sc * 2.0 * z_alpha * lse", "zl = w * 2.0 * z_alpha * lse"),
    ("row weight ignored", "w = sc if weight is None else weight[rows]", "w = sc"),
    ("gradient not scaled", "sc = scale[rows]", "sc = np.ones(rows.size)"),
    ("mask array ignored", "valid &= np.asarray(mask).reshape(T) != 0", "pass"),
    ("segment scale multiplies by the length",
     "scale = float(grad_scale) / lens[seg].astype(np.float64)",
     "scale = float(grad_scale) * lens[seg].astype(np.float64)"),
    ("segment sums take the loss, not the NLL",
     "np.add.at(seg_nll, seg[valid], nll[valid])", "np.add.at(seg_nll, seg[valid], loss[valid])"),
    ("segment sums include ignored rows' neighbours (index shifted)",
     "np.add.at(seg_nll, seg[valid], nll[valid])",
     "np.add.at(seg_nll, np.roll(seg, 1)[valid], nll[valid])"),
    ("non-target probability uses the non-target lse",
     "p = np.exp(z_nt - lse[:, None])", "p = np.exp(z_nt - lse_nt[:, None])"),
    ("out-of-range targets not poisoned", "loss[bad] = np.nan", "pass"),
]


def _load_mutant(old, new):
    src_path = os.path.join(os.path.dirname(oracle.__file__), "ce_oracle.py")
    with open(src_path) as f:
        src = f.read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = {}
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), mod)
    return mod["ce_oracle"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    fn = _load_mutant(old, new)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(fn)
        except Exception as e:  # AssertionError, or a shape error the mistake causes
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"mutant {name!r} passed every pin"


def test_pin_lmhead():
    from oracle_pins import pin_lmhead
    pin_lmhead(oracle.lmhead_ce)


LM_MUTANTS = [
    ("logits use a permuted hidden index", "z = X @ W.T", "z = X @ W[:, ::-1].T"),
    ("dX uses the weight rows in the wrong order", 'out["dhidden"] = G @ W',
     'out["dhidden"] = G @ W[::-1]'),
    ("dW rows in the wrong order", 'out["dweight"] = G.T @ X', 'out["dweight"] = G.T[::-1] @ X'),
    ("dW misses the scale", 'out["dweight"] = G.T @ X', 'out["dweight"] = G.T @ X / 0.125'),
]


@pytest.mark.parametrize("name,old,new", LM_MUTANTS, ids=[m[0] for m in LM_MUTANTS])
def test_lmhead_mutant_is_caught(name, old, new):
    import importlib.util
    import types
    from oracle_pins import pin_lmhead
    path = os.path.join(os.path.dirname(oracle.__file__), "lmhead_oracle.py")
    with open(path) as f:
        src = f.read()
    assert old in src, old
    src = src.replace(old, new).replace("from .ce_oracle import", "from oracle.ce_oracle import")
    mod = types.ModuleType("lmhead_mutant")
    exec(compile(src, path, "exec"), mod.__dict__)
    with pytest.raises(Exception):
        pin_lmhead(mod.lmhead_ce)


def test_pin_distill():
    from oracle_pins import pin_distill
    pin_distill(oracle.distill_oracle)


DISTILL_MUTANTS = [
    ("KL gradient sign flipped", "d = ps - pt", "d = pt - ps"),
    ("teacher and student swapped in KL", "terms = np.where(pt > 0, pt * (lpt - lps), 0.0)",
     "terms = np.where(ps > 0, ps * (lps - lpt), 0.0)"),
    ("target term of KL dropped", "kl[rows] = terms.sum(axis=1) + tgt", "kl[rows] = terms.sum(axis=1)"),
    ("KL not weighted in the loss", "loss = r[\"loss\"] + kl_beta * np.where(valid, kl, 0.0)",
     "loss = r[\"loss\"] + np.where(valid, kl, 0.0)"),
    ("KL gradient misses the row scale", "grad[rows] += (r[\"scale\"][rows] * kl_beta)[:, None] * d",
     "grad[rows] += kl_beta * d"),
    ("target column keeps the raw difference only for the student",
     "d[ar, ti] = pt_nt - ps_nt", "d[ar, ti] = -ps_nt"),
]


@pytest.mark.parametrize("name,old,new", DISTILL_MUTANTS, ids=[m[0] for m in DISTILL_MUTANTS])
def test_distill_mutant_is_caught(name, old, new):
    import types
    from oracle_pins import pin_distill
    path = os.path.join(os.path.dirname(oracle.__file__), "distill_oracle.py")
    with open(path) as f:
        src = f.read()
    assert old in src, old
    src = src.replace(old, new).replace("from .ce_oracle import", "from oracle.ce_oracle import")
    mod = types.ModuleType("distill_mutant")
    exec(compile(src, path, "exec"), mod.__dict__)
    with pytest.raises(Exception):
        pin_distill(mod.distill_oracle)
