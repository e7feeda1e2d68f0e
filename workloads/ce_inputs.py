"""Workload definitions and seeded generators for [T, V] logit matrices.

The five workloads mirror the shapes the pages discuss: torchtitan PR #5661
"fix softmax collapse with improved CE perf" measures T=16384, V=128256 (the
H100 table of its revised PR description) and names Llama-3 / Qwen-3 / gpt-oss
style vocabularies in its golden-file list; the collapse regime is the second
review's margin example; per-segment sums follow Fast-LLM PR #552 "Fuse GSPO
into the monolithic compiled loss" (PR body, GSPO seam).

Recipe (also stated in the design notes):

* logits: standard normal draws in fp32 scaled by sigma, rounded to nearest
  even when the workload is bf16; generated in row chunks, each chunk from its
  own seeded torch generator on the target device;
* targets: uniform over [0, V), or Zipf(s) over vocabulary ids on the finite
  support (P(k) proportional to (k + 1)^-s, inverse-CDF sampled);
* ignored rows: an exact count round(f * T) chosen without replacement, marked
  with ``IGNORE_INDEX`` in the targets;
* planted rows: the target logit set to (row max before planting) + U(a, b),
  computed in fp32 and rounded to the logits dtype; chosen among valid rows;
* segments: S sorted ids whose lengths are ``min_len + Multinomial(T - S *
  min_len, uniform)``.

Nothing here computes any part of the loss.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

IGNORE_INDEX = -100
BASE_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # seed stream id
    T: int
    V: int
    dtype: str                 # "f32" | "bf16"
    sigma: float
    targets: str               # "uniform" | "zipf"
    zipf_s: float = 1.1
    mask_frac: float = 0.0
    plant_frac: float = 0.0    # fraction of rows whose target is planted
    plant_lo: float = 0.0
    plant_hi: float = 0.0
    z_alpha: float = 0.0
    grad: str = "same"         # "f32" | "bf16" | "inplace"
    num_segments: int = 0
    seg_min_len: int = 0
    reduction: str = "mean"    # "mean" (gamma = 1/n_valid) | "segment_mean" (gamma = 1, / len)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def grad_torch_dtype(self):
        if self.grad == "inplace":
            return self.torch_dtype
        return torch.float32 if self.grad == "f32" else torch.bfloat16

    @property
    def n_masked(self):
        return int(round(self.mask_frac * self.T))

    @property
    def n_valid(self):
        return self.T - self.n_masked

    @property
    def grad_scale(self):
        if self.reduction == "segment_mean":
            return 1.0
        return 1.0 / max(1, self.n_valid)

    def scaled(self, T=None, V=None, num_segments=None):
        """The same recipe at another size (for small parity cases)."""
        kw = {}
        if T is not None:
            kw["T"] = T
        if V is not None:
            kw["V"] = V
        if num_segments is not None:
            kw["num_segments"] = num_segments
        return dataclasses.replace(self, name=self.name + "_scaled", **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("ce_f32_T256_V4096_mask10", 0, 256, 4096, "f32", 2.0, "uniform",
                 mask_frac=0.10, grad="f32"),
        Workload("cez_bf16_T8192_V32000_collapse", 1, 8192, 32000, "bf16", 3.0, "uniform",
                 mask_frac=0.15, plant_frac=0.05, plant_lo=20.0, plant_hi=40.0,
                 z_alpha=1e-4, grad="bf16"),
        Workload("ce_bf16_T16384_V128256_zipf_inplace", 2, 16384, 128256, "bf16", 2.0, "zipf",
                 zipf_s=1.1, mask_frac=0.20, grad="inplace"),
        Workload("cez_f32_T32768_V151936_peaked", 3, 32768, 151936, "f32", 1.0, "uniform",
                 plant_frac=1.0, plant_lo=0.0, plant_hi=40.0, z_alpha=1e-4, grad="f32"),
        Workload("cezseg_bf16_T65536_V201088_seg512", 4, 65536, 201088, "bf16", 2.0, "uniform",
                 mask_frac=0.10, z_alpha=1e-4, grad="bf16", num_segments=512,
                 seg_min_len=16, reduction="segment_mean"),
    ]
}

# Order of the workloads above (smallest first).
ORDER = list(WORKLOADS)


def workload(name):
    return WORKLOADS[name]


def _gen(device, *stream):
    """A torch generator on ``device`` seeded from (BASE_SEED, *stream)."""
    seed = BASE_SEED
    for s in stream:
        seed = (seed * 1_000_003 + int(s) + 1) % (2**62)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _np_rng(*stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *stream])))


def _zipf_targets(T, V, s, rng):
    k = np.arange(V, dtype=np.float64)
    w = (k + 1.0) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(T)
    idx = np.searchsorted(cdf, u, side="right")
    return np.minimum(idx, V - 1).astype(np.int64)


def make_inputs(w: Workload, device="cpu", seed_offset=0, chunk_rows=1024):
    """Generate the inputs of workload ``w`` on ``device``.

    Returns a dict: ``logits`` [T, V] (w.torch_dtype), ``targets`` [T] int64,
    ``segment_ids`` [T] int32 or None, ``num_segments``, ``planted`` [T] bool,
    ``z_alpha``, ``grad_scale``, ``segment_mean``.
    """
    T, V = w.T, w.V
    dev = torch.device(device)
    k = w.index * 1000 + seed_offset

    # Targets and row structure are drawn on the host (small), then moved.
    rng = _np_rng(k, 1)
    if w.targets == "zipf":
        tgt = _zipf_targets(T, V, w.zipf_s, rng)
    else:
        tgt = rng.integers(0, V, size=T, dtype=np.int64)
    n_mask = w.n_masked
    masked_rows = rng.choice(T, size=n_mask, replace=False) if n_mask else np.zeros(0, np.int64)
    valid = np.ones(T, dtype=bool)
    valid[masked_rows] = False

    planted = np.zeros(T, dtype=bool)
    n_plant = int(round(w.plant_frac * T))
    if n_plant:
        valid_rows = np.nonzero(valid)[0]
        n_plant = min(n_plant, valid_rows.size)
        planted[rng.choice(valid_rows, size=n_plant, replace=False)] = True
    margins = rng.uniform(w.plant_lo, w.plant_hi, size=T).astype(np.float32)

    seg = None
    if w.num_segments:
        S = w.num_segments
        extra = T - S * w.seg_min_len
        if extra < 0:
            raise ValueError("T too small for the segment minimum length")
        lens = w.seg_min_len + rng.multinomial(extra, np.full(S, 1.0 / S))
        seg = np.repeat(np.arange(S, dtype=np.int32), lens)

    logits = torch.empty((T, V), dtype=w.torch_dtype, device=dev)
    for c0 in range(0, T, chunk_rows):
        c1 = min(T, c0 + chunk_rows)
        g = _gen(dev, k, 2, c0 // chunk_rows)
        block = torch.randn((c1 - c0, V), generator=g, dtype=torch.float32, device=dev)
        block.mul_(w.sigma)
        rows_here = np.nonzero(planted[c0:c1])[0]
        if rows_here.size:
            ri = torch.as_tensor(rows_here, device=dev)
            # Row max before planting; the planted value is rounded to the
            # logits dtype after the fp32 addition.
            rmax = block[ri].amax(dim=1)
            val = rmax + torch.as_tensor(margins[c0:c1][rows_here], device=dev)
            ti = torch.as_tensor(tgt[c0:c1][rows_here], device=dev)
            block[ri, ti] = val
        logits[c0:c1].copy_(block)   # RNE to bf16 where needed
        del block

    tgt_out = tgt.copy()
    tgt_out[~valid] = IGNORE_INDEX
    return {
        "logits": logits,
        "targets": torch.as_tensor(tgt_out, device=dev),
        "segment_ids": None if seg is None else torch.as_tensor(seg, device=dev),
        "num_segments": w.num_segments,
        "planted": torch.as_tensor(planted),
        "z_alpha": w.z_alpha,
        "grad_scale": w.grad_scale,
        "segment_mean": w.reduction == "segment_mean",
    }


def alg_bytes(w: Workload):
    """Algorithmic HBM bytes of one fused fwd+bwd call on workload ``w``.

    Valid rows are read once; every row's gradient is written once; targets
    (8 B) and the per-row loss (4 B) are read/written once; segment ids (4 B)
    and the per-row NLL staging (4 B write + 4 B read) when segments are on.
    """
    b_in = 4 if w.dtype == "f32" else 2
    b_out = 4 if w.grad_torch_dtype == torch.float32 else 2
    nbytes = w.n_valid * w.V * b_in + w.T * w.V * b_out + w.T * (8 + 4)
    if w.num_segments:
        nbytes += w.T * (4 + 8) + w.num_segments * 4
    return nbytes



# ---------------------------------------------------------------------------
# Inputs of the loss behind a linear LM head: hidden states and head weight.
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LmHeadWorkload:
    """Hidden states X [T, H] ~ N(0, 1) and head weight W [V, H] ~ N(0,
    (sigma / sqrt(H))^2), both bf16 (RNE from fp32 draws), so the logits are
    ~ N(0, sigma^2); targets Zipf(s) over [0, V) with an exact count of
    ignored rows. The shape is the pages' measured one (T = 16384, V = 128256)
    with a Llama-3-8B hidden size (H = 4096)."""
    name: str
    index: int
    T: int
    V: int
    H: int
    sigma: float = 2.0
    zipf_s: float = 1.1
    mask_frac: float = 0.2
    z_alpha: float = 0.0

    @property
    def n_masked(self):
        return int(round(self.mask_frac * self.T))

    @property
    def n_valid(self):
        return self.T - self.n_masked

    def scaled(self, T=None, V=None, H=None):
        kw = {k: v for k, v in (("T", T), ("V", V), ("H", H)) if v is not None}
        return dataclasses.replace(self, name=self.name + "_scaled", **kw)


LMHEAD_WORKLOADS = {
    w.name: w for w in [
        LmHeadWorkload("lmhead_bf16_T16384_V128256_H4096", 10, 16384, 128256, 4096),
    ]
}


def lmhead_flops(w: LmHeadWorkload, backward=True, recompute=True):
    """Matrix-core flops of one call: the logit product forward (2 T V H),
    dX = G W and dW = G^T X backward (4 T V H), and with ``recompute`` the
    logit product once more in the backward (executed, not algorithmic)."""
    if not backward:
        return 2 * w.T * w.V * w.H
    return (8 if recompute else 6) * w.T * w.V * w.H


def make_lmhead_inputs(w: LmHeadWorkload, device="cpu", seed_offset=0, rows=None):
    """``hidden`` [T, H] bf16, ``weight`` [V, H] bf16, ``targets`` [T] int64.
    ``rows`` (optional) generates only the first ``rows`` rows of hidden and
    targets (the weight is always whole)."""
    T = w.T if rows is None else rows
    dev = torch.device(device)
    k = w.index * 1000 + seed_offset
    rng = _np_rng(k, 1)
    tgt = _zipf_targets(w.T, w.V, w.zipf_s, rng)
    masked = rng.choice(w.T, size=w.n_masked, replace=False) if w.n_masked else np.zeros(0, np.int64)
    tgt[masked] = IGNORE_INDEX
    hidden = torch.empty((T, w.H), dtype=torch.bfloat16, device=dev)
    for c0 in range(0, T, 4096):
        c1 = min(T, c0 + 4096)
        g = _gen(dev, k, 2, c0 // 4096)
        hidden[c0:c1].copy_(torch.randn((c1 - c0, w.H), generator=g, dtype=torch.float32, device=dev))
    weight = torch.empty((w.V, w.H), dtype=torch.bfloat16, device=dev)
    for c0 in range(0, w.V, 8192):
        c1 = min(w.V, c0 + 8192)
        g = _gen(dev, k, 3, c0 // 8192)
        block = torch.randn((c1 - c0, w.H), generator=g, dtype=torch.float32, device=dev)
        weight[c0:c1].copy_(block.mul_(w.sigma / np.sqrt(w.H)))
    return {"hidden": hidden, "weight": weight,
            "targets": torch.as_tensor(tgt[:T], device=dev), "z_alpha": w.z_alpha,
            "grad_scale": 1.0 / max(1, w.n_valid)}
