"""Seeded random configurations of every call against the fp64 oracle.

Each case draws, from its own seed: the logits dtype, a row length from one
kernel tier (row kernel, row-resident rows in registers or with LDS slots,
two-workgroup fp32 rows, the long-row kernel), a row count, the gradient
dtype or an in-place gradient, 16-byte-aligned padded rows or packed ones, a
mask (starting at an odd address) or none, ignored rows, confident rows, the
z-loss weight and segments with or without the segment mean. Every output is
held to the same bars as the hand-written parity cases (per-row loss,
segment sums, every gradient element, ignored rows bit-exact). The same
draws feed the forward-only call, the split form (random shard counts and
alignments) and the distillation child (a teacher of the same dtype, random
weight). The loss behind the LM head gets draws of its own: row, vocabulary
and hidden sizes that are ragged against its 256 x 256 x 64 tiles, column
chunks, ignored and confident rows, a mask, the z-loss weight and the dX
dtype, on "grid" inputs whose logits are exact in fp32.
"""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from parity_utils import run_oracle, to_np64
from test_gpu_distill import compare as compare_distill
from test_gpu_forward import compare_forward
from test_gpu_lmhead import grid_inputs, run_and_compare
from test_gpu_parity import _inp, compare_all
from test_gpu_split import _split_case

pytestmark = pytest.mark.gpu

DEV = "cuda"

# Row lengths (elements) per kernel tier: the row kernel (two ranges), the
# row-resident kernel in registers and with LDS slots, fp32 rows on two
# workgroups, and the long-row kernel.
TIERS = {
    torch.float32: [(1, 300), (301, 32771), (32772, 65536), (65537, 102403), (102404, 204803),
                    (204804, 230000)],
    torch.bfloat16: [(1, 300), (301, 65543), (65544, 131072), (131073, 204807), (204808, 240000)],
}
# CE_FUZZ_CASES raises the number of cases for a longer search (default 32).
SEEDS = list(range(int(os.environ.get("CE_FUZZ_CASES", "32"))))


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = (torch.float32, torch.bfloat16)[seed % 2]
    tiers = TIERS[dtype]
    lo, hi = tiers[(seed // 2) % len(tiers)]
    V = int(rng.integers(lo, hi + 1))
    T = int(rng.integers(1, 33 if V < 70000 else 10))
    sigma = float(rng.choice([0.5, 2.0, 4.0]))
    g = torch.Generator(device=DEV).manual_seed(seed)
    z = (torch.randn(T, V, generator=g, device=DEV) * sigma).to(dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    ign = rng.random(T) < 0.2
    t[torch.as_tensor(ign, device=DEV)] = -100
    # a few confident rows: the target raised above the row maximum
    for r in np.flatnonzero(rng.random(T) < 0.2):
        if int(t[r]) >= 0:
            z[r, int(t[r])] = (z[r].float().max() + float(rng.uniform(5.0, 40.0))).to(dtype)
    mask = None
    if rng.random() < 0.5:
        off = int(rng.integers(1, 4))
        buf = torch.ones(T + 8, dtype=torch.uint8, device=DEV)
        mask = buf[off:off + T]
        mask[torch.as_tensor(rng.random(T) < 0.25, device=DEV)] = 0
    seg, S, seg_mean = None, 0, False
    if rng.random() < 0.35 and T > 1:
        S = int(rng.integers(1, T + 1))
        ids = np.sort(rng.integers(0, S, T)).astype(np.int32)
        seg = torch.as_tensor(ids, device=DEV)
        seg_mean = bool(rng.random() < 0.5)
    alpha = float(rng.choice([0.0, 1e-4]))
    n_valid = max(1, int((~ign).sum()))
    inp = _inp(z, t, alpha=alpha, gamma=1.0 / n_valid, seg=seg, S=S, seg_mean=seg_mean)
    in_place = bool(rng.random() < 0.25)
    grad_dtype = None if in_place else (torch.float32, torch.bfloat16, dtype)[int(rng.integers(3))]
    pad = bool(rng.random() < 0.5)
    desc = (f"seed={seed} {str(dtype)[6:]} T={T} V={V} sigma={sigma} mask={mask is not None} S={S} "
            f"seg_mean={seg_mean} alpha={alpha} grad={'in place' if in_place else str(grad_dtype)[6:]} "
            f"pad={pad}")
    return dict(inp=inp, mask=mask, grad_dtype=grad_dtype, in_place=in_place, pad=pad, desc=desc,
                rng=rng, dtype=dtype, n_valid=n_valid)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_fused_call(seed):
    c = _case(seed)
    print(f"[fuzz] {c['desc']}", flush=True)
    compare_all(c["inp"], grad_dtype=c["grad_dtype"], in_place=c["in_place"], mask=c["mask"],
                what=f"fuzz {c['desc']}", pad=c["pad"])


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_forward(seed):
    c = _case(seed)
    inp = c["inp"]
    print(f"[fuzz forward] {c['desc']}", flush=True)
    compare_forward(inp["logits"], inp["targets"], mask=c["mask"], seg=inp["segment_ids"],
                    S=inp["num_segments"], alpha=inp["z_alpha"], what=f"fuzz forward {c['desc']}",
                    pad=c["pad"])


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_split(seed):
    import loss_vocab_amd as L
    c = _case(seed)
    inp, rng = c["inp"], c["rng"]
    z, t = inp["logits"], inp["targets"]
    T, V = z.shape
    shards = int(rng.integers(1, 5))
    align = int(rng.choice([1, 8 if c["dtype"] == torch.bfloat16 else 4]))
    seg, S = inp["segment_ids"], inp["num_segments"]
    print(f"[fuzz split] {c['desc']} shards={shards} align={align}", flush=True)
    ref = run_oracle(to_np64(z), t.cpu().numpy(), segment_ids=None if seg is None else seg.cpu().numpy(),
                     num_segments=S, z_alpha=inp["z_alpha"], grad_scale=inp["grad_scale"],
                     segment_mean=S > 0)
    _split_case(L, z, t, seg, S, shards, align, inp["z_alpha"], inp["grad_scale"], c["dtype"], ref,
                c["pad"])


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_distill(seed):
    c = _case(seed)
    inp, rng = c["inp"], c["rng"]
    zs, t = inp["logits"], inp["targets"]
    g = torch.Generator(device=DEV).manual_seed(10_000 + seed)
    zt = (torch.randn(zs.shape, generator=g, device=DEV) * float(rng.choice([0.5, 2.0]))).to(zs.dtype)
    beta = float(rng.choice([0.0, 0.5, 1.0]))
    print(f"[fuzz distill] {c['desc']} beta={beta}", flush=True)
    compare_distill(zs, zt, t, mask=c["mask"], alpha=inp["z_alpha"], beta=beta, gamma=inp["grad_scale"],
                    grad_dtype=c["grad_dtype"], in_place=c["in_place"], what=f"fuzz distill {c['desc']}",
                    pad=c["pad"])


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_lmhead(seed):
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.integers(1, 600))
    V = int(rng.integers(1, 2100))
    H = 8 * int(rng.integers(1, 26))
    chunk = int(rng.choice([0, 256, 512, 768]))
    ignore = tuple(int(r) for r in np.flatnonzero(rng.random(T) < 0.15))
    X, W, t = grid_inputs(T, V, H, seed=seed, ignore=ignore)
    # confident rows: the target's weight row set to the row's hidden state
    for r in np.flatnonzero(rng.random(T) < 0.1):
        if int(t[r]) >= 0:
            W[int(t[r])] = X[r]
    mask = None
    if rng.random() < 0.3:
        mask = torch.as_tensor(rng.random(T) >= 0.2, device=DEV).to(torch.uint8)
    z_alpha = float(rng.choice([0.0, 1e-3]))
    dh_dtype = (torch.float32, torch.bfloat16)[int(rng.integers(2))]
    desc = (f"seed={seed} T={T} V={V} H={H} chunk={chunk} ignored={len(ignore)} "
            f"mask={mask is not None} alpha={z_alpha} dX={str(dh_dtype)[6:]}")
    print(f"[fuzz lmhead] {desc}", flush=True)
    run_and_compare(X, W, t, mask=mask, z_alpha=z_alpha, grad_scale=1.0 / T, chunk_cols=chunk,
                    dhidden_dtype=dh_dtype, what=f"fuzz lmhead {desc}")
