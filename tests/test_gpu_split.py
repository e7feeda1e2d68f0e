"""The split form (per-shard statistics, per-row finish, per-shard gradient)
against the fp64 oracle on the GPU.

The unique part of a shard's statistics is its non-target logsumexp
(shift / log2(e) + log(sum)) and the owner's target logit; the float shift
itself is arbitrary, so only those are compared. The finished losses,
segment sums and gradients are compared element by element.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import shard_nontarget_lse
from parity_utils import (PAD_GRAD, ROW_ALIGN, check_grad, check_loss, check_zero_rows,
                          padded_rows, row_scales, run_oracle, to_np64)
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
L2E_F = float(np.float32(1.4426950408889634))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import loss_vocab_amd  # noqa: F401
    yield
    torch.cuda.empty_cache()


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


CASES = [
    # (dtype, T, V, shards, align, alpha, segments)
    (torch.bfloat16, 40, 3001, 1, 8, 1e-4, 0),
    (torch.bfloat16, 40, 3001, 2, 8, 1e-4, 0),
    (torch.bfloat16, 33, 20011, 3, 8, 0.0, 5),
    (torch.float32, 33, 9999, 4, 4, 1e-3, 0),
    (torch.bfloat16, 25, 1003, 3, 1, 1e-4, 0),    # unaligned shard starts: one-element kernel
    (torch.float32, 25, 777, 5, 1, 0.0, 4),
    (torch.bfloat16, 12, 70001, 2, 8, 1e-4, 0),
    # shard rows on both sides of the 4096-chunk shape boundary in one call
    (torch.bfloat16, 20, 65537, 2, 8, 1e-4, 0),
    # shard rows past 14000 chunks (the deepest statistics shape)
    (torch.bfloat16, 12, 230011, 2, 8, 1e-4, 0),
    (torch.float32, 10, 120001, 2, 4, 1e-4, 3),
]


@pytest.mark.parametrize("dtype,T,V,shards,align,alpha,S", CASES,
                         ids=[f"{c[0]}-T{c[1]}-V{c[2]}-P{c[3]}-a{c[4]}".replace("torch.", "") for c in CASES])
def test_split_matches_oracle(dtype, T, V, shards, align, alpha, S):
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(V + shards)
    z = torch.randn(T, V, generator=g, device=DEV) * 2.5
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    bounds = L.shard_bounds(V, shards, align)
    # targets at shard edges, confident rows, ignored rows
    for i, (a, b) in enumerate(bounds):
        if 2 * i + 1 < T:
            t[2 * i] = a
            t[2 * i + 1] = b - 1
    z[3, t[3]] = z[3].max() + 35.0
    z[5, t[5]] = z[5].max() + 18.0
    t[T - 1] = -100
    z = z.to(dtype)
    seg = None
    if S:
        seg = torch.sort(torch.randint(0, S, (T,), generator=g, device=DEV)).values.to(torch.int32)
    gamma = 1.0 / (T - 1)
    z64 = to_np64(z)
    ref = run_oracle(z64, _np(t), segment_ids=_np(seg), num_segments=S, z_alpha=alpha,
                     grad_scale=gamma, segment_mean=S > 0)
    # packed rows of a ragged V run the one-element kernels; padded 16-byte
    # rows (NaN padding) run the chunk kernels on aligned shards
    for pad in ((False, True) if V % ROW_ALIGN else (False,)):
        _split_case(L, z, t, seg, S, shards, align, alpha, gamma, dtype, ref, pad)


def _split_case(L, z, t, seg, S, shards, align, alpha, gamma, dtype, ref, pad):
    T, V = z.shape
    gout = padded_rows(torch.empty_like(z), fill=PAD_GRAD) if pad else None
    loss, grad, segsum, row_state = L.ce_split(padded_rows(z) if pad else z, t, shards=shards,
                                               segment_ids=seg, num_segments=S,
                                               z_alpha=alpha, grad_scale=gamma,
                                               segment_mean=S > 0, align=align, grad_out=gout)
    torch.cuda.synchronize()
    if pad:
        ld = gout.stride(0)
        rest = gout.as_strided((T, ld - V), (ld, 1), gout.storage_offset() + V)
        assert bool((rest == PAD_GRAD).all()), "padding columns of the gradient were written"
    check_loss(_np(loss), ref["loss"], "split loss")
    check_grad(to_np64(grad), ref["grad"], dtype, "split grad",
               scale=row_scales(T, gamma, _np(seg), S, S > 0), targets=_np(t))
    inv = torch.as_tensor(~ref["valid"], device=DEV)
    check_zero_rows(loss[inv], grad[inv])
    if S:
        check_loss(_np(segsum), ref["seg_nll"], "split seg")
    rs = _np(row_state)
    assert np.all(rs[~ref["valid"], 5] == 1.0) and np.all(rs[ref["valid"], 5] == 0.0)
    # [0] + [6]: lse log2(e) as a float and its rounding residue
    v = ref["valid"]
    l2 = rs[v, 0].astype(np.float64) + rs[v, 6].astype(np.float64)
    check_loss(l2 / float(np.float32(L2E_F)), ref["lse"][v], "split row-state lse")
    assert np.all(np.abs(rs[v, 6]) <= np.spacing(np.abs(rs[v, 0])) / 2)


@pytest.mark.parametrize("dtype,align", [(torch.bfloat16, 8), (torch.float32, 4), (torch.bfloat16, 1)])
def test_shard_stats_unique_part(dtype, align):
    """shift / log2(e) + log(sum) is the shard's non-target logsumexp; the
    third value is the target logit in the owning shard and -inf elsewhere."""
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(17)
    T, V = 30, 5003
    z = (torch.randn(T, V, generator=g, device=DEV) * 3).to(dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[4] = -100
    mask = torch.ones(T, dtype=torch.uint8, device=DEV)
    mask[7] = 0
    for a, b in L.shard_bounds(V, 3, align):
        st = torch.empty(T, 3, device=DEV)
        L.ce_shard_stats(z[:, a:b], t, mask, st, v0=a)
        torch.cuda.synchronize()
        st = st.double().cpu().numpy()
        lse_ref, zt_ref = shard_nontarget_lse(to_np64(z[:, a:b]), _np(t), a, mask=_np(mask))
        lse = np.where(st[:, 0] == -np.inf, -np.inf, st[:, 0] / L2E_F + np.log(np.maximum(st[:, 1], 1e-300)))
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.all(np.abs(lse[fin] - lse_ref[fin]) <= 2e-6 * np.maximum(1.0, np.abs(lse_ref[fin])))
        assert np.array_equal(st[:, 2], zt_ref)


def test_backward_scale_is_applied_at_gradient_time():
    """One saved row state, two upstream scales: gradients scale exactly."""
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(5)
    T, V = 20, 4001
    z = torch.randn(T, V, generator=g, device=DEV)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    _, g1, _, rs = L.ce_split(z, t, shards=2, z_alpha=1e-3, grad_scale=0.25, align=4)
    g2 = torch.empty_like(g1)
    for a, b in L.shard_bounds(V, 2, 4):
        L.ce_shard_grad(z[:, a:b], t, rs, 0.5, g2[:, a:b], v0=a)
    torch.cuda.synchronize()
    assert torch.equal(g2, 2 * g1)


def test_split_in_place_and_forward_agrees_with_fused():
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(6)
    T, V = 64, 32000
    z = (torch.randn(T, V, generator=g, device=DEV) * 3).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[::9] = -100
    loss_f, grad_f, _ = L.ce_fused(z, t, z_alpha=1e-4, grad_scale=1 / 57)
    zc = z.clone()
    loss_s, grad_s, _, _ = L.ce_split(zc, t, shards=2, z_alpha=1e-4, grad_scale=1 / 57, in_place=True)
    torch.cuda.synchronize()
    assert grad_s.data_ptr() == zc.data_ptr()
    ref = run_oracle(to_np64(z), _np(t), z_alpha=1e-4, grad_scale=1 / 57)
    check_loss(_np(loss_s), ref["loss"])
    check_grad(to_np64(grad_s), ref["grad"], torch.bfloat16)
    # the two forms agree closely (different summation orders)
    assert torch.allclose(loss_s, loss_f, rtol=2e-6, atol=0)


def test_split_pages_share_full_size():
    """The pages' measured shape, T = 16384, V = 128256 bf16, in two shards of
    64128 columns (one tensor-parallel rank's share each): sampled rows vs the
    oracle, and ignored rows exactly zero."""
    import loss_vocab_amd as L
    wl = WORKLOADS["ce_bf16_T16384_V128256_zipf_inplace"]
    print("[split] full size", flush=True)
    inp = make_inputs(wl, device=DEV)
    T, V = wl.T, wl.V
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(T, size=24, replace=False))
    ri = torch.as_tensor(rows, device=DEV)
    z_rows = to_np64(inp["logits"][ri])
    loss, grad, _, _ = L.ce_split(inp["logits"], inp["targets"], shards=2, z_alpha=1e-4,
                                  grad_scale=inp["grad_scale"], grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    t_np = _np(inp["targets"])
    ref = run_oracle(z_rows, t_np[rows], z_alpha=1e-4, grad_scale=inp["grad_scale"])
    check_loss(_np(loss)[rows], ref["loss"], "split full loss")
    check_grad(to_np64(grad[ri]), ref["grad"], torch.bfloat16, "split full grad")
    inv = torch.as_tensor(t_np == -100, device=DEV)
    check_zero_rows(loss[inv], grad[inv])
    del inp, grad
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,shards,V", [(torch.bfloat16, 2, 5003), (torch.float32, 3, 5003),
                                            (torch.bfloat16, 2, 70001)])
def test_weighted_backward(dtype, shards, V):
    """A deferred child sharing the softmax: forward (statistics + finish with
    per-segment NLL sums), then per-row weights fixed between forward and
    backward (here seeded per-segment weights broadcast to their rows, as a
    GSPO-style seam would produce), then the weighted gradient."""
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(31 + shards)
    T, S = (200 if V < 10000 else 40), 8
    z = (torch.randn(T, V, generator=g, device=DEV) * 2).to(dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[[3, T // 4, T // 4 + 1]] = -100
    seg = torch.sort(torch.randint(0, S, (T,), generator=g, device=DEV)).values.to(torch.int32)
    w_seg = torch.randn(S, generator=torch.Generator().manual_seed(7), dtype=torch.float32)
    w_row = w_seg.to(DEV)[seg.long()].contiguous()
    alpha, gamma = 1e-3, 0.5
    loss, grad, segsum, rs = L.ce_split(z, t, shards=shards, segment_ids=seg, num_segments=S,
                                        z_alpha=alpha, grad_scale=gamma, row_weight=w_row,
                                        align=8 if dtype == torch.bfloat16 else 4)
    torch.cuda.synchronize()
    ref = run_oracle(to_np64(z), _np(t), segment_ids=_np(seg), num_segments=S, z_alpha=alpha,
                     grad_scale=gamma)
    ref_w = __import__("oracle").ce_oracle(to_np64(z), _np(t), segment_ids=_np(seg),
                                           num_segments=S, z_alpha=alpha, grad_scale=gamma,
                                           row_weight=_np(w_row).astype(np.float64))
    check_loss(_np(loss), ref["loss"], "weighted loss")
    check_loss(_np(segsum), ref["seg_nll"], "weighted seg")
    # unit scale of a row: the larger of its NLL weight and its z-loss weight
    # unit scale of a row: the larger of its NLL weight and its z-loss weight;
    # a weight of either sign makes the row factor w + u 2 alpha lse a float
    # sum that may cancel, so no relative bar here
    check_grad(to_np64(grad), ref_w["grad"], dtype, "weighted grad",
               scale=np.maximum(np.abs(_np(w_row).astype(np.float64)), gamma), rel=False)


@pytest.mark.parametrize("dtype,V,shards", [(torch.float32, 30001, 2), (torch.float32, 230011, 3),
                                            (torch.bfloat16, 230011, 2)])
def test_split_fp32_grad_unit_scale_large_lse(dtype, V, shards):
    """The split form at grad_scale 1 on rows near +-50 (|lse| > 40) whose
    largest softmax value, 0.6-0.95, is a non-target column in either shard,
    fp32 gradient, padded rows: every element within 1e-6 absolute and 2^-16
    relative of the oracle (the row state carries lse log2 e as a float and
    its residue)."""
    import loss_vocab_amd as L
    print(f"[split] unit scale V={V} {dtype} shards={shards}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V + shards)
    T = 10
    z = torch.randn(T, V, generator=g, device=DEV) * 2
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    cols = [3, V // 2 + 5, V - 2, 1100, 2 * V // 3]
    for r in range(T):
        j = cols[r % len(cols)]
        if int(t[r]) == j:
            t[r] = (j + 1) % V
        z[r, j] = float(torch.logsumexp(z[r], 0)) + 0.5 + 0.5 * (r % 6)
        z[r] += 50.0 if r % 2 == 0 else -55.0
    z = z.to(dtype)
    ref = run_oracle(to_np64(z), _np(t), z_alpha=1e-4, grad_scale=1.0)
    gout = padded_rows(torch.empty(T, V, device=DEV), fill=PAD_GRAD)
    loss, grad, _, _ = L.ce_split(padded_rows(z), t, shards=shards, z_alpha=1e-4, grad_scale=1.0,
                                  align=8, grad_out=gout)
    torch.cuda.synchronize()
    check_loss(_np(loss), ref["loss"], "split unit loss")
    check_grad(to_np64(grad), ref["grad"], torch.float32, "split unit grad", scale=1.0,
               targets=_np(t))
