"""Distillation child on the shared softmax vs the fp64 oracle.

Tolerances (derived from the arithmetic):
* the CE part of the loss and of the gradient keeps the fused path's bars
  (loss relative 1e-5; fp32 gradient absolute 1e-6; bf16 gradient 2 ulp);
* KL is assembled from fp32 row statistics whose relative error is ~1e-6, in
  pieces of size up to pT_nt (|lse_z| + |lse_y| + max|y - z|) + |pT_t (NLL_z -
  NLL_y)|; its error is held to 1e-5 |KL| + 4e-6 times that size;
* each gradient element s ((1 + 2 alpha lse + beta) pS - beta pT) carries
  relative error ~1e-6 in each of its two terms: 4e-6 s ((1 + 2 alpha lse +
  beta) pS + beta pT) is added to the element's bar.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import distill_oracle
from distill_checks import check_rows
from parity_utils import PAD_GRAD, ROW_ALIGN, bf16_ulp, padded_rows, to_np64
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import loss_vocab_amd  # noqa: F401
    yield
    torch.cuda.empty_cache()


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


def compare(zs, zt, t, *, mask=None, alpha=0.0, beta=1.0, gamma=1.0, grad_dtype=None,
            in_place=False, what="", pad=False):
    """``pad``: student, teacher and gradient as the first V columns of
    16-byte aligned rows (the chunk kernels and their ragged tail; packed
    rows of a ragged V take the one-element kernel)."""
    import loss_vocab_amd as L
    zs64, zt64, t_np = to_np64(zs), to_np64(zt), _np(t)
    gdt = grad_dtype or zs.dtype
    if pad:
        T, V = zs.shape
        zsp, ztp = padded_rows(zs), padded_rows(zt)
        loss = torch.empty(T, device=DEV)
        kl = torch.empty(T, device=DEV)
        grad = zsp if in_place else padded_rows(torch.empty(T, V, dtype=gdt, device=DEV),
                                                fill=PAD_GRAD)
        L.ce_fused_distill(zsp, ztp, t, mask, alpha, beta, gamma, loss, kl, grad)
        torch.cuda.synchronize()
        if not in_place:
            ld = grad.stride(0)
            rest = grad.as_strided((T, ld - V), (ld, 1), grad.storage_offset() + V)
            assert bool((rest == PAD_GRAD).all()), "padding columns of the gradient were written"
    else:
        loss, kl, grad = L.ce_distill(zs, zt, t, mask=mask, z_alpha=alpha, kl_beta=beta,
                                      grad_scale=gamma, grad_dtype=gdt, in_place=in_place)
        torch.cuda.synchronize()
    ref = distill_oracle(zs64, zt64, t_np, mask=_np(mask), z_alpha=alpha, kl_beta=beta,
                         grad_scale=gamma)
    check_rows(zs64, zt64, t_np, _np(loss), _np(kl), to_np64(grad), ref, alpha=alpha, beta=beta,
               gamma=gamma, gdt=gdt, what=what)
    return loss, kl, grad, ref


def _pair(T, V, dtype, tdtype=None, seed=0, sz=2.0, st=2.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    zs = (torch.randn(T, V, generator=g, device=DEV) * sz).to(dtype)
    zt = (torch.randn(T, V, generator=g, device=DEV) * st).to(tdtype or dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    return zs, zt, t


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [1, 2, 7, 8, 9, 513, 4099, 32000])
def test_vocab_sizes(dtype, V):
    print(f"[distill] V={V} {dtype}", flush=True)
    zs, zt, t = _pair(6, V, dtype, seed=V)
    t[2] = -100
    for pad in ((False, True) if V % ROW_ALIGN else (False,)):
        compare(zs, zt, t, alpha=1e-3, beta=0.7, gamma=0.2, what=f"V={V} pad={pad}", pad=pad)


@pytest.mark.parametrize("sd,td,gd", [(torch.float32, torch.bfloat16, torch.float32),
                                      (torch.bfloat16, torch.float32, torch.bfloat16),
                                      (torch.bfloat16, torch.bfloat16, torch.float32)])
def test_mixed_dtypes(sd, td, gd):
    zs, zt, t = _pair(9, 3001, sd, td, seed=3)
    compare(zs, zt, t, alpha=1e-4, beta=1.5, gamma=0.1, grad_dtype=gd, what="mixed")


def test_unaligned_rows_take_the_element_path():
    g = torch.Generator(device=DEV).manual_seed(5)
    base = torch.randn(7, 2001 + 3, generator=g, device=DEV)
    zs = base[:, 1:2002]
    zt = torch.randn(7, 2001, generator=g, device=DEV).to(torch.bfloat16)
    t = torch.randint(0, 2001, (7,), generator=g, device=DEV)
    compare(zs, zt, t, beta=0.5, gamma=1.0, what="unaligned")


def test_teacher_equal_to_student():
    """KL is 0 and the gradient is the CE gradient: the two statistics are
    computed identically, so the KL pieces cancel exactly."""
    zs, _, t = _pair(8, 5000, torch.bfloat16, seed=7)
    loss, kl, grad, ref = compare(zs, zs.clone(), t, alpha=1e-3, beta=2.0, gamma=0.5, what="same")
    assert bool((kl == 0).all())


def test_beta_zero_skips_the_teacher_in_the_gradient():
    import loss_vocab_amd as L
    zs, zt, t = _pair(8, 5000, torch.bfloat16, seed=8)
    _, kl, grad, ref = compare(zs, zt, t, alpha=1e-3, beta=0.0, gamma=0.5, what="beta0")
    g2 = L.ce_fused(zs, t, z_alpha=1e-3, grad_scale=0.5)[1]
    torch.cuda.synchronize()
    r = ref["grad"]
    d = np.abs(to_np64(grad) - to_np64(g2))
    assert np.all(d <= 2 * bf16_ulp(r) + 2.0 ** -126)


def test_confident_rows_and_infinities():
    g = torch.Generator(device=DEV).manual_seed(9)
    T, V = 12, 3000
    zs = torch.randn(T, V, generator=g, device=DEV) * 2
    zt = torch.randn(T, V, generator=g, device=DEV) * 2
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    ar = torch.arange(T, device=DEV)
    zs[ar[:6], t[:6]] = zs[ar[:6]].amax(1) + torch.linspace(18, 40, 6, device=DEV)
    zt[ar[:6], t[:6]] = zt[ar[:6]].amax(1) + torch.linspace(20, 36, 6, device=DEV)
    zt[6, :100] = float("-inf")            # teacher rules columns out
    zs[7, 5] = float("-inf")
    zs[7, t[7]] = 3.0
    t[8] = -100
    t[9] = V + 4                           # out of range: NaN row
    compare(zs, zt, t, alpha=1e-4, beta=0.8, gamma=0.3, what="confident")


def test_in_place_and_mask():
    zs, zt, t = _pair(64, 8192, torch.bfloat16, seed=11)
    mask = (torch.arange(64, device=DEV) % 3 != 0).to(torch.uint8)
    compare(zs.clone(), zt, t, mask=mask, alpha=1e-4, beta=0.5, gamma=1 / 40, in_place=True,
            what="in place")


@pytest.mark.parametrize("V,dtype", [(8192, torch.bfloat16), (70001, torch.bfloat16),
                                     (30000, torch.float32)])
@pytest.mark.parametrize("offset", [1, 3])
def test_unaligned_mask(V, dtype, offset):
    """A mask that starts at an odd address over 13 rows: its bytes are read
    within aligned 4-byte words where the word lies inside the mask, by byte
    at the ends (chunk kernel for the aligned rows, element kernel for the
    odd row length)."""
    zs, zt, t = _pair(13, V, dtype, seed=40 + offset)
    buf = torch.ones(13 + 8, dtype=torch.uint8, device=DEV)
    mask = buf[offset:offset + 13]
    assert mask.data_ptr() % 4 == offset % 4
    mask[[0, 3, 4, 7, 12]] = 0
    t[6] = -100
    compare(zs, zt, t, mask=mask, alpha=1e-4, beta=0.5, gamma=1 / 7, what=f"unaligned mask +{offset}")


@pytest.mark.parametrize("name", ["cez_bf16_T8192_V32000_collapse",
                                  "ce_bf16_T16384_V128256_zipf_inplace",
                                  "cez_f32_T32768_V151936_peaked"])
def test_full_shape_sampled(name):
    """The benchmarked workloads at full size, a second draw of the recipe as
    teacher: sampled rows against the oracle, every loss finite."""
    import loss_vocab_amd as L
    print(f"[distill] full {name}", flush=True)
    wl = WORKLOADS[name]
    s = make_inputs(wl, device=DEV)
    te = make_inputs(wl, device=DEV, seed_offset=1)["logits"]
    zs, t = s["logits"], s["targets"]
    alpha, gamma = s["z_alpha"], s["grad_scale"]
    loss, kl, grad = L.ce_distill(zs, te, t, z_alpha=alpha, kl_beta=0.5, grad_scale=gamma)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(wl.T, size=24, replace=False))
    ri = torch.as_tensor(rows, device=DEV)
    t_np = _np(t)
    zs64, zt64 = to_np64(zs[ri]), to_np64(te[ri])
    ref = distill_oracle(zs64, zt64, t_np[rows], z_alpha=alpha, kl_beta=0.5, grad_scale=gamma)
    check_rows(zs64, zt64, t_np[rows], _np(loss)[rows], _np(kl)[rows], to_np64(grad[ri]), ref,
               alpha=alpha, beta=0.5, gamma=gamma, gdt=zs.dtype, what=f"full {name}")
    valid = torch.as_tensor(t_np != -100, device=DEV)
    assert bool(torch.isfinite(loss[valid]).all()) and bool((kl[valid] > -1e-3).all())
    assert math.isfinite(float(loss.sum()))
    del s, te, zs, loss, kl, grad
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,gdt,V", [(torch.bfloat16, torch.bfloat16, 32003),
                                         (torch.bfloat16, torch.bfloat16, 128259),
                                         (torch.bfloat16, torch.float32, 70001),
                                         (torch.float32, torch.float32, 151937),
                                         (torch.float32, torch.bfloat16, 20001),
                                         (torch.bfloat16, torch.bfloat16, (1 << 21) + 5)])
def test_target_positions(dtype, gdt, V):
    """One row per target position: the first chunks (kept on chip), each
    later step of streamed chunks, the row's last whole chunk and its tail,
    for every row-length and dtype shape of the chunked kernel."""
    W = 16 // (4 if dtype == torch.float32 else 2)
    nchunk = V // W
    pos = sorted({0, W - 1, W * 256 + 3, W * 1024 * 3 + 5, W * 256 * 9 + 1, W * 4096 + 2,
                  V // 2, (nchunk - 1) * W, (nchunk - 1) * W + W - 1, V - 1})
    pos = [q for q in pos if q < V]
    print(f"[distill positions] V={V} {dtype} -> {gdt}: {pos}", flush=True)
    zs, zt, _ = _pair(len(pos), V, dtype, seed=V % 97)
    t = torch.as_tensor(pos, device=DEV)
    for pad in (False, True):
        compare(zs, zt, t, alpha=1e-4, beta=0.6, gamma=0.05, grad_dtype=gdt,
                what=f"pos V={V} pad={pad}", pad=pad)
