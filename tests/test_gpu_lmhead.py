"""Loss behind a linear LM head on the matrix cores vs the fp64 oracle.

Tolerances (derived from the arithmetic):
* "grid" inputs take values k/8 (|k| <= 8), so every product is a multiple of
  2^-6 and every logit sum is exact in fp32: the logits are exact and the loss
  and logsumexp are held to the loss tolerance, relative 1e-5;
* dL/dz is rounded to bf16 (relative 2^-9) before the two products, so dX and
  dW are held to 2^-8 (|G| |W|) and 2^-8 (|G|^T |X|) elementwise (a factor 2
  over the rounding bound), plus the fp32 accumulation and, for a bf16 dX,
  one more bf16 rounding of the result;
* Gaussian inputs add the fp32 error of each logit, at most K 2^-24 (|X| |W|^T)
  per element; it enters the loss at most twice and each G element relatively.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import lmhead_ce
from parity_utils import check_loss, to_np64

pytestmark = pytest.mark.gpu

DEV = "cuda"
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import loss_vocab_amd  # noqa: F401
    yield
    torch.cuda.empty_cache()


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


def grid_inputs(T, V, H, seed, ignore=(), oor=()):
    g = torch.Generator(device="cpu").manual_seed(seed)
    X = (torch.randint(-8, 9, (T, H), generator=g).double() / 8).to(torch.bfloat16)
    W = (torch.randint(-8, 9, (V, H), generator=g).double() / 8 / 4).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=g)
    for r in ignore:
        t[r] = -100
    for r in oor:
        t[r] = V + 5
    return X.to(DEV), W.to(DEV), t.to(DEV)


def gauss_inputs(T, V, H, seed, sigma_z=2.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    X = torch.randn(T, H, generator=g).to(torch.bfloat16)
    W = (torch.randn(V, H, generator=g) * (sigma_z / math.sqrt(H))).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=g)
    return X.to(DEV), W.to(DEV), t.to(DEV)


def check_products(got, ref, bound, what):
    got = np.asarray(got, dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    m = ~nan_ref
    err = np.abs(got[m] - ref[m])
    b = bound[m]
    bad = err > b
    if bad.any():
        i = np.argmax(err / np.maximum(b, 1e-300))
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} off; worst got {got[m][i]!r} "
                             f"ref {ref[m][i]!r} bound {b[i]:.3e}")


def run_and_compare(X, W, t, *, mask=None, z_alpha=0.0, grad_scale=1.0, chunk_cols=0,
                    dhidden_dtype=torch.float32, exact_logits=True, what=""):
    import loss_vocab_amd as L
    loss, lse, dh, dw = L.ce_lmhead(X, W, t, mask=mask, z_alpha=z_alpha, grad_scale=grad_scale,
                                    chunk_cols=chunk_cols, dhidden_dtype=dhidden_dtype)
    torch.cuda.synchronize()
    X64, W64 = to_np64(X), to_np64(W)
    ref = lmhead_ce(X64, W64, _np(t), mask=_np(mask), z_alpha=z_alpha, grad_scale=grad_scale)
    G = ref["grad_logits"]
    K = X64.shape[1]
    if exact_logits:
        zerr = np.zeros(X64.shape[0])
        check_loss(_np(loss), ref["loss"], what + " loss")
        check_loss(_np(lse), ref["lse"], what + " lse")
    else:
        zerr = K * U * (np.abs(X64) @ np.abs(W64).T).max(axis=1)
        for name, got, r in (("loss", loss, ref["loss"]), ("lse", lse, ref["lse"])):
            got = _np(got).astype(np.float64)
            fin = np.isfinite(r)
            assert np.array_equal(np.isnan(got), np.isnan(r)), f"{what} {name}: NaN pattern"
            tol = 1e-5 * np.abs(r[fin]) + 2 * zerr[fin] * (1 + 2 * z_alpha * np.abs(
                ref["lse"][fin]))
            assert np.all(np.abs(got[fin] - r[fin]) <= tol), f"{what} {name}"
    absG = np.abs(G)
    gre = 2.0 ** -8 + 2 * zerr[:, None]                   # relative error of each G element
    bx = (gre * absG) @ np.abs(W64) + K * U * (absG @ np.abs(W64))
    if dhidden_dtype == torch.bfloat16:
        bx = bx + 2.0 ** -8 * np.abs(ref["dhidden"]) + 2.0 ** -133
    bw = (gre * absG).T @ np.abs(X64) + X64.shape[0] * U * (absG.T @ np.abs(X64))
    check_products(to_np64(dh), ref["dhidden"], bx + 1e-30, what + " dX")
    check_products(to_np64(dw), ref["dweight"], bw + 1e-30, what + " dW")
    inv = ~ref["valid"]
    if inv.any():
        lb = loss[torch.as_tensor(inv, device=DEV)].cpu().view(torch.int32)
        assert int(lb.abs().max()) == 0, "ignored loss not +0.0"
        assert np.all(to_np64(dh)[inv] == 0), "ignored dX row not 0"
    return loss, lse, dh, dw, ref


@pytest.mark.parametrize("T,V,H,chunk", [
    (128, 128, 64, 0),        # one tile
    (300, 1000, 72, 128),     # ragged rows, vocabulary and K; four column chunks
    (257, 4099, 136, 0),      # one chunk, ragged everything
    (64, 50, 256, 0),         # vocabulary inside one tile
])
def test_grid_inputs(T, V, H, chunk):
    print(f"[lmhead] grid T={T} V={V} H={H} chunk={chunk}", flush=True)
    X, W, t = grid_inputs(T, V, H, seed=T + V + H, ignore=(3, T - 1))
    run_and_compare(X, W, t, z_alpha=1e-3, grad_scale=1.0 / T, chunk_cols=chunk,
                    what=f"T{T} V{V} H{H}")


@pytest.mark.parametrize("T,V", [(2048, 8448), (4096, 5000), (1950, 8300)])
def test_grouped_ranges_every_row(T, V):
    """Row tiles in groups of 8 take the grouped statistics grid (8 row tiles
    by 4 ranges per XCD, ranges of balanced length): every row's loss and lse,
    and dX and dW, against the oracle."""
    print(f"[lmhead] grouped ranges T={T} V={V}", flush=True)
    X, W, t = grid_inputs(T, V, 64, seed=T + V, ignore=(0, T // 2))
    run_and_compare(X, W, t, z_alpha=1e-3, grad_scale=1.0 / T, what=f"grouped T{T} V{V}")


def test_strided_operands():
    """hidden and weight as column slices of wider buffers (row strides 80
    and 96 elements, still 16-byte aligned)."""
    Xb, Wb, t = grid_inputs(150, 333, 96, seed=19, ignore=(0,))
    X = Xb[:, :64]
    W = Wb[:, 16:80]
    assert X.stride(0) == 96 and W.stride(0) == 96
    Xs = torch.empty((150, 80), dtype=torch.bfloat16, device=DEV)[:, :64]
    Xs.copy_(X)
    run_and_compare(Xs, W, t, z_alpha=1e-3, grad_scale=0.25, chunk_cols=256, what="strided")


def test_mask_and_bf16_dhidden():
    X, W, t = grid_inputs(200, 777, 64, seed=5)
    mask = (torch.arange(200, device=DEV) % 7 != 0).to(torch.uint8)
    run_and_compare(X, W, t, mask=mask, z_alpha=0.0, grad_scale=0.5,
                    dhidden_dtype=torch.bfloat16, what="mask bf16")


def test_forward_only_matches():
    import loss_vocab_amd as L
    X, W, t = grid_inputs(130, 600, 64, seed=9, ignore=(1,))
    loss, lse, _, _ = L.ce_lmhead(X, W, t, z_alpha=1e-4, want_grad=False)
    loss2, lse2, _, _ = L.ce_lmhead(X, W, t, z_alpha=1e-4)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2) and torch.equal(lse, lse2)
    ref = lmhead_ce(to_np64(X), to_np64(W), _np(t), z_alpha=1e-4, want_grad=False)
    check_loss(_np(loss), ref["loss"], "forward-only loss")


def test_partial_backward_and_null_lse():
    """dX alone, dW alone and no lse output give exactly the values of the
    full call (the same kernels run; the skipped products are not needed)."""
    import loss_vocab_amd as L
    X, W, t = grid_inputs(200, 700, 64, seed=29, ignore=(2,))
    T, H, V = 200, 64, 700
    full = L.ce_lmhead(X, W, t, z_alpha=1e-3, grad_scale=0.1, chunk_cols=256)
    loss = torch.empty(T, device=DEV)
    dh = torch.empty((T, H), device=DEV)
    dw = torch.empty((V, H), device=DEV)
    L.ce_lmhead_fwd_bwd(X, W, t, None, 1e-3, 0.1, loss, None, dh, None, chunk_cols=256)
    torch.cuda.synchronize()
    assert torch.equal(loss, full[0]) and torch.equal(dh, full[2])
    L.ce_lmhead_fwd_bwd(X, W, t, None, 1e-3, 0.1, loss, None, None, dw, chunk_cols=256)
    torch.cuda.synchronize()
    assert torch.equal(dw, full[3])


def test_out_of_range_target_poisons():
    X, W, t = grid_inputs(130, 300, 64, seed=11, oor=(7,))
    loss, lse, dh, dw, ref = run_and_compare(X, W, t, what="oor")
    assert math.isnan(float(loss[7])) and bool(torch.isnan(dh[7]).all())
    assert bool(torch.isnan(dw).all())


def test_confident_rows_exact_logits():
    """A third of the rows get W[t_r] = X_r, so z_t = |X_r|^2 stands ~20 above
    the rest: the NLL falls to ~1e-7 and below and keeps relative 1e-5, since
    grid logits are exact."""
    X, W, t = grid_inputs(128, 512, 64, seed=13)
    # make W[t_r] a scaled copy of X_r for a third of the rows: z_t = c |X_r|^2
    Wn = W.clone()
    rows = torch.arange(0, 128, 3, device=DEV)
    for r in rows.tolist():
        Wn[t[r]] = X[r]
    run_and_compare(X, Wn, t, what="confident")


def test_gaussian_inputs():
    X, W, t = gauss_inputs(384, 3000, 512, seed=17)
    t[5] = -100
    run_and_compare(X, W, t, z_alpha=1e-4, grad_scale=1.0 / 383, exact_logits=False,
                    chunk_cols=256, what="gauss")


def test_zero_rows():
    import loss_vocab_amd as L
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    W = torch.randn(100, 64, device=DEV).to(torch.bfloat16)
    t = torch.empty(0, dtype=torch.int64, device=DEV)
    loss, lse, dh, dw = L.ce_lmhead(X, W, t)
    torch.cuda.synchronize()
    assert loss.numel() == 0 and bool((dw == 0).all())


def test_mid_size_complete():
    """T = 1024, V = 32000, H = 1024, eight column chunks: every element of
    loss, lse, dX and dW against the oracle."""
    print("[lmhead] mid T=1024 V=32000 H=1024", flush=True)
    X, W, t = gauss_inputs(1024, 32000, 1024, seed=23)
    t[::9] = -100
    run_and_compare(X, W, t, z_alpha=1e-4, grad_scale=1.0 / 900, exact_logits=False,
                    chunk_cols=4096, what="mid")


def test_full_shape_sampled():
    """T = 16384 rows of a Llama-3-8B-sized head (V = 128256, H = 4096), four
    column chunks: loss, lse and dX on sampled rows vs the oracle (its logits
    for those rows in fp64); every output finite."""
    import loss_vocab_amd as L
    T, V, H = 16384, 128256, 4096
    print(f"[lmhead] full T={T} V={V} H={H}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(2024)
    X = torch.randn(T, H, generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn(V, H, generator=g, device=DEV) * (2.0 / math.sqrt(H))).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[torch.arange(0, T, 5, device=DEV)] = -100
    n_valid = int((t != -100).sum())
    loss, lse, dh, dw = L.ce_lmhead(X, W, t, z_alpha=1e-4, grad_scale=1.0 / n_valid)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(T, size=16, replace=False))
    ri = torch.as_tensor(rows, device=DEV)
    W64 = to_np64(W)
    absW = np.abs(W64)
    X64 = to_np64(X[ri])
    ref = lmhead_ce(X64, W64, _np(t)[rows], z_alpha=1e-4, grad_scale=1.0 / n_valid)
    zerr = H * U * (np.abs(X64) @ absW.T).max(axis=1)
    for name, got, r in (("loss", loss, ref["loss"]), ("lse", lse, ref["lse"])):
        got = _np(got)[rows].astype(np.float64)
        tol = 1e-5 * np.abs(r) + 2 * zerr * (1 + 2e-4 * np.abs(ref["lse"]))
        assert np.all(np.abs(got - r) <= tol), f"full {name}"
    absG = np.abs(ref["grad_logits"])
    bx = ((2.0 ** -8 + 2 * zerr[:, None]) * absG) @ absW + V * U * (absG @ absW)
    check_products(to_np64(dh[ri]), ref["dhidden"], bx + 1e-30, "full dX")
    assert bool(torch.isfinite(dw).all()) and bool(torch.isfinite(dh).all())
    assert bool(torch.isfinite(loss).all())
