"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
the same inputs, compare to the stated tolerances.

Tolerances (fixed by the benchmark spec of this path):
* fp32 losses (per row, means, segment sums): relative 1e-5;
* fp32 gradients: absolute 1e-6;
* bf16 gradients: 2 bf16 ulp of the fp64 reference, where
  ulp_bf16(x) = 2^(max(floor(log2|x|), -126) - 7); below 2^-126 an absolute
  2^-126 is also accepted (fp32/bf16 subnormal range, flush to zero allowed);
* ignored rows and segment indexing: bit-exact (+0.0 everywhere).
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import ce_oracle

LOSS_REL = 1e-5
GRAD_F32_ABS = 1e-6
BF16_ULPS = 2.0


def bf16_ulp(x):
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


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


def check_grad(got, ref, dtype, what="grad"):
    """got: float64 array of the GPU's values; ref: float64 oracle values."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nan_ok = np.isnan(got) == np.isnan(ref)
    assert nan_ok.all(), f"{what}: NaN pattern differs"
    m = ~np.isnan(ref)
    err = np.abs(got[m] - ref[m])
    if dtype == torch.float32:
        bound = np.full_like(err, GRAD_F32_ABS)
    else:
        bound = BF16_ULPS * bf16_ulp(ref[m])
        tiny = np.abs(ref[m]) < 2.0 ** -126
        bound = np.where(tiny, np.maximum(bound, 2.0 ** -126), bound)
    bad = err > bound
    if bad.any():
        i = np.argmax(err / bound)
        idx = np.argwhere(m)[i]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} off; worst at {tuple(idx)} "
                             f"got {got[m][i]!r} ref {ref[m][i]!r} bound {bound[i]:.3e}")


def check_zero_rows(loss_rows, grad_rows):
    """Ignored rows are +0.0 bit for bit."""
    if loss_rows is not None:
        lb = loss_rows.detach().cpu().contiguous().view(torch.int32)
        assert int(lb.abs().max()) == 0 if lb.numel() else True, "ignored loss not +0.0"
    if grad_rows is not None and grad_rows.numel():
        g = grad_rows.detach()
        bits = g.view(torch.int16) if g.dtype == torch.bfloat16 else g.view(torch.int32)
        assert int((bits != 0).sum()) == 0, "ignored gradient row not +0.0"


def run_hip(inp, grad_dtype=None, in_place=False, want_grad=True, mask=None):
    import loss_vocab_amd as L
    return L.ce_fused(inp["logits"], inp["targets"], mask=mask,
                      segment_ids=inp.get("segment_ids"), num_segments=inp.get("num_segments", 0),
                      z_alpha=inp["z_alpha"], grad_scale=inp["grad_scale"],
                      segment_mean=inp.get("segment_mean", False), grad_dtype=grad_dtype,
                      in_place=in_place, want_grad=want_grad)


def run_oracle(logits_cpu64, targets, *, mask=None, segment_ids=None, num_segments=0,
               z_alpha=0.0, grad_scale=1.0, segment_mean=False, want_grad=True):
    return ce_oracle(logits_cpu64, targets, mask=mask, segment_ids=segment_ids,
                     num_segments=num_segments, z_alpha=z_alpha, grad_scale=grad_scale,
                     segment_mean=segment_mean, want_grad=want_grad)
