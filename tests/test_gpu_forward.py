"""Forward-only entry (loss, full logsumexp, softmax entropy) vs the fp64 oracle.

The logsumexp is checked to the loss tolerance (relative 1e-5), and so is the
entropy, plus an absolute term derived from its fp32 inputs: the non-target
part of H comes from the pass-1 partials (shift, sum S, sum U of e d), whose
relative error is at most one 2^-24 rounding per step of a row's accumulation
chain (fewer than 64 steps at the row lengths here: 2^-18). Carried through
H_nt = ln2 2^(M - L2) ((L2 - M) S - U), that is at most
2^-18 p_nt (1 + |lse - max_{j != t} z_j|) absolute; it matters only where
one non-target column holds nearly all the mass (H small, p_nt ~ 1), and on
confident rows (H ~ p_nt margin) it is about 2^-18 H, so they keep their
relative accuracy. Ignored rows are +0.0 bit for bit and out-of-range
targets NaN. Cases:
the five workload recipes at oracle-sized shapes, vocabulary sizes across
every kernel shape and the one-element path (unaligned strides), confident
rows past the fp32 collapse point (where the entropy is ~1e-8 and must keep
its relative accuracy), infinities, segments, and the full workload shapes on
sampled rows plus bounds every row satisfies.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import ce_oracle, row_entropy
from parity_utils import ROW_ALIGN, check_entropy, check_loss, padded_rows, to_np64
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
W = WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    import loss_vocab_amd  # noqa: F401  (raises if the HIP library is missing)
    yield
    torch.cuda.empty_cache()


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


def _bits_zero(x):
    return bool((x.detach().cpu().contiguous().view(torch.int32) == 0).all())


def compare_forward(z, t, *, mask=None, seg=None, S=0, alpha=0.0, what="", pad=False):
    """``pad``: the call reads z as the first V columns of 16-byte aligned
    rows with NaN padding (the chunk kernels and their ragged tail; packed
    rows of a ragged V take the one-element kernel)."""
    import loss_vocab_amd as L
    loss, lse, ent, segl = L.ce_forward(padded_rows(z) if pad else z, t, mask=mask,
                                        segment_ids=seg, num_segments=S, z_alpha=alpha)
    torch.cuda.synchronize()
    z64, t_np, m_np = to_np64(z), _np(t), _np(mask)
    ref = ce_oracle(z64, t_np, mask=m_np, segment_ids=_np(seg), num_segments=S, z_alpha=alpha,
                    want_grad=False)
    H, lse_ref = row_entropy(z64, t_np, mask=m_np)
    check_loss(_np(loss), ref["loss"], what + " loss")
    check_loss(_np(lse), lse_ref, what + " lse")
    check_entropy(_np(ent), H, z64, t_np, lse_ref, what + " entropy")
    inv = torch.as_tensor(~ref["valid"], device=z.device)
    for name, x in (("loss", loss), ("lse", lse), ("entropy", ent)):
        assert _bits_zero(x[inv]), f"{what}: ignored {name} not +0.0"
    if segl is not None:
        check_loss(_np(segl), ref["seg_nll"], what + " seg")
    return loss, lse, ent, segl, H


SMALL = [
    ("f32_mask10_T256_V4096", W["ce_f32_T256_V4096_mask10"]),
    ("bf16_collapse_zloss_ragged", W["cez_bf16_T8192_V32000_collapse"].scaled(T=300, V=3001)),
    ("bf16_zipf_V10007", W["ce_bf16_T16384_V128256_zipf_inplace"].scaled(T=200, V=10007)),
    ("f32_peaked_zloss_V5003", W["cez_f32_T32768_V151936_peaked"].scaled(T=128, V=5003)),
    ("bf16_segments", W["cezseg_bf16_T65536_V201088_seg512"].scaled(T=2000, V=515, num_segments=37)),
]


@pytest.mark.parametrize("name,wl", SMALL, ids=[s[0] for s in SMALL])
def test_small_workloads_forward(name, wl):
    print(f"[forward] {name} T={wl.T} V={wl.V}", flush=True)
    inp = make_inputs(wl, device=DEV)
    for pad in ((False, True) if wl.V % ROW_ALIGN else (False,)):
        compare_forward(inp["logits"], inp["targets"], seg=inp["segment_ids"],
                        S=inp["num_segments"], alpha=inp["z_alpha"], what=f"{name} pad={pad}",
                        pad=pad)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [1, 2, 3, 7, 64, 65, 4097, 8193, 50001])
def test_forward_vocab_sizes(dtype, V):
    print(f"[forward] vocab V={V} {dtype}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(100 + V)
    T = 5
    z = (torch.randn(T, V, generator=g, device=DEV) * 2).to(dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[1] = -100
    for pad in ((False, True) if V % ROW_ALIGN else (False,)):
        compare_forward(z, t, alpha=1e-3, what=f"V={V} pad={pad}", pad=pad)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_forward_unaligned_rows(dtype):
    """A row stride that is not a multiple of 16 bytes takes the one-element
    kernel; an offset start does too."""
    g = torch.Generator(device=DEV).manual_seed(7)
    T, V = 9, 3001
    base = (torch.randn(T, V + 13, generator=g, device=DEV) * 3).to(dtype)
    z = base[:, 1:V + 1]
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[4] = -100
    compare_forward(z, t, alpha=1e-4, what="unaligned")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_forward_confident_rows(dtype):
    """Target margins 17..80: p_nt falls to ~e^-80 and so does the entropy;
    both the loss and the entropy keep relative 1e-5."""
    g = torch.Generator(device=DEV).manual_seed(21)
    T, V = 48, 9000
    z = torch.randn(T, V, generator=g, device=DEV) * 2
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    margin = torch.linspace(17, 80, T, device=DEV)
    z[torch.arange(T, device=DEV), t] = z.amax(dim=1) + margin
    z = z.to(dtype)
    loss, lse, ent, _, H = compare_forward(z, t, what="confident")
    assert bool((ent > 0).all())


def test_forward_infinities_and_bad_targets():
    T, V = 7, 300
    z = torch.randn(T, V, device=DEV, generator=torch.Generator(device=DEV).manual_seed(8))
    t = torch.tensor([5, 17, 299, 0, 150, 3, 1000], device=DEV)
    z[0, :100] = float("-inf")
    z[1, 17] = float("-inf")             # -inf target: the target term is 0
    z[2, :299] = float("-inf")           # one finite column: H = 0, lse = z_t
    z[3, 1::2] = float("-inf")
    loss, lse, ent, _, H = compare_forward(z, t, alpha=1e-2, what="inf")
    assert float(ent[2]) == 0.0 and float(lse[2]) == float(z[2, 299])
    assert math.isnan(float(ent[6])) and math.isnan(float(lse[6]))


def test_forward_uniform_rows_entropy_is_log_v():
    """Equal logits: the softmax is uniform and H = ln V, lse = c + ln V."""
    for V in (1000, 32000, 100003):
        z = torch.full((3, V), 1.5, device=DEV)
        t = torch.tensor([0, V // 2, V - 1], device=DEV)
        import loss_vocab_amd as L
        _, lse, ent, _ = L.ce_forward(z, t)
        torch.cuda.synchronize()
        check_loss(_np(ent), np.full(3, math.log(V)), f"uniform V={V} entropy")
        check_loss(_np(lse), np.full(3, 1.5 + math.log(V)), f"uniform V={V} lse")


def test_forward_matches_fused_loss_and_mask():
    """The loss of the forward entry equals the fused call's on the same rows
    (both to the oracle's tolerance), with the mask array in use."""
    import loss_vocab_amd as L
    wl = W["cez_bf16_T8192_V32000_collapse"].scaled(T=256)
    inp = make_inputs(wl, device=DEV)
    mask = (torch.arange(wl.T, device=DEV) % 5 != 0).to(torch.uint8)
    loss_f, _, _ = L.ce_fused(inp["logits"], inp["targets"], mask=mask, z_alpha=inp["z_alpha"],
                              want_grad=False)
    loss, lse, ent, _, H = compare_forward(inp["logits"], inp["targets"], mask=mask,
                                           alpha=inp["z_alpha"], what="mask")
    check_loss(_np(loss), to_np64(loss_f), "forward vs fused", rel=2e-6)


@pytest.mark.parametrize("V,dtype", [(2050, torch.bfloat16), (140005, torch.bfloat16),
                                     (70003, torch.float32)])
def test_forward_unaligned_mask(V, dtype):
    """A mask that starts at an odd address over 13 rows (bytes read within
    aligned 4-byte words inside the mask, by byte at the ends)."""
    g = torch.Generator(device=DEV).manual_seed(21)
    z = (2 * torch.randn(13, V, generator=g, device=DEV)).to(dtype)
    t = torch.randint(0, V, (13,), generator=g, device=DEV)
    t[6] = -100
    buf = torch.ones(13 + 8, dtype=torch.uint8, device=DEV)
    mask = buf[3:16]
    mask[[0, 3, 4, 7, 12]] = 0
    compare_forward(z, t, mask=mask, alpha=1e-4, what="unaligned mask", pad=True)
    compare_forward(z, t, mask=mask, alpha=1e-4, what="unaligned mask packed")


def test_forward_without_entropy():
    """entropy_out NULL runs the plain forward; lse alone is still written."""
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(3)
    z = torch.randn(33, 20000, generator=g, device=DEV).to(torch.bfloat16)
    t = torch.randint(0, 20000, (33,), generator=g, device=DEV)
    loss, lse, ent, _ = L.ce_forward(z, t, entropy=False)
    torch.cuda.synchronize()
    assert ent is None
    H, lse_ref = row_entropy(to_np64(z), _np(t))
    check_loss(_np(lse), lse_ref, "lse without entropy")


SHAPES = [(torch.float32, 50001), (torch.bfloat16, 100003), (torch.float32, 170003),
          (torch.bfloat16, 170003), (torch.bfloat16, (1 << 22) + 3), (torch.float32, (1 << 21) + 1)]


@pytest.mark.parametrize("dtype,V", SHAPES, ids=[f"{str(d)[6:]}-{v}" for d, v in SHAPES])
def test_forward_row_shapes(dtype, V):
    """Medium and long rows take the LDS-staged forward shapes (as padded
    16-byte rows; packed ragged rows take the one-element kernel): with and
    without the entropy output, and the fused call without a gradient."""
    import loss_vocab_amd as L
    print(f"[forward] shapes V={V} {dtype}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V)
    T = 6
    z = (torch.randn(T, V, generator=g, device=DEV) * 2).to(dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[2] = -100
    z[4, t[4]] = z[4].max() + 30          # a confident row
    compare_forward(z, t, alpha=1e-4, what=f"shape V={V}")
    compare_forward(z, t, alpha=1e-4, what=f"shape V={V} padded", pad=True)
    zp = padded_rows(z)
    loss2, lse2, ent2, _ = L.ce_forward(zp, t, z_alpha=1e-4, entropy=False)
    loss3, _, _ = L.ce_fused(zp, t, z_alpha=1e-4, want_grad=False)
    torch.cuda.synchronize()
    z64 = to_np64(z)
    ref = ce_oracle(z64, _np(t), z_alpha=1e-4, want_grad=False)
    _, lse_ref = row_entropy(z64, _np(t))
    check_loss(_np(loss2), ref["loss"], "forward without entropy")
    check_loss(_np(lse2), lse_ref, "lse without entropy")
    check_loss(_np(loss3), ref["loss"], "fused without gradient")


FULL = ["ce_f32_T256_V4096_mask10", "cez_bf16_T8192_V32000_collapse",
        "ce_bf16_T16384_V128256_zipf_inplace", "cez_f32_T32768_V151936_peaked",
        "cezseg_bf16_T65536_V201088_seg512"]


@pytest.mark.parametrize("name", FULL)
def test_forward_full_size(name):
    import loss_vocab_amd as L
    wl = W[name]
    print(f"[forward] full {name}", flush=True)
    inp = make_inputs(wl, device=DEV)
    T, V = wl.T, wl.V
    t_all = _np(inp["targets"])
    rng = np.random.default_rng(T + 1)
    valid = np.nonzero(t_all != -100)[0]
    rows = set(rng.choice(valid, size=min(40, valid.size), replace=False).tolist())
    planted = np.nonzero(inp["planted"].numpy())[0]
    if planted.size:
        rows |= set(rng.choice(planted, size=min(8, planted.size), replace=False).tolist())
    rows = np.array(sorted(rows | {0, T - 1}))
    ri = torch.as_tensor(rows, device=DEV)
    z_rows = to_np64(inp["logits"][ri])
    loss, lse, ent, seg = L.ce_forward(inp["logits"], inp["targets"],
                                       segment_ids=inp["segment_ids"],
                                       num_segments=inp["num_segments"], z_alpha=inp["z_alpha"])
    torch.cuda.synchronize()
    ref = ce_oracle(z_rows, t_all[rows], z_alpha=inp["z_alpha"], want_grad=False)
    H, lse_ref = row_entropy(z_rows, t_all[rows])
    check_loss(_np(loss)[rows], ref["loss"], f"{name} sampled loss")
    check_loss(_np(lse)[rows], lse_ref, f"{name} sampled lse")
    check_loss(_np(ent)[rows], H, f"{name} sampled entropy")
    # every row: 0 <= H <= ln V (up to the float rounding), ignored rows +0.0
    inv = torch.as_tensor(t_all == -100, device=DEV)
    e = ent[~inv]
    assert bool((e >= 0).all()) and bool((e <= math.log(V) * (1 + 1e-6)).all())
    assert _bits_zero(ent[inv]) and _bits_zero(lse[inv]) and _bits_zero(loss[inv])
    del inp, loss, lse, ent, seg
    torch.cuda.empty_cache()
