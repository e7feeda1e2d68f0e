"""HIP path vs the fp64 oracle, element by element, on seeded inputs.

Small cases span several chunks per thread, the register-resident and the
streamed kernel variants, and ragged tails (V not a multiple of the 16-byte
width). Edge cases cover empty/degenerate shapes, strides, masks, infinities,
in-place and forward-only calls, segments and determinism. Full-size cases run
the five workload shapes in the benchmark's launch configuration and compare
sampled rows (and sampled segments) with the oracle, plus properties that hold
for every row.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from parity_utils import (ROW_ALIGN, check_grad, check_loss, check_zero_rows, padded_rows,
                          row_scales, run_hip, run_oracle, to_np64)
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


def compare_all(inp, *, grad_dtype=None, in_place=False, mask=None, want_grad=True, what="",
                pad=False):
    logits = inp["logits"]
    z64 = to_np64(logits)
    gdt = grad_dtype or logits.dtype
    loss, grad, seg = run_hip(inp, grad_dtype=gdt, in_place=in_place, want_grad=want_grad,
                              mask=mask, pad=pad)
    torch.cuda.synchronize()
    ref = run_oracle(z64, _np(inp["targets"]), mask=_np(mask), segment_ids=_np(inp.get("segment_ids")),
                     num_segments=inp.get("num_segments", 0), z_alpha=inp["z_alpha"],
                     grad_scale=inp["grad_scale"], segment_mean=inp.get("segment_mean", False),
                     want_grad=want_grad)
    check_loss(_np(loss), ref["loss"], what + " loss")
    inv = torch.as_tensor(~ref["valid"], device=DEV)
    check_zero_rows(loss[inv], grad[inv] if grad is not None else None)
    if want_grad:
        sc = row_scales(logits.shape[0], inp["grad_scale"], _np(inp.get("segment_ids")),
                        inp.get("num_segments", 0), inp.get("segment_mean", False))
        check_grad(to_np64(grad), ref["grad"], gdt, what + " grad", scale=sc,
                   targets=_np(inp["targets"]))
    if seg is not None:
        check_loss(_np(seg), ref["seg_nll"], what + " seg")
        empty = ref["seg_nll"] == 0
        assert np.all(_np(seg)[empty] == 0.0)
    return loss, grad, seg, ref


# ---------------------------------------------------------------------------
# The five workload recipes at sizes the oracle finishes in seconds
# ---------------------------------------------------------------------------

SMALL = [
    ("f32_mask10_T256_V4096", W["ce_f32_T256_V4096_mask10"], {}),
    ("bf16_collapse_zloss_ragged", W["cez_bf16_T8192_V32000_collapse"].scaled(T=300, V=3001), {}),
    ("bf16_collapse_zloss_V32000", W["cez_bf16_T8192_V32000_collapse"].scaled(T=48), {}),
    ("bf16_zipf_inplace_streamed", W["ce_bf16_T16384_V128256_zipf_inplace"].scaled(T=200, V=10007),
     {"in_place": True}),
    ("f32_peaked_zloss_streamed", W["cez_f32_T32768_V151936_peaked"].scaled(T=128, V=5003), {}),
    ("bf16_segments", W["cezseg_bf16_T65536_V201088_seg512"].scaled(T=2000, V=515, num_segments=37),
     {}),
]


@pytest.mark.parametrize("name,wl,opt", SMALL, ids=[s[0] for s in SMALL])
def test_small_workloads(name, wl, opt):
    print(f"[parity] {name} T={wl.T} V={wl.V}", flush=True)
    inp = make_inputs(wl, device=DEV)
    for pad in ((False, True) if wl.V % ROW_ALIGN else (False,)):
        compare_all(inp, in_place=opt.get("in_place", False), what=f"{name} pad={pad}", pad=pad)


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

def _inp(z, t, alpha=0.0, gamma=1.0, seg=None, S=0, seg_mean=False):
    return {"logits": z, "targets": t, "z_alpha": alpha, "grad_scale": gamma,
            "segment_ids": seg, "num_segments": S, "segment_mean": seg_mean}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [1, 2, 3, 7, 63, 64, 65, 4095, 4097, 8193])
def test_vocab_sizes(dtype, V):
    print(f"[parity] vocab V={V} {dtype}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V)
    T = 5
    z = (torch.randn(T, V, generator=g, device=DEV) * 2).to(dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[1] = -100
    compare_all(_inp(z, t, alpha=1e-3, gamma=0.25), what=f"V={V}")


@pytest.mark.parametrize("T", [1, 3, 257])
def test_row_counts(T):
    g = torch.Generator(device=DEV).manual_seed(T)
    z = torch.randn(T, 777, generator=g, device=DEV).to(torch.bfloat16)
    t = torch.randint(0, 777, (T,), generator=g, device=DEV)
    compare_all(_inp(z, t, alpha=1e-4, gamma=1.0 / T), what=f"T={T}")


def test_zero_rows():
    import loss_vocab_amd as L
    z = torch.empty(0, 100, device=DEV)
    t = torch.empty(0, dtype=torch.int64, device=DEV)
    loss, grad, _ = L.ce_fused(z, t)
    torch.cuda.synchronize()
    assert loss.numel() == 0 and grad.numel() == 0
    # T = 0 with segments still writes zero segment sums
    seg = torch.empty(0, dtype=torch.int32, device=DEV)
    out = torch.full((4,), 7.0, device=DEV)
    L.ce_fused_fwd_bwd(z, t, None, seg, 0.0, 1.0, torch.empty(0, device=DEV), out, None,
                       num_segments=4)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


@pytest.mark.parametrize("dtype,pad", [(torch.float32, 13), (torch.bfloat16, 13),
                                       (torch.float32, 7), (torch.bfloat16, 7)])
def test_row_stride_larger_than_V(dtype, pad):
    """V = 1001 in rows of 1014 elements (misaligned: the one-element path)
    or of 1008 (16-byte rows: the chunk kernel with a 1- or 9-column tail)."""
    g = torch.Generator(device=DEV).manual_seed(pad)
    T, V = 33, 1001
    big = (torch.randn(T, V + pad, generator=g, device=DEV) * 2).to(dtype)
    z = big[:, :V]
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[4] = -100
    gbig = torch.full((T, V + 7), 5.0, dtype=torch.float32, device=DEV)
    gout = gbig[:, :V]
    import loss_vocab_amd as L
    loss = torch.empty(T, device=DEV)
    L.ce_fused_fwd_bwd(z, t, None, None, 1e-4, 0.5, loss, None, gout)
    torch.cuda.synchronize()
    ref = run_oracle(to_np64(z), _np(t), z_alpha=1e-4, grad_scale=0.5)
    check_loss(_np(loss), ref["loss"])
    check_grad(to_np64(gout), ref["grad"], torch.float32, scale=0.5, targets=_np(t))
    assert torch.all(gbig[:, V:] == 5.0), "padding columns of the gradient were written"
    # the padding of the logits is never part of the result
    big[:, V:] = float("nan")
    loss2 = torch.empty(T, device=DEV)
    L.ce_fused_fwd_bwd(z, t, None, None, 1e-4, 0.5, loss2, None, None)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2)


def test_mask_array_and_ignore_index():
    g = torch.Generator(device=DEV).manual_seed(3)
    T, V = 64, 2050
    z = torch.randn(T, V, generator=g, device=DEV).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[[0, 9]] = -100
    mask = torch.ones(T, dtype=torch.uint8, device=DEV)
    mask[[1, 9, 40]] = 0
    z[1] = float("nan")            # an ignored row is never read
    z[40] = float("-inf")
    compare_all(_inp(z, t, alpha=1e-4, gamma=1 / 59), mask=mask, what="mask")


# A mask that starts at an odd address, over a row count that is not a
# multiple of 4: the kernels read a mask byte within its aligned 4-byte word
# when that word lies inside the mask, and with a byte load at the ends.
# Masked rows at the first and last rows and next to word edges; each shape
# runs one kernel tier (row kernel; row-resident in registers, with LDS
# slots; fp32 half rows in pairs).
MASK_TIER_CASES = [
    ("rows_bf16", torch.bfloat16, 2050),
    ("resident_reg_bf16", torch.bfloat16, 70001),
    ("resident_lds_bf16", torch.bfloat16, 140005),
    ("pair_f32", torch.float32, 110003),
]


@pytest.mark.parametrize("name,dtype,V", MASK_TIER_CASES, ids=[c[0] for c in MASK_TIER_CASES])
@pytest.mark.parametrize("offset", [1, 3])
def test_unaligned_mask(name, dtype, V, offset):
    g = torch.Generator(device=DEV).manual_seed(31 + offset)
    T = 13
    z = (2 * torch.randn(T, V, generator=g, device=DEV)).to(dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[6] = -100
    buf = torch.ones(T + 8, dtype=torch.uint8, device=DEV)
    mask = buf[offset:offset + T]
    assert mask.data_ptr() % 4 == offset % 4
    mask[[0, 3, 4, 7, 12]] = 0
    z[3] = float("nan")            # a masked row is never read
    inp = _inp(z, t, alpha=1e-4, gamma=1 / 7)
    compare_all(inp, mask=mask, what=f"unaligned mask {name}", pad=True)
    compare_all(inp, mask=mask, what=f"unaligned mask {name} packed")


@pytest.mark.parametrize("all_masked", [True, False])
def test_all_or_none_masked(all_masked):
    g = torch.Generator(device=DEV).manual_seed(4)
    T, V = 40, 3000
    z = torch.randn(T, V, generator=g, device=DEV)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    if all_masked:
        t[:] = -100
    loss, grad, _, _ = compare_all(_inp(z, t, alpha=1e-4), grad_dtype=torch.bfloat16,
                                   what="all/none")
    if all_masked:
        check_zero_rows(loss, grad)


def test_infinite_logits():
    T, V = 6, 300
    z = torch.randn(T, V, device=DEV, generator=torch.Generator(device=DEV).manual_seed(6))
    t = torch.tensor([5, 17, 299, 0, 150, 3], device=DEV)
    z[0, :100] = float("-inf")           # many -inf non-targets
    z[1, 17] = float("-inf")             # -inf target: NLL = +inf, target grad = -gamma
    z[2, :299] = float("-inf")           # every non-target -inf (acts as V = 1)
    z[3, 1::2] = float("-inf")
    compare_all(_inp(z, t, alpha=1e-2, gamma=0.5), what="inf")


def test_margin20_example_on_gpu():
    """The pages' worked example (torchtitan #5661, second review)."""
    z = torch.tensor([[0.0, 20.0]], device=DEV)
    t = torch.tensor([1], device=DEV)
    loss, grad, _, ref = compare_all(_inp(z, t), what="margin20")
    assert abs(float(loss[0]) - 2.06e-9) < 0.005e-9
    assert abs(float(grad[0, 1]) + 2.06e-9) < 0.005e-9
    assert abs(float(grad[0].double().sum())) < 1e-15


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_collapse_regime_nll(dtype):
    """Planted margins 17..45 (past the fp32 collapse point) without z-loss,
    so the stored loss is the tiny NLL itself and is checked to rel 1e-5."""
    g = torch.Generator(device=DEV).manual_seed(11)
    T, V = 64, 9000
    z = torch.randn(T, V, generator=g, device=DEV) * 2
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    margin = torch.linspace(17, 45, T, device=DEV)
    z[torch.arange(T, device=DEV), t] = z.amax(dim=1) + margin
    z = z.to(dtype)
    loss, grad, _, ref = compare_all(_inp(z, t, gamma=1 / T), what="collapse")
    assert torch.all(loss > 0)
    assert torch.all(grad[torch.arange(T, device=DEV), t] < 0)


@pytest.mark.parametrize("src,dst", [(torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)])
def test_mixed_dtypes(src, dst):
    g = torch.Generator(device=DEV).manual_seed(8)
    z = torch.randn(70, 4099, generator=g, device=DEV).to(src)
    t = torch.randint(0, 4099, (70,), generator=g, device=DEV)
    compare_all(_inp(z, t, alpha=1e-4, gamma=1 / 70), grad_dtype=dst, what="mixed")


@pytest.mark.parametrize("V", [4096, 50001])
def test_in_place_equals_out_of_place_and_forward_only(V):
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(V)
    z = (torch.randn(77, V, generator=g, device=DEV) * 3).to(torch.bfloat16)
    t = torch.randint(0, V, (77,), generator=g, device=DEV)
    t[5] = -100
    loss_a, grad_a, _ = L.ce_fused(z, t, z_alpha=1e-4, grad_scale=1 / 76)
    loss_f, none, _ = L.ce_fused(z, t, z_alpha=1e-4, grad_scale=1 / 76, want_grad=False)
    zc = z.clone()
    loss_b, grad_b, _ = L.ce_fused(zc, t, z_alpha=1e-4, grad_scale=1 / 76, in_place=True)
    torch.cuda.synchronize()
    assert none is None
    assert grad_b.data_ptr() == zc.data_ptr()
    # in place and out of place run one kernel: bit for bit
    assert torch.equal(loss_a, loss_b)
    assert torch.equal(grad_a.view(torch.int16), grad_b.view(torch.int16))
    # the forward-only call keeps nothing on chip and runs another workgroup
    # shape, so its partial sums merge in another order: equal up to the
    # fp32 rounding of the row statistics (the loss bar, rel 1e-5, holds)
    rel = ((loss_f - loss_a).abs() / loss_a.abs().clamp_min(1e-30)).max()
    assert float(rel) <= 2e-6
    assert float(loss_f[5]) == 0.0 and float(loss_a[5]) == 0.0


def test_z_alpha_zero_loss_is_nll():
    g = torch.Generator(device=DEV).manual_seed(12)
    z = torch.randn(50, 1234, generator=g, device=DEV)
    t = torch.randint(0, 1234, (50,), generator=g, device=DEV)
    seg = torch.zeros(50, dtype=torch.int32, device=DEV)
    seg[25:] = 1
    import loss_vocab_amd as L
    loss, _, segsum = L.ce_fused(z, t, segment_ids=seg, num_segments=2, z_alpha=0.0)
    torch.cuda.synchronize()
    ref = run_oracle(to_np64(z), _np(t), z_alpha=0.0)
    check_loss(_np(loss), ref["nll"])
    check_loss(_np(segsum), [ref["nll"][:25].sum(), ref["nll"][25:].sum()])


def test_out_of_range_targets_are_nan():
    z = torch.randn(4, 100, device=DEV)
    t = torch.tensor([100, -3, 7, 1000], device=DEV)
    compare_all(_inp(z, t), what="oob")


@pytest.mark.parametrize("layout", ["one", "singletons", "masked_segment", "empty_segments"])
def test_segment_layouts(layout):
    g = torch.Generator(device=DEV).manual_seed(21)
    T, V = 96, 700
    z = (torch.randn(T, V, generator=g, device=DEV) * 2).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    if layout == "one":
        seg, S = torch.zeros(T, dtype=torch.int32), 1
    elif layout == "singletons":
        seg, S = torch.arange(T, dtype=torch.int32), T
    elif layout == "masked_segment":
        seg, S = torch.arange(T, dtype=torch.int32) // 12, 8
        t[24:36] = -100                 # segment 2 fully ignored
    else:
        seg, S = torch.arange(T, dtype=torch.int32) // 12 * 2, 20   # odd ids and 16..19 empty
    inp = _inp(z, t, alpha=1e-4, gamma=1.0, seg=seg.to(DEV), S=S, seg_mean=True)
    _, _, segsum, ref = compare_all(inp, what=layout)
    if layout == "masked_segment":
        assert float(segsum[2]) == 0.0


DET_CASES = [("cez_bf16_T8192_V32000_collapse", 512, None),          # 512-lane tier
             ("ce_bf16_T16384_V128256_zipf_inplace", 700, None),    # registers only, fixed stride
             ("cezseg_bf16_T65536_V201088_seg512", 700, 16),        # 16 + 9 slots, dealt by ticket
             ("cez_f32_T32768_V151936_peaked", 600, None)]          # half rows, dealt by ticket


@pytest.mark.parametrize("name,T,S", DET_CASES, ids=[c[0] for c in DET_CASES])
def test_deterministic(name, T, S):
    """Two calls on the same inputs agree bit for bit, also where rows are
    dealt to workgroups in whatever order they ask (each row's arithmetic
    does not depend on which workgroup runs it)."""
    wl = W[name].scaled(T=T) if S is None else W[name].scaled(T=T, num_segments=S)
    inp = make_inputs(wl, device=DEV)
    a = run_hip(inp)
    b = run_hip(inp)
    torch.cuda.synchronize()
    bits = torch.int16 if a[1].dtype == torch.bfloat16 else torch.int32
    assert torch.equal(a[0].nan_to_num(7.0), b[0].nan_to_num(7.0))
    assert torch.equal(a[1].view(bits), b[1].view(bits))
    if a[2] is not None:
        assert torch.equal(a[2], b[2])


# ---------------------------------------------------------------------------
# Kernel tiers by row length in 16-byte chunks: up to 8192 chunks (512 lanes,
# 8 LDS slots per lane, rest streamed); up to 25600 (the row-resident kernel:
# 1024 lanes, 16 register slots then 9 LDS slots, the whole row on chip);
# beyond (1024 lanes, 4 VGPR + 9 LDS slots, rest streamed), and for fp32 rows
# up to 51200 chunks two workgroups per row, each row-resident on its half.
# Targets are placed in each kind of slot: register, LDS, streamed, the row's
# partial last slot and the tail past the last whole chunk.
# ---------------------------------------------------------------------------

TIER_CASES = [
    (torch.bfloat16, 4096 * 8), (torch.bfloat16, 4096 * 8 + 9), (torch.float32, 4096 * 4 - 3),
    (torch.bfloat16, 8192 * 8), (torch.bfloat16, 8192 * 8 + 8), (torch.bfloat16, 70001),
    (torch.bfloat16, 16384 * 8), (torch.bfloat16, 16384 * 8 + 3), (torch.bfloat16, 150000),
    (torch.float32, 8192 * 4 + 1), (torch.float32, 40000), (torch.float32, 70003),
    # row-resident rows: the end in the first LDS slot (16385 chunks), in a
    # middle one, and exactly filling all 25 slots (25600 chunks)
    (torch.bfloat16, 16385 * 8 + 5), (torch.bfloat16, (13312 + 8192) * 8),
    (torch.bfloat16, (13312 + 12288) * 8),
    # past one workgroup's chip space: bf16 rows take the streamed long-row
    # shape, fp32 rows two workgroups (halves of 13313 and 17408 chunks)
    (torch.bfloat16, 25601 * 8 + 3),
    (torch.float32, 2 * (13312 + 1) * 4), (torch.float32, 2 * (13312 + 4096) * 4),
]


def _tier_targets(V, W):
    nchunk = V // W
    lanes = 512 if nchunk <= 8192 else 1024
    marks = [0, 1, lanes - 1, lanes, 4 * lanes - 1, 4 * lanes, 8 * lanes - 1, 8 * lanes,
             13 * lanes - 1, 13 * lanes, 16 * lanes - 1, 16 * lanes, 17 * lanes + 5,
             24 * lanes + 3, nchunk - 1]
    elems = sorted({min(V - 1, c * W + (c % W)) for c in marks if c < max(nchunk, 1)})
    return elems + [V - 1, V // 2]


@pytest.mark.parametrize("dtype,V", TIER_CASES, ids=[f"{d}-{v}".replace("torch.", "") for d, v in TIER_CASES])
def test_kernel_tiers(dtype, V):
    W = 4 if dtype == torch.float32 else 8
    tg = _tier_targets(V, W)
    T = len(tg) + 2
    print(f"[parity] tier V={V} {dtype} T={T}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V)
    z = (torch.randn(T, V, generator=g, device=DEV) * 2.5)
    t = torch.tensor(tg + [-100, 3], device=DEV)
    # half the rows confident (collapse regime), so a wrong exclusion of the
    # target column shows in the NLL
    for i in range(0, len(tg), 2):
        z[i, tg[i]] = z[i].max() + 30.0
    z = z.to(dtype)
    # a ragged V with packed rows takes the one-element kernel; as the first
    # V columns of 16-byte aligned rows it takes the tier's chunk kernel and
    # its tail of V % W columns
    for pad in ((False, True) if V % ROW_ALIGN else (False,)):
        compare_all(_inp(z, t, alpha=1e-4, gamma=1.0 / (T - 1)), what=f"tier V={V} pad={pad}",
                    pad=pad)
        compare_all(_inp(z, t, alpha=1e-4, gamma=1.0 / (T - 1)),
                    grad_dtype=torch.float32 if dtype == torch.bfloat16 else torch.bfloat16,
                    what=f"tier V={V} mixed pad={pad}", pad=pad)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, (1 << 22) + 3), (torch.float32, (1 << 21) + 1)])
def test_very_long_rows(dtype, V):
    """Rows of millions of columns: hundreds of streamed slots per lane in
    the long-row tier, targets at the start, the middle and the last column."""
    print(f"[parity] long rows V={V} {dtype}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V % 1000)
    z = (torch.randn(4, V, generator=g, device=DEV) * 2).to(dtype)
    t = torch.tensor([0, V // 2 + 1, V - 1, -100], device=DEV)
    z[1, V // 2 + 1] = float(z[1].float().max()) + 30.0
    compare_all(_inp(z, t, alpha=1e-4, gamma=1.0 / 3), what=f"long V={V}")


def test_long_fp32_rows_two_workgroups_per_row():
    """fp32 rows past 25600 chunks run two workgroups per row that exchange
    their halves' statistics: segments, a mask, ignored and out-of-range rows,
    targets in either half and at the split, in place equal to out of place."""
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(71)
    T, V, S = 40, 110001, 3
    split = (V // 4 // 2) * 4
    z = torch.randn(T, V, generator=g, device=DEV) * 2
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[0], t[1], t[2], t[3] = split - 1, split, 0, V - 1
    t[5] = -100
    t[6] = V + 3                                  # out of range: NaN row
    z[7, t[7]] = z[7].max() + 35.0                # confident row
    mask = (torch.arange(T, device=DEV) % 9 != 4).to(torch.uint8)
    seg = (torch.arange(T, device=DEV) * S // T).to(torch.int32)
    inp = _inp(z, t, alpha=1e-4, gamma=1.0, seg=seg, S=S, seg_mean=True)
    # padded 16-byte rows (a ragged V as it runs on the pair kernel), then
    # packed rows (the one-element kernel) for comparison
    loss_a, grad_a, seg_a, _ = compare_all(inp, mask=mask, what="pair rows", pad=True)
    compare_all(inp, mask=mask, what="pair rows packed")
    zc = padded_rows(z)
    loss_b, grad_b, seg_b = L.ce_fused(zc, t, mask=mask, segment_ids=seg, num_segments=S,
                                       z_alpha=1e-4, grad_scale=1.0, segment_mean=True,
                                       in_place=True)
    torch.cuda.synchronize()
    assert torch.equal(loss_a.nan_to_num(7.0), loss_b.nan_to_num(7.0))
    assert torch.equal(grad_a.nan_to_num(7.0), grad_b.nan_to_num(7.0))
    assert torch.equal(seg_a.nan_to_num(7.0), seg_b.nan_to_num(7.0))   # a NaN row poisons its segment


def test_pair_give_up_is_reported(monkeypatch):
    """The two-workgroup fp32 rows' bounded wait, forced from the host: with
    the poll limit at 0 every half row gives up at once (no kernel waits),
    those rows come out NaN, and a validating call returns CE_ERR_TIMEOUT.
    With the limit restored the same validating call succeeds and matches
    the plain call bit for bit."""
    import loss_vocab_amd as L
    from loss_vocab_amd._lib import CE_ERR_TIMEOUT, CeError
    print("[parity] pair give-up report V=110003", flush=True)
    g = torch.Generator(device=DEV).manual_seed(17)
    T, V = 12, 110003
    z = padded_rows(torch.randn(T, V, generator=g, device=DEV))   # 16-byte rows: the pair kernel
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[3] = -100

    def call(validate=False):
        loss = torch.empty(T, device=DEV)
        grad = padded_rows(torch.empty(T, V, device=DEV), fill=0.0)
        L.ce_fused_fwd_bwd(z, t, None, None, 1e-4, 0.5, loss, None, grad, validate=validate)
        torch.cuda.synchronize()
        return loss, grad

    ref_loss, ref_grad = call()
    assert torch.isfinite(ref_loss).all()
    monkeypatch.setenv("CE_PAIR_SPIN_LIMIT", "0")
    loss, grad = call()
    live = t != -100
    assert torch.isnan(loss[live]).all() and torch.isnan(grad[live]).all()
    assert (loss[~live] == 0).all() and (grad[~live] == 0).all()
    with pytest.raises(CeError) as err:
        call(validate=True)
    assert err.value.status == CE_ERR_TIMEOUT
    monkeypatch.delenv("CE_PAIR_SPIN_LIMIT")
    loss_v, grad_v = call(validate=True)
    assert torch.equal(loss_v, ref_loss) and torch.equal(grad_v, ref_grad)


@pytest.mark.parametrize("dtype,V,T", [(torch.bfloat16, 201088, 600), (torch.float32, 151936, 520),
                                       (torch.bfloat16, 70001, 900)])
def test_row_resident_many_rows(dtype, V, T):
    """More rows than workgroups on the row-resident kernel (whole rows, and
    fp32 half rows in pairs): a workgroup issues its next read row's loads
    during the gradient pass and fills the ignored, masked and out-of-range
    rows it skips in between. Runs of skipped rows, a skipped last row,
    segments, and in place equal to out of place."""
    import loss_vocab_amd as L
    print(f"[parity] row-resident many rows V={V} T={T} {dtype}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V + T)
    z = (torch.randn(T, V, generator=g, device=DEV) * 2).to(dtype)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[::10] = -100                                 # every tenth row ignored
    t[256:262] = -100                              # a run of ignored rows
    t[T - 1] = -100                                # the last row is not read
    t[300] = V + 5                                 # out of range: NaN row
    mask = torch.ones(T, dtype=torch.uint8, device=DEV)
    mask[[7, 263, 511]] = 0
    for r in (5, 299, T - 3):
        z[r, t[r]] = float(z[r].float().max()) + 33.0
    S = 9
    seg = (torch.arange(T, device=DEV) * S // T).to(torch.int32)
    inp = _inp(z, t, alpha=1e-4, gamma=1.0, seg=seg, S=S, seg_mean=True)
    pad = V % ROW_ALIGN != 0                       # a ragged V runs as padded 16-byte rows
    loss_a, grad_a, seg_a, _ = compare_all(inp, mask=mask, what=f"rowres V={V}", pad=pad)
    zc = padded_rows(z) if pad else z.clone()
    loss_b, grad_b, seg_b = L.ce_fused(zc, t, mask=mask, segment_ids=seg, num_segments=S,
                                       z_alpha=1e-4, grad_scale=1.0, segment_mean=True,
                                       in_place=True)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(loss_a.nan_to_num(7.0), loss_b.nan_to_num(7.0))
    assert torch.equal(grad_a.nan_to_num(7.0).view(bits), grad_b.nan_to_num(7.0).view(bits))
    assert torch.equal(seg_a.nan_to_num(7.0), seg_b.nan_to_num(7.0))


def test_many_rows_per_workgroup():
    """More rows than workgroups: every workgroup loops over several rows."""
    g = torch.Generator(device=DEV).manual_seed(99)
    T, V = 40000, 77
    z = (torch.randn(T, V, generator=g, device=DEV) * 2).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[::7] = -100
    compare_all(_inp(z, t, alpha=1e-4, gamma=1.0 / T), what="many rows")


# ---------------------------------------------------------------------------
# Full sizes, as the benchmark launches them: sampled rows vs the oracle
# ---------------------------------------------------------------------------

def _sample_rows(inp, T, k=24):
    rng = np.random.default_rng(T)
    t = _np(inp["targets"])
    valid = np.nonzero(t != -100)[0]
    masked = np.nonzero(t == -100)[0]
    planted = np.nonzero(inp["planted"].numpy())[0]
    rows = {0, 1, T - 1, T - 2}
    rows |= set(rng.choice(valid, size=min(k, valid.size), replace=False).tolist())
    if masked.size:
        rows |= set(rng.choice(masked, size=min(6, masked.size), replace=False).tolist())
    if planted.size:
        rows |= set(rng.choice(planted, size=min(8, planted.size), replace=False).tolist())
    return np.array(sorted(rows))


FULL = ["ce_f32_T256_V4096_mask10", "cez_bf16_T8192_V32000_collapse",
        "ce_bf16_T16384_V128256_zipf_inplace", "cez_f32_T32768_V151936_peaked",
        "cezseg_bf16_T65536_V201088_seg512"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    import loss_vocab_amd as L
    wl = W[name]
    print(f"[parity] full {name}", flush=True)
    inp = make_inputs(wl, device=DEV)
    T, V = wl.T, wl.V
    rows = _sample_rows(inp, T)
    ri = torch.as_tensor(rows, device=DEV)
    z_rows = to_np64(inp["logits"][ri])
    seg_ids = inp["segment_ids"]
    # whole segments to check the sums on: first, last and two in between
    seg_check = []
    if seg_ids is not None:
        ids = _np(seg_ids)
        for s in (0, wl.num_segments // 3, 2 * wl.num_segments // 3, wl.num_segments - 1):
            r = np.nonzero(ids == s)[0]
            seg_check.append((s, r, to_np64(inp["logits"][torch.as_tensor(r, device=DEV)])))
    in_place = wl.grad == "inplace"
    loss, grad, seg = L.ce_fused(inp["logits"], inp["targets"], segment_ids=seg_ids,
                                 num_segments=wl.num_segments, z_alpha=inp["z_alpha"],
                                 grad_scale=inp["grad_scale"], segment_mean=inp["segment_mean"],
                                 grad_dtype=wl.grad_torch_dtype, in_place=in_place)
    torch.cuda.synchronize()
    t_all = _np(inp["targets"])
    # per-row scale: the segment length of each sampled row counts all rows of its id
    scale = np.full(rows.size, inp["grad_scale"])
    if inp["segment_mean"]:
        lens = np.bincount(_np(seg_ids), minlength=wl.num_segments)
        scale = inp["grad_scale"] / lens[_np(seg_ids)[rows]]
    ref = run_oracle(z_rows, t_all[rows], z_alpha=inp["z_alpha"], grad_scale=1.0)
    check_loss(_np(loss)[rows], ref["loss"], f"{name} sampled loss")
    # the oracle ran with scale 1; apply each row's scale (exact in fp64 for
    # the power-of-two-free factors up to rounding far below the tolerance)
    g_ref = ref["grad"] * scale[:, None]
    check_grad(to_np64(grad[ri]), g_ref, wl.grad_torch_dtype, f"{name} sampled grad", scale=scale,
               targets=t_all[rows])
    # every ignored row is +0.0, every valid loss finite
    inv = torch.as_tensor(t_all == -100, device=DEV)
    check_zero_rows(loss[inv], grad[inv])
    assert bool(torch.isfinite(loss[~inv]).all())
    # without z-loss every valid gradient row sums to zero (torchtitan #5661,
    # second review), up to the rounding of the stored values
    if inp["z_alpha"] == 0.0:
        eps = 2.0 ** -8 if wl.grad_torch_dtype == torch.bfloat16 else 1e-6
        vrows = torch.nonzero(~inv).flatten()
        for c0 in range(0, vrows.numel(), 1024):
            gb = grad[vrows[c0:c0 + 1024]].double()
            sums, absg = gb.sum(dim=1), gb.abs().sum(dim=1)
            assert bool((sums.abs() <= eps * absg + 1e-12).all())
            del gb
    if seg is not None:
        for s, r, zr in seg_check:
            o = run_oracle(zr, t_all[r], z_alpha=inp["z_alpha"], grad_scale=1.0, want_grad=False)
            ref_s = math.fsum(o["nll"][o["valid"]])
            check_loss([float(seg[s])], [ref_s], f"{name} segment {s}")
    del inp, loss, grad, seg
    torch.cuda.empty_cache()


def test_validate_flag():
    """CE_FLAG_VALIDATE: clean inputs give exactly the unchecked outputs; an
    out-of-range target, an id outside [0, S) or a decreasing id is refused
    with CE_ERR_INVALID_ARG before any output is written."""
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(33)
    T, V, S = 700, 1001, 9
    z = (torch.randn(T, V, generator=g, device=DEV) * 2).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[::7] = -100
    seg = (torch.arange(T, device=DEV) * S // T).to(torch.int32)
    kw = dict(segment_ids=seg, num_segments=S, z_alpha=1e-4, grad_scale=0.5)
    ref = L.ce_fused(z, t, **kw)
    got = L.ce_fused(z, t, validate=True, **kw)
    fwd_ref = L.ce_forward(z, t, segment_ids=seg, num_segments=S, z_alpha=1e-4)
    fwd = L.ce_forward(z, t, segment_ids=seg, num_segments=S, z_alpha=1e-4, validate=True)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    for a, b in zip(fwd_ref, fwd):
        assert torch.equal(a, b)

    def refused(targets, ids):
        loss = torch.full((T,), 7.0, device=DEV)
        grad = torch.full((T, V), 3.0, device=DEV, dtype=torch.bfloat16)
        segl = torch.full((S,), 5.0, device=DEV)
        with pytest.raises(L.CeError) as e:
            L.ce_fused_fwd_bwd(z, targets, None, ids, 0.0, 1.0, loss, segl, grad, num_segments=S,
                               validate=True)
        assert e.value.status == 1
        torch.cuda.synchronize()
        assert bool((loss == 7.0).all()) and bool((grad == 3.0).all()) and bool((segl == 5.0).all())

    bad_t = t.clone()
    bad_t[T - 1] = V
    refused(bad_t, seg)
    bad_t = t.clone()
    bad_t[300] = -5
    refused(bad_t, seg)
    bad_s = seg.clone()
    bad_s[T - 1] = S
    refused(t, bad_s)
    bad_s = seg.clone()
    bad_s[400] = 0                      # decreasing once
    refused(t, bad_s)


# ---------------------------------------------------------------------------
# lse_out on the fused call; fp32 gradients at unit scale with a large lse
# ---------------------------------------------------------------------------

LSE_CASES = [(torch.float32, 4099), (torch.bfloat16, 3001), (torch.bfloat16, 70001),
             (torch.bfloat16, 16385 * 8 + 5), (torch.float32, 70003)]


@pytest.mark.parametrize("dtype,V", LSE_CASES, ids=[f"{d}-{v}".replace("torch.", "") for d, v in LSE_CASES])
def test_lse_out_on_fused_call(dtype, V):
    """The optional lse_out of ce_fused_fwd_bwd: each valid row's full
    logsumexp (rel 1e-5 against the oracle), +0.0 for ignored rows and NaN for
    an out-of-range target, from the same pass, on every row-length tier (the
    last one is the two-workgroup fp32 mode). Loss and gradient are bit for
    bit those of the call without it."""
    import loss_vocab_amd as L
    print(f"[parity] lse_out V={V} {dtype}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V + 1)
    T = 24
    z = (torch.randn(T, V, generator=g, device=DEV) * 2.5)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[3] = -100
    t[7] = V + 2
    z[5, t[5]] = z[5].max() + 30.0
    z = z.to(dtype)
    lse = torch.full((T,), 9.0, device=DEV)
    loss_a, grad_a, _ = L.ce_fused(z, t, z_alpha=1e-4, grad_scale=0.25, lse_out=lse)
    loss_b, grad_b, _ = L.ce_fused(z, t, z_alpha=1e-4, grad_scale=0.25)
    torch.cuda.synchronize()
    ref = run_oracle(to_np64(z), _np(t), z_alpha=1e-4, grad_scale=0.25)
    check_loss(_np(lse), ref["lse"], "lse_out")
    assert float(lse[3]) == 0.0 and math.copysign(1.0, float(lse[3])) == 1.0
    assert math.isnan(float(lse[7]))
    assert torch.equal(loss_a.nan_to_num(7.0), loss_b.nan_to_num(7.0))
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(grad_a.view(bits), grad_b.view(bits))


# short rows (512-lane tier), register-only and register + LDS row-resident
# rows, two-workgroup fp32 rows, and the streamed long-row tier (fp32 past
# 51200 chunks, bf16 past 25600); ragged lengths run packed (one-element
# kernel) and padded (the chunk kernels and their tails)
FP32_UNIT_CASES = [(torch.float32, 3001), (torch.float32, 40000), (torch.float32, 70003),
                   (torch.bfloat16, 16385 * 8 + 5), (torch.float32, 8192 * 4 + 1),
                   (torch.float32, 110003), (torch.float32, 210001), (torch.bfloat16, 205001)]


@pytest.mark.parametrize("dtype,V", FP32_UNIT_CASES,
                         ids=[f"{d}-{v}".replace("torch.", "") for d, v in FP32_UNIT_CASES])
def test_fp32_grad_unit_scale_large_lse(dtype, V):
    """fp32 gradients at grad_scale 1 on rows whose logits sit near +-50 (so
    |lse| > 40, where one float carries lse log2(e) only to ~4e-6) and whose
    largest softmax value, 0.6-0.95, belongs to a non-target column placed in
    an on-chip slot, a streamed slot or the last chunk: every element within
    1e-6 absolute (and 2^-16 relative) of the oracle."""
    print(f"[parity] fp32 unit scale V={V} {dtype}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V + 7)
    T = 12
    z = torch.randn(T, V, generator=g, device=DEV) * 2
    W = 4 if dtype == torch.float32 else 8
    cols = [5, V // 2 + 3, V - 1 - (V % W) - 2, V - 1, 1100, 9 * 1024 * W + 17]
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    for r in range(T):
        j = cols[r % len(cols)] % V
        if int(t[r]) == j:
            t[r] = (j + 1) % V
        # dominant non-target: softmax value sigmoid(0.5 + 0.5 (r mod 6)) in 0.62..0.95
        z[r, j] = float(torch.logsumexp(z[r], 0)) + 0.5 + 0.5 * (r % 6)
        z[r] += 50.0 if r % 2 == 0 else -55.0
    z = z.to(dtype)
    for pad in ((False, True) if V % ROW_ALIGN else (False,)):
        compare_all(_inp(z, t, alpha=1e-4, gamma=1.0), grad_dtype=torch.float32,
                    what=f"unit V={V} pad={pad}", pad=pad)


def test_side_stream_without_workspace():
    """The binding allocates the segment workspace itself when none is given;
    on a stream other than torch's current one the block must not be handed
    out again before the call has run. The side stream is held busy first,
    so the call's kernels run late, and an allocation of the same size on
    the current stream is filled right after the call returns."""
    import loss_vocab_amd as L
    g = torch.Generator(device=DEV).manual_seed(21)
    T, V, S = 4096, 2048, 64
    z = torch.randn(T, V, generator=g, device=DEV)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    seg = (torch.arange(T, device=DEV) * S // T).to(torch.int32)
    need = L.workspace_bytes(z, num_segments=S)
    assert need > 0
    loss = torch.empty(T, device=DEV)
    segl = torch.empty(S, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)           # ~10 ms of spinning on the side stream
    L.ce_fused_fwd_bwd(z, t, None, seg, 0.0, 1.0, loss, segl, None, num_segments=S,
                       stream=side.cuda_stream)
    junk = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)   # current stream
    torch.cuda.synchronize()
    del junk
    ref = run_oracle(to_np64(z), _np(t), segment_ids=_np(seg), num_segments=S, want_grad=False)
    check_loss(_np(loss), ref["loss"], "side stream loss")
    check_loss(_np(segl), ref["seg_nll"], "side stream segments")
