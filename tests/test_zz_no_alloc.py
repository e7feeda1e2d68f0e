"""The allocation-free entry point (ce_fused_fwd_bwd_noalloc) against the
workspace entry point (ce_fused_fwd_bwd) through the C ABI: the same kernels,
so every output must agree bit for bit. Two calls in a row on each kernel
path that uses scratch (segment sums; two-workgroup fp32 rows with segments;
the debug scan), the second with a smaller input, so the second call runs on
scratch the first one left behind."""

from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import loss_vocab_amd  # noqa: F401  (raises if the HIP library is missing)
    yield
    torch.cuda.empty_cache()


def _bits(x):
    if x is None:
        return None
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def _rows(T, V, dtype, fill):
    """[T, V] as the first V columns of 16-byte aligned rows (ld a multiple
    of 8), so a ragged V still runs the chunk kernels."""
    ld = -(-V // 8) * 8
    return torch.full((T, ld), fill, dtype=dtype, device=DEV)[:, :V]


def _case(T, V, S, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    z = _rows(T, V, dtype, float("nan"))
    z.copy_(torch.randn(T, V, generator=g, device=DEV) * 2)
    t = torch.randint(0, V, (T,), generator=g, device=DEV)
    t[::11] = -100
    z[1, t[1]] = z[1].float().max() + 30.0
    seg = (torch.arange(T, device=DEV) * S // T).to(torch.int32) if S else None
    return z, t, seg


def _both(z, t, seg, S, gdt, validate=False):
    import loss_vocab_amd as L
    T, V = z.shape
    outs = []
    for fn in (L.ce_fused_fwd_bwd, L.ce_fused_fwd_bwd_noalloc):
        loss = torch.full((T,), 7.0, device=DEV)
        lse = torch.full((T,), 7.0, device=DEV)
        segl = torch.full((S,), 7.0, device=DEV) if S else None
        grad = _rows(T, V, gdt, 3.0)
        fn(z, t, None, seg, 1e-4, 1.0, loss, segl, grad, lse_out=lse, num_segments=S,
           segment_mean=S > 0, validate=validate)
        outs.append((loss, lse, segl, grad))
    torch.cuda.synchronize()
    (a, b) = outs
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        assert torch.equal(_bits(x), _bits(y))
    assert bool(torch.isfinite(a[0]).all())


@pytest.mark.parametrize("dtype,gdt,sizes", [
    (torch.bfloat16, torch.bfloat16, [(3000, 4099, 37), (1000, 3001, 5)]),
    (torch.float32, torch.float32, [(40, 110003, 3), (12, 110003, 2)]),   # two workgroups per row
    (torch.bfloat16, torch.float32, [(500, 16385 * 8 + 5, 4), (64, 2050, 1)]),
])
def test_noalloc_matches_workspace_call(dtype, gdt, sizes):
    for i, (T, V, S) in enumerate(sizes):
        print(f"[noalloc] T={T} V={V} S={S} {dtype}->{gdt}", flush=True)
        z, t, seg = _case(T, V, S, dtype, seed=T + V + i)
        _both(z, t, seg, S, gdt)


def test_noalloc_without_scratch_and_with_validate():
    """No segments and short rows (no scratch used), then the debug scan,
    which keeps its words in the scratch array, and its refusal."""
    import loss_vocab_amd as L
    z, t, _ = _case(300, 5003, 0, torch.bfloat16, seed=3)
    _both(z, t, None, 0, torch.bfloat16)
    z, t, seg = _case(700, 1001, 9, torch.bfloat16, seed=4)
    _both(z, t, seg, 9, torch.bfloat16, validate=True)
    bad = t.clone()
    bad[5] = 1001
    loss = torch.full((700,), 7.0, device=DEV)
    with pytest.raises(L.CeError) as e:
        L.ce_fused_fwd_bwd_noalloc(z, bad, None, seg, 0.0, 1.0, loss, None, None,
                                   num_segments=9, validate=True)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert bool((loss == 7.0).all())
