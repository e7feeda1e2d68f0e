"""The entry points under HIP graph capture.

A captured call enqueues only this library's kernels on the capturing
stream (no allocation, no memset: the workspace comes from the caller), so a
graph of it replays to the eager result. Each graph is replayed several times
with other device work and synchronisation between the replays, and every
replay is compared with the eager call bit for bit.
"""

from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import loss_vocab_amd  # noqa: F401
    yield
    torch.cuda.empty_cache()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _replay_matches(g, outs, ref, what):
    for rep in range(3):
        for o in outs:
            o.fill_(-7.0)                               # stale values must be rewritten
        junk = torch.randn(1 << 20, device=DEV).sum()   # other eager work in between
        g.replay()
        torch.cuda.synchronize()
        float(junk)
        for o, r in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(r)), f"{what}: replay {rep} differs"


def test_fused_call_with_segments_replays():
    import loss_vocab_amd as L
    gen = torch.Generator(device=DEV).manual_seed(5)
    T, V, S = 640, 20011, 11
    z = (torch.randn(T, V, generator=gen, device=DEV) * 2).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=gen, device=DEV)
    t[::9] = -100
    seg = (torch.arange(T, device=DEV) * S // T).to(torch.int32)
    loss = torch.empty(T, device=DEV)
    segl = torch.empty(S, device=DEV)
    grad = torch.empty(T, V, device=DEV, dtype=torch.bfloat16)
    ws = torch.empty(L.workspace_bytes(z, num_segments=S), dtype=torch.uint8, device=DEV)

    def call():
        L.ce_fused_fwd_bwd(z, t, None, seg, 1e-4, 1.0, loss, segl, grad, num_segments=S,
                           segment_mean=True, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = (loss.clone(), segl.clone(), grad.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                          # warm the launch paths off-capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replay_matches(g, (loss, segl, grad), ref, "fused")


def test_forward_and_distill_calls_replay():
    import loss_vocab_amd as L
    gen = torch.Generator(device=DEV).manual_seed(6)
    T, V = 300, 50021
    z = (torch.randn(T, V, generator=gen, device=DEV) * 2).to(torch.bfloat16)
    y = (torch.randn(T, V, generator=gen, device=DEV) * 2).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=gen, device=DEV)
    t[::5] = -100
    loss, lse, ent = (torch.empty(T, device=DEV) for _ in range(3))
    dl, kl = torch.empty(T, device=DEV), torch.empty(T, device=DEV)
    grad = torch.empty(T, V, device=DEV, dtype=torch.bfloat16)

    def call():
        L.ce_fused_forward(z, t, None, None, 1e-4, loss, None, lse, ent)
        L.ce_fused_distill(z, y, t, None, 1e-4, 0.5, 1.0 / T, dl, kl, grad)

    call()
    torch.cuda.synchronize()
    ref = tuple(x.clone() for x in (loss, lse, ent, dl, kl, grad))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replay_matches(g, (loss, lse, ent, dl, kl, grad), ref, "forward + distill")


def test_long_fp32_rows_replay():
    """fp32 rows past 25600 chunks run two workgroups per row, which take the
    row halves in ticket order and exchange statistics; the same ordinary
    launch is recorded under capture (a fill kernel resets the slots and the
    ticket counter). Every replay equals the eager call bit for bit: which
    workgroup takes which half does not change a half's arithmetic, and the
    merge of the two halves is symmetric."""
    import loss_vocab_amd as L
    gen = torch.Generator(device=DEV).manual_seed(7)
    T, V = 96, 110003
    # 16-byte aligned rows (ld 110008), as the two-workgroup kernel needs
    z = torch.empty(T, V + 5, device=DEV)[:, :V]
    z.copy_(torch.randn(T, V, generator=gen, device=DEV) * 2)
    t = torch.randint(0, V, (T,), generator=gen, device=DEV)
    t[::7] = -100
    loss = torch.empty(T, device=DEV)
    grad = torch.empty(T, V + 5, device=DEV)[:, :V]
    ws = torch.empty(max(1, L.workspace_bytes(z)), dtype=torch.uint8, device=DEV)

    def call():
        L.ce_fused_fwd_bwd(z, t, None, None, 1e-4, 1.0 / T, loss, None, grad, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = (loss.clone(), grad.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(_bits(loss), _bits(eager[0])), "loss vs eager"
    assert torch.equal(_bits(grad), _bits(eager[1])), "grad vs eager"
    _replay_matches(g, (loss, grad), eager, "long fp32 rows")


@pytest.mark.parametrize("V", [70001, 140005], ids=["registers", "registers_and_lds"])
def test_row_resident_rows_replay(V):
    """Whole rows of 8193..25600 chunks: one workgroup per CU takes rows in
    ticket order (a fill kernel resets the counter inside the call, so the
    call records into a graph). Ignored rows take their next ticket before
    their zero fill. Every replay equals the eager call bit for bit: which
    workgroup takes a row does not change the row's arithmetic."""
    import loss_vocab_amd as L
    gen = torch.Generator(device=DEV).manual_seed(8)
    T = 700
    # 16-byte aligned rows (ld V + 7), as the row-resident kernel needs
    z = torch.empty(T, V + 7, device=DEV, dtype=torch.bfloat16)[:, :V]
    z.copy_(torch.randn(T, V, generator=gen, device=DEV) * 2)
    t = torch.randint(0, V, (T,), generator=gen, device=DEV)
    t[::6] = -100
    loss = torch.empty(T, device=DEV)
    grad = torch.empty(T, V + 7, device=DEV, dtype=torch.bfloat16)[:, :V]
    ws = torch.empty(max(1, L.workspace_bytes(z)), dtype=torch.uint8, device=DEV)
    assert L.workspace_bytes(z) > 0, "row-resident rows are dealt by a ticket in the workspace"

    def call():
        L.ce_fused_fwd_bwd(z, t, None, None, 1e-4, 1.0 / T, loss, None, grad, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = (loss.clone(), grad.clone())
    g = _capture(call)
    _replay_matches(g, (loss, grad), eager, f"row-resident rows V={V}")


def _capture(call):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                          # warm the launch paths off-capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    return g


def test_split_calls_replay():
    """Per-shard statistics, the finish and per-shard gradients in one graph."""
    import loss_vocab_amd as L
    gen = torch.Generator(device=DEV).manual_seed(8)
    T, V = 200, 20011
    z = (torch.randn(T, V, generator=gen, device=DEV) * 2).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=gen, device=DEV)
    t[::6] = -100
    bounds = L.shard_bounds(V, 2, 8)
    stats = torch.empty(len(bounds), T, 3, device=DEV)
    row_state = torch.empty(T, L._lib.ROW_STATE, device=DEV)
    loss = torch.empty(T, device=DEV)
    grad = torch.empty(T, V, device=DEV, dtype=torch.bfloat16)

    def call():
        for k, (a, b) in enumerate(bounds):
            L.ce_shard_stats(z[:, a:b], t, None, stats[k], v0=a)
        L.ce_rows_finish(len(bounds), stats, t, None, None, 1e-4, loss, None, row_state, vocab=V)
        for a, b in bounds:
            L.ce_shard_grad(z[:, a:b], t, row_state, 1.0 / T, grad[:, a:b], v0=a)

    call()
    torch.cuda.synchronize()
    ref = (loss.clone(), row_state.clone(), grad.clone())
    g = _capture(call)
    _replay_matches(g, (loss, row_state, grad), ref, "split")


def test_lmhead_call_replays():
    """The LM-head loss (statistics, finish, chunked backward with dX and dW)
    with a caller-owned workspace."""
    import loss_vocab_amd as L
    gen = torch.Generator(device=DEV).manual_seed(9)
    T, V, H = 256, 1000, 128
    X = (torch.randn(T, H, generator=gen, device=DEV)).to(torch.bfloat16)
    W = (torch.randn(V, H, generator=gen, device=DEV) * 0.1).to(torch.bfloat16)
    t = torch.randint(0, V, (T,), generator=gen, device=DEV)
    t[::5] = -100
    loss, lse = torch.empty(T, device=DEV), torch.empty(T, device=DEV)
    dh = torch.empty(T, H, device=DEV)
    dw = torch.empty(V, H, device=DEV)
    p = L.make_lmhead(X, W, dhidden_dtype=torch.float32)
    ws = torch.empty(max(1, L._lib.lmhead_workspace_bytes(p, True)), dtype=torch.uint8, device=DEV)

    def call():
        L.ce_lmhead_fwd_bwd(X, W, t, None, 1e-4, 1.0 / T, loss, lse, dh, dw, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = (loss.clone(), lse.clone(), dh.clone(), dw.clone())
    g = _capture(call)
    _replay_matches(g, (loss, lse, dh, dw), ref, "lmhead")
