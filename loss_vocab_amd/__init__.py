"""Fused vocabulary cross-entropy forward + backward on MI355X (gfx950).

The only compute path is the HIP library ``libce_fused.so`` built from
``csrc/ce_fused.hip``; this package marshals torch tensors into its C ABI
(``include/ce_fused.h``). torch provides device memory and the stream.
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import (  # noqa: F401
    CE_DTYPE_BF16,
    CE_DTYPE_F32,
    CE_FLAG_SEGMENT_MEAN,
    CE_FLAG_VALIDATE,
    CE_OK,
    CeError,
    CeLmhead,
    CeProblem,
    CeShard,
    status_string,
)

IGNORE_INDEX = -100

_DTYPES = {torch.float32: CE_DTYPE_F32, torch.bfloat16: CE_DTYPE_BF16}


def _ptr(t):
    return 0 if t is None else int(t.data_ptr())


def _rows(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0)


def make_problem(logits, grad_out=None, *, num_segments=0, segment_mean=False,
                 ignore_index=IGNORE_INDEX, validate=False):
    if logits.dtype not in _DTYPES:
        raise TypeError(f"logits dtype {logits.dtype} is not float32/bfloat16")
    T, V = logits.shape
    p = CeProblem()
    p.T, p.V = T, V
    p.ld_logits = _rows(logits, "logits")
    p.logits_dtype = _DTYPES[logits.dtype]
    if grad_out is not None:
        if grad_out.dtype not in _DTYPES:
            raise TypeError(f"grad_out dtype {grad_out.dtype} is not float32/bfloat16")
        if tuple(grad_out.shape) != (T, V):
            raise ValueError("grad_out must have the shape of logits")
        p.ld_grad = _rows(grad_out, "grad_out")
        p.grad_dtype = _DTYPES[grad_out.dtype]
    else:
        p.ld_grad = p.ld_logits
        p.grad_dtype = p.logits_dtype
    p.ignore_index = int(ignore_index)
    p.num_segments = int(num_segments)
    p.flags = (CE_FLAG_SEGMENT_MEAN if segment_mean else 0) | (CE_FLAG_VALIDATE if validate else 0)
    return p


def workspace_bytes(logits, *, num_segments=0, validate=False):
    return _lib.workspace_bytes(make_problem(logits, num_segments=num_segments, validate=validate))


def _workspace(need, device, stream):
    """A uint8 workspace of ``need`` bytes for a call enqueued on ``stream``
    (a hipStream_t as an integer). torch's caching allocator ties a block to
    the current stream; when the call goes to another stream the block is
    recorded on it, so it is not handed out again before the call has run."""
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    if int(stream) != int(torch.cuda.current_stream(device).cuda_stream):
        ws.record_stream(torch.cuda.ExternalStream(int(stream), device=device))
    return ws


def ce_fused_fwd_bwd(logits, targets, mask, segment_ids, z_alpha, grad_scale,
                     loss_out, seg_loss_out, grad_out, *, lse_out=None, num_segments=0,
                     segment_mean=False, ignore_index=IGNORE_INDEX, workspace=None,
                     stream=None, validate=False):
    """Same-named wrapper of the C entry point on torch tensors.

    logits [T, V] f32/bf16 (row stride free, unit column stride); targets [T]
    int64; mask [T] uint8 or None; segment_ids [T] int32 or None; loss_out [T]
    f32; seg_loss_out [S] f32 or None; grad_out [T, V] f32/bf16, ``logits``
    itself (in place) or None (forward only); lse_out [T] f32 or None (each
    row's full logsumexp); workspace: a uint8 device tensor of at least
    ``workspace_bytes`` bytes when segments are used (allocated here when
    None). The call is asynchronous on ``stream`` (default: torch's current
    stream). ``validate`` sets CE_FLAG_VALIDATE: a device scan of the targets
    and segment ids, after which the call waits for the stream and raises
    CeError(CE_ERR_INVALID_ARG) before writing anything if one is out of range
    or the ids are unsorted; on fp32 rows of 102404..204803 columns (two
    workgroups per row) it also waits for the kernels and raises
    CeError(CE_ERR_TIMEOUT) if a half row gave up waiting for its partner.
    Raises CeError on a non-OK status.
    """
    p = make_problem(logits, grad_out, num_segments=num_segments,
                     segment_mean=segment_mean, ignore_index=ignore_index, validate=validate)
    for name, t, dt in (("targets", targets, torch.int64), ("mask", mask, torch.uint8),
                        ("segment_ids", segment_ids, torch.int32),
                        ("loss_out", loss_out, torch.float32),
                        ("seg_loss_out", seg_loss_out, torch.float32),
                        ("lse_out", lse_out, torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous {dt} tensor")
    stream = _stream(logits, stream)
    need = _lib.workspace_bytes(p)
    if need and workspace is None:
        workspace = _workspace(need, logits.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.call_raw(p, _ptr(logits), _ptr(targets), _ptr(mask), _ptr(segment_ids),
                       z_alpha, grad_scale, _ptr(loss_out), _ptr(seg_loss_out),
                       _ptr(grad_out), _ptr(lse_out), _ptr(workspace), ws_bytes, stream)
    if st != CE_OK:
        raise CeError(st)


def ce_fused_fwd_bwd_noalloc(logits, targets, mask, segment_ids, z_alpha, grad_scale,
                             loss_out, seg_loss_out, grad_out, *, lse_out=None, num_segments=0,
                             segment_mean=False, ignore_index=IGNORE_INDEX, stream=None,
                             validate=False):
    """Same-named wrapper of the allocation-free C entry point: arguments as
    for ``ce_fused_fwd_bwd`` without a workspace (the library's fixed per-GPU
    scratch array serves instead; calls that may overlap on one GPU race on
    it). Allocates nothing; raises CeError(CE_ERR_WORKSPACE) when the problem
    needs more than ``_lib.NOALLOC_SCRATCH_BYTES`` of workspace."""
    p = make_problem(logits, grad_out, num_segments=num_segments,
                     segment_mean=segment_mean, ignore_index=ignore_index, validate=validate)
    for name, t, dt in (("targets", targets, torch.int64), ("mask", mask, torch.uint8),
                        ("segment_ids", segment_ids, torch.int32),
                        ("loss_out", loss_out, torch.float32),
                        ("seg_loss_out", seg_loss_out, torch.float32),
                        ("lse_out", lse_out, torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous {dt} tensor")
    st = _lib.noalloc_raw(p, _ptr(logits), _ptr(targets), _ptr(mask), _ptr(segment_ids),
                          z_alpha, grad_scale, _ptr(loss_out), _ptr(seg_loss_out),
                          _ptr(grad_out), _ptr(lse_out), _stream(logits, stream))
    if st != CE_OK:
        raise CeError(st, "ce_fused_fwd_bwd_noalloc")


def ce_fused(logits, targets, *, mask=None, segment_ids=None, num_segments=0,
             z_alpha=0.0, grad_scale=1.0, segment_mean=False, grad_dtype=None,
             in_place=False, want_grad=True, ignore_index=IGNORE_INDEX, validate=False,
             lse_out=None):
    """Allocate the outputs and run one fused call.

    Returns ``(loss[T] f32, grad[T, V] or None, seg_loss[S] f32 or None)``.
    With ``in_place`` the gradient overwrites ``logits`` and is returned;
    ``lse_out`` ([T] f32, optional) receives each row's full logsumexp.
    """
    T, V = logits.shape
    dev = logits.device
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    seg = torch.empty(num_segments, dtype=torch.float32, device=dev) if segment_ids is not None else None
    if not want_grad:
        grad = None
    elif in_place:
        grad = logits
    else:
        grad = torch.empty((T, V), dtype=grad_dtype or logits.dtype, device=dev)
    ce_fused_fwd_bwd(logits, targets, mask, segment_ids, z_alpha, grad_scale, loss, seg, grad,
                     lse_out=lse_out, num_segments=num_segments, segment_mean=segment_mean,
                     ignore_index=ignore_index, validate=validate)
    return loss, grad, seg


def ce_fused_forward(logits, targets, mask, segment_ids, z_alpha, loss_out, seg_loss_out,
                     lse_out, entropy_out, *, num_segments=0, ignore_index=IGNORE_INDEX,
                     workspace=None, stream=None, validate=False):
    """Same-named wrapper of the forward-only C entry point: loss_out [T] f32,
    seg_loss_out [S] f32 or None, lse_out / entropy_out [T] f32 or None;
    ``validate`` as for ``ce_fused_fwd_bwd``."""
    p = make_problem(logits, num_segments=num_segments, ignore_index=ignore_index,
                     validate=validate)
    for name, t, dt in (("targets", targets, torch.int64), ("mask", mask, torch.uint8),
                        ("segment_ids", segment_ids, torch.int32),
                        ("loss_out", loss_out, torch.float32),
                        ("seg_loss_out", seg_loss_out, torch.float32),
                        ("lse_out", lse_out, torch.float32),
                        ("entropy_out", entropy_out, torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous {dt} tensor")
    stream = _stream(logits, stream)
    need = _lib.workspace_bytes(p)
    if need and workspace is None:
        workspace = _workspace(need, logits.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.forward_raw(p, _ptr(logits), _ptr(targets), _ptr(mask), _ptr(segment_ids), z_alpha,
                          _ptr(loss_out), _ptr(seg_loss_out), _ptr(lse_out), _ptr(entropy_out),
                          _ptr(workspace), ws_bytes, stream)
    if st != CE_OK:
        raise CeError(st, "ce_fused_forward")


def ce_forward(logits, targets, *, mask=None, segment_ids=None, num_segments=0, z_alpha=0.0,
               entropy=True, ignore_index=IGNORE_INDEX, validate=False):
    """Allocate and run the forward-only call.

    Returns ``(loss[T], lse[T], entropy[T] or None, seg_loss[S] or None)``.
    """
    T = logits.shape[0]
    dev = logits.device
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev) if entropy else None
    seg = (torch.empty(num_segments, dtype=torch.float32, device=dev)
           if segment_ids is not None else None)
    ce_fused_forward(logits, targets, mask, segment_ids, z_alpha, loss, seg, lse, ent,
                     num_segments=num_segments, ignore_index=ignore_index, validate=validate)
    return loss, lse, ent, seg


# ---------------------------------------------------------------------------
# Split form: per-shard statistics, per-row finish, per-shard gradient.
# ---------------------------------------------------------------------------

def _stream(t, stream):
    return int(stream if stream is not None else torch.cuda.current_stream(t.device).cuda_stream)


def make_shard(logits, v0, grad_out=None, ignore_index=IGNORE_INDEX):
    if logits.dtype not in _DTYPES:
        raise TypeError(f"logits dtype {logits.dtype} is not float32/bfloat16")
    T, V = logits.shape
    s = CeShard()
    s.T, s.V, s.v0 = T, V, int(v0)
    s.ld_logits = _rows(logits, "logits")
    s.logits_dtype = _DTYPES[logits.dtype]
    if grad_out is not None:
        if grad_out.dtype not in _DTYPES or tuple(grad_out.shape) != (T, V):
            raise ValueError("grad_out must be float32/bfloat16 with the shard's shape")
        s.ld_grad = _rows(grad_out, "grad_out")
        s.grad_dtype = _DTYPES[grad_out.dtype]
    else:
        s.ld_grad, s.grad_dtype = s.ld_logits, s.logits_dtype
    s.ignore_index = int(ignore_index)
    return s


def ce_shard_stats(logits, targets, mask, stats, *, v0, ignore_index=IGNORE_INDEX, stream=None):
    """Pass 1 over the column shard ``logits`` = columns [v0, v0 + V) of the
    vocabulary; writes ``stats`` [T, 3] f32 (shift, sum, target logit)."""
    sh = make_shard(logits, v0, ignore_index=ignore_index)
    st = _lib.shard_stats_raw(sh, _ptr(logits), _ptr(targets), _ptr(mask), _ptr(stats),
                              _stream(logits, stream))
    if st != CE_OK:
        raise CeError(st, "ce_shard_stats")


def ce_rows_finish(num_shards, stats, targets, mask, segment_ids, z_alpha, loss_out, seg_loss_out,
                   row_state, *, vocab, num_segments=0, segment_mean=False,
                   ignore_index=IGNORE_INDEX, workspace=None, stream=None):
    """Merge ``stats`` [num_shards, T, 3] into loss_out [T], seg_loss_out [S]
    and row_state [T, 8] for a vocabulary of ``vocab`` columns."""
    p = CeProblem()
    p.T, p.V = targets.shape[0], int(vocab)
    p.ld_logits = p.ld_grad = p.V
    p.ignore_index = int(ignore_index)
    p.num_segments = int(num_segments)
    p.flags = CE_FLAG_SEGMENT_MEAN if segment_mean else 0
    stream = _stream(targets, stream)
    need = _lib.workspace_bytes(p)
    if need and workspace is None:
        workspace = _workspace(need, targets.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.rows_finish_raw(p, num_shards, _ptr(stats), _ptr(targets), _ptr(mask),
                              _ptr(segment_ids), z_alpha, _ptr(loss_out), _ptr(seg_loss_out),
                              _ptr(row_state), _ptr(workspace), ws_bytes, stream)
    if st != CE_OK:
        raise CeError(st, "ce_rows_finish")


def ce_shard_grad(logits, targets, row_state, grad_scale, grad_out, *, v0, row_weight=None,
                  ignore_index=IGNORE_INDEX, stream=None):
    """Pass 2 over a column shard from the saved ``row_state``; ``row_weight``
    [T] f32 (optional) weights each row's NLL gradient."""
    sh = make_shard(logits, v0, grad_out, ignore_index=ignore_index)
    st = _lib.shard_grad_raw(sh, _ptr(logits), _ptr(targets), _ptr(row_state), _ptr(row_weight),
                             grad_scale, _ptr(grad_out), _stream(logits, stream))
    if st != CE_OK:
        raise CeError(st, "ce_shard_grad")


def shard_bounds(V, num_shards, align=8):
    """Contiguous column ranges of ``num_shards`` shards, boundaries rounded to
    ``align`` columns (so shards of a 16-byte aligned row stay aligned)."""
    base = -(-V // num_shards)
    base = -(-base // align) * align
    out, v = [], 0
    while v < V:
        out.append((v, min(V, v + base)))
        v += base
    return out


def ce_split(logits, targets, *, shards=2, mask=None, segment_ids=None, num_segments=0,
             z_alpha=0.0, grad_scale=1.0, segment_mean=False, grad_dtype=None, in_place=False,
             align=8, row_weight=None, ignore_index=IGNORE_INDEX, grad_out=None):
    """The split form on one device: the columns of ``logits`` cut into shards,
    statistics per shard, one finish, gradient per shard.

    ``grad_out`` ([T, V], any row stride) receives the gradient when given
    (otherwise a new tensor, or ``logits`` itself with ``in_place``).
    Returns ``(loss[T], grad[T, V], seg_loss[S] or None, row_state[T, 8])``.
    """
    T, V = logits.shape
    dev = logits.device
    bounds = shard_bounds(V, shards, align)
    stats = torch.empty((len(bounds), T, 3), dtype=torch.float32, device=dev)
    for k, (a, b) in enumerate(bounds):
        ce_shard_stats(logits[:, a:b], targets, mask, stats[k], v0=a, ignore_index=ignore_index)
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    seg = (torch.empty(num_segments, dtype=torch.float32, device=dev)
           if segment_ids is not None else None)
    row_state = torch.empty((T, _lib.ROW_STATE), dtype=torch.float32, device=dev)
    ce_rows_finish(len(bounds), stats, targets, mask, segment_ids, z_alpha, loss, seg, row_state,
                   vocab=V, num_segments=num_segments, segment_mean=segment_mean,
                   ignore_index=ignore_index)
    if in_place:
        grad = logits
    elif grad_out is not None:
        grad = grad_out
    else:
        grad = torch.empty((T, V), dtype=grad_dtype or logits.dtype, device=dev)
    for a, b in bounds:
        ce_shard_grad(logits[:, a:b], targets, row_state, grad_scale, grad[:, a:b], v0=a,
                      row_weight=row_weight, ignore_index=ignore_index)
    return loss, grad, seg, row_state


# ---------------------------------------------------------------------------
# Loss behind a linear LM head (logits never stored whole).
# ---------------------------------------------------------------------------

def make_lmhead(hidden, weight, *, dhidden_dtype=torch.float32, chunk_cols=0,
                ignore_index=IGNORE_INDEX):
    for name, t in (("hidden", hidden), ("weight", weight)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    T, H = hidden.shape
    V, H2 = weight.shape
    if H != H2:
        raise ValueError("hidden and weight disagree on the hidden size")
    p = CeLmhead()
    p.T, p.V, p.H = T, V, H
    p.ld_hidden = _rows(hidden, "hidden")
    p.ld_weight = _rows(weight, "weight")
    p.ignore_index = int(ignore_index)
    p.dhidden_dtype = _DTYPES[dhidden_dtype]
    p.chunk_cols = int(chunk_cols)
    return p


def ce_lmhead_fwd_bwd(hidden, weight, targets, mask, z_alpha, grad_scale, loss_out, lse_out,
                      dhidden, dweight, *, chunk_cols=0, ignore_index=IGNORE_INDEX,
                      workspace=None, stream=None):
    """Same-named wrapper of the C entry point: hidden [T, H] bf16, weight
    [V, H] bf16, targets [T] int64, mask [T] uint8 or None, loss_out [T] f32,
    lse_out [T] f32 or None, dhidden [T, H] f32/bf16 or None, dweight [V, H]
    f32 or None (both None: forward only)."""
    p = make_lmhead(hidden, weight, dhidden_dtype=dhidden.dtype if dhidden is not None
                    else torch.float32, chunk_cols=chunk_cols, ignore_index=ignore_index)
    backward = dhidden is not None or dweight is not None
    stream = _stream(hidden, stream)
    need = _lib.lmhead_workspace_bytes(p, backward)
    if workspace is None:
        workspace = _workspace(max(need, 1), hidden.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    for name, t in (("dhidden", dhidden), ("dweight", dweight)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    st = _lib.lmhead_raw(p, _ptr(hidden), _ptr(weight), _ptr(targets), _ptr(mask), z_alpha,
                         grad_scale, _ptr(loss_out), _ptr(lse_out), _ptr(dhidden), _ptr(dweight),
                         _ptr(workspace), ws_bytes, stream)
    if st != CE_OK:
        raise CeError(st, "ce_lmhead_fwd_bwd")


def ce_lmhead(hidden, weight, targets, *, mask=None, z_alpha=0.0, grad_scale=1.0,
              want_grad=True, dhidden_dtype=torch.float32, chunk_cols=0,
              ignore_index=IGNORE_INDEX):
    """Allocate and run. Returns ``(loss[T], lse[T], dhidden or None, dweight or None)``."""
    T, H = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    dh = torch.empty((T, H), dtype=dhidden_dtype, device=dev) if want_grad else None
    dw = torch.empty((V, H), dtype=torch.float32, device=dev) if want_grad else None
    ce_lmhead_fwd_bwd(hidden, weight, targets, mask, z_alpha, grad_scale, loss, lse, dh, dw,
                      chunk_cols=chunk_cols, ignore_index=ignore_index)
    return loss, lse, dh, dw


# ---------------------------------------------------------------------------
# Distillation child on the same softmax pass.
# ---------------------------------------------------------------------------

def ce_fused_distill(logits, teacher, targets, mask, z_alpha, kl_beta, grad_scale, loss_out,
                     kl_out, grad_out, *, ignore_index=IGNORE_INDEX, stream=None):
    """Same-named wrapper of the C entry point: logits / teacher [T, V]
    f32/bf16 (unit column stride), loss_out [T] f32, kl_out [T] f32 or None,
    grad_out [T, V] f32/bf16, ``logits`` (in place) or None."""
    if teacher.dtype not in _DTYPES or tuple(teacher.shape) != tuple(logits.shape):
        raise ValueError("teacher must be float32/bfloat16 with the logits' shape")
    p = make_problem(logits, grad_out, ignore_index=ignore_index)
    for name, t, dt in (("targets", targets, torch.int64), ("mask", mask, torch.uint8),
                        ("loss_out", loss_out, torch.float32), ("kl_out", kl_out, torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous {dt} tensor")
    st = _lib.distill_raw(p, _ptr(logits), _ptr(teacher), _rows(teacher, "teacher"),
                          _DTYPES[teacher.dtype], _ptr(targets), _ptr(mask), z_alpha, kl_beta,
                          grad_scale, _ptr(loss_out), _ptr(kl_out), _ptr(grad_out),
                          _stream(logits, stream))
    if st != CE_OK:
        raise CeError(st, "ce_fused_distill")


def ce_distill(logits, teacher, targets, *, mask=None, z_alpha=0.0, kl_beta=1.0, grad_scale=1.0,
               grad_dtype=None, in_place=False, want_grad=True, ignore_index=IGNORE_INDEX):
    """Allocate and run. Returns ``(loss[T], kl[T], grad[T, V] or None)``."""
    T, V = logits.shape
    dev = logits.device
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    kl = torch.empty(T, dtype=torch.float32, device=dev)
    if not want_grad:
        grad = None
    elif in_place:
        grad = logits
    else:
        grad = torch.empty((T, V), dtype=grad_dtype or logits.dtype, device=dev)
    ce_fused_distill(logits, teacher, targets, mask, z_alpha, kl_beta, grad_scale, loss, kl, grad,
                     ignore_index=ignore_index)
    return loss, kl, grad
