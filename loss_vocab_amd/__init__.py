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
    CE_OK,
    CeError,
    CeProblem,
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
                 ignore_index=IGNORE_INDEX):
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
    p.flags = CE_FLAG_SEGMENT_MEAN if segment_mean else 0
    return p


def workspace_bytes(logits, *, num_segments=0):
    return _lib.workspace_bytes(make_problem(logits, num_segments=num_segments))


def ce_fused_fwd_bwd(logits, targets, mask, segment_ids, z_alpha, grad_scale,
                     loss_out, seg_loss_out, grad_out, *, num_segments=0,
                     segment_mean=False, ignore_index=IGNORE_INDEX, workspace=None,
                     stream=None):
    """Same-named wrapper of the C entry point on torch tensors.

    logits [T, V] f32/bf16 (row stride free, unit column stride); targets [T]
    int64; mask [T] uint8 or None; segment_ids [T] int32 or None; loss_out [T]
    f32; seg_loss_out [S] f32 or None; grad_out [T, V] f32/bf16, ``logits``
    itself (in place) or None (forward only); workspace: a uint8 device tensor
    of at least ``workspace_bytes`` bytes when segments are used (allocated
    here when None). The call is asynchronous on ``stream`` (default: torch's
    current stream). Raises CeError on a non-OK status.
    """
    p = make_problem(logits, grad_out, num_segments=num_segments,
                     segment_mean=segment_mean, ignore_index=ignore_index)
    for name, t, dt in (("targets", targets, torch.int64), ("mask", mask, torch.uint8),
                        ("segment_ids", segment_ids, torch.int32),
                        ("loss_out", loss_out, torch.float32),
                        ("seg_loss_out", seg_loss_out, torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous {dt} tensor")
    need = _lib.workspace_bytes(p)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(logits.device).cuda_stream
    st = _lib.call_raw(p, _ptr(logits), _ptr(targets), _ptr(mask), _ptr(segment_ids),
                       z_alpha, grad_scale, _ptr(loss_out), _ptr(seg_loss_out),
                       _ptr(grad_out), _ptr(workspace), ws_bytes, int(stream or 0))
    if st != CE_OK:
        raise CeError(st)


def ce_fused(logits, targets, *, mask=None, segment_ids=None, num_segments=0,
             z_alpha=0.0, grad_scale=1.0, segment_mean=False, grad_dtype=None,
             in_place=False, want_grad=True, ignore_index=IGNORE_INDEX):
    """Allocate the outputs and run one fused call.

    Returns ``(loss[T] f32, grad[T, V] or None, seg_loss[S] f32 or None)``.
    With ``in_place`` the gradient overwrites ``logits`` and is returned.
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
                     num_segments=num_segments, segment_mean=segment_mean,
                     ignore_index=ignore_index)
    return loss, grad, seg
