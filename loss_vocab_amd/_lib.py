"""ctypes view of the C ABI declared in include/ce_fused.h.

Loading never touches the GPU. There is no fallback: if the built library is
absent, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libce_fused.so")

CE_DTYPE_F32 = 0
CE_DTYPE_BF16 = 1

CE_OK = 0
CE_ERR_INVALID_ARG = 1
CE_ERR_UNSUPPORTED = 2
CE_ERR_ALIAS = 3
CE_ERR_WORKSPACE = 4
CE_ERR_HIP = 5
CE_ERR_TIMEOUT = 6

CE_FLAG_SEGMENT_MEAN = 0x1
CE_FLAG_VALIDATE = 0x2

ROW_STATE = 8   # floats of saved state per row (ce_rows_finish)

# Every symbol include/ce_fused.h declares.
EXPORTS = ("ce_workspace_bytes", "ce_fused_fwd_bwd", "ce_fused_fwd_bwd_noalloc", "ce_fused_forward",
           "ce_shard_stats", "ce_rows_finish", "ce_shard_grad", "ce_lmhead_workspace_bytes",
           "ce_lmhead_fwd_bwd", "ce_fused_distill", "ce_status_string")

# Size of the library's fixed scratch array (CE_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 8 << 20


class CeProblem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("ld_logits", ctypes.c_int64),
        ("ld_grad", ctypes.c_int64),
        ("logits_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
        ("ignore_index", ctypes.c_int64),
        ("num_segments", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class CeShard(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("v0", ctypes.c_int64),
        ("ld_logits", ctypes.c_int64),
        ("ld_grad", ctypes.c_int64),
        ("logits_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
        ("ignore_index", ctypes.c_int64),
    ]


class CeLmhead(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("ld_hidden", ctypes.c_int64),
        ("ld_weight", ctypes.c_int64),
        ("ignore_index", ctypes.c_int64),
        ("dhidden_dtype", ctypes.c_int32),
        ("chunk_cols", ctypes.c_int32),
    ]


class CeError(RuntimeError):
    def __init__(self, status, where="ce_fused_fwd_bwd"):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)} ({status})")


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python loss_vocab_amd/build.py` "
            "(the fused CE has no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.ce_workspace_bytes.argtypes = [ctypes.POINTER(CeProblem)]
    lib.ce_workspace_bytes.restype = ctypes.c_size_t
    lib.ce_fused_fwd_bwd.argtypes = [
        ctypes.POINTER(CeProblem), vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
        vp, vp, vp, vp, vp, ctypes.c_size_t, vp,
    ]
    lib.ce_fused_fwd_bwd.restype = ctypes.c_int
    lib.ce_fused_fwd_bwd_noalloc.argtypes = [
        ctypes.POINTER(CeProblem), vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
        vp, vp, vp, vp, vp,
    ]
    lib.ce_fused_fwd_bwd_noalloc.restype = ctypes.c_int
    lib.ce_fused_forward.argtypes = [
        ctypes.POINTER(CeProblem), vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp,
        ctypes.c_size_t, vp,
    ]
    lib.ce_fused_forward.restype = ctypes.c_int
    lib.ce_shard_stats.argtypes = [ctypes.POINTER(CeShard), vp, vp, vp, vp, vp]
    lib.ce_shard_stats.restype = ctypes.c_int
    lib.ce_rows_finish.argtypes = [
        ctypes.POINTER(CeProblem), ctypes.c_int32, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
        vp, ctypes.c_size_t, vp,
    ]
    lib.ce_rows_finish.restype = ctypes.c_int
    lib.ce_shard_grad.argtypes = [ctypes.POINTER(CeShard), vp, vp, vp, vp, ctypes.c_float, vp, vp]
    lib.ce_shard_grad.restype = ctypes.c_int
    lib.ce_lmhead_workspace_bytes.argtypes = [ctypes.POINTER(CeLmhead), ctypes.c_int32]
    lib.ce_lmhead_workspace_bytes.restype = ctypes.c_size_t
    lib.ce_lmhead_fwd_bwd.argtypes = [
        ctypes.POINTER(CeLmhead), vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp, vp, vp, vp,
        vp, ctypes.c_size_t, vp,
    ]
    lib.ce_lmhead_fwd_bwd.restype = ctypes.c_int
    lib.ce_fused_distill.argtypes = [
        ctypes.POINTER(CeProblem), vp, vp, ctypes.c_int64, ctypes.c_int32, vp, vp, ctypes.c_float,
        ctypes.c_float, ctypes.c_float, vp, vp, vp, vp,
    ]
    lib.ce_fused_distill.restype = ctypes.c_int
    lib.ce_status_string.argtypes = [ctypes.c_int]
    lib.ce_status_string.restype = ctypes.c_char_p
    return lib


LIB = _load()


def status_string(status):
    return LIB.ce_status_string(int(status)).decode()


def workspace_bytes(problem):
    return int(LIB.ce_workspace_bytes(ctypes.byref(problem)))


def call_raw(problem, logits, targets, mask, segment_ids, z_alpha, grad_scale,
             loss_out, seg_loss_out, grad_out, lse_out, workspace, workspace_bytes_, stream):
    """Call ce_fused_fwd_bwd with integer addresses (0 = NULL); returns the status."""
    return int(LIB.ce_fused_fwd_bwd(
        ctypes.byref(problem), logits or None, targets or None, mask or None,
        segment_ids or None, float(z_alpha), float(grad_scale), loss_out or None,
        seg_loss_out or None, grad_out or None, lse_out or None, workspace or None,
        int(workspace_bytes_), stream or None))


def noalloc_raw(problem, logits, targets, mask, segment_ids, z_alpha, grad_scale,
                loss_out, seg_loss_out, grad_out, lse_out, stream):
    """Call ce_fused_fwd_bwd_noalloc with integer addresses (0 = NULL)."""
    return int(LIB.ce_fused_fwd_bwd_noalloc(
        ctypes.byref(problem), logits or None, targets or None, mask or None,
        segment_ids or None, float(z_alpha), float(grad_scale), loss_out or None,
        seg_loss_out or None, grad_out or None, lse_out or None, stream or None))


def forward_raw(problem, logits, targets, mask, segment_ids, z_alpha, loss_out, seg_loss_out,
                lse_out, entropy_out, workspace, workspace_bytes_, stream):
    """Call ce_fused_forward with integer addresses (0 = NULL); returns the status."""
    return int(LIB.ce_fused_forward(
        ctypes.byref(problem), logits or None, targets or None, mask or None,
        segment_ids or None, float(z_alpha), loss_out or None, seg_loss_out or None,
        lse_out or None, entropy_out or None, workspace or None, int(workspace_bytes_),
        stream or None))


def shard_stats_raw(shard, logits, targets, mask, stats, stream):
    return int(LIB.ce_shard_stats(ctypes.byref(shard), logits or None, targets or None,
                                  mask or None, stats or None, stream or None))


def rows_finish_raw(problem, num_shards, stats, targets, mask, segment_ids, z_alpha, loss_out,
                    seg_loss_out, row_state, workspace, workspace_bytes_, stream):
    return int(LIB.ce_rows_finish(
        ctypes.byref(problem), int(num_shards), stats or None, targets or None, mask or None,
        segment_ids or None, float(z_alpha), loss_out or None, seg_loss_out or None,
        row_state or None, workspace or None, int(workspace_bytes_), stream or None))


def shard_grad_raw(shard, logits, targets, row_state, row_weight, grad_scale, grad_out, stream):
    return int(LIB.ce_shard_grad(ctypes.byref(shard), logits or None, targets or None,
                                 row_state or None, row_weight or None, float(grad_scale),
                                 grad_out or None, stream or None))


def lmhead_workspace_bytes(problem, backward):
    return int(LIB.ce_lmhead_workspace_bytes(ctypes.byref(problem), int(bool(backward))))


def lmhead_raw(problem, hidden, weight, targets, mask, z_alpha, grad_scale, loss_out, lse_out,
               dhidden, dweight, workspace, workspace_bytes_, stream):
    return int(LIB.ce_lmhead_fwd_bwd(
        ctypes.byref(problem), hidden or None, weight or None, targets or None, mask or None,
        float(z_alpha), float(grad_scale), loss_out or None, lse_out or None, dhidden or None,
        dweight or None, workspace or None, int(workspace_bytes_), stream or None))


def distill_raw(problem, logits, teacher, ld_teacher, teacher_dtype, targets, mask, z_alpha,
                kl_beta, grad_scale, loss_out, kl_out, grad_out, stream):
    return int(LIB.ce_fused_distill(
        ctypes.byref(problem), logits or None, teacher or None, int(ld_teacher), int(teacher_dtype),
        targets or None, mask or None, float(z_alpha), float(kl_beta), float(grad_scale),
        loss_out or None, kl_out or None, grad_out or None, stream or None))
