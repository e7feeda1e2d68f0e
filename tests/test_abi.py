"""The C ABI on the CPU: the library loads, exports what the header declares,
its struct layout matches the binding, and every host validation error comes
back as a status code before any HIP call (no kernel is launched here)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ce_fused.h")


def _lib():
    from loss_vocab_amd import _lib
    return _lib


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ce_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(_lib().EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib().LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib().LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported, name


@pytest.mark.parametrize("ctype,pytype", [("ce_problem", "CeProblem"), ("ce_shard", "CeShard"),
                                          ("ce_lmhead", "CeLmhead")])
def test_struct_layout_matches_header(tmp_path, ctype, pytype):
    """Compile a C probe with gcc against the header and compare offsets."""
    L = _lib()
    cls = getattr(L, pytype)
    fields = [f[0] for f in cls._fields_]
    src = tmp_path / "probe.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ce_fused.h"', 'int main(void){',
             f'printf("%zu\\n", sizeof({ctype}));']
    lines += [f'printf("%zu\\n", offsetof({ctype}, {f}));' for f in fields]
    lines += ["return 0;}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(cls)
    for f, off in zip(fields, vals[1:]):
        assert getattr(cls, f).offset == off, f


def test_status_strings():
    L = _lib()
    for code, name in [(0, "CE_OK"), (1, "CE_ERR_INVALID_ARG"), (2, "CE_ERR_UNSUPPORTED"),
                       (3, "CE_ERR_ALIAS"), (4, "CE_ERR_WORKSPACE"), (5, "CE_ERR_HIP"),
                       (6, "CE_ERR_TIMEOUT")]:
        assert L.status_string(code) == name
    assert L.status_string(99) == "CE_ERR_UNKNOWN"


def _problem(T=8, V=100, ld=None, ldg=None, dt=0, gdt=0, S=0, flags=0):
    L = _lib()
    p = L.CeProblem()
    p.T, p.V = T, V
    p.ld_logits = V if ld is None else ld
    p.ld_grad = V if ldg is None else ldg
    p.logits_dtype, p.grad_dtype = dt, gdt
    p.ignore_index = -100
    p.num_segments = S
    p.flags = flags
    return p


def test_workspace_bytes():
    L = _lib()
    assert L.workspace_bytes(_problem()) == 0
    # [T] floats and [S+1] int32 offsets, each rounded up to 256 bytes
    assert L.workspace_bytes(_problem(T=1000, S=7)) == 4096 + 256
    assert L.workspace_bytes(_problem(T=65536, S=512)) == 262144 + 2304
    assert L.LIB.ce_workspace_bytes(None) == 0
    # the debug scan's per-block words come after the segment arrays
    assert L.workspace_bytes(_problem(flags=2)) == 4096
    assert L.workspace_bytes(_problem(T=1000, S=7, flags=3)) == 4096 + 256 + 4096


# Fake device addresses: validation compares them, never dereferences them.
A_LOGITS = 0x10000000
A_TGT = 0x20000000
A_LOSS = 0x30000000
A_GRAD = 0x40000000
A_SEG = 0x50000000
A_WS = 0x60000000


def _call(p, logits=A_LOGITS, targets=A_TGT, mask=0, seg=0, za=0.0, gs=1.0, loss=A_LOSS,
          seg_out=0, grad=A_GRAD, lse=0, ws=0, ws_bytes=0):
    return _lib().call_raw(p, logits, targets, mask, seg, za, gs, loss, seg_out, grad, lse, ws,
                           ws_bytes, 0)


@pytest.mark.parametrize("case,kwargs,pkw,expect", [
    ("null problem", {}, None, 1),
    ("T < 0", {}, dict(T=-1), 1),
    ("V < 1", {}, dict(V=0), 1),
    ("ld_logits < V", {}, dict(ld=99), 1),
    ("ld_grad < V", {}, dict(ldg=50), 1),
    ("bad logits dtype", {}, dict(dt=7), 1),
    ("bad grad dtype", {}, dict(gdt=-1), 1),
    ("unknown flag", {}, dict(flags=0x8), 1),
    ("null logits", dict(logits=0), {}, 1),
    ("null targets", dict(targets=0), {}, 1),
    ("null loss_out", dict(loss=0), {}, 1),
    ("segments without ids", {}, dict(S=4), 1),
    ("ids without segments", dict(seg=A_SEG), {}, 1),
    ("negative segments", {}, dict(S=-2), 1),
    ("seg_loss_out without ids", dict(seg_out=A_LOSS + 4096), {}, 1),
    ("segment mean without ids", {}, dict(flags=1), 1),
    ("non-finite z_alpha", dict(za=float("nan")), {}, 1),
    ("non-finite grad_scale", dict(gs=float("inf")), {}, 1),
    ("grad overlaps logits (shifted)", dict(grad=A_LOGITS + 64), {}, 3),
    ("lse_out overlaps logits", dict(lse=A_LOGITS + 32), {}, 3),
    ("in place with another dtype", dict(grad=A_LOGITS), dict(gdt=1), 3),
    ("in place with another stride", dict(grad=A_LOGITS), dict(ldg=128, ld=100), 3),
    ("workspace missing", dict(seg=A_SEG), dict(S=4), 4),
    ("workspace too small", dict(seg=A_SEG, ws=A_WS, ws_bytes=100), dict(S=4), 4),
    ("V past the 2^28 in-row offset bound", {}, dict(V=(1 << 28) + 1), 2),
    ("validate without workspace", {}, dict(flags=2), 4),
    ("validate, workspace for segments only", dict(seg=A_SEG, ws=A_WS, ws_bytes=4096 + 256),
     dict(T=1000, S=7, flags=2), 4),
])
def test_validation_errors(case, kwargs, pkw, expect):
    p = None if pkw is None else _problem(**pkw)
    if p is None:
        st = _lib().LIB.ce_fused_fwd_bwd(None, None, None, None, None, 0.0, 1.0, None, None,
                                         None, None, None, 0, None)
    else:
        st = _call(p, **kwargs)
    assert st == expect, (case, _lib().status_string(st))


def test_product_path_has_no_fallback(monkeypatch, tmp_path):
    """Without the built library, importing the binding fails loudly."""
    import importlib
    import loss_vocab_amd._lib as lib_mod
    monkeypatch.setattr(os.path, "exists", lambda p: False if p.endswith("libce_fused.so") else True)
    with pytest.raises(ImportError):
        importlib.reload(lib_mod)
    monkeypatch.undo()
    importlib.reload(lib_mod)


def test_package_does_not_import_the_oracle():
    """The product package never references the oracle."""
    pkg = os.path.join(ROOT, "loss_vocab_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(dirpath, fn)) as f:
                    text = f.read()
                assert "oracle" not in text, fn


def _shard(T=8, V=100, v0=0, ld=None, ldg=None, dt=0, gdt=0):
    L = _lib()
    s = L.CeShard()
    s.T, s.V, s.v0 = T, V, v0
    s.ld_logits = V if ld is None else ld
    s.ld_grad = V if ldg is None else ldg
    s.logits_dtype, s.grad_dtype = dt, gdt
    s.ignore_index = -100
    return s


@pytest.mark.parametrize("case,kw,expect", [
    ("V < 1", dict(V=0), 1),
    ("negative v0", dict(v0=-1), 1),
    ("ld < V", dict(ld=50), 1),
    ("bad dtype", dict(dt=3), 1),
    ("huge V", dict(V=1 << 29, ld=1 << 29), 2),
])
def test_shard_stats_validation(case, kw, expect):
    st = _lib().shard_stats_raw(_shard(**kw), A_LOGITS, A_TGT, 0, A_LOSS, 0)
    assert st == expect, case


def test_shard_stats_null_pointers():
    L = _lib()
    assert L.shard_stats_raw(_shard(), 0, A_TGT, 0, A_LOSS, 0) == 1
    assert L.shard_stats_raw(_shard(), A_LOGITS, 0, 0, A_LOSS, 0) == 1
    assert L.shard_stats_raw(_shard(), A_LOGITS, A_TGT, 0, 0, 0) == 1
    assert L.LIB.ce_shard_stats(None, None, None, None, None, None) == 1


@pytest.mark.parametrize("case,kw,grad,expect", [
    ("no grad", {}, 0, 1),
    ("bad grad dtype", dict(gdt=5), A_GRAD, 1),
    ("ld_grad < V", dict(ldg=10), A_GRAD, 1),
    ("overlap", {}, A_LOGITS + 32, 3),
    ("in place other dtype", dict(gdt=1), A_LOGITS, 3),
])
def test_shard_grad_validation(case, kw, grad, expect):
    st = _lib().shard_grad_raw(_shard(**kw), A_LOGITS, A_TGT, A_WS, 0, 1.0, grad, 0)
    assert st == expect, case


def test_shard_grad_nonfinite_scale():
    assert _lib().shard_grad_raw(_shard(), A_LOGITS, A_TGT, A_WS, 0, float("nan"), A_GRAD, 0) == 1


@pytest.mark.parametrize("case,pkw,kw,expect", [
    ("no shards", {}, dict(n=0), 1),
    ("null stats", {}, dict(stats=0), 1),
    ("null row state", {}, dict(rs=0), 1),
    ("segments without ids", dict(S=3), {}, 1),
    ("workspace missing", dict(S=3), dict(seg=A_SEG), 4),
    ("bad flag", dict(flags=4), {}, 1),
    ("validate is for the fused calls", dict(flags=2), {}, 1),
])
def test_rows_finish_validation(case, pkw, kw, expect):
    p = _problem(**pkw)
    st = _lib().rows_finish_raw(p, kw.get("n", 2), kw.get("stats", A_LOGITS), A_TGT, 0,
                                kw.get("seg", 0), 0.0, A_LOSS, 0, kw.get("rs", A_GRAD), 0, 0, 0)
    assert st == expect, case


def test_build_script_does_not_import_the_package():
    """The build must run where the library is absent or stale, so loading
    build.py may not import the package (which loads the library)."""
    code = ("import sys, importlib.util;"
            f"spec = importlib.util.spec_from_file_location('b', {os.path.join(ROOT, 'loss_vocab_amd', 'build.py')!r});"
            "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m);"
            "assert 'loss_vocab_amd' not in sys.modules and 'loss_vocab_amd._lib' not in sys.modules;"
            "assert callable(m.build)")
    subprocess.run(["python", "-c", code], check=True, cwd="/")


def _fwd(p, logits=A_LOGITS, targets=A_TGT, loss=A_LOSS, lse=0, ent=0, seg=0, seg_out=0, ws=0,
         ws_bytes=0, za=0.0):
    return _lib().forward_raw(p, logits, targets, 0, seg, za, loss, seg_out, lse, ent, ws,
                              ws_bytes, 0)


@pytest.mark.parametrize("case,kw,pkw,expect", [
    ("null loss", dict(loss=0), {}, 1),
    ("null logits", dict(logits=0), {}, 1),
    ("lse overlaps logits", dict(lse=A_LOGITS + 16), {}, 3),
    ("entropy overlaps logits", dict(ent=A_LOGITS + 8 * 100 * 4 - 4), {}, 3),
    ("loss overlaps logits", dict(loss=A_LOGITS), {}, 3),
    ("non-finite z_alpha", dict(za=float("inf")), {}, 1),
    ("segments without workspace", dict(seg=A_SEG), dict(S=2), 4),
    ("bad logits dtype", {}, dict(dt=2), 1),
])
def test_forward_validation(case, kw, pkw, expect):
    st = _fwd(_problem(**pkw), **kw)
    assert st == expect, (case, _lib().status_string(st))


def test_forward_ignores_grad_fields():
    """grad_dtype and ld_grad are not read by the forward entry: a problem
    whose gradient fields are invalid still fails only on other checks."""
    p = _problem(gdt=9, ldg=1)
    assert _fwd(p, loss=0) == 1
    assert _fwd(p, lse=A_LOGITS) == 3


def _lm(T=8, V=100, H=64, ldh=None, ldw=None, dt=0, chunk=0):
    L = _lib()
    p = L.CeLmhead()
    p.T, p.V, p.H = T, V, H
    p.ld_hidden = H if ldh is None else ldh
    p.ld_weight = H if ldw is None else ldw
    p.ignore_index = -100
    p.dhidden_dtype = dt
    p.chunk_cols = chunk
    return p


A_W = 0x70000000
A_DW = 0x90000000


def _lmcall(p, hidden=A_LOGITS, weight=A_W, targets=A_TGT, loss=A_LOSS, lse=0, dh=0, dw=0,
            ws=A_WS, ws_bytes=1 << 40, za=0.0, gs=1.0):
    return _lib().lmhead_raw(p, hidden, weight, targets, 0, za, gs, loss, lse, dh, dw, ws,
                             ws_bytes, 0)


@pytest.mark.parametrize("case,pkw,kw,expect", [
    ("V < 1", dict(V=0), {}, 1),
    ("H < 1", dict(H=0), {}, 1),
    ("ld_hidden < H", dict(ldh=32), {}, 1),
    ("ld_weight < H", dict(ldw=8), {}, 1),
    ("bad dhidden dtype", dict(dt=4), {}, 1),
    ("negative chunk", dict(chunk=-1), {}, 1),
    ("H not a multiple of 8", dict(H=60), {}, 2),
    ("unaligned hidden", {}, dict(hidden=A_LOGITS + 2), 2),
    ("odd weight stride", dict(ldw=66), {}, 2),
    ("null weight", {}, dict(weight=0), 1),
    ("null loss", {}, dict(loss=0), 1),
    ("non-finite scale", {}, dict(gs=float("nan")), 1),
    ("workspace too small", {}, dict(ws_bytes=16), 4),
    ("unaligned workspace", {}, dict(ws=A_WS + 64), 4),
    ("dweight overlaps weight", {}, dict(dw=A_W + 128), 3),
    ("dhidden overlaps hidden", {}, dict(dh=A_LOGITS), 3),
    ("loss inside the workspace", {}, dict(loss=A_WS + 256), 3),
])
def test_lmhead_validation(case, pkw, kw, expect):
    st = _lmcall(_lm(**pkw), **kw)
    assert st == expect, (case, _lib().status_string(st))


def test_lmhead_workspace_grows_with_backward_and_chunk():
    L = _lib()
    p = _lm(T=1000, V=50000, H=256)
    fwd = L.lmhead_workspace_bytes(p, False)
    bwd = L.lmhead_workspace_bytes(p, True)
    assert 0 < fwd < bwd
    p.chunk_cols = 256
    assert L.lmhead_workspace_bytes(p, True) < bwd
    p.chunk_cols = 0
    p.dhidden_dtype = 1      # a bf16 dX adds an fp32 accumulator
    assert L.lmhead_workspace_bytes(p, True) > bwd
    assert L.LIB.ce_lmhead_workspace_bytes(None, 1) == 0


A_TEACH = 0xA0000000
A_KL = 0xB0000000


def _dcall(p, logits=A_LOGITS, teacher=A_TEACH, ldt=None, tdt=0, targets=A_TGT, loss=A_LOSS,
           kl=0, grad=A_GRAD, za=0.0, kb=1.0, gs=1.0):
    return _lib().distill_raw(p, logits, teacher, p.V if ldt is None else ldt, tdt, targets, 0, za,
                              kb, gs, loss, kl, grad, 0)


@pytest.mark.parametrize("case,pkw,kw,expect", [
    ("segments are not supported", dict(S=2), {}, 2),
    ("flags", dict(flags=1), {}, 1),
    ("bad teacher dtype", {}, dict(tdt=5), 1),
    ("teacher stride < V", {}, dict(ldt=50), 1),
    ("null teacher", {}, dict(teacher=0), 1),
    ("null loss", {}, dict(loss=0), 1),
    ("non-finite beta", {}, dict(kb=float("nan")), 1),
    ("grad over the teacher", {}, dict(grad=A_TEACH + 64), 3),
    ("grad overlapping logits (shifted)", {}, dict(grad=A_LOGITS + 4), 3),
    ("kl inside the logits", {}, dict(kl=A_LOGITS + 16), 3),
    ("loss inside the teacher", {}, dict(loss=A_TEACH), 3),
])
def test_distill_validation(case, pkw, kw, expect):
    st = _dcall(_problem(**pkw), **kw)
    assert st == expect, (case, _lib().status_string(st))


def test_distill_in_place_allowed():
    """grad_out == logits with the same dtype and stride passes validation
    (checked with T = 0 so nothing is launched)."""
    assert _dcall(_problem(T=0), grad=A_LOGITS) == 0


NO_DEVICE_PROBE = r"""
import sys
sys.path.insert(0, sys.argv[1])
from loss_vocab_amd import _lib as L
p = L.CeProblem()
p.T, p.V, p.ld_logits, p.ld_grad = 8, 100, 100, 100
p.logits_dtype = p.grad_dtype = 0
p.ignore_index = -100
out = {}
out["fused"] = L.call_raw(p, 0x10000000, 0x20000000, 0, 0, 0.0, 1.0, 0x30000000, 0, 0x40000000,
                          0x50000000, 0, 0, 0)
out["forward"] = L.forward_raw(p, 0x10000000, 0x20000000, 0, 0, 0.0, 0x30000000, 0, 0, 0, 0, 0, 0)
s = L.CeShard()
s.T, s.V, s.v0, s.ld_logits, s.ld_grad = 8, 100, 0, 100, 100
s.logits_dtype = s.grad_dtype = 0
s.ignore_index = -100
out["shard_stats"] = L.shard_stats_raw(s, 0x10000000, 0x20000000, 0, 0x30000000, 0)
out["rows_finish"] = L.rows_finish_raw(p, 1, 0x10000000, 0x20000000, 0, 0, 0.0, 0x30000000, 0,
                                       0x40000000, 0, 0, 0)
out["shard_grad"] = L.shard_grad_raw(s, 0x10000000, 0x20000000, 0x30000000, 0, 1.0, 0x40000000, 0)
out["noalloc"] = L.noalloc_raw(p, 0x10000000, 0x20000000, 0, 0, 0.0, 1.0, 0x30000000, 0,
                               0x40000000, 0, 0)
ps = L.CeProblem()
ps.T, ps.V, ps.ld_logits, ps.ld_grad, ps.num_segments = 8, 100, 100, 100, 2
ps.ignore_index = -100
out["noalloc_segments"] = L.noalloc_raw(ps, 0x10000000, 0x20000000, 0, 0x70000000, 0.0, 1.0,
                                        0x30000000, 0x80000000, 0x40000000, 0, 0)
out["distill"] = L.distill_raw(p, 0x10000000, 0x60000000, 100, 0, 0x20000000, 0, 0.0, 1.0, 1.0,
                               0x30000000, 0, 0x40000000, 0)
print(out)
"""


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present: the probe's fake "
                    "addresses would reach real kernels")
def test_valid_calls_without_a_device_return_ce_err_hip(tmp_path):
    """A call that passes every host check, made where no GPU exists, comes
    back as CE_ERR_HIP from its first HIP call and does not crash the process
    (a subprocess, so a crash would show as its exit status)."""
    import ast
    probe = tmp_path / "nodev.py"
    probe.write_text(NO_DEVICE_PROBE)
    res = subprocess.run(["python", str(probe), ROOT], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    got = ast.literal_eval(res.stdout.strip().splitlines()[-1])
    assert got == {k: 5 for k in ("fused", "forward", "shard_stats", "rows_finish", "shard_grad",
                                  "noalloc", "noalloc_segments", "distill")}, got


def test_forward_only_needs_no_pair_slots():
    """The gradient pass's row scheduling space: a 4-byte ticket counter
    (256 bytes) for rows of 8193..25600 16-byte chunks, and for fp32 rows of
    25601..51200 chunks (two workgroups per row) 32 bytes of exchange slots
    per row before it, and a give-up count after it. ce_workspace_bytes counts it; a call without a
    gradient (fused with grad_out NULL, or the forward entry) does not ask
    for it, while a gradient call still does. T = 0 keeps every call on the
    host (segment-free, so nothing is enqueued)."""
    L = _lib()
    p = _problem(T=1000, V=110000)
    assert L.workspace_bytes(p) == (1000 * 32 + 8 + 255) // 256 * 256
    assert L.workspace_bytes(_problem(T=1000, V=204800)) > 256
    for v, want in ((32768, 0), (32771, 0), (32772, 256), (65536, 256), (65540, 256),
                    (70000, 256), (102400, 256), (204804, 0), (300000, 0)):
        assert L.workspace_bytes(_problem(T=1000, V=v)) == want, v
    for v, want in ((65536, 0), (65543, 0), (65544, 256), (131072, 256), (131080, 256),
                    (201088, 256), (204800, 256), (204808, 0)):
        assert L.workspace_bytes(_problem(T=1000, V=v, dt=1)) == want, v
    p0 = _problem(T=0, V=110000)
    assert _call(p0, grad=A_GRAD) == 0 and _fwd(p0) == 0
    # rows present: without the slots a gradient call is refused, a
    # forward-only call is not refused for the workspace (it fails later, at
    # its first HIP call, where no device exists; it is not run where one does)
    assert _call(p, grad=A_GRAD) == 4
    if not os.path.exists("/dev/kfd"):
        assert _call(p, grad=0) == 5
        assert _fwd(p) == 5


def _noalloc(p, logits=A_LOGITS, targets=A_TGT, seg=0, loss=A_LOSS, seg_out=0, grad=A_GRAD, lse=0):
    return _lib().noalloc_raw(p, logits, targets, 0, seg, 0.0, 1.0, loss, seg_out, grad, lse, 0)


def test_noalloc_limits_and_validation():
    """The allocation-free entry refuses, before any HIP call, a problem whose
    workspace would exceed the fixed scratch (CE_ERR_WORKSPACE), and
    validates like the workspace entry."""
    L = _lib()
    assert L.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert L.LIB.ce_fused_fwd_bwd_noalloc(None, None, None, None, None, 0.0, 1.0, None, None,
                                          None, None, None) == 1
    # segments: 4 T bytes of staging past 8 MiB
    big = _problem(T=2_200_000, V=100, S=4, flags=1)
    assert _noalloc(big, seg=A_SEG, seg_out=A_LOSS + (1 << 24)) == 4
    # two-workgroup fp32 rows: 32 T + 8 bytes of slots past 8 MiB with a gradient
    pair = _problem(T=300_000, V=110000)
    assert _noalloc(pair) == 4
    # within the limit, host validation still applies first
    assert _noalloc(_problem(V=0)) == 1
    assert _noalloc(_problem(), grad=A_LOGITS + 64) == 3
    assert _noalloc(_problem(), lse=A_LOGITS) == 3
