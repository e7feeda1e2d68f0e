"""Build the in-tree HIP library ``libce_fused.so`` for gfx950.

Run ``python loss_vocab_amd/build.py`` (or ``__graft_entry__.build()``); not
``python -m``, which imports the package and with it the library this builds.
The library is compiled by hipcc straight from ``csrc/*.hip``; it needs
no GPU to build. This file imports nothing of the package.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("ce_fused.hip", "lmhead_ce.hip", "distill_ce.hip")]
INC = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libce_fused.so")
ARCH = "gfx950"

# Packed-FP32 VALU forms are switched off for all device code. Machine-level
# loop-invariant code motion is off: the kernels are persistent loops over
# rows, and hoisting per-slot lane masks, offsets and fp64 constants out of
# the row loop only moved them into spilled registers (the row-resident
# kernel keeps a whole row in 64 VGPRs per lane and has none to spare).
HIP_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-disable-machine-licm",
    # Atomic read-modify-writes stay single-lane operations: the wave-level
    # rewrite would read each result right after issuing it, and on gfx9 that
    # wait drains every earlier load and store of the wave (one in-order
    # counter) -- a row-resident workgroup's ticket would hold up its row.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose=False, extra=()):
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-I", INC, *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
