"""Compile libcce.so for gfx950 in-tree (hipcc, no JIT cache).

Five translation units: the host API (cce.hip), the logit tile kernel
(tile.hip, built with the VGPR form of MFMA because the VALU rescales its
accumulator every quantization group), the dh contraction (dh.hip, whose
accumulators are best left to AGPRs), the dense head's dW contraction
(dw.hip) and the small kernels (kernels.hip).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
UNITS = {
    "cce.hip": [],
    "tile.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "kernels.hip": [],
    "dh.hip": [],
    "dw.hip": [],
}
HEADERS = [os.path.join(CSRC, "cce_device.h"), os.path.join(ROOT, "include", "cce.h"),
           os.path.join(ROOT, "include", "cce_profile.h")]
LIB = os.path.join(PKG, "libcce.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # no packed-fp32 VALU ops anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(force: bool = True, verbose: bool = False) -> str:
    deps = [os.path.join(CSRC, u) for u in UNITS] + HEADERS
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in deps):
        return LIB
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for unit, extra in UNITS.items():
        obj = os.path.join(BUILD_DIR, unit.replace(".hip", ".%d.o" % os.getpid()))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, unit)])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs], verbose)
    for o in objs:
        os.remove(o)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
