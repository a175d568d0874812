"""ctypes wrapper of the fp64 CPU oracle (cce_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.  See cce_oracle.c for what
is computed and which passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cce_oracle.c")
_LIB = os.path.join(_HERE, "libcce_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load(path: str):
    """Load an oracle build (the default one, or e.g. a test's mutated copy)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.oracle_cce.restype = ctypes.c_int
    lib.oracle_cce.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P, P, ctypes.c_int64,
                               ctypes.c_int, ctypes.c_int, ctypes.c_double, P, P, P, P,
                               ctypes.c_int64, P, P, P]
    lib.oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = load(build())
    return _lib


def threads() -> int:
    return int(_load().oracle_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def cce(inp: dict, tokens: Optional[Sequence[int]] = None, backward: bool = True,
        g: Optional[np.ndarray] = None, softcap: Optional[float] = None, lib=None):
    """Evaluate the head on `inp` (a dict from synthetic.make_inputs).

    Returns (logp, lse, dh) as float64 arrays indexed like `tokens` (all M tokens
    when tokens is None); dh is None when backward is False.
    """
    lib = _load() if lib is None else lib
    h = np.ascontiguousarray(inp["h"], dtype=np.uint16)
    wq = np.ascontiguousarray(inp["wq"], dtype=np.uint32)
    sc = np.ascontiguousarray(inp["scales"], dtype=np.float32)
    bi = np.ascontiguousarray(inp["biases"], dtype=np.float32)
    tg = np.ascontiguousarray(inp["targets"], dtype=np.int32)
    mk = inp.get("mask")
    mk = None if mk is None else np.ascontiguousarray(mk, dtype=np.uint8)
    gg = None if g is None else np.ascontiguousarray(g, dtype=np.float64)
    M, H, V = int(inp["M"]), int(inp["H"]), int(inp["V"])
    cap = float(inp["softcap"] if softcap is None else softcap)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = M if tok is None else len(tok)
    logp = np.zeros(n, np.float64)
    lse = np.zeros(n, np.float64)
    dh = np.zeros((n, H), np.float64) if backward else None
    rc = lib.oracle_cce(_ptr(h), M, H, _ptr(wq), _ptr(sc), _ptr(bi), V, int(inp["bits"]),
                        int(inp["group"]), cap, _ptr(tg), _ptr(mk), _ptr(gg), _ptr(tok), n,
                        _ptr(logp), _ptr(lse), _ptr(dh))
    if rc != 0:
        raise ValueError("oracle_cce rejected its arguments (rc=%d)" % rc)
    return logp, lse, dh
