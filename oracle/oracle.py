"""fp64 CPU oracle: ctypes wrapper of cce_oracle.c, plus the approximate
backward (block skip, coefficient filter) written out on dense matrices.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.  See cce_oracle.c for what
is computed and which passages of the pages each step follows; the skip rules
and their readings are described above `cce_skip` below.
"""
from __future__ import annotations

import ctypes
import math
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


def _sb_f32(a, sb_dtype: str) -> np.ndarray:
    """Stored scales or biases widened exactly to fp32 (fp32, or the raw bits
    of bf16 / fp16)."""
    if sb_dtype == "f32":
        return np.asarray(a, np.float32)
    b = np.asarray(a, np.uint16)
    if sb_dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32)
    if sb_dtype == "f16":
        return b.view(np.float16).astype(np.float32)
    raise ValueError(sb_dtype)


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
    sc = np.ascontiguousarray(_sb_f32(inp["scales"], inp.get("sb_dtype", "f32")))
    bi = np.ascontiguousarray(_sb_f32(inp["biases"], inp.get("sb_dtype", "f32")))
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


# ---------------------------------------------------------------------------
# The approximate backward (opt-in skips), written out on dense fp64 matrices.
#
# Page "mlx-bun 0.0.4 -> 0.0.6", src/train/flash-cce.ts, the notes on the two
# backward skips and the scalar backward kernel's phase 1 / phase 2:
#   * block early exit: a (token block, vocabulary block) pair contributes
#     nothing when, for every token of the token block, the largest softmax
#     probability inside the vocabulary block is below eps and the token's
#     target lies outside it;
#   * coefficient filter: the contraction of a (token block, vocabulary block)
#     pair is skipped when every coefficient in it is below eps in magnitude.
# Readings fixed here (the pages' blocks are their own kernel tiles):
#   * token blocks are runs of TOKEN_TILE consecutive supervised tokens (in
#     index order; masked tokens are not counted); vocabulary blocks are rows
#     [BLOCK_V*b, BLOCK_V*(b+1)) clipped to V;
#   * "largest probability below eps" is block_max - lse < log(eps), where
#     block_max is the largest softcapped logit of the block;
#   * the filter looks at the non-target coefficients only, and a target's
#     term g*(1 - p)*c'*w is always kept: dropping it is never "small";
#   * eps = 0 turns a skip off; both skips on: the block rule first, the
#     filter on the pairs that stay.
# Dense [M, V] matrices: small inputs only.
# ---------------------------------------------------------------------------
BLOCK_V = 256
TOKEN_TILE = 256


def dequantize(inp: dict, v0: int = 0, v1: Optional[int] = None) -> np.ndarray:
    """W[v][d] = scale * q + bias in fp64 from the packed words (little-endian
    codes within each uint32, per-group scale and bias), rows [v0, v1)."""
    bits, group = int(inp["bits"]), int(inp["group"])
    v1 = int(inp["V"]) if v1 is None else v1
    wq = np.asarray(inp["wq"], dtype=np.uint32)[v0:v1]
    V, wpr = wq.shape
    per = 32 // bits
    shifts = (np.arange(per, dtype=np.uint32) * bits).astype(np.uint32)
    q = (wq[:, :, None] >> shifts[None, None, :]) & np.uint32((1 << bits) - 1)
    q = q.reshape(V, wpr * per).astype(np.float64)
    sbt = inp.get("sb_dtype", "f32")
    s = np.repeat(_sb_f32(inp["scales"][v0:v1], sbt).astype(np.float64), group, axis=1)
    b = np.repeat(_sb_f32(inp["biases"][v0:v1], sbt).astype(np.float64), group, axis=1)
    return s * q + b


def dense(inp: dict, g: Optional[np.ndarray] = None, softcap: Optional[float] = None) -> dict:
    """Every quantity of the plain definition as dense fp64 matrices over the
    supervised tokens: z, y, lse, logp, coefficients and the block maxima."""
    W = dequantize(inp)
    M, V = int(inp["M"]), int(inp["V"])
    cap = float(inp["softcap"] if softcap is None else softcap)
    mk = inp.get("mask")
    act = np.arange(M) if mk is None else np.flatnonzero(np.asarray(mk) != 0)
    hb = np.asarray(inp["h"], dtype=np.uint16)[act]
    hd = (hb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    z = hd @ W.T
    if cap > 0:
        th = np.tanh(z / cap)
        y, dc = cap * th, 1.0 - th * th
    else:
        y, dc = z, np.ones_like(z)
    mx = y.max(axis=1, keepdims=True)
    lse = (mx + np.log(np.exp(y - mx).sum(axis=1, keepdims=True)))[:, 0]
    tg = np.asarray(inp["targets"], np.int64)[act]
    t_in = (tg >= 0) & (tg < V)
    rows = np.arange(len(act))
    logp = np.where(t_in, y[rows, np.clip(tg, 0, V - 1)], 0.0) - lse
    gt = np.ones(len(act)) if g is None else np.asarray(g, np.float64)[act]
    p = np.exp(y - lse[:, None])
    coeff = -gt[:, None] * p * dc           # non-target part of every coefficient
    tcoef = np.zeros(len(act))              # the target's whole coefficient g*(1-p)*c'
    tcoef[t_in] = gt[t_in] * (1.0 - p[rows[t_in], tg[t_in]]) * dc[rows[t_in], tg[t_in]]
    coeff[rows[t_in], tg[t_in]] = 0.0
    nb = (V + BLOCK_V - 1) // BLOCK_V
    bmax = np.full((len(act), nb), -np.inf)
    for b in range(nb):
        bmax[:, b] = y[:, b * BLOCK_V:min(V, (b + 1) * BLOCK_V)].max(axis=1)
    return dict(W=W, act=act, z=z, y=y, lse=lse, logp=logp, coeff=coeff, tcoef=tcoef, tgt=tg,
                t_in=t_in, block_max=bmax)


def block_max(inp: dict, softcap: Optional[float] = None, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """[M, ceil(V/BLOCK_V)] largest softcapped logit per vocabulary block of
    each token; rows of masked tokens are 0.  With `tokens`, only those rows
    ([len(tokens), n_blocks]), computed over the head in row chunks so that a
    full-size head fits in memory."""
    if tokens is None:
        d = dense(inp, softcap=softcap)
        out = np.zeros((int(inp["M"]), d["block_max"].shape[1]))
        out[d["act"]] = d["block_max"]
        return out
    V = int(inp["V"])
    cap = float(inp["softcap"] if softcap is None else softcap)
    tok = np.asarray(tokens, np.int64)
    hb = np.asarray(inp["h"], dtype=np.uint16)[tok]
    hd = (hb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nb = (V + BLOCK_V - 1) // BLOCK_V
    out = np.zeros((len(tok), nb))
    step = 64 * BLOCK_V
    for v0 in range(0, V, step):
        v1 = min(V, v0 + step)
        z = hd @ dequantize(inp, v0, v1).T
        y = cap * np.tanh(z / cap) if cap > 0 else z
        for b in range(v0 // BLOCK_V, (v1 + BLOCK_V - 1) // BLOCK_V):
            out[:, b] = y[:, b * BLOCK_V - v0:min(v1, (b + 1) * BLOCK_V) - v0].max(axis=1)
    mk = inp.get("mask")
    if mk is not None:
        out[np.asarray(mk)[tok] == 0] = 0.0
    return out


def _pair_cold(bmax_tile, lse_tile, tgt_tile, b, block_eps):
    """Block rule for one (token tile, vocabulary block b) pair."""
    lo, hi = b * BLOCK_V, (b + 1) * BLOCK_V
    if np.any((tgt_tile >= lo) & (tgt_tile < hi)):
        return False
    return bool(np.all(bmax_tile[:, b] - lse_tile < math.log(block_eps)))


def _pair_filtered(coeff_pair, filter_eps):
    """Filter rule for one pair: every non-target coefficient below eps."""
    return bool(np.max(np.abs(coeff_pair), initial=0.0) < filter_eps)


def cce_skip(inp: dict, g: Optional[np.ndarray] = None, block_eps: float = 0.0,
             filter_eps: float = 0.0, softcap: Optional[float] = None):
    """(logp, lse, dh, dropped) over all M tokens with the two skips applied.

    `dropped` is the boolean [n_token_tiles, n_blocks] table of the pairs whose
    non-target coefficients were left out.
    """
    d = dense(inp, g=g, softcap=softcap)
    M, V, H = int(inp["M"]), int(inp["V"]), int(inp["H"])
    coeff = d["coeff"].copy()
    n = len(d["act"])
    nt = (n + TOKEN_TILE - 1) // TOKEN_TILE
    nb = d["block_max"].shape[1]
    dropped = np.zeros((nt, nb), dtype=bool)
    for k in range(nt):
        r0, r1 = k * TOKEN_TILE, min(n, (k + 1) * TOKEN_TILE)
        for b in range(nb):
            c0, c1 = b * BLOCK_V, min(V, (b + 1) * BLOCK_V)
            drop = block_eps > 0 and _pair_cold(d["block_max"][r0:r1], d["lse"][r0:r1],
                                                d["tgt"][r0:r1], b, block_eps)
            if not drop and filter_eps > 0:
                drop = _pair_filtered(coeff[r0:r1, c0:c1], filter_eps)
            if drop:
                coeff[r0:r1, c0:c1] = 0.0
                dropped[k, b] = True
    W = d["W"]
    dh_act = coeff @ W
    ti = np.flatnonzero(d["t_in"])
    dh_act[ti] += d["tcoef"][ti, None] * W[d["tgt"][ti]]
    logp = np.zeros(M)
    lse = np.zeros(M)
    dh = np.zeros((M, H))
    logp[d["act"]] = d["logp"]
    lse[d["act"]] = d["lse"]
    dh[d["act"]] = dh_act
    return logp, lse, dh, dropped


# ---------------------------------------------------------------------------
# Trainable dense head: W a bf16 [V, H] matrix instead of a quantized one.
# The same plain definition (page "mlx-bun 0.0.4 -> 0.0.6",
# src/train/flash-cce.ts, header comment: log-softmax of the softcapped logits,
# its gradient through the coefficient g * (1[v = target] - p_v) * c'(z_v)),
# plus the weight gradient that a frozen head does not need,
#     dW[v] = sum over supervised tokens t of coeff[t, v] * h[t],
# i.e. dW = coeff^T . h with the target's term inside the coefficient.
# W and h are widened exactly to fp64; numpy's fp64 matmul is the only library
# step.  Full-vocabulary rows are formed in chunks of V only to bound memory.
# ---------------------------------------------------------------------------
def _widen_bf16(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dense_core(hd: np.ndarray, Wd: np.ndarray, tgt: np.ndarray, gt: np.ndarray, cap: float,
               dw_rows: Optional[Sequence[int]] = None, need_dw: bool = True):
    """The definition on fp64 arrays: hd [n, H] supervised tokens, Wd [V, H],
    tgt [n] (outside [0, V): no target term), gt [n] cotangents.  Returns
    (logp, lse, dh, dw) with dw [V, H], or only the rows `dw_rows`."""
    n, V = hd.shape[0], Wd.shape[0]
    step = 16384
    Z = np.empty((n, V))
    for v0 in range(0, V, step):
        Z[:, v0:v0 + step] = hd @ Wd[v0:v0 + step].T
    if cap > 0:
        th = np.tanh(Z / cap)
        Y, DC = cap * th, 1.0 - th * th
    else:
        Y, DC = Z, np.ones_like(Z)
    mx = Y.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(Y - mx).sum(axis=1))
    rows = np.arange(n)
    t_in = (tgt >= 0) & (tgt < V)
    tc = np.clip(tgt, 0, V - 1)
    logp = np.where(t_in, Y[rows, tc], 0.0) - lse
    onehot = np.zeros_like(Y)
    onehot[rows[t_in], tgt[t_in]] = 1.0
    C = gt[:, None] * (onehot - np.exp(Y - lse[:, None])) * DC
    dh = np.zeros((n, Wd.shape[1]))
    for v0 in range(0, V, step):
        dh += C[:, v0:v0 + step] @ Wd[v0:v0 + step]
    dw = None
    if need_dw:
        dw = C.T @ hd if dw_rows is None else C[:, np.asarray(dw_rows)].T @ hd
    return logp, lse, dh, dw


def cce_dense(inp: dict, g: Optional[np.ndarray] = None, need_dw: bool = True,
              dw_rows: Optional[Sequence[int]] = None, tokens: Optional[Sequence[int]] = None):
    """(logp [M], lse [M], dh [M, H], dw) for a dict from synthetic.make_dense;
    masked tokens get 0 and add nothing to dw.  With `tokens`, only those
    tokens are evaluated (the others read as masked, in dw too); dw is [V, H],
    or its rows `dw_rows`."""
    M, H = int(inp["M"]), int(inp["H"])
    mk = inp.get("mask")
    sel = np.ones(M, bool) if mk is None else np.asarray(mk) != 0
    if tokens is not None:
        keep = np.zeros(M, bool)
        keep[np.asarray(tokens, np.int64)] = True
        sel &= keep
    act = np.flatnonzero(sel)
    hd = _widen_bf16(np.asarray(inp["h"])[act])
    Wd = _widen_bf16(inp["w"])
    tgt = np.asarray(inp["targets"], np.int64)[act]
    gt = np.ones(len(act)) if g is None else np.asarray(g, np.float64)[act]
    lp, ls, dh_a, dw = dense_core(hd, Wd, tgt, gt, float(inp["softcap"]), dw_rows, need_dw)
    logp, lse, dh = np.zeros(M), np.zeros(M), np.zeros((M, H))
    logp[act], lse[act], dh[act] = lp, ls, dh_a
    return logp, lse, dh, dw
