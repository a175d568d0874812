"""Thin Python binding of libcce (include/cce.h), same names as the C ABI.

Argument marshalling only: every step of the head runs in the HIP kernels of
libcce.so.  PyTorch supplies device memory and the current stream.  There is
no fallback: if libcce.so cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcce.so")

CCE_OK, CCE_ERR_INVALID_ARG, CCE_ERR_UNSUPPORTED, CCE_ERR_WORKSPACE, CCE_ERR_HIP = range(5)

EXPORTS = ("cce_forward", "cce_backward", "cce_forward_ex", "cce_backward_ex",
           "cce_forward_workspace_bytes", "cce_backward_workspace_bytes", "cce_status_str",
           "cce_abi_version", "cce_profile_enable", "cce_profile_read",
           "cce_dense_forward", "cce_dense_backward", "cce_dense_forward_workspace_bytes",
           "cce_dense_backward_workspace_bytes", "cce_forward_backward", "cce_forward_backward_workspace_bytes",
           "cce_forward_static", "cce_head_prepare", "cce_head_prepare_bytes",
           "cce_dense_forward_backward", "cce_dense_forward_backward_workspace_bytes")

BLOCK_V = 256      # CCE_BLOCK_V: vocabulary rows per block of block_max
TOKEN_TILE = 256   # CCE_TOKEN_TILE: supervised tokens per token tile of the skips


SB_DTYPES = {"f32": 0, "bf16": 1, "f16": 2}   # cce_sb_dtype
DH_DTYPES = {"f32": 0, "bf16": 1}            # cce_dh_dtype


class cce_head(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("V", ctypes.c_int64), ("H", ctypes.c_int64), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("softcap", ctypes.c_float), ("sb_dtype", ctypes.c_int32),
                ("prep", ctypes.c_void_p), ("prep_bytes", ctypes.c_size_t)]


class cce_dense_head(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("V", ctypes.c_int64), ("H", ctypes.c_int64), ("softcap", ctypes.c_float)]


class cce_skip(ctypes.Structure):
    _fields_ = [("block_eps", ctypes.c_float), ("filter_eps", ctypes.c_float)]


class cce_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class CceError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__("libcce status %d: %s" % (status, text))
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libcce.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libcce.so not built (%s); run linear_cross_entropy_libcce_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    HP = ctypes.POINTER(cce_head)
    lib.cce_forward.restype = ctypes.c_int
    lib.cce_forward.argtypes = [HP, P, I64, P, P, P, P, P, SZ, P]
    lib.cce_backward.restype = ctypes.c_int
    lib.cce_backward.argtypes = [HP, P, I64, P, P, P, P, P, P, SZ, P]
    lib.cce_forward_ex.restype = ctypes.c_int
    lib.cce_forward_ex.argtypes = [HP, P, I64, P, P, P, P, P, P, SZ, P]
    lib.cce_backward_ex.restype = ctypes.c_int
    lib.cce_backward_ex.argtypes = [HP, P, I64, P, P, P, P, P, ctypes.POINTER(cce_skip), P, ctypes.c_int32, P, SZ,
                                    P]
    lib.cce_forward_workspace_bytes.restype = SZ
    lib.cce_forward_workspace_bytes.argtypes = [HP, I64]
    lib.cce_backward_workspace_bytes.restype = SZ
    lib.cce_backward_workspace_bytes.argtypes = [HP, I64]
    lib.cce_forward_backward.restype = ctypes.c_int
    lib.cce_forward_backward.argtypes = [HP, P, I64, P, P, P, P, P, P, ctypes.c_int32, P, SZ, P]
    lib.cce_forward_backward_workspace_bytes.restype = SZ
    lib.cce_forward_backward_workspace_bytes.argtypes = [HP, I64]
    lib.cce_forward_static.restype = ctypes.c_int
    lib.cce_forward_static.argtypes = [HP, P, I64, P, P, P, P, P]
    lib.cce_head_prepare_bytes.restype = SZ
    lib.cce_head_prepare_bytes.argtypes = [HP]
    lib.cce_head_prepare.restype = ctypes.c_int
    lib.cce_head_prepare.argtypes = [HP, P, SZ, P]
    DP = ctypes.POINTER(cce_dense_head)
    lib.cce_dense_forward.restype = ctypes.c_int
    lib.cce_dense_forward.argtypes = [DP, P, I64, P, P, P, P, P, SZ, P]
    lib.cce_dense_backward.restype = ctypes.c_int
    lib.cce_dense_backward.argtypes = [DP, P, I64, P, P, P, P, P, P, P, SZ, P]
    lib.cce_dense_forward_workspace_bytes.restype = SZ
    lib.cce_dense_forward_workspace_bytes.argtypes = [DP, I64]
    lib.cce_dense_backward_workspace_bytes.restype = SZ
    lib.cce_dense_backward_workspace_bytes.argtypes = [DP, I64]
    lib.cce_dense_forward_backward.restype = ctypes.c_int
    lib.cce_dense_forward_backward.argtypes = [DP, P, I64, P, P, P, P, P, P, P, P, SZ, P]
    lib.cce_dense_forward_backward_workspace_bytes.restype = SZ
    lib.cce_dense_forward_backward_workspace_bytes.argtypes = [DP, I64]
    lib.cce_status_str.restype = ctypes.c_char_p
    lib.cce_status_str.argtypes = [ctypes.c_int]
    lib.cce_abi_version.restype = ctypes.c_int
    lib.cce_profile_enable.restype = ctypes.c_int
    lib.cce_profile_enable.argtypes = [ctypes.c_int]
    lib.cce_profile_read.restype = ctypes.c_int
    lib.cce_profile_read.argtypes = [ctypes.POINTER(cce_kernel_time), ctypes.c_int]
    _lib = lib
    return lib


def _check(status: int):
    if status != CCE_OK:
        raise CceError(status, load().cce_status_str(status).decode())


@dataclasses.dataclass
class Head:
    """Device tensors of a quantized head: wq uint32-as-int32 [V, H*bits/32],
    scales/biases [V, H/group] stored as float32, or as bf16 / fp16 (torch
    bfloat16 / float16, or their raw bits in int16 with sb_dtype set)."""
    wq: "object"
    scales: "object"
    biases: "object"
    bits: int
    softcap: float = 0.0
    group: int = 64
    sb_dtype: str = "f32"
    prep: "object" = None   # uint8 device tensor written by cce_head_prepare, or None

    @property
    def V(self) -> int:
        return int(self.scales.shape[0])

    @property
    def H(self) -> int:
        return int(self.scales.shape[1]) * self.group

    def c_struct(self) -> cce_head:
        return cce_head(self.wq.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr(),
                        self.V, self.H, self.bits, self.group, float(self.softcap), SB_DTYPES[self.sb_dtype],
                        _ptr(self.prep), 0 if self.prep is None else self.prep.numel())


@dataclasses.dataclass
class DenseHead:
    """A trainable dense head: w a contiguous bfloat16 [V, H] device tensor."""
    w: "object"
    softcap: float = 0.0

    @property
    def V(self) -> int:
        return int(self.w.shape[0])

    @property
    def H(self) -> int:
        return int(self.w.shape[1])

    def c_struct(self) -> cce_dense_head:
        return cce_dense_head(self.w.data_ptr(), self.V, self.H, float(self.softcap))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _expect(t, dtype, device, shape, name):
    if t.dtype != dtype or t.device != device or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s (got %s %s %s)"
                         % (name, dtype, tuple(shape), device, t.dtype, tuple(t.shape), t.device))


def _workspace(nbytes: int, device, workspace=None):
    import torch
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise CceError(CCE_ERR_WORKSPACE, "workspace too small")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def forward_workspace_bytes(head: Head, M: int) -> int:
    return int(load().cce_forward_workspace_bytes(ctypes.byref(head.c_struct()), M))


def backward_workspace_bytes(head: Head, M: int) -> int:
    return int(load().cce_backward_workspace_bytes(ctypes.byref(head.c_struct()), M))


def forward_backward_workspace_bytes(head: Head, M: int) -> int:
    return int(load().cce_forward_backward_workspace_bytes(ctypes.byref(head.c_struct()), M))


def dense_forward_workspace_bytes(head: DenseHead, M: int) -> int:
    return int(load().cce_dense_forward_workspace_bytes(ctypes.byref(head.c_struct()), M))


def dense_backward_workspace_bytes(head: DenseHead, M: int) -> int:
    return int(load().cce_dense_backward_workspace_bytes(ctypes.byref(head.c_struct()), M))


def dense_forward_backward_workspace_bytes(head: DenseHead, M: int) -> int:
    return int(load().cce_dense_forward_backward_workspace_bytes(ctypes.byref(head.c_struct()), M))


def n_blocks(head: Head) -> int:
    """Blocks per row of block_max: ceil(V / BLOCK_V)."""
    return (head.V + BLOCK_V - 1) // BLOCK_V


def _tokens(h, head: Head, targets, mask):
    import torch
    M, dev = int(h.shape[0]), h.device
    _expect(h, torch.bfloat16, dev, (M, head.H), "h")
    _expect(targets, torch.int32, dev, (M,), "targets")
    if mask is not None:
        _expect(mask, torch.uint8, dev, (M,), "mask")
    return M, dev


def _fwd_out(M, dev, out):
    import torch
    if out is not None:
        return out
    return torch.empty(M, dtype=torch.float32, device=dev), torch.empty(M, dtype=torch.float32, device=dev)


def _bwd_in(head: Head, M, dev, lse, g, out, dtype=None):
    import torch
    dtype = torch.float32 if dtype is None else dtype
    _expect(lse, torch.float32, dev, (M,), "lse")
    if g is not None:
        _expect(g, torch.float32, dev, (M,), "g")
    if out is not None:
        _expect(out, dtype, dev, (M, head.H), "out")
        return out
    return torch.empty((M, head.H), dtype=dtype, device=dev)


def cce_forward(h, head: Head, targets, mask=None, workspace=None, out=None):
    """(logp, lse), each float32 [M], for bf16 h [M, H] and int32 targets [M]."""
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    logp, lse = _fwd_out(M, dev, out)
    hs = head.c_struct()
    ws = _workspace(lib.cce_forward_workspace_bytes(ctypes.byref(hs), M), dev, workspace)
    _check(lib.cce_forward(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(logp), _ptr(lse),
                           _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return logp, lse


STATIC_SCRATCH_BYTES = 128 << 20   # CCE_STATIC_SCRATCH_BYTES


def cce_head_prepare_bytes(head: Head) -> int:
    """Bytes of the head's prepared buffer (0 for an invalid head)."""
    hs = head.c_struct()
    hs.prep, hs.prep_bytes = None, 0
    return int(load().cce_head_prepare_bytes(ctypes.byref(hs)))


def cce_head_prepare(head: Head, prep=None):
    """Write the head's preparation (into `prep`, a uint8 device tensor, or a
    new one) on the current stream and attach it to `head`: later calls skip
    the per-call preparation.  Returns the buffer.  Call again after changing
    wq, scales or biases (or set head.prep = None)."""
    import torch
    lib = load()
    dev = head.scales.device
    nb = cce_head_prepare_bytes(head)
    if nb == 0:
        raise CceError(CCE_ERR_INVALID_ARG, "invalid head")
    if prep is None:
        prep = torch.empty(nb, dtype=torch.uint8, device=dev)
    hs = head.c_struct()
    hs.prep, hs.prep_bytes = None, 0
    _check(lib.cce_head_prepare(ctypes.byref(hs), _ptr(prep), prep.numel(), _stream(dev)))
    head.prep = prep
    return prep


def cce_forward_static(h, head: Head, targets, mask=None, out=None):
    """(logp, lse) like cce_forward, with the library's own device scratch as
    the workspace (no workspace argument, nothing allocated by the library)."""
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    logp, lse = _fwd_out(M, dev, out)
    hs = head.c_struct()
    _check(lib.cce_forward_static(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(logp), _ptr(lse),
                                  _stream(dev)))
    return logp, lse


def cce_forward_ex(h, head: Head, targets, mask=None, block_max=True, workspace=None, out=None):
    """(logp, lse, block_max): block_max float32 [M, n_blocks(head)], allocated
    (True), given as a tensor to write into, or not produced (None)."""
    import torch
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    logp, lse = _fwd_out(M, dev, out)
    bmx = None
    if block_max is True:
        bmx = torch.empty((M, n_blocks(head)), dtype=torch.float32, device=dev)
    elif block_max is not None and block_max is not False:
        _expect(block_max, torch.float32, dev, (M, n_blocks(head)), "block_max")
        bmx = block_max
    hs = head.c_struct()
    ws = _workspace(lib.cce_forward_workspace_bytes(ctypes.byref(hs), M), dev, workspace)
    _check(lib.cce_forward_ex(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(logp), _ptr(lse),
                              _ptr(bmx), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return logp, lse, bmx


def cce_backward(h, head: Head, targets, lse, g=None, mask=None, workspace=None, out=None):
    """dh float32 [M, H] = g * d logp / d h (g = None means all ones)."""
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    dh = _bwd_in(head, M, dev, lse, g, out)
    hs = head.c_struct()
    ws = _workspace(lib.cce_backward_workspace_bytes(ctypes.byref(hs), M), dev, workspace)
    _check(lib.cce_backward(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(lse), _ptr(g),
                            _ptr(dh), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return dh


def cce_backward_ex(h, head: Head, targets, lse, g=None, mask=None, block_max=None, block_eps=0.0,
                    filter_eps=0.0, workspace=None, out=None, dh_dtype="f32"):
    """dh with the opt-in skips (block_eps needs block_max from cce_forward_ex), as
    float32 or, with dh_dtype="bf16", bfloat16 (the fp32 result rounded once)."""
    import torch
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    if dh_dtype not in DH_DTYPES:
        raise ValueError("dh_dtype must be one of %s" % sorted(DH_DTYPES))
    dh = _bwd_in(head, M, dev, lse, g, out, torch.float32 if dh_dtype == "f32" else torch.bfloat16)
    if block_max is not None:
        _expect(block_max, torch.float32, dev, (M, n_blocks(head)), "block_max")
    hs = head.c_struct()
    sk = cce_skip(float(block_eps), float(filter_eps))
    ws = _workspace(lib.cce_backward_workspace_bytes(ctypes.byref(hs), M), dev, workspace)
    _check(lib.cce_backward_ex(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(lse), _ptr(g),
                               _ptr(block_max), ctypes.byref(sk), _ptr(dh), DH_DTYPES[dh_dtype], _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(dev)))
    return dh


def cce_forward_backward(h, head: Head, targets, g=None, mask=None, workspace=None, out=None, dh_dtype="f32"):
    """(logp, lse, dh) in one call for a g known up front (None: all ones, so
    dh = d logp / d h, which the caller may scale row by row later)."""
    import torch
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    if dh_dtype not in DH_DTYPES:
        raise ValueError("dh_dtype must be one of %s" % sorted(DH_DTYPES))
    if out is not None:
        logp, lse, dh = out
        _expect(logp, torch.float32, dev, (M,), "logp")
    else:
        logp, lse = _fwd_out(M, dev, None)
        dh = None
    dh = _bwd_in(head, M, dev, lse, g, dh, torch.float32 if dh_dtype == "f32" else torch.bfloat16)
    hs = head.c_struct()
    ws = _workspace(lib.cce_forward_backward_workspace_bytes(ctypes.byref(hs), M), dev, workspace)
    _check(lib.cce_forward_backward(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(g), _ptr(logp),
                                    _ptr(lse), _ptr(dh), DH_DTYPES[dh_dtype], _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(dev)))
    return logp, lse, dh


def cce_dense_forward(h, head: DenseHead, targets, mask=None, workspace=None, out=None):
    """(logp, lse), each float32 [M], on a dense bf16 head."""
    import torch
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    _expect(head.w, torch.bfloat16, dev, (head.V, head.H), "w")
    logp, lse = _fwd_out(M, dev, out)
    hs = head.c_struct()
    ws = _workspace(lib.cce_dense_forward_workspace_bytes(ctypes.byref(hs), M), dev, workspace)
    _check(lib.cce_dense_forward(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(logp), _ptr(lse),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return logp, lse


def cce_dense_backward(h, head: DenseHead, targets, lse, g=None, mask=None, need_dw=True, workspace=None,
                       out=None, dw_out=None):
    """(dh float32 [M, H], dW float32 [V, H] or None) on a dense bf16 head."""
    import torch
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    _expect(head.w, torch.bfloat16, dev, (head.V, head.H), "w")
    dh = _bwd_in(head, M, dev, lse, g, out)
    dw = None
    if need_dw:
        if dw_out is not None:
            _expect(dw_out, torch.float32, dev, (head.V, head.H), "dw_out")
            dw = dw_out
        else:
            dw = torch.empty((head.V, head.H), dtype=torch.float32, device=dev)
    hs = head.c_struct()
    ws = _workspace(lib.cce_dense_backward_workspace_bytes(ctypes.byref(hs), M), dev, workspace)
    _check(lib.cce_dense_backward(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(lse), _ptr(g),
                                  _ptr(dh), _ptr(dw), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return dh, dw


def cce_dense_forward_backward(h, head: DenseHead, targets, g=None, mask=None, need_dw=True, workspace=None,
                               out=None, dw_out=None):
    """(logp, lse, dh, dW or None) in one call on a dense bf16 head; g float32
    [M] or None (all ones).  out: (logp, lse, dh) to write into."""
    import torch
    lib = load()
    M, dev = _tokens(h, head, targets, mask)
    _expect(head.w, torch.bfloat16, dev, (head.V, head.H), "w")
    if g is not None:
        _expect(g, torch.float32, dev, (M,), "g")
    if out is not None:
        logp, lse, dh = out
        _expect(dh, torch.float32, dev, (M, head.H), "dh")
    else:
        logp, lse = _fwd_out(M, dev, None)
        dh = torch.empty((M, head.H), dtype=torch.float32, device=dev)
    dw = None
    if need_dw:
        if dw_out is not None:
            _expect(dw_out, torch.float32, dev, (head.V, head.H), "dw_out")
            dw = dw_out
        else:
            dw = torch.empty((head.V, head.H), dtype=torch.float32, device=dev)
    hs = head.c_struct()
    ws = _workspace(lib.cce_dense_forward_backward_workspace_bytes(ctypes.byref(hs), M), dev, workspace)
    _check(lib.cce_dense_forward_backward(ctypes.byref(hs), _ptr(h), M, _ptr(targets), _ptr(mask), _ptr(g),
                                          _ptr(logp), _ptr(lse), _ptr(dh), _ptr(dw), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(dev)))
    return logp, lse, dh, dw


def dense_head_from_numpy(inp: dict, device="cuda") -> DenseHead:
    """Upload the bf16 head of a synthetic.make_dense dict."""
    import torch
    w = torch.from_numpy(inp["w"].view("int16")).to(device).view(torch.bfloat16)
    return DenseHead(w=w, softcap=float(inp["softcap"]))


def head_from_numpy(inp: dict, device="cuda") -> Head:
    """Upload the head arrays of a synthetic.make_inputs dict."""
    import torch
    wq = torch.from_numpy(inp["wq"].view("int32")).to(device)
    sbt = inp.get("sb_dtype", "f32")

    def up(a):
        return torch.from_numpy(a if sbt == "f32" else a.view("int16")).to(device)
    return Head(wq=wq, scales=up(inp["scales"]), biases=up(inp["biases"]), bits=int(inp["bits"]),
                softcap=float(inp["softcap"]), group=int(inp["group"]), sb_dtype=sbt)


def tokens_from_numpy(inp: dict, device="cuda"):
    """(h bf16 [M,H], targets int32 [M], mask uint8 [M] or None) on the device."""
    import torch
    h = torch.from_numpy(inp["h"].view("int16")).to(device).view(torch.bfloat16)
    t = torch.from_numpy(inp["targets"]).to(device)
    m = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).to(device)
    return h, t, m


def profile_enable(on: bool) -> bool:
    """Opt-in per-kernel event timing (include/cce_profile.h); returns the old state."""
    return bool(load().cce_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{kernel family: (launches, total_ms)} since the last read (waits for the GPU)."""
    buf = (cce_kernel_time * 32)()
    n = load().cce_profile_read(buf, 32)
    if n < 0:
        raise CceError(CCE_ERR_HIP, "event timing failed")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n)}
