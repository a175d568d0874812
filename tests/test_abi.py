"""The C ABI without a GPU: the library loads, exports what include/cce.h
declares, and rejects bad arguments with status codes before any HIP call."""
import ctypes
import os
import re

import pytest

from linear_cross_entropy_libcce_amd import build, cce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    build.build(force=False)
    return cce.load()


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(cce_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(cce.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.cce_abi_version() == 8


def head(**kw):
    d = dict(wq=0x1000, scales=0x2000, biases=0x3000, V=1000, H=256, bits=4, group=64, softcap=0.0, sb_dtype=0)
    d.update(kw)
    return cce.cce_head(**d)


def fwd(lib, hd, M=4, h=0x4000, targets=0x5000, logp=0x6000, lse=0x7000, ws=None, nbytes=None):
    if ws is None:
        ws, nbytes = 0x100000, 1 << 40
    return lib.cce_forward(ctypes.byref(hd), h, M, targets, None, logp, lse, ws, nbytes, None)


def test_head_prepare_sizes_and_errors(lib):
    # the prepared head side: its size depends on the head's shape only, and a
    # head that carries it needs less workspace; the checks return before any
    # launch (no GPU needed)
    hd = head()
    nb = lib.cce_head_prepare_bytes(ctypes.byref(hd))
    assert nb > 0 and nb % 256 == 0
    assert lib.cce_head_prepare_bytes(ctypes.byref(head(V=100000))) > nb
    assert lib.cce_head_prepare_bytes(ctypes.byref(head(bits=3))) == 0
    assert lib.cce_head_prepare_bytes(ctypes.byref(head(prep=0x9000, prep_bytes=1))) == nb  # prep fields ignored
    for M in (16, 100000):
        plain = lib.cce_forward_workspace_bytes(ctypes.byref(hd), M)
        prepd = lib.cce_forward_workspace_bytes(ctypes.byref(head(prep=0x900000, prep_bytes=nb)), M)
        assert 0 < prepd < plain and plain - prepd >= nb - 256
        plain = lib.cce_forward_backward_workspace_bytes(ctypes.byref(hd), M)
        prepd = lib.cce_forward_backward_workspace_bytes(ctypes.byref(head(prep=0x900000, prep_bytes=nb)), M)
        assert 0 < prepd < plain
    # a prepared buffer too small, or misaligned: no workspace size, and calls refuse
    assert lib.cce_forward_workspace_bytes(ctypes.byref(head(prep=0x900000, prep_bytes=nb - 256)), 16) == 0
    assert fwd(lib, head(prep=0x900000, prep_bytes=nb - 256)) == cce.CCE_ERR_WORKSPACE
    assert fwd(lib, head(prep=0x900010, prep_bytes=nb)) == cce.CCE_ERR_INVALID_ARG
    # cce_head_prepare's own checks
    assert lib.cce_head_prepare(ctypes.byref(hd), None, nb, None) == cce.CCE_ERR_INVALID_ARG
    assert lib.cce_head_prepare(ctypes.byref(hd), 0x900010, nb, None) == cce.CCE_ERR_INVALID_ARG
    assert lib.cce_head_prepare(ctypes.byref(hd), 0x900000, nb - 1, None) == cce.CCE_ERR_WORKSPACE
    assert lib.cce_head_prepare(ctypes.byref(head(bits=3)), 0x900000, nb, None) == cce.CCE_ERR_UNSUPPORTED
    assert lib.cce_head_prepare(ctypes.byref(head(H=250)), 0x900000, nb, None) == cce.CCE_ERR_INVALID_ARG


def test_workspace_sizes(lib):
    hd = head()
    a = lib.cce_forward_workspace_bytes(ctypes.byref(hd), 16)
    b = lib.cce_backward_workspace_bytes(ctypes.byref(hd), 16)
    assert a > 0 and b > 0 and a % 256 == 0 and b % 256 == 0
    assert lib.cce_forward_workspace_bytes(ctypes.byref(hd), 100000) > a
    assert lib.cce_forward_workspace_bytes(ctypes.byref(head(bits=5)), 16) == 0
    assert lib.cce_backward_workspace_bytes(ctypes.byref(hd), -1) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(bits=5), cce.CCE_ERR_UNSUPPORTED),
    (dict(bits=2), cce.CCE_ERR_UNSUPPORTED),
    (dict(group=16), cce.CCE_ERR_UNSUPPORTED),
    (dict(group=256), cce.CCE_ERR_UNSUPPORTED),
    (dict(group=32, H=96), cce.CCE_ERR_UNSUPPORTED),   # a multiple of the group, not of the 64-wide K step
    (dict(sb_dtype=3), cce.CCE_ERR_UNSUPPORTED),
    (dict(sb_dtype=0, scales=0x2002), cce.CCE_ERR_INVALID_ARG),   # fp32 scales need 4-byte alignment
    (dict(sb_dtype=1, scales=0x2001), cce.CCE_ERR_INVALID_ARG),   # 16-bit ones 2-byte alignment
    (dict(H=100), cce.CCE_ERR_INVALID_ARG),      # not a multiple of the group
    (dict(H=32768), cce.CCE_ERR_UNSUPPORTED),
    (dict(V=0), cce.CCE_ERR_INVALID_ARG),
    (dict(softcap=-1.0), cce.CCE_ERR_INVALID_ARG),
    (dict(softcap=float("inf")), cce.CCE_ERR_INVALID_ARG),
    (dict(softcap=float("nan")), cce.CCE_ERR_INVALID_ARG),
    (dict(wq=0), cce.CCE_ERR_INVALID_ARG),
    (dict(wq=0x1004), cce.CCE_ERR_INVALID_ARG),  # not 16-byte aligned
    (dict(scales=0), cce.CCE_ERR_INVALID_ARG),
])
def test_bad_head_is_rejected(lib, kw, status):
    assert fwd(lib, head(**kw)) == status


def test_bad_token_arguments_are_rejected(lib):
    hd = head()
    assert fwd(lib, hd, M=-1) == cce.CCE_ERR_INVALID_ARG
    assert fwd(lib, hd, h=0) == cce.CCE_ERR_INVALID_ARG
    assert fwd(lib, hd, h=0x4001) == cce.CCE_ERR_INVALID_ARG
    assert fwd(lib, hd, targets=0) == cce.CCE_ERR_INVALID_ARG
    assert fwd(lib, hd, logp=0) == cce.CCE_ERR_INVALID_ARG
    assert fwd(lib, hd, ws=0x100010, nbytes=1 << 40) == cce.CCE_ERR_INVALID_ARG   # misaligned workspace
    need = lib.cce_forward_workspace_bytes(ctypes.byref(hd), 4)
    assert fwd(lib, hd, ws=0x100000, nbytes=need - 1) == cce.CCE_ERR_WORKSPACE
    assert lib.cce_forward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x6000, 0x7000, None, 1 << 40, None) \
        == cce.CCE_ERR_WORKSPACE
    # M = 0 is a successful no-op
    assert fwd(lib, hd, M=0, h=0, targets=0) == cce.CCE_OK
    bneed = lib.cce_backward_workspace_bytes(ctypes.byref(hd), 4)
    assert lib.cce_backward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0, None, 0x8000, 0x100000, bneed, None) \
        == cce.CCE_ERR_INVALID_ARG   # lse missing
    assert lib.cce_backward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x7000, 0x9002, 0x8000, 0x100000, bneed,
                            None) == cce.CCE_ERR_INVALID_ARG   # misaligned g
    assert lib.cce_backward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x7000, None, 0x8000, 0x100000, bneed - 256,
                            None) == cce.CCE_ERR_WORKSPACE


def bwd_ex(lib, hd, block_max=None, skip=None, ws=0x100000, nbytes=None, dh=0x8000, dh_dtype=0):
    if nbytes is None:
        nbytes = lib.cce_backward_workspace_bytes(ctypes.byref(hd), 4)
    sk = None if skip is None else ctypes.byref(cce.cce_skip(*skip))
    return lib.cce_backward_ex(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x7000, None, block_max, sk, dh,
                               dh_dtype, ws, nbytes, None)


def test_dh_dtype_is_checked(lib):
    hd = head()
    need = lib.cce_backward_workspace_bytes(ctypes.byref(hd), 4)
    for bad in (-1, 2, 7):
        assert bwd_ex(lib, hd, dh_dtype=bad) == cce.CCE_ERR_INVALID_ARG, bad
    # fp32 dh needs 4-byte alignment, bf16 dh 2-byte; past those checks a short
    # workspace is the next error (nothing is launched)
    assert bwd_ex(lib, hd, dh=0x8002, dh_dtype=cce.DH_DTYPES["f32"]) == cce.CCE_ERR_INVALID_ARG
    assert bwd_ex(lib, hd, dh=0x8001, dh_dtype=cce.DH_DTYPES["bf16"]) == cce.CCE_ERR_INVALID_ARG
    assert bwd_ex(lib, hd, dh=0x8002, dh_dtype=cce.DH_DTYPES["bf16"], nbytes=need - 256) == cce.CCE_ERR_WORKSPACE


def dense(**kw):
    d = dict(w=0x1000, V=1000, H=256, softcap=0.0)
    d.update(kw)
    return cce.cce_dense_head(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(w=0), cce.CCE_ERR_INVALID_ARG),
    (dict(w=0x1008), cce.CCE_ERR_INVALID_ARG),       # 16-byte alignment
    (dict(V=0), cce.CCE_ERR_INVALID_ARG),
    (dict(H=0), cce.CCE_ERR_INVALID_ARG),
    (dict(softcap=-1.0), cce.CCE_ERR_INVALID_ARG),
    (dict(softcap=float("inf")), cce.CCE_ERR_INVALID_ARG),
    (dict(H=96), cce.CCE_ERR_UNSUPPORTED),           # not a multiple of 64
    (dict(H=16384 + 64), cce.CCE_ERR_UNSUPPORTED),
])
def test_bad_dense_head_is_rejected(lib, kw, status):
    hd = dense(**kw)
    assert lib.cce_dense_forward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x6000, 0x7000, 0x100000, 1 << 40,
                                 None) == status
    assert lib.cce_dense_backward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x7000, None, 0x8000, 0x9000,
                                  0x100000, 1 << 40, None) == status
    assert lib.cce_dense_forward_workspace_bytes(ctypes.byref(hd), 4) == 0


def test_dense_arguments_and_workspace(lib):
    hd = dense()
    f = lib.cce_dense_forward_workspace_bytes(ctypes.byref(hd), 300)
    b = lib.cce_dense_backward_workspace_bytes(ctypes.byref(hd), 300)
    # the backward also holds the transposed h and coefficient chunk of dW
    assert 0 < f < b and b % 256 == 0
    # M = 0 is a no-op; negative M is rejected
    assert lib.cce_dense_forward(ctypes.byref(hd), 0, 0, 0, None, 0, 0, None, 0, None) == cce.CCE_OK
    assert lib.cce_dense_backward(ctypes.byref(hd), 0, -1, 0, None, 0, None, 0, 0, None, 0, None) \
        == cce.CCE_ERR_INVALID_ARG
    need = lib.cce_dense_backward_workspace_bytes(ctypes.byref(hd), 4)
    # misaligned dw (fp32) is rejected; past the checks a short workspace is the next error
    assert lib.cce_dense_backward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x7000, None, 0x8000, 0x9002,
                                  0x100000, need, None) == cce.CCE_ERR_INVALID_ARG
    assert lib.cce_dense_backward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x7000, None, 0x8000, 0x9000,
                                  0x100000, need - 256, None) == cce.CCE_ERR_WORKSPACE
    assert lib.cce_dense_backward(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x7000, None, 0x8000, None,
                                  0x100000, need - 256, None) == cce.CCE_ERR_WORKSPACE
    # dW needs M <= 2^21
    big = (1 << 21) + 1
    nb = lib.cce_dense_backward_workspace_bytes(ctypes.byref(hd), big)
    assert lib.cce_dense_backward(ctypes.byref(hd), 0x4000, big, 0x5000, None, 0x7000, None, 0x8000, 0x9000,
                                  0x100000, nb, None) == cce.CCE_ERR_UNSUPPORTED
    # a quantized head cannot claim 16 bits
    q = head(bits=16)
    assert lib.cce_forward_workspace_bytes(ctypes.byref(q), 4) == 0


def test_bad_skip_arguments_are_rejected(lib):
    hd = head()
    for sk in [(-1.0, 0.0), (0.0, -1e-5), (float("nan"), 0.0), (0.0, float("inf"))]:
        assert bwd_ex(lib, hd, block_max=0xA000, skip=sk) == cce.CCE_ERR_INVALID_ARG, sk
    # the block skip needs block_max (4-byte aligned); the filter alone does not
    assert bwd_ex(lib, hd, block_max=None, skip=(1e-5, 0.0)) == cce.CCE_ERR_INVALID_ARG
    assert bwd_ex(lib, hd, block_max=0xA002, skip=(1e-5, 0.0)) == cce.CCE_ERR_INVALID_ARG
    need = lib.cce_backward_workspace_bytes(ctypes.byref(hd), 4)
    assert bwd_ex(lib, hd, skip=(0.0, 1e-5), nbytes=need - 256) == cce.CCE_ERR_WORKSPACE
    # the forward's block_max must be 4-byte aligned
    assert lib.cce_forward_ex(ctypes.byref(hd), 0x4000, 4, 0x5000, None, 0x6000, 0x7000, 0xA002, 0x100000,
                              1 << 40, None) == cce.CCE_ERR_INVALID_ARG
    assert lib.cce_forward_ex(ctypes.byref(hd), 0x4000, 0, 0, None, 0x6000, 0x7000, 0xA000, 0x100000,
                              1 << 40, None) == cce.CCE_OK    # M = 0


def test_profile_api_without_launches(lib):
    assert lib.cce_profile_enable(0) == 0
    assert cce.profile_read() == {}


def test_status_strings(lib):
    for s in range(5):
        assert lib.cce_status_str(s)


def fwdbwd(lib, hd, M=4, logp=0x6000, lse=0x7000, dh=0x8000, dh_dtype=0, g=None, ws=0x100000, nbytes=1 << 40):
    return lib.cce_forward_backward(ctypes.byref(hd), 0x4000, M, 0x5000, None, g, logp, lse, dh, dh_dtype, ws,
                                    nbytes, None)


def test_forward_backward_arguments(lib):
    # the one-call forward + backward checks like its two halves, before any launch
    hd = head(softcap=30.0)
    n = lib.cce_forward_backward_workspace_bytes(ctypes.byref(hd), 1000)
    # the single pass (softcap <= 40) keeps the forward partials of every
    # chunk next to the backward's buffers; other heads keep the forward's
    # partials after the backward's buffers (their backward tiles merge them)
    assert n >= lib.cce_backward_workspace_bytes(ctypes.byref(hd), 1000) and n % 256 == 0
    plain = head(softcap=0.0)
    assert lib.cce_forward_backward_workspace_bytes(ctypes.byref(plain), 1000) > \
        lib.cce_backward_workspace_bytes(ctypes.byref(plain), 1000)
    assert lib.cce_forward_backward_workspace_bytes(ctypes.byref(head(bits=3)), 16) == 0
    assert fwdbwd(lib, head(bits=5)) == cce.CCE_ERR_UNSUPPORTED
    assert fwdbwd(lib, hd, M=-1) == cce.CCE_ERR_INVALID_ARG
    assert fwdbwd(lib, hd, M=0) == cce.CCE_OK
    assert fwdbwd(lib, hd, logp=None) == cce.CCE_ERR_INVALID_ARG
    assert fwdbwd(lib, hd, dh=None) == cce.CCE_ERR_INVALID_ARG
    assert fwdbwd(lib, hd, dh=0x8002) == cce.CCE_ERR_INVALID_ARG        # fp32 dh: 4-byte aligned
    assert fwdbwd(lib, hd, dh_dtype=2) == cce.CCE_ERR_INVALID_ARG
    assert fwdbwd(lib, hd, g=0x9002) == cce.CCE_ERR_INVALID_ARG
    assert fwdbwd(lib, hd, ws=None) == cce.CCE_ERR_WORKSPACE
    assert fwdbwd(lib, hd, nbytes=n - 1, M=1000) == cce.CCE_ERR_WORKSPACE


def test_static_forward_size_limit(lib):
    # the no-allocation forward rejects a plan larger than its device scratch
    # before any HIP call (so this runs without a GPU)
    big = head(V=400000, H=4096, bits=8)
    assert lib.cce_forward_workspace_bytes(ctypes.byref(big), 8) > cce.STATIC_SCRATCH_BYTES
    assert lib.cce_forward_static(ctypes.byref(big), 0x4000, 8, 0x5000, None, 0x6000, 0x7000, None) == \
        cce.CCE_ERR_WORKSPACE
    assert lib.cce_forward_static(ctypes.byref(head(bits=5)), 0x4000, 8, 0x5000, None, 0x6000, 0x7000, None) == \
        cce.CCE_ERR_UNSUPPORTED
    assert lib.cce_forward_static(ctypes.byref(head()), 0x4000, 0, 0x5000, None, 0x6000, 0x7000, None) == cce.CCE_OK
