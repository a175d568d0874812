"""A prepared head (cce_head_prepare) on the GPU, through the C ABI.

The preparation is the per-call derivation of the head's per-row data (fold
ratios, last scales, bias-block digits and their block maxima) written once
into the caller's buffer; every call given it must write exactly what it
writes without one, bit for bit, and the oracle still bounds the result.
"""
import sys

import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import cce
from linear_cross_entropy_libcce_amd import synthetic as syn
from test_parity_gpu import check

pytestmark = pytest.mark.gpu


def say(msg):
    print("[prepared] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cce.load()
    return torch


def outputs(torch, head, inp, g):
    """Every call's outputs on these inputs, as host arrays."""
    h, t, m = cce.tokens_from_numpy(inp)
    gg = torch.from_numpy(np.asarray(g, np.float32)).cuda()
    logp, lse = cce.cce_forward(h, head, t, m)
    dh = cce.cce_backward(h, head, t, lse, gg, m)
    logp_x, lse_x, bmx = cce.cce_forward_ex(h, head, t, m, block_max=True)
    dh_x = cce.cce_backward_ex(h, head, t, lse_x, gg, m, block_max=bmx, block_eps=1e-5, filter_eps=1e-6)
    logp_f, lse_f, dh_f = cce.cce_forward_backward(h, head, t, gg, m)
    logp_s, lse_s = cce.cce_forward_static(h, head, t, m)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in dict(
        logp=logp, lse=lse, dh=dh, logp_x=logp_x, lse_x=lse_x, bmx=bmx, dh_x=dh_x,
        logp_f=logp_f, lse_f=lse_f, dh_f=dh_f, logp_s=logp_s, lse_s=lse_s).items()}


CASES = {
    "8bit_cap30_affine_randmask": dict(M=300, H=512, V=1300, bits=8, softcap=30.0, bias="affine", mask="random",
                                       mask_frac=0.2),
    "4bit_nocap_affine": dict(M=300, H=768, V=900, bits=4, bias="affine"),
    "8bit_cap50_symmetric": dict(M=257, H=512, V=700, bits=8, softcap=50.0),
    "4bit_cap30_group32_bf16_affine": dict(M=200, H=512, V=800, bits=4, softcap=30.0, group=32, sb_dtype="bf16",
                                           bias="affine"),
    "8bit_group128_f16_affine": dict(M=100, H=1024, V=600, bits=8, group=128, sb_dtype="f16", bias="affine"),
    "M16_8bit_cap30_affine": dict(M=16, H=2560, V=4097, bits=8, softcap=30.0, bias="affine"),
    "M40_4bit_cap30": dict(M=40, H=512, V=3000, bits=4, softcap=30.0),
    # no softcap at small M: the dh contraction scales the coefficients as it stages them
    "M24_8bit_nocap_affine_randmask": dict(M=24, H=768, V=5000, bits=8, bias="affine", mask="random",
                                           mask_frac=0.25),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prepared_head_writes_the_same_bits(torch_cuda, name):
    kw = dict(CASES[name])
    inp = syn.make_custom(seed=90 + sorted(CASES).index(name), **kw)
    g = np.random.default_rng(5).uniform(-1.5, 1.5, size=inp["M"])
    head = cce.head_from_numpy(inp)
    ref = outputs(torch_cuda, head, inp, g)
    prep = cce.cce_head_prepare(head)
    assert head.prep is prep and prep.numel() == cce.cce_head_prepare_bytes(head)
    got = outputs(torch_cuda, head, inp, g)
    for k in ref:
        assert np.array_equal(ref[k], got[k], equal_nan=True), k
    say("%s: %d outputs bitwise equal with the prepared head" % (name, len(ref)))
    # and still the oracle's result
    check(inp, (got["logp_f"].astype(np.float64), got["lse_f"].astype(np.float64), got["dh_f"].astype(np.float64)),
          oracle.cce(inp, g=g), np.arange(inp["M"]), "prepared_" + name)


def test_prepared_head_serves_other_token_batches(torch_cuda):
    # one preparation, then calls with other M (other workspace sizes and launch
    # plans), each equal to the unprepared call
    inp = syn.make_custom(M=600, H=512, V=2000, bits=8, seed=99, softcap=30.0, bias="affine")
    head = cce.head_from_numpy(inp)
    cce.cce_head_prepare(head)
    plain = cce.head_from_numpy(inp)
    for M in (600, 33, 1, 300):
        sub = dict(inp)
        sub["M"] = M
        sub["h"] = inp["h"][:M]
        sub["targets"] = inp["targets"][:M]
        g = np.linspace(-1.0, 1.0, M)
        a = outputs(torch_cuda, plain, sub, g)
        b = outputs(torch_cuda, head, sub, g)
        for k in a:
            assert np.array_equal(a[k], b[k], equal_nan=True), (M, k)
    say("one preparation served M = 600, 33, 1, 300 bit for bit")
