"""Seeded random shapes on the GPU, through the C ABI, against the fp64 oracle.

Forty configurations drawn once from a fixed seed (the list below is the same
on every run): token counts from 1 to 700 (the one- and two-block small-M
variants, one and several token tiles), H any multiple of 64 up to 3072, V
from 1 to 6000 (vocabulary tiles cut anywhere), 4- and 8-bit codes, groups
32 / 64 / 128, fp32 / bf16 / fp16 scales and biases, symmetric and affine
heads, softcaps 0 (none), 10, 30 (the single pass) and 60 (above the fixed
reference), no mask, random and prefix masks, uniform and Zipf targets.
Each runs the two calls and the combined call; both are held to the
tolerances of test_parity_gpu.py on every token.
"""
import sys

import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import cce
from linear_cross_entropy_libcce_amd import synthetic as syn
from test_parity_gpu import check, run_gpu

pytestmark = pytest.mark.gpu


def say(msg):
    print("[random] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cce.load()
    return torch


def draw_cases(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(rng.choice([1, 2, 7, 16, 31, 32, 33, 50, 64, 65, 100, 255, 256, 257, 400, 700]))
        group = int(rng.choice([32, 64, 128]))
        H = 64 * int(rng.integers(1, 49))
        if H % group:
            H = group * max(1, H // group)
        V = int(rng.choice([1, 2, 255, 256, 257, 1000, 2049, 3001, 4096, 6000]))
        cases.append(dict(
            M=M, H=H, V=V, group=group,
            bits=int(rng.choice([4, 8])),
            sb_dtype=str(rng.choice(["f32", "f32", "bf16", "f16"])),
            bias=str(rng.choice(["symmetric", "affine"])),
            softcap=float(rng.choice([0.0, 10.0, 30.0, 30.0, 60.0])),
            mask=str(rng.choice(["none", "none", "random", "prefix"])),
            mask_frac=0.3,
            targets=str(rng.choice(["uniform", "zipf"])),
            seed=1000 + i))
    return cases


CASES = draw_cases()


def name_of(kw):
    return "M%d_H%d_V%d_%dbit_g%d_%s_%s_cap%g_%s_%s" % (kw["M"], kw["H"], kw["V"], kw["bits"], kw["group"],
                                                        kw["sb_dtype"], kw["bias"][:3], kw["softcap"], kw["mask"],
                                                        kw["targets"])


@pytest.mark.parametrize("kw", CASES, ids=[name_of(k) for k in CASES])
def test_random_shape_against_oracle(torch_cuda, kw):
    kw = dict(kw)
    if kw["mask"] == "none":
        kw["mask_frac"] = 0.0
    inp = syn.make_custom(**kw)
    M = inp["M"]
    g = np.random.default_rng(kw["seed"]).uniform(-1.5, 1.5, size=M)
    tag = name_of(kw)
    say("%s: oracle" % tag)
    orc = oracle.cce(inp, g=g)
    rows = np.arange(M)
    check(inp, run_gpu(torch_cuda, inp, g=g), orc, rows, tag + "_calls")
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    gg = torch_cuda.from_numpy(np.asarray(g, np.float32)).cuda()
    logp, lse, dh = cce.cce_forward_backward(h, head, t, gg, m)
    torch_cuda.cuda.synchronize()
    fused = (logp.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
             dh.cpu().numpy().astype(np.float64))
    check(inp, fused, orc, rows, tag + "_combined")
