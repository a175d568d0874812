"""Parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (stated for the head): |logp_gpu - logp_oracle| <= 5e-3 and the
same for lse, max over supervised tokens; masked tokens exactly 0; dh relative
L2 error ||dh_gpu - dh_oracle||_F / ||dh_oracle||_F <= 1e-2 over the compared
rows, masked rows exactly 0.  Each dh row is also bounded on its own:
||row error|| <= 5e-2 ||row||, with rows far below the typical norm (1e-3 of
the median, e.g. a token whose softmax puts all its mass on the target)
measured against that floor instead.

Heads come in two kinds (synthetic.py): "sym" heads (uniform codes, bias =
-zero_point * scale, so b' = 0 and the tiles skip the bias block) and
"affine" heads (a float head quantized with bias = group minimum, so every
row carries b' != 0 and every tile runs the bias block).
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import cce
from linear_cross_entropy_libcce_amd import synthetic as syn

pytestmark = pytest.mark.gpu

LOGP_TOL = 5e-3
DH_TOL = 1e-2
ROW_TOL = 5e-2
BIAS = {"sym": "symmetric", "affine": "affine"}


def say(msg):
    print("[parity] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cce.load()
    return torch


def run_gpu(torch, inp, g=None, backward=True):
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    gg = None if g is None else torch.from_numpy(np.asarray(g, np.float32)).cuda()
    logp, lse = cce.cce_forward(h, head, t, m)
    dh = cce.cce_backward(h, head, t, lse, gg, m) if backward else None
    torch.cuda.synchronize()
    out = (logp.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
           None if dh is None else dh.cpu().numpy().astype(np.float64))
    del head, h, t, m, logp, lse, dh
    return out


def check(inp, gpu, orc, rows, tag):
    glogp, glse, gdh = gpu
    ologp, olse, odh = orc
    mask = inp["mask"]
    active = np.ones(len(rows), bool) if mask is None else mask[rows] != 0
    rows = np.asarray(rows)
    el = np.abs(glogp[rows] - ologp)[active]
    es = np.abs(glse[rows] - olse)[active]
    say("%s: max|dlogp|=%.3g max|dlse|=%.3g over %d tokens" % (tag, el.max(initial=0), es.max(initial=0),
                                                               active.sum()))
    assert np.all(np.isfinite(glogp)) and np.all(np.isfinite(glse))
    assert el.max(initial=0) <= LOGP_TOL and es.max(initial=0) <= LOGP_TOL
    if mask is not None:
        assert np.all(glogp[mask == 0] == 0) and np.all(glse[mask == 0] == 0)
    if gdh is not None:
        assert np.all(np.isfinite(gdh))
        if mask is not None:
            assert np.all(gdh[mask == 0] == 0)
        a, b = gdh[rows][active], odh[active]
        if a.size:
            num, den = np.linalg.norm(a - b), np.linalg.norm(b)
            rel = num / den if den > 0 else num
            nb = np.linalg.norm(b, axis=1)
            floor = 1e-3 * np.median(nb)
            row = np.linalg.norm(a - b, axis=1) / np.maximum(nb, max(floor, 1e-30))
            say("%s: dh rel L2 = %.3g (worst row %.3g, row %d)" % (tag, rel, row.max(), int(np.argmax(row))))
            assert rel <= DH_TOL
            if den > 0:
                assert row.max() <= ROW_TOL


SMALL = {
    "H256_V1000_4bit": dict(M=600, H=256, V=1000, bits=4),
    "H1536_V777_8bit_cap_zipf_randmask": dict(M=300, H=1536, V=777, bits=8, softcap=30.0, targets="zipf",
                                             mask="random", mask_frac=0.3),
    "H2560_V400_4bit_cap_prefixmask": dict(M=520, H=2560, V=400, bits=4, softcap=30.0, mask="prefix",
                                          mask_frac=0.5),
    "H4096_V300_4bit": dict(M=257, H=4096, V=300, bits=4),
    "H2560_V260_8bit_cap_small_scales": dict(M=140, H=2560, V=260, bits=8, softcap=30.0),
    # M above 4096: many token tiles, ragged token and vocabulary tails
    "wide_H256_V700_4bit": dict(M=4200, H=256, V=700, bits=4),
    "wide_H512_V389_8bit_cap_randmask": dict(M=4500, H=512, V=389, bits=8, softcap=30.0, mask="random",
                                             mask_frac=0.4),
    # quantization groups of 32 (32-wide K steps) and 128, bf16 / fp16 scales and biases
    "H512_V900_8bit_group32": dict(M=300, H=512, V=900, bits=8, group=32),
    "H768_V700_4bit_cap_group32_bf16_randmask": dict(M=400, H=768, V=700, bits=4, softcap=30.0, group=32,
                                                     sb_dtype="bf16", mask="random", mask_frac=0.3),
    "H1024_V600_8bit_group128_f16": dict(M=270, H=1024, V=600, bits=8, group=128, sb_dtype="f16"),
    "H384_V500_4bit_group128_bf16_zipf": dict(M=100, H=384, V=500, bits=4, group=128, sb_dtype="bf16",
                                              targets="zipf"),
    "H2560_V300_8bit_cap_f16": dict(M=200, H=2560, V=300, bits=8, softcap=30.0, sb_dtype="f16"),
    "M40_H512_V900_8bit_group32": dict(M=40, H=512, V=900, bits=8, group=32),
    "M50_H640_V333_4bit_group128_bf16": dict(M=50, H=640, V=333, bits=4, group=128, sb_dtype="bf16"),
    # at most 33 tokens (the small-M tile: every group size, both widths, narrow
    # scales, softcap, masks, vocabularies that end inside a tile)
    "M1_H256_V1000_4bit": dict(M=1, H=256, V=1000, bits=4),
    "M7_H512_V777_8bit_cap_zipf": dict(M=7, H=512, V=777, bits=8, softcap=30.0, targets="zipf"),
    "M16_H1536_V4097_4bit_group32_bf16": dict(M=16, H=1536, V=4097, bits=4, group=32, sb_dtype="bf16"),
    "M24_H1024_V2049_8bit_group128_f16_randmask": dict(M=24, H=1024, V=2049, bits=8, group=128, sb_dtype="f16",
                                                       mask="random", mask_frac=0.3),
    "M31_H2560_V3001_8bit_cap_group32": dict(M=31, H=2560, V=3001, bits=8, softcap=30.0, group=32),
    "M32_H768_V515_4bit_cap_group128_prefixmask": dict(M=32, H=768, V=515, bits=4, softcap=30.0, group=128,
                                                       mask="prefix", mask_frac=0.5),
    "M32_H640_V64_8bit_f16": dict(M=32, H=640, V=64, bits=8, sb_dtype="f16"),
    "M33_H512_V900_8bit": dict(M=33, H=512, V=900, bits=8),
}


@pytest.mark.parametrize("bias", sorted(BIAS))
@pytest.mark.parametrize("name", sorted(SMALL))
def test_reduced_case_against_full_oracle(torch_cuda, name, bias):
    kw = SMALL[name]
    inp = syn.make_custom(seed=zlib.crc32(name.encode()) % 1000, bias=BIAS[bias], **kw)
    g = np.random.default_rng(1).uniform(-2, 2, size=kw["M"])
    say("case %s (%s head): GPU fwd+bwd" % (name, bias))
    gpu = run_gpu(torch_cuda, inp, g=g)
    orc = oracle.cce(inp, g=g)
    check(inp, gpu, orc, np.arange(kw["M"]), "%s_%s" % (name, bias))


def test_workload0_full(torch_cuda):
    inp = syn.make_inputs(syn.WORKLOADS[0], syn.seed_for(0))
    say("workload 0 (M=16 H=256 V=4096): GPU fwd+bwd")
    gpu = run_gpu(torch_cuda, inp)
    check(inp, gpu, oracle.cce(inp), np.arange(16), "workload0")


def sample_rows(inp, n, seed, every=None):
    """Token rows to compare: the first, middle and last token, two masked
    ones, the first and last supervised ones, one supervised token from every
    token tile (runs of 256 supervised tokens: the kernels' token tiles), or
    every `every`-th supervised token, and n more at random."""
    M = inp["M"]
    rng = np.random.default_rng(seed)
    rows = {0, M - 1, M // 2}
    act = np.arange(M) if inp["mask"] is None else np.flatnonzero(inp["mask"] != 0)
    if inp["mask"] is not None:
        rows |= set(np.flatnonzero(inp["mask"] == 0)[:2].tolist())
    if act.size:
        rows |= {int(act[0]), int(act[-1])}
        if every is not None:
            rows |= set(act[::every].tolist())
        else:
            for t0 in range(0, act.size, 256):  # one random member of every token tile
                rows.add(int(act[t0 + rng.integers(0, min(256, act.size - t0))]))
    rows |= set(rng.choice(M, size=n, replace=False).tolist())
    return np.array(sorted(rows))


# supervised-token stride of the comparison (None: one token per token tile);
# workload 2 has a single token tile spread over hundreds of vocabulary splits
FULL_SAMPLE = {(2, "sym"): 1, (2, "affine"): 4}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("bias", sorted(BIAS))
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_workload_sampled(torch_cuda, cfg, bias):
    import dataclasses
    w = dataclasses.replace(syn.WORKLOADS[cfg], bias=BIAS[bias])
    say("workload %d (%s, %s head): generating inputs" % (cfg, w.name, bias))
    inp = syn.make_inputs(w, syn.seed_for(cfg))
    say("workload %d: GPU fwd+bwd at full size" % cfg)
    gpu = run_gpu(torch_cuda, inp)
    rows = sample_rows(inp, 4, cfg, every=FULL_SAMPLE.get((cfg, bias)))
    say("workload %d: oracle on %d sampled tokens" % (cfg, len(rows)))
    orc = oracle.cce(inp, tokens=rows)
    check(inp, gpu, orc, rows, "workload%d_%s" % (cfg, bias))
    # properties that hold for every token
    glogp, glse, gdh = gpu
    act = np.ones(inp["M"], bool) if inp["mask"] is None else inp["mask"] != 0
    assert np.all(glogp[act] <= 1e-6) and np.all(np.isfinite(glse))
    assert np.all(np.isfinite(gdh))


EDGE = {
    "M1": dict(M=1, H=128, V=300, bits=4),
    "M2": dict(M=2, H=128, V=300, bits=8),
    "M3": dict(M=3, H=192, V=300, bits=4, softcap=5.0),
    "M4": dict(M=4, H=64, V=129, bits=8),
    "M255": dict(M=255, H=64, V=130, bits=4),
    "M256": dict(M=256, H=64, V=128, bits=4),
    "M257": dict(M=257, H=64, V=127, bits=8),
    "V1": dict(M=5, H=64, V=1, bits=4),
    "V2": dict(M=5, H=128, V=2, bits=8, softcap=3.0),
    "V65": dict(M=7, H=320, V=65, bits=4),
    "H64": dict(M=33, H=64, V=1000, bits=8),
    "H320_ragged_dh_tile": dict(M=40, H=320, V=200, bits=4),
    # the largest H (256 K steps, a 12-step bias block), with group 32 the most groups (512)
    "H16384_V200_8bit_cap": dict(M=20, H=16384, V=200, bits=8, softcap=30.0),
    "H16384_V100_4bit_group32": dict(M=10, H=16384, V=100, bits=4, group=32),
    # one row in the last vocabulary tile; the compaction launch just past the fused threshold
    "V65537_tail_row": dict(M=30, H=128, V=65537, bits=4),
    "M2049_separate_compaction": dict(M=2049, H=64, V=300, bits=8, mask="random", mask_frac=0.5),
    # more than 2048 vocabulary tiles: two coefficient chunks (the later one accumulates into the slabs)
    "V600000_two_chunks": dict(M=20, H=64, V=600000, bits=8, softcap=20.0),
}


@pytest.mark.parametrize("bias", sorted(BIAS))
@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_shapes(torch_cuda, name, bias):
    kw = EDGE[name]
    inp = syn.make_custom(seed=7, bias=BIAS[bias], **kw)
    g = np.random.default_rng(2).uniform(-1, 1, size=kw["M"])
    say("edge %s (%s head): GPU fwd+bwd" % (name, bias))
    gpu = run_gpu(torch_cuda, inp, g=g)
    check(inp, gpu, oracle.cce(inp, g=g), np.arange(kw["M"]), "%s_%s" % (name, bias))


def test_all_masked_and_out_of_range_targets(torch_cuda):
    inp = syn.make_custom(M=20, H=128, V=500, bits=4, seed=3)
    inp["mask"] = np.zeros(20, np.uint8)
    say("edge all-masked: GPU fwd+bwd")
    logp, lse, dh = run_gpu(torch_cuda, inp)
    assert np.all(logp == 0) and np.all(lse == 0) and np.all(dh == 0)
    inp["mask"] = None
    inp["targets"] = np.array([-1, 500, 2 ** 31 - 1, -(2 ** 31)] + list(range(16)), np.int32)
    say("edge out-of-range targets: GPU fwd+bwd")
    gpu = run_gpu(torch_cuda, inp)
    orc = oracle.cce(inp)
    check(inp, gpu, orc, np.arange(20), "oob-targets")
    assert np.allclose(gpu[0][:4], -gpu[1][:4], atol=1e-6)


def test_empty_token_batch(torch_cuda):
    # M = 0 through the binding: a successful no-op with empty outputs, for the
    # quantized and the dense head (no workspace is needed)
    torch = torch_cuda
    inp = syn.make_custom(M=0, H=128, V=500, bits=8, seed=4, softcap=30.0)
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    logp, lse = cce.cce_forward(h, head, t, m)
    dh = cce.cce_backward(h, head, t, lse, None, m)
    torch.cuda.synchronize()
    assert logp.shape == (0,) and lse.shape == (0,) and dh.shape == (0, 128)
    d = syn.make_dense(M=0, H=128, V=300, seed=4)
    dhead = cce.dense_head_from_numpy(d)
    h2, t2, _ = cce.tokens_from_numpy(d)
    logp2, lse2 = cce.cce_dense_forward(h2, dhead, t2)
    dh2, dw2 = cce.cce_dense_backward(h2, dhead, t2, lse2)
    torch.cuda.synchronize()
    assert logp2.shape == (0,) and dh2.shape == (0, 128) and dw2.shape == (300, 128)


def test_workspace_reuse_across_sizes(torch_cuda):
    # one caller-owned workspace (sized for the larger call) serves calls of
    # different M back to back, forward and backward, with results equal to
    # calls on fresh workspaces
    import torch
    big = syn.make_custom(M=600, H=256, V=900, bits=8, seed=21, softcap=30.0)
    small = syn.make_custom(M=70, H=256, V=900, bits=8, seed=22, softcap=30.0)
    head = cce.head_from_numpy(big)
    wsf = torch.empty(cce.forward_workspace_bytes(head, 600), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(cce.backward_workspace_bytes(head, 600), dtype=torch.uint8, device="cuda")
    outs = []
    for inp in (big, small, big):
        h, t, m = cce.tokens_from_numpy(inp)
        logp, lse = cce.cce_forward(h, head, t, m, workspace=wsf)
        dh = cce.cce_backward(h, head, t, lse, None, m, workspace=wsb)
        logp0, lse0 = cce.cce_forward(h, head, t, m)
        dh0 = cce.cce_backward(h, head, t, lse0, None, m)
        torch.cuda.synchronize()
        assert torch.equal(logp, logp0) and torch.equal(lse, lse0) and torch.equal(dh, dh0)
        outs.append(logp.cpu().numpy())
    assert np.array_equal(outs[0], outs[2])


def test_repeat_runs_are_bitwise_identical(torch_cuda):
    inp = syn.make_custom(M=300, H=512, V=3000, bits=8, seed=11, softcap=30.0)
    say("determinism: two GPU runs")
    a = run_gpu(torch_cuda, inp)
    b = run_gpu(torch_cuda, inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("case", ["w8_cap_mask", "w4_group32"])
def test_bf16_dh_is_the_fp32_dh_rounded(torch_cuda, case):
    # the bf16 output is the fp32 result rounded once (RNE, as torch rounds),
    # so the two must agree bit for bit; masked rows are exact zeros in both
    torch = torch_cuda
    if case == "w8_cap_mask":
        inp = syn.make_custom(M=300, H=512, V=3000, bits=8, seed=13, softcap=30.0, mask="random", mask_frac=0.3)
    else:
        inp = syn.make_custom(M=200, H=384, V=1500, bits=4, seed=14, group=32)
    say("bf16 dh (%s): GPU backward in both output types" % case)
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    g = torch.from_numpy(np.random.default_rng(3).uniform(-2, 2, size=inp["M"]).astype(np.float32)).cuda()
    _, lse = cce.cce_forward(h, head, t, m)
    d32 = cce.cce_backward(h, head, t, lse, g, m)
    d16 = cce.cce_backward_ex(h, head, t, lse, g, m, dh_dtype="bf16")
    assert d16.dtype == torch.bfloat16 and d16.shape == d32.shape
    assert torch.equal(d16.view(torch.int16), d32.to(torch.bfloat16).view(torch.int16))
    if m is not None:
        assert int((d16[m == 0] != 0).sum()) == 0


@pytest.mark.parametrize("softcap,bias", [(0.0, "sym"), (30.0, "sym"), (0.0, "affine"), (30.0, "affine")])
def test_peaked_softmax(torch_cuda, softcap, bias):
    """Target probability near 1: dh = g (1 - p_t) c'_t w_t - ..., a small
    difference of large terms; the coefficient must be formed before rounding."""
    # With an affine head every row carries b' != 0 (the bias block runs) and
    # the target row leads by ~0.12 * sum(h) (0.14 under the cap):
    # 1 - p_t between ~4e-5 and ~3e-4, where the target term
    # g (1 - p_t) c'_t w_t is a small difference of large numbers and must be
    # formed from the same logit as the lse it is compared with.  The peaked
    # tokens' rows are also bounded among themselves (their norms are far
    # below the other rows').
    M = 64 if bias == "sym" else 300
    inp = syn.make_custom(M=M, H=256, V=300, bits=4, seed=5, softcap=softcap, bias=BIAS[bias])
    hf = np.abs(syn.f32_from_bf16_bits(inp["h"]))
    inp["h"] = syn.bf16_bits_from_f32(hf)
    inp["targets"][:48] = 7
    inp["biases"][7] += np.float32(0.07 if bias == "sym" else (0.14 if softcap > 0 else 0.12))
    say("peaked softmax (cap %g, %s head): GPU fwd+bwd" % (softcap, bias))
    gpu = run_gpu(torch_cuda, inp)
    orc = oracle.cce(inp)
    pt = np.exp(orc[0][:48])
    say("peaked: 1 - p_t in [%.3g, %.3g]" % (1 - pt.max(), 1 - pt.min()))
    assert pt.min() > (0.95 if bias == "sym" else 0.999)   # the case really is peaked
    check(inp, gpu, orc, np.arange(M), "peaked_%s" % bias)
    check(inp, gpu, tuple(x[:48] for x in orc), np.arange(48), "peaked_%s_targets" % bias)


@pytest.mark.parametrize("M,bias", [(1, "sym"), (16, "sym"), (32, "sym"), (40, "sym"), (64, "sym"), (65, "sym"),
                                    (16, "affine"), (65, "affine")])
def test_small_m_on_the_full_head(torch_cuda, M, bias):
    # the small-M launch on workload 3's full head (M <= 64: every wave of the
    # tile and of the dh contraction multiplies all the tokens by its own 32
    # rows or columns, many dh splits) and its neighbour M = 65; every token
    # against the oracle
    import dataclasses
    w = dataclasses.replace(syn.WORKLOADS[3], bias=BIAS[bias])
    say("small M=%d on workload 3's head (%s): generating inputs" % (M, bias))
    inp = syn.make_inputs(w, syn.seed_for(3), M=M)
    g = np.random.default_rng(M).uniform(-1.5, 1.5, size=M)
    gpu = run_gpu(torch_cuda, inp, g=g)
    say("small M=%d: oracle on all tokens" % M)
    check(inp, gpu, oracle.cce(inp, g=g), np.arange(M), "smallM%d_%s" % (M, bias))


@pytest.mark.parametrize("bias", sorted(BIAS))
@pytest.mark.parametrize("cap", [0.5, 40.0, 50.0, 100.0, 1000.0])
def test_softcap_range(torch_cuda, cap, bias):
    # every logit far below a large cap: e^{c(z) - cap} of the largest logit
    # is below fp32's smallest normal once 2 cap exceeds ~87, so such caps
    # need a running maximum; a cap of 0.5 saturates nearly every logit.
    # Against the oracle, several vocabulary tiles and splits, a ragged tail
    # and masked tokens, 4- and 8-bit heads, groups of 32 and the small-M launch
    for bits, H, V, M, group in ((8, 512, 2300, 150, 64), (4, 768, 1500, 150, 64), (4, 512, 900, 150, 32),
                                 (8, 512, 1100, 20, 64)):
        inp = syn.make_custom(M=M, H=H, V=V, bits=bits, seed=int(cap) + bits + group + M, softcap=cap,
                              mask="random", mask_frac=0.2, group=group, bias=BIAS[bias])
        g = np.random.default_rng(7).uniform(-1.5, 1.5, size=M)
        say("softcap %g, %d-bit, group %d, M=%d, %s head: GPU" % (cap, bits, group, M, bias))
        gpu = run_gpu(torch_cuda, inp, g=g)
        assert np.all(np.isfinite(gpu[0])) and np.all(np.isfinite(gpu[1])) and np.all(np.isfinite(gpu[2]))
        check(inp, gpu, oracle.cce(inp, g=g), np.arange(M), "cap%g_%dbit_g%d_M%d" % (cap, bits, group, M))


@pytest.mark.parametrize("bits,cap", [(8, 30.0), (4, 0.0)])
def test_zero_and_tiny_scales(torch_cuda, bits, cap):
    # the fold divides consecutive group scales (a zero scale stands in as
    # 1e-30): groups of scale exactly 0 first, in the middle (two in a row)
    # and last, rows whose every scale is 0 (constant per group: the bias
    # alone), and rows of scales near 1e-20, against the oracle, which uses
    # the stored values as they are
    M, H, V = 120, 512, 1300
    inp = syn.make_custom(M=M, H=H, V=V, bits=bits, seed=91 + bits, softcap=cap, mask="random", mask_frac=0.2)
    sc = inp["scales"]
    sc[0:100, 0] = 0.0
    sc[100:200, 3:5] = 0.0
    sc[200:210, :] = 0.0
    sc[300:320, -1] = 0.0
    sc[400:420, :] *= np.float32(1e-20)
    sc[500:520, 1::2] = 0.0
    inp["targets"][:20] = np.arange(200, 220)  # some targets on the all-zero-scale rows
    g = np.random.default_rng(3).uniform(-1.5, 1.5, size=M)
    say("zero and tiny scales, %d-bit, cap %g: GPU" % (bits, cap))
    gpu = run_gpu(torch_cuda, inp, g=g)
    assert all(np.all(np.isfinite(x)) for x in gpu)
    check(inp, gpu, oracle.cce(inp, g=g), np.arange(M), "zeroscale%d" % bits)


@pytest.mark.parametrize("where,H,bits,M,group", [
    ("none", 512, 8, 150, 64), ("first", 512, 8, 150, 64), ("middle", 512, 8, 150, 64),
    ("last", 512, 8, 150, 64), ("none", 64, 8, 150, 64), ("middle", 512, 4, 150, 64),
    ("middle", 512, 8, 40, 64), ("last", 768, 4, 40, 64), ("middle", 512, 8, 150, 32),
    ("first", 512, 4, 40, 128)])
def test_zero_bias_block_start(torch_cuda, where, H, bits, M, group):
    # a symmetric head (b = -128 s or -8 s: every b' is 0) starts each tile at
    # its first code step, and its front stores no bias digits; one row with
    # b' != 0 in the first, a middle or the last 64-row block must bring the
    # bias steps back for every tile, the other blocks' zero digits then read
    # through an empty buffer resource.  Ten tokens target that row, whose
    # logit moves by the sum of h.  H = 64 has a single code step and keeps
    # the bias steps.  M = 40 takes the small-M tile, group 32 the 32-wide step.
    V = 1333
    inp = syn.make_custom(M=M, H=H, V=V, bits=bits, seed=23 + H + bits + M + group, softcap=30.0, mask="random",
                          mask_frac=0.2, group=group)
    s, b = inp["scales"], inp["biases"]
    shift = np.float32(128.0 if bits == 8 else 8.0)
    row = {"none": None, "first": 3, "middle": 700, "last": V - 1}[where]
    if row is not None:
        b[row, :] = np.float32(1.0) - shift * s[row, :]
        inp["targets"][:10] = row
    g = np.random.default_rng(9).uniform(-1.5, 1.5, size=M)
    say("zero bias block, nonzero row %s, H=%d, %d-bit, M=%d, group %d: GPU" % (where, H, bits, M, group))
    gpu = run_gpu(torch_cuda, inp, g=g)
    orc = oracle.cce(inp, g=g)
    name = "biasstart_%s_%d_%d_%d_%d" % (where, H, bits, M, group)
    check(inp, gpu, orc, np.arange(M), name)
    # the single pass (softcap 30) reads the same bias block
    torch = torch_cuda
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    lp, ls, dh = cce.cce_forward_backward(h, head, t, torch.from_numpy(g.astype(np.float32)).cuda(), m)
    torch.cuda.synchronize()
    one = tuple(x.cpu().numpy().astype(np.float64) for x in (lp, ls, dh))
    check(inp, one, orc, np.arange(M), name + "_single_pass")


@pytest.mark.parametrize("bits", [8, 4])
def test_outlier_group_biases(torch_cuda, bits):
    # the bias block holds each row's b' (b plus 128 s for 8-bit codes, 8 s for 4-bit) in
    # 16-bit fixed point relative to the row's largest |b'|: one group per row
    # with b' = 1 (20-40x the others) loosens it for the whole row and must
    # still meet the tolerance
    M, H, V = 64, 2560, 2000
    inp = syn.make_custom(M=M, H=H, V=V, bits=bits, seed=5, softcap=0.0)
    s, b = inp["scales"], inp["biases"]
    rows = np.arange(V)
    grp = rows % s.shape[1]
    shift = np.float32(128.0 if bits == 8 else 8.0)
    b[rows, grp] = np.float32(1.0) - shift * s[rows, grp]
    g = np.random.default_rng(4).uniform(-1.5, 1.5, size=M)
    say("outlier group biases, %d-bit: GPU" % bits)
    gpu = run_gpu(torch_cuda, inp, g=g)
    check(inp, gpu, oracle.cce(inp, g=g), np.arange(M), "outlier_b%d" % bits)


def test_large_token_count(torch_cuda):
    # 300000 tokens (1172 token tiles after compaction; the mask compacted by
    # its own launch): sampled tokens, the first and last supervised ones
    # among them, against the oracle, and properties of every token
    M = 300000
    inp = syn.make_custom(M=M, H=256, V=700, bits=8, seed=17, softcap=30.0, mask="random", mask_frac=0.25)
    g = np.random.default_rng(8).uniform(-1.5, 1.5, size=M)
    say("M=%d: GPU" % M)
    gpu = run_gpu(torch_cuda, inp, g=g)
    rows = sample_rows(inp, 40, 17)
    rows = np.unique(np.concatenate([rows, np.arange(M - 40, M)]))
    say("M=%d: oracle on %d tokens" % (M, len(rows)))
    check(inp, gpu, oracle.cce(inp, g=g, tokens=rows), rows, "largeM")
    glogp, glse, gdh = gpu
    act = inp["mask"] != 0
    assert np.all(glogp[act] <= 1e-6) and np.all(np.isfinite(glse)) and np.all(np.isfinite(gdh))
    assert not np.any(glogp[~act]) and not np.any(glse[~act]) and not np.any(gdh[~act])


def test_dh_output_with_element_alignment_only(torch_cuda):
    # the ABI asks dh for element alignment only: an output one element into a
    # larger buffer (fp32 4-byte, bf16 2-byte aligned) gets the same bits as an
    # aligned one
    import torch
    inp = syn.make_custom(M=90, H=512, V=800, bits=8, seed=61, softcap=30.0, mask="random", mask_frac=0.2)
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    M, H = inp["M"], inp["H"]
    _, lse = cce.cce_forward(h, head, t, m)
    for dtype, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        ref = cce.cce_backward_ex(h, head, t, lse, None, m, dh_dtype=name)
        buf = torch.full((M * H + 1,), 7.0, dtype=dtype, device="cuda")
        out = buf[1:].view(M, H)
        assert out.data_ptr() % 16 != 0
        cce.cce_backward_ex(h, head, t, lse, None, m, out=out, dh_dtype=name)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and buf[0].item() == 7.0


def test_hip_graph_capture_and_replay(torch_cuda):
    # the calls enqueue kernels only (no allocation, no host synchronization,
    # no memset), so a forward + backward can be captured in a HIP graph; every
    # replay, with eager work and synchronizations between them, must match
    # the eager result bit for bit
    import torch
    inp = syn.make_custom(M=300, H=512, V=2000, bits=8, seed=31, softcap=30.0, mask="random", mask_frac=0.2)
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    M, H = inp["M"], inp["H"]
    wsf = torch.empty(cce.forward_workspace_bytes(head, M), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(cce.backward_workspace_bytes(head, M), dtype=torch.uint8, device="cuda")
    logp = torch.empty(M, dtype=torch.float32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    dh = torch.empty((M, H), dtype=torch.float32, device="cuda")

    def step():
        cce.cce_forward(h, head, t, m, workspace=wsf, out=(logp, lse))
        cce.cce_backward(h, head, t, lse, None, m, workspace=wsb, out=dh)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # warm-up on a side stream, as graph capture wants
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = (logp.clone(), lse.clone(), dh.clone())
    say("graph: capture forward + backward")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        logp.zero_(); lse.zero_(); dh.zero_()
        junk = torch.randn(1000, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("graph: replay %d" % rep)
        assert torch.equal(logp, ref[0]) and torch.equal(lse, ref[1]) and torch.equal(dh, ref[2])
    del junk


def _with_bias_offsets(inp, B, seed):
    """Give every (row, group) of the head a shifted bias b' = b + zero_point * s
    drawn uniform in (-B, B): the bias term then carries the logits."""
    s = syn.sb_as_f32(inp["scales"], inp["sb_dtype"])
    shift = np.float32(128.0 if inp["bits"] == 8 else 8.0)
    bp = np.random.default_rng(seed).uniform(-B, B, size=s.shape).astype(np.float32)
    inp["biases"] = (bp - shift * s).astype(np.float32)
    return inp


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("B,hs", [(0.01, 1.0), (0.1, 8.0), (1.0, 1.0), (1.0, 8.0), (10.0, 1.0), (10.0, 8.0),
                                  (100.0, 8.0)])
def test_bias_precision_sweep(torch_cuda, bits, B, hs):
    """Shifted biases |b'| up to 100 on every group, hidden states scaled by up
    to 8.  The bias block holds b' in per-row fixed point; its error bound is
    2^-15 B T (coarse half) or 2^-22 B T (with the refinement half), B the
    largest |b'|, T = sum_g |S_g|.  Bound on |dlogp|: 5e-4, plus, where the
    logits reach the thousands, the fp32 floor of the accumulation itself:
    every logit passes through n = Ka/16 MFMA k-steps, the per-step folds and
    the final scale, each a rounding of at most 2^-24 of a partial sum that
    can be as large as the logit, so 2 n 2^-24 max_v |z_v| bounds logp
    (the target's logit and the lse)."""
    M, H, V = 300, 1024, 700
    inp = syn.make_custom(M=M, H=H, V=V, bits=bits, seed=40 + bits, h_scale=hs, mask="random", mask_frac=0.1)
    _with_bias_offsets(inp, B, seed=41 + bits)
    g = np.random.default_rng(42).uniform(-1.5, 1.5, size=M)
    say("bias sweep: %d-bit, |b'| < %g, h x %g: GPU" % (bits, B, hs))
    glogp, glse, gdh = run_gpu(torch_cuda, inp, g=g)
    ologp, olse, odh = oracle.cce(inp, g=g)
    d = oracle.dense(inp, g=g)
    act = d["act"]
    zmax = np.abs(d["z"]).max(axis=1)
    G = H // 64
    Ka = 2 * (-(-3 * G // 64) * 64) + H        # bias block (two halves) + h
    n_round = Ka // 16 + G + 1
    tol = 5e-4 + 2.0 * n_round * 2.0 ** -24 * zmax
    el = np.abs(glogp[act] - ologp[act])
    es = np.abs(glse[act] - olse[act])
    rel = np.linalg.norm(gdh[act] - odh[act]) / np.linalg.norm(odh[act])
    say("bias sweep %d-bit B=%g hs=%g: max|z| %.3g, max|dlogp| %.3g (worst/tol %.3g), max|dlse| %.3g, dh rel %.3g"
        % (bits, B, hs, zmax.max(), el.max(), (el / tol).max(), es.max(), rel))
    assert np.all(el <= tol) and np.all(es <= tol)
    assert rel <= DH_TOL


def test_bias_precision_differs_per_token_tile(torch_cuda):
    """One call whose two token tiles choose differently: with |b'| < 0.02 the
    coarse bound 2^-15 B T stays under 1e-4 for N(0, 1) hidden states (T ~ 100
    at H = 1024) and exceeds it for the tile scaled by 8, which takes the
    refinement half.  Both tiles against the oracle."""
    M, H, V = 512, 1024, 900
    inp = syn.make_custom(M=M, H=H, V=V, bits=8, seed=44, softcap=30.0)
    _with_bias_offsets(inp, 0.02, seed=45)
    hf = syn.f32_from_bf16_bits(inp["h"]).copy()
    hf[256:] *= np.float32(8.0)
    inp["h"] = syn.bf16_bits_from_f32(hf)
    S = hf.reshape(M, H // 64, 64).sum(axis=2)
    T = np.abs(S).sum(axis=1)
    coarse = 2.0 ** -15 * 0.02 * np.array([T[:256].max(), T[256:].max()])
    say("per-tile bias precision: coarse bounds %.3g (tile 0), %.3g (tile 1)" % tuple(coarse))
    assert coarse[0] < 1e-4 < coarse[1]
    g = np.random.default_rng(46).uniform(-1.5, 1.5, size=M)
    gpu = run_gpu(torch_cuda, inp, g=g)
    check(inp, gpu, oracle.cce(inp, g=g), np.arange(M), "tile_precision")
    el = np.abs(gpu[0] - oracle.cce(inp, backward=False)[0])
    say("per-tile bias precision: max|dlogp| tile 0 %.3g, tile 1 %.3g" % (el[:256].max(), el[256:].max()))
    assert el[:256].max() <= 2 * coarse[0] + 1e-5
