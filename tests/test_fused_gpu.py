"""cce_forward_backward on the GPU, through the C ABI, against the fp64 oracle.

With a softcap in (0, 40] the call is a single pass over the head: the
forward's fixed reference e^{y - cap} gives every coefficient up to the
token's factor g e^{cap - lse}, which the split reduce applies once it has
summed the token's split sums into lse (no logit is computed twice, no merge
launch).  Without a softcap it is a single pass too: the coefficients against
each 32-row vocabulary block's largest logit, brought to the token's maximum
after the merge (at small M by the dh contraction as it stages them).  A
softcap above 40 runs a forward and a backward pass after one front; the
backward tiles merge the forward's partials themselves, so the results match
the two separate calls to rounding.
Tolerances as in test_parity_gpu.py (|dlogp|, |dlse| <= 5e-3, dh relative L2
<= 1e-2, worst row <= 5e-2).
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import cce
from linear_cross_entropy_libcce_amd import synthetic as syn
from test_parity_gpu import check, sample_rows

pytestmark = pytest.mark.gpu


def say(msg):
    print("[fused] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cce.load()
    return torch


def run_fused(torch, inp, g=None, dh_dtype="f32"):
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    gg = None if g is None else torch.from_numpy(np.asarray(g, np.float32)).cuda()
    logp, lse, dh = cce.cce_forward_backward(h, head, t, gg, m, dh_dtype=dh_dtype)
    torch.cuda.synchronize()
    return (logp.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            dh.float().cpu().numpy().astype(np.float64))


CASES = {
    "H512_V1000_8bit_cap30": dict(M=600, H=512, V=1000, bits=8, softcap=30.0),
    "H1536_V777_4bit_cap30_zipf_randmask": dict(M=300, H=1536, V=777, bits=4, softcap=30.0, targets="zipf",
                                               mask="random", mask_frac=0.3),
    "H2560_V400_8bit_cap40_prefixmask": dict(M=520, H=2560, V=400, bits=8, softcap=40.0, mask="prefix",
                                            mask_frac=0.5),
    "H512_V900_8bit_cap30_group32": dict(M=300, H=512, V=900, bits=8, softcap=30.0, group=32),
    "H768_V700_4bit_cap30_group32_bf16": dict(M=400, H=768, V=700, bits=4, softcap=30.0, group=32,
                                             sb_dtype="bf16"),
    "H1024_V600_8bit_cap10_group128_f16": dict(M=270, H=1024, V=600, bits=8, softcap=10.0, group=128,
                                               sb_dtype="f16"),
    "H256_V700_4bit_cap0.5_wide": dict(M=4200, H=256, V=700, bits=4, softcap=0.5),
    # small M (the small-M tile) and a vocabulary in two coefficient chunks
    "M1_H256_V1000_8bit_cap30": dict(M=1, H=256, V=1000, bits=8, softcap=30.0),
    "M16_H1536_V4097_4bit_cap30": dict(M=16, H=1536, V=4097, bits=4, softcap=30.0),
    "M64_H512_V3000_8bit_cap30_randmask": dict(M=64, H=512, V=3000, bits=8, softcap=30.0, mask="random",
                                               mask_frac=0.3),
    "M20_H64_V600000_8bit_cap20_two_chunks": dict(M=20, H=64, V=600000, bits=8, softcap=20.0),
    "M300_H64_V600000_4bit_cap30_two_chunks": dict(M=300, H=64, V=600000, bits=4, softcap=30.0),
    # no softcap: the uncapped single pass (coefficients against their block's
    # largest logit, brought to the token's maximum after the merge); a
    # softcap above 40: the call's two passes (the backward tiles merge the
    # forward's partials themselves; no merge launch, one front)
    "M16_H256_V4096_4bit_nocap": dict(M=16, H=256, V=4096, bits=4),
    # the small-M dh contraction scales the uncapped pass's coefficients as it
    # stages them: one and two token blocks, masked, ragged V, several splits
    "M64_H768_V2501_4bit_nocap_randmask": dict(M=64, H=768, V=2501, bits=4, mask="random", mask_frac=0.3),
    "M33_H512_V7000_8bit_nocap_zipf": dict(M=33, H=512, V=7000, bits=8, targets="zipf"),
    "H512_V1000_8bit_nocap_randmask": dict(M=600, H=512, V=1000, bits=8, mask="random", mask_frac=0.3),
    "H768_V700_4bit_cap50_group32_bf16": dict(M=400, H=768, V=700, bits=4, softcap=50.0, group=32, sb_dtype="bf16"),
    "M2100_H256_V900_8bit_nocap_randmask": dict(M=2100, H=256, V=900, bits=8, mask="random", mask_frac=0.4),
    "M20_H64_V600000_8bit_nocap_two_chunks": dict(M=20, H=64, V=600000, bits=8),
    "M40_H512_V3001_4bit_nocap_group128_f16_randmask": dict(M=40, H=512, V=3001, bits=4, group=128, sb_dtype="f16",
                                                            mask="random", mask_frac=0.3),
    "M300_H768_V1000_8bit_nocap_group32_zipf": dict(M=300, H=768, V=1000, bits=8, group=32, targets="zipf"),
    "M300_H64_V600000_4bit_nocap_two_chunks": dict(M=300, H=64, V=600000, bits=4),
}


@pytest.mark.parametrize("bias", ["sym", "affine"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_against_oracle(torch_cuda, name, bias):
    kw = CASES[name]
    inp = syn.make_custom(seed=zlib.crc32(name.encode()) % 1000, bias="symmetric" if bias == "sym" else "affine",
                          **kw)
    g = np.random.default_rng(3).uniform(-2, 2, size=kw["M"])
    say("%s (%s head): fused forward + backward" % (name, bias))
    gpu = run_fused(torch_cuda, inp, g=g)
    check(inp, gpu, oracle.cce(inp, g=g), np.arange(kw["M"]), "fused_%s_%s" % (name, bias))


@pytest.mark.parametrize("cap", [0.0, 50.0])
def test_other_heads_match_the_two_calls(torch_cuda, cap):
    # a softcap above 40: the call runs a forward and a backward pass, the
    # backward tiles merging the forward's partials themselves: the same
    # quantities as cce_forward followed by cce_backward, in another order.
    # No softcap: the uncapped single pass, whose coefficients are rounded to
    # bf16 against their block's reference and again once brought to the
    # token's maximum: within that rounding of the two calls
    torch = torch_cuda
    inp = syn.make_custom(M=300, H=512, V=1300, bits=8, seed=81, softcap=cap, mask="random", mask_frac=0.2,
                          bias="affine")
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    g = torch.from_numpy(np.random.default_rng(5).uniform(-1, 1, size=300).astype(np.float32)).cuda()
    logp, lse, dh = cce.cce_forward_backward(h, head, t, g, m)
    logp0, lse0 = cce.cce_forward(h, head, t, m)
    dh0 = cce.cce_backward(h, head, t, lse0, g, m)
    torch.cuda.synchronize()
    dl = (logp - logp0).abs().max().item()
    ds = (lse - lse0).abs().max().item()
    rel = ((dh - dh0).norm() / dh0.norm()).item()
    say("combined call vs two calls (cap %g): max|dlogp| %.3g max|dlse| %.3g dh rel %.3g" % (cap, dl, ds, rel))
    if cap == 0.0:
        assert dl <= 1e-4 and ds <= 1e-4 and rel <= 5e-3
    else:
        assert dl <= 1e-5 and ds <= 1e-5 and rel <= 1e-5
    mk = m == 0
    assert int((logp[mk] != 0).sum()) == 0 and int((lse[mk] != 0).sum()) == 0 and int((dh[mk] != 0).sum()) == 0


def test_fused_matches_the_two_calls(torch_cuda):
    # under a softcap the single pass and the two calls compute the same
    # quantities in different orders: within rounding of each other
    torch = torch_cuda
    inp = syn.make_custom(M=700, H=1024, V=3000, bits=8, seed=82, softcap=30.0, mask="random", mask_frac=0.2,
                          bias="affine")
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    logp, lse, dh = cce.cce_forward_backward(h, head, t, None, m)
    logp0, lse0 = cce.cce_forward(h, head, t, m)
    dh0 = cce.cce_backward(h, head, t, lse0, None, m)
    torch.cuda.synchronize()
    dl = (logp - logp0).abs().max().item()
    ds = (lse - lse0).abs().max().item()
    rel = ((dh - dh0).norm() / dh0.norm()).item()
    say("fused vs two calls: max|dlogp| %.3g max|dlse| %.3g dh rel %.3g" % (dl, ds, rel))
    assert dl <= 1e-4 and ds <= 1e-4 and rel <= 5e-3


def test_fused_is_linear_in_g(torch_cuda):
    # dh(g) = g * dh(1) row by row (the caller may scale d logp / d h later)
    torch = torch_cuda
    inp = syn.make_custom(M=300, H=512, V=2000, bits=4, seed=83, softcap=30.0, bias="affine")
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    gn = np.random.default_rng(6).uniform(-3, 3, size=300).astype(np.float32)
    g = torch.from_numpy(gn).cuda()
    _, _, dh1 = cce.cce_forward_backward(h, head, t, None, m)
    _, _, dhg = cce.cce_forward_backward(h, head, t, g, m)
    torch.cuda.synchronize()
    ref = dh1 * g[:, None]
    rel = ((dhg - ref).norm() / ref.norm()).item()
    say("linearity in g: rel %.3g" % rel)
    assert rel <= 1e-6


def test_fused_bf16_dh_is_the_fp32_dh_rounded(torch_cuda):
    torch = torch_cuda
    inp = syn.make_custom(M=300, H=512, V=3000, bits=8, seed=84, softcap=30.0, mask="random", mask_frac=0.3)
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    _, _, d32 = cce.cce_forward_backward(h, head, t, None, m)
    _, _, d16 = cce.cce_forward_backward(h, head, t, None, m, dh_dtype="bf16")
    torch.cuda.synchronize()
    assert d16.dtype == torch.bfloat16
    assert torch.equal(d16.view(torch.int16), d32.to(torch.bfloat16).view(torch.int16))


def test_fused_repeat_runs_are_bitwise_identical(torch_cuda):
    inp = syn.make_custom(M=300, H=512, V=3000, bits=8, seed=85, softcap=30.0, bias="affine")
    a = run_fused(torch_cuda, inp)
    b = run_fused(torch_cuda, inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,bias", [(3, "sym"), (3, "affine"), (2, "sym"), (1, "sym"), (4, "affine")])
def test_fused_full_size_workload_sampled(torch_cuda, cfg, bias):
    # workloads at full size (the launches bench.py times): the softcapped ones
    # in the single pass, workloads 1 and 4 (no softcap; 4 in three
    # coefficient chunks) in the uncapped single pass; one supervised token per
    # token tile and the first and last against the oracle
    import dataclasses
    w = dataclasses.replace(syn.WORKLOADS[cfg], bias="symmetric" if bias == "sym" else "affine")
    say("workload %d (%s head): generating inputs" % (cfg, bias))
    inp = syn.make_inputs(w, syn.seed_for(cfg))
    say("workload %d: fused forward + backward at full size" % cfg)
    gpu = run_fused(torch_cuda, inp)
    rows = sample_rows(inp, 4, cfg + 10, every=8 if cfg == 2 else None)
    say("workload %d: oracle on %d sampled tokens" % (cfg, len(rows)))
    check(inp, gpu, oracle.cce(inp, tokens=rows), rows, "fused_workload%d_%s" % (cfg, bias))
    act = np.ones(inp["M"], bool) if inp["mask"] is None else inp["mask"] != 0
    assert np.all(gpu[0][act] <= 1e-6) and np.all(np.isfinite(gpu[1])) and np.all(np.isfinite(gpu[2]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,bias", [(1, "sym"), (16, "sym"), (32, "affine"), (33, "sym"), (64, "affine")])
def test_fused_small_m_on_the_full_head(torch_cuda, M, bias):
    # the single pass at small M on workload 3's full head: one 32-row token
    # block (M <= 32) and two (33..64) in the tile and the dh contraction,
    # with and without the bias block; every token against the oracle
    import dataclasses
    w = dataclasses.replace(syn.WORKLOADS[3], bias="symmetric" if bias == "sym" else "affine")
    say("small M=%d on workload 3's head (%s): generating inputs" % (M, bias))
    inp = syn.make_inputs(w, syn.seed_for(3), M=M)
    g = np.random.default_rng(M + 7).uniform(-1.5, 1.5, size=M)
    gpu = run_fused(torch_cuda, inp, g=g)
    say("small M=%d: oracle on all tokens" % M)
    check(inp, gpu, oracle.cce(inp, g=g), np.arange(M), "fused_smallM%d_%s" % (M, bias))


GRAPH_CASES = {
    "single_pass_cap30": dict(M=300, H=512, V=2000, bits=8, softcap=30.0, mask="random", mask_frac=0.2, seed=41),
    "single_pass_nocap": dict(M=300, H=512, V=2000, bits=4, mask="random", mask_frac=0.2, seed=42),
    "small_M20_cap30": dict(M=20, H=256, V=3000, bits=8, softcap=30.0, seed=43),
    "small_M24_nocap": dict(M=24, H=256, V=3000, bits=8, mask="random", mask_frac=0.2, seed=45),
}


def _replays_match(torch, step, outs):
    """Warm up on a side stream, capture one step in a HIP graph, then replay
    it three times with eager work and synchronizations between the replays;
    every replay must reproduce the eager outputs bit for bit."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(3):
        for o in outs:
            o.zero_()
        junk = torch.randn(1000, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        say("graph: replay %d" % rep)
        for o, r in zip(outs, ref):
            assert torch.equal(o, r)
    del junk


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_combined_call_replays_from_a_hip_graph(torch_cuda, name):
    # the combined call enqueues kernels only (no allocation, no host
    # synchronization, no memset), in every form: the single pass under a
    # softcap and without one (its scaling launch, or at small M the dh
    # contraction's own scaling), the small-M variants
    torch = torch_cuda
    kw = dict(GRAPH_CASES[name])
    seed = kw.pop("seed")
    inp = syn.make_custom(seed=seed, **kw)
    say("%s: capture cce_forward_backward" % name)
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    M, H = inp["M"], inp["H"]
    ws = torch.empty(cce.forward_backward_workspace_bytes(head, M), dtype=torch.uint8, device="cuda")
    g = torch.from_numpy(np.random.default_rng(seed).uniform(-2, 2, M).astype(np.float32)).cuda()
    logp = torch.empty(M, dtype=torch.float32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    dh = torch.empty((M, H), dtype=torch.float32, device="cuda")
    _replays_match(torch, lambda: cce.cce_forward_backward(h, head, t, g, m, workspace=ws, out=(logp, lse, dh)),
                   [logp, lse, dh])


def test_static_forward_replays_from_a_hip_graph(torch_cuda):
    # the forward on the library's own device scratch, which exists for
    # callers such as graph capture that cannot allocate
    torch = torch_cuda
    inp = syn.make_custom(M=64, H=256, V=3000, bits=8, seed=44, softcap=30.0, mask="random", mask_frac=0.25)
    say("static forward: capture")
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    M = inp["M"]
    logp = torch.empty(M, dtype=torch.float32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    _replays_match(torch, lambda: cce.cce_forward_static(h, head, t, m, out=(logp, lse)), [logp, lse])
