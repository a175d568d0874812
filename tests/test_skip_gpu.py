"""The forward's block maxima and the backward's opt-in skips on the GPU,
through the C ABI, against the fp64 oracle (oracle.block_max, oracle.cce_skip).

Tolerances: block_max within 5e-3 of the oracle (the logit tolerance of the
head) and exactly 0 on masked rows; dh relative L2 error <= 1e-2 against the
oracle's skipped dh.  The eps values are chosen so that the skips change dh by
far more than that tolerance, so matching the oracle checks which pairs were
dropped, not only that little was.
"""
import sys

import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import cce
from linear_cross_entropy_libcce_amd import synthetic as syn

pytestmark = pytest.mark.gpu

LOGIT_TOL = 5e-3
DH_TOL = 1e-2


def say(msg):
    print("[skip] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cce.load()
    return torch


def flat_blocks(M, H, V, bits, seed, mask, cap=0.0, bias="symmetric", group=64):
    """Vocabulary blocks 1.. made of one repeated row each, targets mostly in
    block 0 (every 97th token's in block 2): the probability spreads evenly
    over the repeated rows (each below 0.01, the blocks holding ~30% of it), so
    the pairs of blocks 1.. go cold for whole token tiles while carrying enough
    mass that dropping them moves dh by ~35%.  The per-pair maxima sit far from
    the eps values used (warm pairs >= 0.08, cold <= 0.014)."""
    inp = syn.make_custom(M=M, H=H, V=V, bits=bits, seed=seed, mask=mask, mask_frac=0.3, softcap=cap, bias=bias,
                          group=group)
    for k in ("wq", "scales", "biases"):
        a = inp[k]
        for b in range(1, (V + 255) // 256):
            a[256 * b:min(V, 256 * b + 256)] = a[256 * b]
    tg = inp["targets"] % 256
    tg[::97] = 512 + tg[::97] % 100
    inp["targets"] = tg.astype(np.int32)
    return inp


# V and M ragged against the 256-wide blocks and token tiles
CASES = {
    "H256_V1000_8bit_randmask": (600, 256, 1000, 8, 71, "random"),
    "H512_V1100_4bit_cap": (700, 512, 1100, 4, 72, "none", 30.0),
    # affine heads (b' != 0 on every row: the bias block runs), 64- and 32-wide steps
    "H512_V1100_8bit_cap_randmask_affine": (700, 512, 1100, 8, 75, "random", 30.0, "affine"),
    "H512_V1000_4bit_group32_affine": (600, 512, 1000, 4, 76, "none", 0.0, "affine", 32),
}


def gpu_run(torch, inp, g, block_eps, filter_eps):
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    gg = torch.from_numpy(np.asarray(g, np.float32)).cuda()
    logp, lse, bmx = cce.cce_forward_ex(h, head, t, m, block_max=True)
    dh = cce.cce_backward_ex(h, head, t, lse, gg, m, block_max=bmx, block_eps=block_eps, filter_eps=filter_eps)
    torch.cuda.synchronize()
    return bmx.cpu().numpy().astype(np.float64), dh.cpu().numpy().astype(np.float64)


# block maxima also under a softcap above 40 (the forward's running-maximum path)
BMX_CASES = dict(CASES, H512_V1100_4bit_cap100_randmask=(700, 512, 1100, 4, 73, "random", 100.0))


@pytest.mark.parametrize("name", list(BMX_CASES))
def test_block_max_matches_oracle(torch_cuda, name):
    inp = flat_blocks(*BMX_CASES[name])
    say("%s: block_max" % name)
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    logp0, lse0 = cce.cce_forward(h, head, t, m)
    logp, lse, bmx = cce.cce_forward_ex(h, head, t, m, block_max=True)
    torch_cuda.cuda.synchronize()
    # the block maxima ride along: logp and lse are bit-identical to cce_forward
    assert torch_cuda.equal(logp0, logp) and torch_cuda.equal(lse0, lse)
    got = bmx.cpu().numpy().astype(np.float64)
    ref = oracle.block_max(inp)
    act = np.ones(inp["M"], bool) if inp["mask"] is None else inp["mask"] != 0
    err = np.abs(got[act] - ref[act]).max()
    say("%s: max|d block_max| = %.3g over %d x %d" % (name, err, act.sum(), ref.shape[1]))
    assert np.all(np.isfinite(got)) and err <= LOGIT_TOL
    assert np.all(got[~act] == 0)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("block_eps,filter_eps", [(2e-2, 0.0), (0.0, 3e-2), (2e-2, 3e-2)])
def test_skips_match_oracle(torch_cuda, name, block_eps, filter_eps):
    inp = flat_blocks(*CASES[name])
    g = np.linspace(-1.0, 1.5, inp["M"])
    say("%s: block_eps=%g filter_eps=%g" % (name, block_eps, filter_eps))
    _, gdh = gpu_run(torch_cuda, inp, g, block_eps, filter_eps)
    _, _, odh, dropped = oracle.cce_skip(inp, g=g, block_eps=block_eps, filter_eps=filter_eps)
    _, _, exact = oracle.cce(inp, g=g)
    act = np.ones(inp["M"], bool) if inp["mask"] is None else inp["mask"] != 0
    moved = np.linalg.norm(odh[act] - exact[act]) / np.linalg.norm(exact[act])
    rel = np.linalg.norm(gdh[act] - odh[act]) / np.linalg.norm(odh[act])
    say("%s: %d of %d pairs dropped, skip moves dh by %.3g, GPU vs oracle %.3g"
        % (name, dropped.sum(), dropped.size, moved, rel))
    assert moved > 5 * DH_TOL        # the case exercises the skips
    assert np.all(np.isfinite(gdh)) and rel <= DH_TOL
    assert np.all(gdh[~act] == 0)


def test_skips_off_are_exact(torch_cuda):
    # eps = 0 (and no block_max) is the exact backward, bit for bit
    inp = flat_blocks(*CASES["H256_V1000_8bit_randmask"])
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    logp, lse, bmx = cce.cce_forward_ex(h, head, t, m, block_max=True)
    dh0 = cce.cce_backward(h, head, t, lse, None, m)
    dh1 = cce.cce_backward_ex(h, head, t, lse, None, m)
    dh2 = cce.cce_backward_ex(h, head, t, lse, None, m, block_max=bmx, block_eps=0.0, filter_eps=0.0)
    torch_cuda.cuda.synchronize()
    assert torch_cuda.equal(dh0, dh1) and torch_cuda.equal(dh0, dh2)


def test_tiny_eps_keeps_exact_tolerance(torch_cuda):
    # the pages' default eps (1e-5) on a peaked head: within the exact tolerance
    inp = syn.make_custom(M=700, H=512, V=2000, bits=4, seed=62, boost_rows=256, boost=4.0, targets="zipf",
                          softcap=30.0)
    g = np.ones(inp["M"])
    _, gdh = gpu_run(torch_cuda, inp, g, 1e-5, 1e-5)
    _, _, exact = oracle.cce(inp, g=g)
    rel = np.linalg.norm(gdh - exact) / np.linalg.norm(exact)
    say("eps 1e-5: GPU skip vs exact oracle %.3g" % rel)
    assert rel <= DH_TOL


def test_peaked_workload_full_size(torch_cuda):
    # the full-size peaked workload in bench's launch configuration: exact
    # forward/backward within the head's tolerances on sampled tokens, block
    # maxima on those tokens, and the skipped backward at the pages' eps
    # (1e-5, 1e-5) within the exact dh tolerance
    cfg = 5
    w = syn.WORKLOADS[cfg]
    say("workload %d (%s): generating inputs" % (cfg, w.name))
    inp = syn.make_inputs(w, syn.seed_for(cfg))
    head = cce.head_from_numpy(inp)
    h, t, m = cce.tokens_from_numpy(inp)
    say("workload %d: GPU forward with block maxima, exact and skipped backward" % cfg)
    logp, lse, bmx = cce.cce_forward_ex(h, head, t, m, block_max=True)
    dh_exact = cce.cce_backward(h, head, t, lse, None, m)
    dh_skip = cce.cce_backward_ex(h, head, t, lse, None, m, block_max=bmx, block_eps=1e-5, filter_eps=1e-5)
    torch_cuda.cuda.synchronize()
    rng = np.random.default_rng(cfg)
    rows = np.array(sorted({0, inp["M"] - 1, inp["M"] // 2} | set(rng.choice(inp["M"], 5, replace=False).tolist())))
    say("workload %d: oracle on %d sampled tokens" % (cfg, len(rows)))
    ologp, olse, odh = oracle.cce(inp, tokens=rows)
    glogp = logp.cpu().numpy()[rows].astype(np.float64)
    glse = lse.cpu().numpy()[rows].astype(np.float64)
    assert np.abs(glogp - ologp).max() <= 5e-3 and np.abs(glse - olse).max() <= 5e-3
    ge = dh_exact.cpu().numpy()[rows].astype(np.float64)
    gs = dh_skip.cpu().numpy()[rows].astype(np.float64)
    rel_e = np.linalg.norm(ge - odh) / np.linalg.norm(odh)
    rel_s = np.linalg.norm(gs - odh) / np.linalg.norm(odh)
    say("workload %d: dh rel L2 exact %.3g, skipped %.3g" % (cfg, rel_e, rel_s))
    assert rel_e <= DH_TOL and rel_s <= DH_TOL
    say("workload %d: oracle block maxima of the sampled tokens" % cfg)
    ob = oracle.block_max(inp, tokens=rows)
    gb = bmx.cpu().numpy()[rows].astype(np.float64)
    err = np.abs(gb - ob).max()
    say("workload %d: max|d block_max| = %.3g" % (cfg, err))
    assert err <= LOGIT_TOL


def two_chunk_head():
    """V = 530000 (2071 vocabulary tiles: two coefficient chunks of at most
    2048).  Block 3 (in the first chunk) and block 2052 (in the second) have
    8x scales, so they are hot for every token; the flat rest is cold at
    block_eps = 2e-2 except where targets fall.  Reading the second chunk's
    flags at a wrong offset drops block 2052 or keeps cold ones."""
    inp = syn.make_custom(M=40, H=64, V=530000, bits=8, seed=74, targets="zipf")
    for b in (3, 2052):
        inp["scales"][256 * b:256 * b + 256] *= np.float32(8.0)
    inp["biases"] = (-128.0 * inp["scales"]).astype(np.float32)
    return inp


def test_skips_across_two_coefficient_chunks(torch_cuda):
    inp = two_chunk_head()
    g = np.linspace(-1.0, 1.5, inp["M"])
    say("two chunks: block_eps=2e-2")
    _, gdh = gpu_run(torch_cuda, inp, g, 2e-2, 0.0)
    _, _, odh, dropped = oracle.cce_skip(inp, g=g, block_eps=2e-2)
    rel = np.linalg.norm(gdh - odh) / np.linalg.norm(odh)
    say("two chunks: %d of %d pairs dropped (blocks 3, 2052 kept: %s), GPU vs oracle %.3g"
        % (dropped.sum(), dropped.size, (not dropped[0, 3]) and (not dropped[0, 2052]), rel))
    assert not dropped[0, 3] and not dropped[0, 2052] and dropped.sum() > 1000
    assert rel <= DH_TOL
