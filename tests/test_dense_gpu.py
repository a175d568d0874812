"""GPU parity of the trainable dense head (cce_dense_forward / cce_dense_backward)
against the fp64 oracle (oracle.cce_dense).

Tolerances are those of the quantized head: |d logp| <= 5e-3 absolute, dh rows
and dW within 1e-2 relative L2; masked tokens are exact zeros.  The kernels
round every coefficient to bf16 once (dh adds the target's term in fp32, dW
takes it rounded like the rest), which is what bounds dW's error.
"""
import sys

import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import cce
from linear_cross_entropy_libcce_amd import synthetic as syn

pytestmark = pytest.mark.gpu

LOGP_TOL = 5e-3
DH_TOL = 1e-2
DW_TOL = 1e-2


def say(msg):
    print("[dense] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cce.load()
    return torch


def run(torch, inp, g=None, mask=None, need_dw=True):
    head = cce.dense_head_from_numpy(inp)
    h = torch.from_numpy(inp["h"].view("int16")).cuda().view(torch.bfloat16)
    t = torch.from_numpy(inp["targets"]).cuda()
    mk = inp["mask"] if mask is None else mask
    m = None if mk is None else torch.from_numpy(mk).cuda()
    gg = None if g is None else torch.from_numpy(np.asarray(g, np.float32)).cuda()
    logp, lse = cce.cce_dense_forward(h, head, t, m)
    dh, dw = cce.cce_dense_backward(h, head, t, lse, gg, m, need_dw=need_dw)
    torch.cuda.synchronize()
    out = (logp.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
           dh.cpu().numpy().astype(np.float64), None if dw is None else dw.cpu().numpy().astype(np.float64))
    del head, h, t, m, gg, logp, lse, dh, dw
    return out


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def check_tokens(gpu, orc, rows, mask, tag):
    rows = np.asarray(rows)
    act = np.ones(len(rows), bool) if mask is None else mask[rows] != 0
    el = np.abs(gpu[0][rows] - orc[0][rows])[act]
    es = np.abs(gpu[1][rows] - orc[1][rows])[act]
    say("%s: max|dlogp|=%.3g max|dlse|=%.3g over %d tokens" % (tag, el.max(initial=0), es.max(initial=0), act.sum()))
    assert el.max(initial=0) <= LOGP_TOL and es.max(initial=0) <= LOGP_TOL
    worst = 0.0
    for k, r in enumerate(rows):
        if act[k]:
            worst = max(worst, rel_l2(gpu[2][r], orc[2][r]))
        else:
            assert gpu[0][r] == 0 and gpu[1][r] == 0 and not np.any(gpu[2][r])
    say("%s: worst dh row rel L2 %.3g" % (tag, worst))
    assert worst <= DH_TOL


SMALL = {
    # name: (M, H, V, softcap, mask, targets)
    "cap30_masked": (300, 512, 3000, 30.0, "random", "uniform"),
    "nocap_ragged_zipf": (200, 256, 1000, 0.0, "none", "zipf"),
    "prefix_masked_H1536": (260, 1536, 2304, 0.0, "prefix", "uniform"),
    "H16384_max": (70, 16384, 700, 30.0, "random", "uniform"),
    "cap100_randmask": (250, 512, 1500, 100.0, "random", "uniform"),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_dense_small_against_oracle(torch_cuda, name):
    M, H, V, cap, mask, tg = SMALL[name]
    inp = syn.make_dense(M=M, H=H, V=V, seed=31, softcap=cap, mask=mask, mask_frac=0.4, targets=tg)
    inp["targets"][3] = V + 5            # out of range: no target term
    g = np.random.default_rng(2).uniform(-2, 2, size=M)
    say("%s: GPU fwd+bwd+dW" % name)
    gpu = run(torch_cuda, inp, g=g)
    orc = oracle.cce_dense(inp, g=g)
    check_tokens(gpu, orc, np.arange(M), inp["mask"], name)
    e = rel_l2(gpu[3], orc[3])
    say("%s: dW rel L2 %.3g" % (name, e))
    assert e <= DW_TOL
    # rows that no supervised token reaches with any weight still come out finite
    assert np.all(np.isfinite(gpu[3]))


def test_dense_degenerate_and_repeatable(torch_cuda):
    # one vocabulary row (p = 1, every coefficient 0 except out-of-range
    # targets' -g p c'), H = 64, a single token tile; then two runs bitwise
    inp = syn.make_dense(M=17, H=64, V=1, seed=3, softcap=0.0)
    inp["targets"][:] = 0
    inp["targets"][5] = -1
    say("degenerate V=1: GPU")
    gpu = run(torch_cuda, inp)
    orc = oracle.cce_dense(inp)
    # most gradient rows are exactly zero here (p = 1 at the target), so the
    # comparison is absolute, against the scale of W and h
    assert np.abs(gpu[0] - orc[0]).max() <= LOGP_TOL and np.abs(gpu[1] - orc[1]).max() <= LOGP_TOL
    wmax = np.abs(syn.f32_from_bf16_bits(inp["w"])).max()
    assert np.abs(gpu[2] - orc[2]).max() <= 1e-4 * wmax
    assert np.abs(gpu[2][5] - orc[2][5]).max() <= 1e-2 * np.abs(orc[2][5]).max()   # the nonzero row
    assert np.allclose(gpu[3], orc[3], rtol=0, atol=1e-2 * np.abs(orc[3]).max())
    inp = syn.make_dense(M=300, H=256, V=777, seed=4, softcap=30.0)
    a = run(torch_cuda, inp)
    b = run(torch_cuda, inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_dense_all_masked_gives_zero_gradients(torch_cuda):
    inp = syn.make_dense(M=40, H=128, V=500, seed=6, softcap=30.0)
    inp["mask"] = np.zeros(40, np.uint8)
    gpu = run(torch_cuda, inp)
    assert not np.any(gpu[0]) and not np.any(gpu[1]) and not np.any(gpu[2]) and not np.any(gpu[3])


def test_dense_skipping_dw_matches(torch_cuda):
    inp = syn.make_dense(M=100, H=256, V=900, seed=8, softcap=30.0)
    a = run(torch_cuda, inp, need_dw=False)
    b = run(torch_cuda, inp, need_dw=True)
    assert a[3] is None and np.array_equal(a[2], b[2]) and np.array_equal(a[0], b[0])


FULL = dict(M=8192, H=2560, V=262144)


def test_dense_full_size_sampled_tokens_and_dw_properties(torch_cuda):
    # the full shape in the bench's launch configuration: sampled tokens'
    # logp and dh against the oracle; dW through a property that holds at any
    # size (no softcap: every column of dW sums to zero up to the bf16
    # rounding of the coefficients; a missing or misplaced target term breaks
    # it by orders of magnitude)
    say("full size dense: generating inputs")
    inp = syn.make_dense(seed=41, softcap=0.0, **FULL)
    g = np.random.default_rng(5).uniform(0.5, 1.5, size=FULL["M"])
    say("full size dense: GPU fwd+bwd+dW")
    gpu = run(torch_cuda, inp, g=g)
    rows = np.random.default_rng(9).choice(FULL["M"], size=24, replace=False)
    say("full size dense: oracle on %d sampled tokens" % len(rows))
    orc = oracle.cce_dense(inp, g=g, tokens=rows, need_dw=False)
    check_tokens(gpu, orc, rows, None, "full")
    dw = gpu[3]
    col = np.abs(dw.sum(axis=0)).max()
    scale = np.abs(dw).sum(axis=0).max()
    say("full size dense: max |column sum of dW| %.3g against %.3g" % (col, scale))
    # each token's coefficients sum to ~0 up to the bf16 rounding of its
    # target coefficient (~1e-3 g), so a column sum is ~1e-3 sqrt(M) times the
    # largest of H such sums: ~5e-5 of the column's absolute sum here; a
    # dropped target term would leave sum_t g_t h_t, ~1e-2 of it
    assert col <= 4e-4 * scale


def test_dense_full_vocabulary_dw_rows(torch_cuda):
    # full V, H and M (M_pad = 8192: four coefficient chunks of 65536 rows),
    # dW rows compared element by element: a mask keeps 48 tokens so the
    # oracle's dW over them is cheap
    M = FULL["M"]
    say("full vocabulary dW rows: generating inputs")
    inp = syn.make_dense(M=M, H=FULL["H"], V=FULL["V"], seed=43, softcap=30.0)
    keep = np.random.default_rng(10).choice(M, size=48, replace=False)
    inp["mask"] = np.zeros(M, np.uint8)
    inp["mask"][keep] = 1
    # some kept tokens share a target, one sits in the last (ragged) tile
    inp["targets"][keep[:6]] = 1234
    inp["targets"][keep[6]] = FULL["V"] - 1
    g = np.random.default_rng(11).uniform(-1.5, 1.5, size=M)
    say("full vocabulary dW rows: GPU")
    gpu = run(torch_cuda, inp, g=g)
    tg = inp["targets"][keep]
    rows = np.unique(np.concatenate([tg, np.random.default_rng(12).choice(FULL["V"], 40, replace=False),
                                     [0, 65535, 65536, 131072, FULL["V"] - 1]]))
    say("full vocabulary dW rows: oracle over the 48 tokens, %d rows" % len(rows))
    orc = oracle.cce_dense(inp, g=g, dw_rows=rows)
    check_tokens(gpu, orc, np.arange(M), inp["mask"], "fullV")
    e = rel_l2(gpu[3][rows], orc[3])
    worst_t = max(rel_l2(gpu[3][v], orc[3][k]) for k, v in enumerate(rows) if v in set(tg))
    say("full vocabulary dW rows: rel L2 %.3g (target rows worst %.3g)" % (e, worst_t))
    assert e <= DW_TOL and worst_t <= DW_TOL


# ---- cce_dense_forward_backward: one call (the single pass under a softcap <= 40 or without one)

def run_combined(torch, inp, g=None, need_dw=True):
    head = cce.dense_head_from_numpy(inp)
    h = torch.from_numpy(inp["h"].view("int16")).cuda().view(torch.bfloat16)
    t = torch.from_numpy(inp["targets"]).cuda()
    m = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).cuda()
    gg = None if g is None else torch.from_numpy(np.asarray(g, np.float32)).cuda()
    logp, lse, dh, dw = cce.cce_dense_forward_backward(h, head, t, gg, m, need_dw=need_dw)
    torch.cuda.synchronize()
    out = (logp.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
           dh.cpu().numpy().astype(np.float64), None if dw is None else dw.cpu().numpy().astype(np.float64))
    del head, h, t, m, gg, logp, lse, dh, dw
    return out


@pytest.mark.parametrize("name", sorted(SMALL))
def test_dense_combined_against_oracle(torch_cuda, name):
    # softcap 30: the single pass (dW from the kept chunks and hT scaled by each
    # row's factor); softcap 0: the same against block references brought to
    # each token's maximum; softcap 100: the forward and the backward in turn
    M, H, V, cap, mask, tg = SMALL[name]
    inp = syn.make_dense(M=M, H=H, V=V, seed=31, softcap=cap, mask=mask, mask_frac=0.4, targets=tg)
    inp["targets"][3] = V + 5
    g = np.random.default_rng(2).uniform(-2, 2, size=M)
    gpu = run_combined(torch_cuda, inp, g=g)
    orc = oracle.cce_dense(inp, g=g)
    check_tokens(gpu, orc, np.arange(M), inp["mask"], "combined_" + name)
    e = rel_l2(gpu[3], orc[3])
    say("combined_%s: dW rel L2 %.3g" % (name, e))
    assert e <= DW_TOL and np.all(np.isfinite(gpu[3]))


def test_dense_combined_masked_and_without_dw(torch_cuda):
    inp = syn.make_dense(M=40, H=128, V=500, seed=6, softcap=30.0)
    inp["mask"] = np.zeros(40, np.uint8)
    gpu = run_combined(torch_cuda, inp)
    assert not np.any(gpu[0]) and not np.any(gpu[1]) and not np.any(gpu[2]) and not np.any(gpu[3])
    inp = syn.make_dense(M=100, H=256, V=900, seed=8, softcap=30.0)
    a = run_combined(torch_cuda, inp, need_dw=False)
    b = run_combined(torch_cuda, inp, need_dw=True)
    assert a[3] is None and np.array_equal(a[2], b[2]) and np.array_equal(a[0], b[0])
    c = run_combined(torch_cuda, inp, need_dw=True)
    for x, y in zip(b, c):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("cap", [30.0, 0.0])
def test_dense_combined_full_vocabulary_dw_rows(torch_cuda, cap):
    # the single pass at full V, H and M (four coefficient chunks, all kept
    # until dW; without a softcap brought to each token's maximum first), 48
    # supervised tokens, dW rows element by element
    M = FULL["M"]
    inp = syn.make_dense(M=M, H=FULL["H"], V=FULL["V"], seed=44, softcap=cap)
    keep = np.random.default_rng(13).choice(M, size=48, replace=False)
    inp["mask"] = np.zeros(M, np.uint8)
    inp["mask"][keep] = 1
    inp["targets"][keep[:6]] = 4321
    inp["targets"][keep[6]] = FULL["V"] - 1
    g = np.random.default_rng(14).uniform(-1.5, 1.5, size=M)
    say("combined full vocabulary: GPU")
    gpu = run_combined(torch_cuda, inp, g=g)
    tg = inp["targets"][keep]
    rows = np.unique(np.concatenate([tg, np.random.default_rng(15).choice(FULL["V"], 40, replace=False),
                                     [0, 65535, 65536, 131072, FULL["V"] - 1]]))
    orc = oracle.cce_dense(inp, g=g, dw_rows=rows)
    check_tokens(gpu, orc, np.arange(M), inp["mask"], "combined_fullV_cap%g" % cap)
    e = rel_l2(gpu[3][rows], orc[3])
    worst_t = max(rel_l2(gpu[3][v], orc[3][k]) for k, v in enumerate(rows) if v in set(tg))
    say("combined full vocabulary dW rows: rel L2 %.3g (target rows worst %.3g)" % (e, worst_t))
    assert e <= DW_TOL and worst_t <= DW_TOL
