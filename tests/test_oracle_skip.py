"""Pins of the oracle's approximate backward (block skip, coefficient filter).

The dense fp64 path (numpy matmuls over the dequantized head) is pinned to the
C oracle's loops, which test_oracle.py pins to closed forms and finite
differences.  The skip rules are pinned on hand-built heads whose logits are
set code by code, so that which (token tile, vocabulary block) pairs drop out,
and what that removes from dh, can be read off by hand; a bound pins the size
of what the skips may remove on random peaked heads.  Each test names the
mistake it catches; test_skip_rule_mutants plants those mistakes.
"""
import math

import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import synthetic as syn

GROUP = 64


def head_from_first_codes(first_codes, scale, V_rows_codes=None):
    """8-bit head with H = 64 (one group): row v's code at d = 0 is
    first_codes[v], every other code 0; scale s and bias 0 for every row, so
    with h = e_0 the logit of row v is exactly s * first_codes[v]."""
    V = len(first_codes)
    q = np.zeros((V, GROUP), dtype=np.uint64)
    q[:, 0] = first_codes
    if V_rows_codes is not None:
        for v, codes in V_rows_codes.items():
            q[v, 1:1 + len(codes)] = codes
    words = np.zeros((V, GROUP // 4), dtype=np.uint64)
    for k in range(4):
        words |= q[:, k::4] << np.uint64(8 * k)
    return words.astype(np.uint32), np.full((V, 1), scale, np.float32), np.zeros((V, 1), np.float32)


def inputs(M, targets, first_codes, scale=0.1, mask=None, h_extra=None, hot=None):
    """h = e_0 for every token, or e_{hot[t]} for token t when `hot` is given."""
    wq, sc, bi = head_from_first_codes(first_codes, scale, h_extra)
    h = np.zeros((M, GROUP), np.float32)
    h[np.arange(M), 0 if hot is None else np.asarray(hot)] = 1.0
    return dict(h=syn.bf16_bits_from_f32(h), wq=wq, scales=sc, biases=bi,
                targets=np.asarray(targets, np.int32), mask=mask, M=M, H=GROUP,
                V=len(first_codes), bits=8, group=GROUP, softcap=0.0)


def three_block_codes():
    """V = 768: block 0 holds ten rows at logit 20 (code 200) and the rest at
    0; block 1 is all at logit 0; block 2 is at 0 except row 600 at logit 10."""
    c = np.zeros(768, np.int64)
    c[:10] = 200
    c[600] = 100
    return c


def block_sum(d, rows, t):
    """sum over `rows` of p_v * w_v for token t, from the closed-form softmax
    of the hand-set logits (z_v = 0.1 * code_v)."""
    z = 0.1 * three_block_codes().astype(np.float64)
    p = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    W = oracle.dequantize(d)
    return (p[rows, None] * W[rows]).sum(axis=0)


@pytest.mark.parametrize("seed,bits,cap,mask,group,sbt", [(1, 4, 0.0, "none", 64, "f32"),
                                                      (2, 8, 20.0, "random", 64, "f32"),
                                                      (3, 8, 0.0, "none", 32, "bf16"),
                                                      (4, 4, 10.0, "random", 128, "f16")])
def test_dense_path_matches_c_oracle(seed, bits, cap, mask, group, sbt):
    # catches a numpy dequantization or a softmax/coefficient that differs from
    # the pinned C oracle (code order, group axis, 16-bit widening, sign of the
    # softmax term)
    d = syn.make_custom(300, 128, 700, bits, seed, softcap=cap, mask=mask, mask_frac=0.3,
                        boost_rows=64, boost=4.0, group=group, sb_dtype=sbt)
    g = np.linspace(-1.5, 1.0, d["M"])
    l0, s0, h0 = oracle.cce(d, g=g)
    l1, s1, h1, dropped = oracle.cce_skip(d, g=g)
    assert not dropped.any()
    assert np.abs(l0 - l1).max() < 1e-10 and np.abs(s0 - s1).max() < 1e-10
    assert np.abs(h0 - h1).max() < 1e-10 * max(1.0, np.abs(h0).max())


def check_block_rule():
    # one token tile (M = 2), both targets in block 0
    d = inputs(2, [3, 4], three_block_codes())
    _, _, exact = oracle.cce(d)
    _, _, dh, dropped = oracle.cce_skip(d, block_eps=1e-6)
    # lse ~ 20 + log 10; block 1's rows carry p = e^-lse ~ 2e-10 each: cold;
    # block 2 holds p ~ 4.5e-6 (row 600): warm at 1e-6; block 0 holds the
    # targets: warm
    assert dropped.tolist() == [[False, True, False]]
    # dh lost exactly block 1's share: coeff_v = -p_v, so dh gains sum p_v w_v
    for t in range(2):
        np.testing.assert_allclose(dh[t], exact[t] + block_sum(d, np.arange(256, 512), t), atol=1e-15)
    # at eps = 1e-3 block 2 goes cold too
    _, _, dh2, dropped2 = oracle.cce_skip(d, block_eps=1e-3)
    assert dropped2.tolist() == [[False, True, True]]
    np.testing.assert_allclose(dh2[0], exact[0] + block_sum(d, np.arange(256, 768), 0), atol=1e-15)


def check_one_hot_token_keeps_block_warm():
    # token 0 sees the three-block logits (block 1 cold for it); token 1 reads
    # column 1, where only row 300 (block 1) has a code: logit 25, so block 1
    # is hot for token 1 and the pair stays warm for the whole tile
    d = inputs(2, [3, 4], three_block_codes(), h_extra={300: [250]}, hot=[0, 1])
    _, _, exact = oracle.cce(d)
    _, _, dh, dropped = oracle.cce_skip(d, block_eps=1e-6)
    assert not dropped[0, 1]
    np.testing.assert_allclose(dh[:, :], exact, atol=1e-15)


def check_target_keeps_block_warm():
    # a target inside block 1 keeps the whole pair warm for the tile
    d = inputs(2, [3, 300], three_block_codes())
    _, _, exact = oracle.cce(d)
    _, _, dh, dropped = oracle.cce_skip(d, block_eps=1e-6)
    assert dropped.tolist() == [[False, False, False]]
    np.testing.assert_allclose(dh, exact, atol=1e-15)


def check_tiles_are_runs_of_supervised_tokens():
    # M = 300 with the first 44 tokens masked: 256 supervised tokens, one tile;
    # the last token's target in block 1 keeps block 1 warm for all of them
    mask = np.ones(300, np.uint8)
    mask[:44] = 0
    tg = np.full(300, 3)
    tg[299] = 300
    d = inputs(300, tg, three_block_codes(), mask=mask)
    _, _, _, dropped = oracle.cce_skip(d, block_eps=1e-6)
    assert dropped.shape == (1, 3) and not dropped[0, 1]
    # unmasked, the same 300 tokens make two tiles: [0, 256) and [256, 300);
    # only the second holds token 299's target
    d = inputs(300, tg, three_block_codes())
    _, _, _, dropped = oracle.cce_skip(d, block_eps=1e-6)
    assert dropped.tolist() == [[False, True, False], [False, False, False]]


def check_filter_rule():
    # token 1's target is in block 1: the filter drops block 1's non-target
    # coefficients (all ~2e-9) but keeps the target's own term g (1 - p) w
    d = inputs(2, [3, 300], three_block_codes())
    _, _, exact = oracle.cce(d)
    _, _, dh, dropped = oracle.cce_skip(d, filter_eps=1e-6)
    assert dropped.tolist() == [[False, True, False]]
    rows = np.setdiff1d(np.arange(256, 512), [300])
    np.testing.assert_allclose(dh[1], exact[1] + block_sum(d, rows, 1), atol=1e-15)
    np.testing.assert_allclose(dh[0], exact[0] + block_sum(d, np.arange(256, 512), 0), atol=1e-15)
    # block 2's largest coefficient is p_600 = e^(10 - lse) ~ 4.5e-6: kept at
    # 1e-6 (above), dropped at 1e-5
    assert oracle.cce_skip(d, filter_eps=1e-5)[3][0, 2]


def test_block_rule_drops_exactly_the_cold_block():
    # catches a flipped threshold, a per-token instead of per-tile decision and
    # a decision on z instead of z - lse
    check_block_rule()


def test_one_warm_token_keeps_the_pair():
    # catches a rule that drops a pair when any (not every) token finds it cold
    check_one_hot_token_keeps_block_warm()


def test_target_in_block_keeps_it_warm():
    # catches a block rule that ignores where the targets are
    check_target_keeps_block_warm()


def test_token_tiles_count_supervised_tokens_only():
    # catches tiles cut over all positions instead of supervised ranks
    check_tiles_are_runs_of_supervised_tokens()


def test_filter_drops_small_coefficients_but_never_the_target_term():
    # catches a filter that drops the one-hot term or compares p instead of |coeff|
    check_filter_rule()


@pytest.mark.parametrize("kind", ["block", "filter"])
def test_what_the_skips_remove_is_bounded(kind):
    # each dropped coefficient is below eps (block: |coeff| = |g| p c' <= p <
    # eps), so |dh_skip - dh_exact|_t <= eps * (dropped rows of t) * max_v |w_v|
    d = syn.make_custom(520, 128, 1536, 8, 5, boost_rows=256, boost=8.0, targets="zipf")
    _, _, exact = oracle.cce(d)
    eps = 1e-3
    kw = dict(block_eps=eps) if kind == "block" else dict(filter_eps=eps)
    _, _, dh, dropped = oracle.cce_skip(d, **kw)
    assert dropped.sum() > 0
    wmax = np.linalg.norm(oracle.dequantize(d), axis=1).max()
    for t in range(d["M"]):
        k = t // oracle.TOKEN_TILE
        n_rows = sum(min(d["V"], (b + 1) * 256) - b * 256 for b in np.flatnonzero(dropped[k]))
        assert np.linalg.norm(dh[t] - exact[t]) <= eps * n_rows * wmax + 1e-12  # + rounding of the two paths


def test_skip_rule_mutants(monkeypatch):
    """Planted mistakes in the two rules must fail the hand-built pins."""
    mutants = {
        "threshold flipped": ("_pair_cold", lambda bm, l, tg, b, e: bool(np.all(bm[:, b] - l >= math.log(e)))),
        "targets ignored": ("_pair_cold", lambda bm, l, tg, b, e: bool(np.all(bm[:, b] - l < math.log(e)))),
        "z instead of z - lse": ("_pair_cold", lambda bm, l, tg, b, e: (not np.any((tg >= 256 * b) & (tg < 256 * b + 256)))
                                 and bool(np.all(bm[:, b] < math.log(e)))),
        "any token instead of every token": ("_pair_cold", lambda bm, l, tg, b, e: (not np.any((tg >= 256 * b) & (tg < 256 * b + 256)))
                                             and bool(np.any(bm[:, b] - l < math.log(e)))),
        "filter on the mean": ("_pair_filtered", lambda c, e: bool(np.mean(np.abs(c)) < e)),
    }
    checks = [check_block_rule, check_one_hot_token_keeps_block_warm, check_target_keeps_block_warm,
              check_tiles_are_runs_of_supervised_tokens, check_filter_rule]
    for name, (fn, bad) in mutants.items():
        with monkeypatch.context() as mp:
            mp.setattr(oracle, fn, bad)
            failed = 0
            for c in checks:
                try:
                    c()
                except AssertionError:
                    failed += 1
            assert failed > 0, "mutant survived: " + name


def test_sampled_block_max_matches_dense():
    # the row-chunked path (used at full size) against the dense one: catches a
    # block cut wrong at a chunk boundary (V = 20000 is ragged against both the
    # 16384-row chunks and the 256-row blocks) and masked rows left non-zero
    d = syn.make_custom(300, 128, 20000, 8, 3, boost_rows=128, boost=8.0, targets="zipf", mask="random",
                        mask_frac=0.3, softcap=20.0)
    rows = [0, 5, 7, 150, 299]
    full = oracle.block_max(d)
    part = oracle.block_max(d, tokens=rows)
    assert part.shape == (len(rows), (20000 + 255) // 256)
    assert np.array_equal(full[rows], part)
    # a block's maximum is attained by one of its rows: the largest softcapped
    # logit read straight off the dense logits of the plain definition
    y = oracle.dense(d)["y"]
    act = np.flatnonzero(d["mask"] != 0)
    r = int(np.searchsorted(act, 150))
    assert act[r] == 150 or d["mask"][150] == 0
    if d["mask"][150] != 0:
        np.testing.assert_allclose(full[150, 78], y[r, 78 * 256:20000].max(), rtol=0, atol=0)
