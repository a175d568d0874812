"""Pins of the dense-head oracle (oracle.cce_dense / oracle.dense_core).

* A quantized head whose dequantized values are exact in bf16 (4-bit codes,
  scale 2^-6, bias -8 * 2^-6) is also a dense bf16 head: the dense oracle must
  agree with the independently written, separately pinned C oracle of the
  quantized head on logp, lse and dh.
* dh and dW are the gradients of L = sum_t g_t logp_t: central finite
  differences of L in fp64 must match them (softcap on and off, a target
  outside [0, V), a masked-out token absent).
* Without a softcap the softmax weights of a token sum to one, so for
  in-range targets every column of dW sums to zero.
"""
import numpy as np
import pytest

import oracle
from linear_cross_entropy_libcce_amd import synthetic as syn


def _exact_quantized(M, H, V, seed, softcap, mask="none"):
    q = syn.make_custom(M=M, H=H, V=V, bits=4, seed=seed, softcap=softcap, mask=mask, mask_frac=0.25)
    q["scales"] = np.full_like(q["scales"], np.float32(2.0 ** -6))
    q["biases"] = np.full_like(q["biases"], np.float32(-8 * 2.0 ** -6))
    W = oracle.dequantize(q)                      # (code - 8) / 64: exact in bf16
    w = syn.bf16_bits_from_f32(W.astype(np.float32))
    assert np.array_equal(syn.f32_from_bf16_bits(w).astype(np.float64), W)
    d = dict(w=w, h=q["h"], targets=q["targets"], mask=q["mask"], M=M, H=H, V=V, softcap=float(softcap))
    return q, d


@pytest.mark.parametrize("softcap,mask", [(0.0, "none"), (30.0, "random")])
def test_dense_oracle_matches_quantized_oracle_on_an_exact_head(softcap, mask):
    q, d = _exact_quantized(M=48, H=128, V=300, seed=21, softcap=softcap, mask=mask)
    g = np.random.default_rng(4).uniform(-2, 2, size=48)
    lp_q, ls_q, dh_q = oracle.cce(q, g=g)
    lp_d, ls_d, dh_d, _ = oracle.cce_dense(d, g=g, need_dw=False)
    assert np.allclose(lp_d, lp_q, rtol=0, atol=1e-10)
    assert np.allclose(ls_d, ls_q, rtol=0, atol=1e-10)
    assert np.allclose(dh_d, dh_q, rtol=0, atol=1e-12)
    if q["mask"] is not None:
        off = q["mask"] == 0
        assert np.all(lp_d[off] == 0) and np.all(dh_d[off] == 0)


def _loss(hd, Wd, tgt, gt, cap):
    lp, _, _, _ = oracle.dense_core(hd, Wd, tgt, gt, cap, need_dw=False)
    return float(np.dot(gt, lp))


@pytest.mark.parametrize("cap", [0.0, 3.0])
def test_dense_gradients_match_finite_differences(cap):
    rng = np.random.default_rng(7)
    n, H, V = 3, 8, 5
    hd = rng.standard_normal((n, H))
    Wd = rng.standard_normal((V, H)) * 0.7
    tgt = np.array([2, 4, V + 3])            # the last target matches no row
    gt = np.array([1.0, -0.5, 2.0])
    _, _, dh, dw = oracle.dense_core(hd, Wd, tgt, gt, cap)
    eps = 1e-6
    fd_w = np.zeros_like(Wd)
    for v in range(V):
        for d in range(H):
            Wp, Wm = Wd.copy(), Wd.copy()
            Wp[v, d] += eps
            Wm[v, d] -= eps
            fd_w[v, d] = (_loss(hd, Wp, tgt, gt, cap) - _loss(hd, Wm, tgt, gt, cap)) / (2 * eps)
    assert np.allclose(dw, fd_w, rtol=0, atol=1e-7)
    # dh_t = g_t d logp_t / d h_t: the per-token gradient of the same loss
    fd_h = np.zeros_like(hd)
    for t in range(n):
        for d in range(H):
            hp, hm = hd.copy(), hd.copy()
            hp[t, d] += eps
            hm[t, d] -= eps
            fd_h[t, d] = (_loss(hp, Wd, tgt, gt, cap) - _loss(hm, Wd, tgt, gt, cap)) / (2 * eps)
    assert np.allclose(dh, fd_h, rtol=0, atol=1e-7)


def test_dense_dw_columns_sum_to_zero_without_softcap():
    d = syn.make_dense(M=64, H=96, V=400, seed=5, softcap=0.0)
    g = np.random.default_rng(8).uniform(-1, 1, size=64)
    _, _, _, dw = oracle.cce_dense(d, g=g)
    col = dw.sum(axis=0)
    assert np.abs(col).max() < 1e-12 * np.abs(dw).sum(axis=0).max()
    # a softcap breaks it (c' differs per row): the property is not vacuous
    d["softcap"] = 2.0
    _, _, _, dw2 = oracle.cce_dense(d, g=g)
    assert np.abs(dw2.sum(axis=0)).max() > 1e-6


def test_dense_oracle_token_subset_and_rows():
    d = syn.make_dense(M=40, H=64, V=256, seed=9, softcap=30.0, mask="random", mask_frac=0.3)
    full = oracle.cce_dense(d)
    sub = [1, 5, 7, 30]
    part = oracle.cce_dense(d, tokens=sub, dw_rows=[0, 17, 255])
    act = [t for t in sub if d["mask"][t] != 0]
    assert np.allclose(part[0][act], full[0][act], atol=1e-12)
    assert np.allclose(part[2][act], full[2][act], atol=1e-12)
    # dw over a token subset is the sum of those tokens' terms only
    only = oracle.cce_dense(d, tokens=sub)[3]
    assert np.allclose(part[3], only[[0, 17, 255]], atol=1e-12)
