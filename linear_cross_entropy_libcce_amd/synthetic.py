"""Seeded synthetic inputs for the flash cut-cross-entropy head.

This module draws inputs only; it holds none of the head's arithmetic, so both
the HIP path and the CPU oracle can take its arrays without sharing any code.

Recipe (one ``numpy.random.default_rng(seed)`` stream, draws in this order):

1. packed head words ``wq`` uint32 [V, H*bits/32], each word uniform over all
   32-bit values -- so every ``bits``-wide code inside it is uniform over
   [0, 2**bits), the code distribution of the workloads;
2. per-group scales fp32 [V, H/group] (group 64 unless stated), uniform in
   [lo, hi); biases are derived, not drawn: ``-8*s`` (4-bit) or ``-128*s``
   (8-bit), i.e. the affine zero point sits mid-range as in an MLX affine
   quantizer.  With bf16 / fp16 storage the scales are rounded to that type
   (nearest, ties to even) before the biases are derived, and both are
   returned as raw 16-bit patterns (exact in the narrow type: the zero points
   are powers of two);
3. hidden states drawn fp32 N(0, 1), rounded to bf16 (round-to-nearest-even),
   returned as the raw uint16 bit patterns [M, H];
4. targets int32 [M]: uniform over [0, V), or truncated Zipf(a) over the
   vocabulary (P(id = k-1) proportional to k**-a, sampled by inverse CDF);
5. mask uint8 [M] (1 = supervised token) or None: a contiguous masked prefix,
   or exactly round(frac*M) masked positions chosen by a seeded permutation.

Affine heads (``bias="affine"``) replace steps 1-2 by the quantization of a
float head, the way an asymmetric min/max quantizer (MLX's affine mode) makes
one: row means mu_v ~ N(0, row_mean_std^2) are drawn first, then the float
rows w_v = mu_v + N(0, w_std^2) [V, H] in row chunks; per group the bias is
the group minimum and the scale (max - min) / (2**bits - 1), both rounded to
the storage type, and each code is round((w - bias) / scale) clipped to
[0, 2**bits).  Codes are then bell-shaped rather than uniform, every group
holds a 0 and (nearly always) a top code, and the bias is not a multiple of
the scale, so the zero point is arbitrary -- the head every real quantized
LM head is.

A peaked workload multiplies the scales (and so the biases) of the first
``boost_rows`` vocabulary rows by ``boost`` after step 2.  Their logits then
dominate every token's softmax, as the frequent tokens of a trained model's
head do, and most vocabulary blocks carry almost no probability: the regime
in which the backward's block skip and coefficient filter fire.

Workloads 0-4 mirror the sizes the pages validate (H=1536 and H=2560 heads
with V up to 262144; page "mlx-bun 0.0.4 -> 0.0.6", src/train/flash-cce.ts,
the header comment and the H_MAX note) plus a tail-mask case; workload 5 is
workload 3's shape with a peaked head and Zipf targets, the stand-in for the
real text on which the pages measure their backward skips.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

GROUP = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    H: int
    V: int
    bits: int
    scale_lo: float
    scale_hi: float
    softcap: float = 0.0
    targets: str = "uniform"      # "uniform" | "zipf"
    zipf_a: float = 1.1
    mask: str = "none"            # "none" | "prefix" | "random"
    mask_frac: float = 0.0
    boost_rows: int = 0           # peaked head: rows [0, boost_rows) get scales * boost
    boost: float = 1.0
    group: int = GROUP            # quantization group: 32, 64 or 128
    sb_dtype: str = "f32"         # storage of scales and biases: "f32" | "bf16" | "f16"
    bias: str = "symmetric"       # "symmetric" (b = -zero_point*s) | "affine" (min/max quantized float head)
    w_std: float = 0.02           # affine: spread of a float row around its mean
    row_mean_std: float = 0.02    # affine: spread of the row means

    @property
    def G(self) -> int:
        return self.H // self.group

    @property
    def words_per_row(self) -> int:
        return self.H * self.bits // 32


def _w4(name, M, H, V, **kw):
    return Workload(name, M, H, V, 4, 0.005, 0.02, **kw)


WORKLOADS = {
    0: _w4("tiny: M=16 H=256 V=4096 4-bit", 16, 256, 4096),
    1: _w4("M=2048 H=1536 V=65536 4-bit", 2048, 1536, 65536),
    2: _w4("M=512 H=2560 V=262144 4-bit cap30 prefix-masked", 512, 2560, 262144,
           softcap=30.0, mask="prefix", mask_frac=0.5),
    3: Workload("M=8192 H=2560 V=262144 8-bit cap30", 8192, 2560, 262144, 8,
                0.0005, 0.002, softcap=30.0),
    4: _w4("M=8192 H=4096 V=151655 4-bit zipf random-masked", 8192, 4096, 151655,
           targets="zipf", mask="random", mask_frac=0.3),
    5: Workload("M=8192 H=2560 V=262144 8-bit peaked (rows < 4096 scaled x8) zipf", 8192, 2560, 262144, 8,
                0.0005, 0.002, targets="zipf", boost_rows=4096, boost=8.0),
}

SEED_BASE = 20261202


def seed_for(cfg: int) -> int:
    return SEED_BASE + cfg


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def sb_as_f32(a: np.ndarray, sb_dtype: str) -> np.ndarray:
    """Scales or biases as fp32 (exact widening of the stored type)."""
    if sb_dtype == "f32":
        return np.asarray(a, np.float32)
    if sb_dtype == "bf16":
        return f32_from_bf16_bits(np.asarray(a, np.uint16))
    return np.asarray(a, np.uint16).view(np.float16).astype(np.float32)


def _targets(rng, M, V, kind, a):
    if kind == "uniform":
        return rng.integers(0, V, size=M, dtype=np.int64).astype(np.int32)
    if kind == "zipf":
        w = np.arange(1, V + 1, dtype=np.float64) ** (-a)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        u = rng.random(M)
        return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int32)
    raise ValueError(kind)


def _mask(rng, M, kind, frac) -> Optional[np.ndarray]:
    if kind == "none":
        return None
    m = np.ones(M, dtype=np.uint8)
    n = int(round(frac * M))
    if kind == "prefix":
        m[:n] = 0
    elif kind == "random":
        m[rng.permutation(M)[:n]] = 0
    else:
        raise ValueError(kind)
    return m


def _round_sb(x: np.ndarray, sb_dtype: str) -> np.ndarray:
    """fp32 values rounded to the storage type (nearest, ties to even), as fp32."""
    if sb_dtype == "bf16":
        return f32_from_bf16_bits(bf16_bits_from_f32(x))
    if sb_dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    return np.asarray(x, np.float32)


def _store_sb(x: np.ndarray, sb_dtype: str) -> np.ndarray:
    """fp32 values exact in the storage type -> the stored array."""
    if sb_dtype == "bf16":
        return bf16_bits_from_f32(x)
    if sb_dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return np.asarray(x, np.float32)


def _affine_head(rng, w: Workload, chunk_rows: int = 4096):
    """Min/max (asymmetric) quantization of a float head drawn row chunk by
    row chunk: returns packed words, scales and biases (stored types)."""
    V, H, G, bits = w.V, w.H, w.G, w.bits
    top = (1 << bits) - 1
    per = 32 // bits
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))
    mu = (rng.standard_normal(V, dtype=np.float32) * np.float32(w.row_mean_std)).astype(np.float32)
    wq = np.empty((V, w.words_per_row), np.uint32)
    scales = np.empty((V, G), np.float32)
    biases = np.empty((V, G), np.float32)
    for v0 in range(0, V, chunk_rows):
        v1 = min(V, v0 + chunk_rows)
        x = rng.standard_normal((v1 - v0, H), dtype=np.float32) * np.float32(w.w_std) + mu[v0:v1, None]
        xg = x.reshape(v1 - v0, G, w.group)
        lo = xg.min(axis=2)
        hi = xg.max(axis=2)
        s = _round_sb(((hi - lo) / np.float32(top)).astype(np.float32), w.sb_dtype)
        b = _round_sb(lo, w.sb_dtype)
        safe = np.where(s > 0, s, np.float32(1.0))
        q = np.rint((xg - b[:, :, None]) / safe[:, :, None])
        q = np.clip(q, 0, top).astype(np.uint32).reshape(v1 - v0, w.words_per_row, per)
        wq[v0:v1] = np.bitwise_or.reduce(q << shifts, axis=2)
        scales[v0:v1] = s
        biases[v0:v1] = b
    return wq, _store_sb(scales, w.sb_dtype), _store_sb(biases, w.sb_dtype)


def make_inputs(w: Workload, seed: int, M: Optional[int] = None) -> dict:
    """All arrays of one workload (M may be overridden for reduced cases)."""
    M = w.M if M is None else M
    rng = np.random.default_rng(seed)
    if w.bias == "affine":
        wq, scales, biases = _affine_head(rng, w)
        return _tokens(rng, w, M, wq, scales, biases)
    if w.bias != "symmetric":
        raise ValueError(w.bias)
    wq = rng.integers(0, 2**32, size=(w.V, w.words_per_row), dtype=np.uint32)
    scales = rng.uniform(w.scale_lo, w.scale_hi, size=(w.V, w.G)).astype(np.float32)
    if w.boost_rows > 0:
        scales[:w.boost_rows] *= np.float32(w.boost)
    if w.sb_dtype == "bf16":
        scales = f32_from_bf16_bits(bf16_bits_from_f32(scales))
    elif w.sb_dtype == "f16":
        scales = scales.astype(np.float16).astype(np.float32)
    zero_point = np.float32(8.0 if w.bits == 4 else 128.0)
    biases = (-zero_point * scales).astype(np.float32)
    if w.sb_dtype == "bf16":
        scales, biases = bf16_bits_from_f32(scales), bf16_bits_from_f32(biases)
    elif w.sb_dtype == "f16":
        scales, biases = scales.astype(np.float16).view(np.uint16), biases.astype(np.float16).view(np.uint16)
    return _tokens(rng, w, M, wq, scales, biases)


def _tokens(rng, w: Workload, M: int, wq, scales, biases) -> dict:
    """Steps 3-5 of the recipe (hidden states, targets, mask) on the same stream."""
    h = bf16_bits_from_f32(rng.standard_normal((M, w.H), dtype=np.float32))
    targets = _targets(rng, M, w.V, w.targets, w.zipf_a)
    mask = _mask(rng, M, w.mask, w.mask_frac)
    return dict(h=h, wq=wq, scales=scales, biases=biases, targets=targets, mask=mask,
                M=M, H=w.H, V=w.V, bits=w.bits, group=w.group, softcap=float(w.softcap), sb_dtype=w.sb_dtype)


def make_dense(M, H, V, seed, softcap=0.0, w_std=0.02, targets="uniform", zipf_a=1.1, mask="none",
               mask_frac=0.0) -> dict:
    """A trainable dense head and its tokens.  One default_rng(seed) stream:
    W drawn fp32 N(0, w_std^2) [V, H] and rounded to bf16 (the usual
    initialization scale of an LM head: logits of order 1), then h, targets
    and mask as in make_inputs.  W and h are raw bf16 bit patterns."""
    rng = np.random.default_rng(seed)
    w = bf16_bits_from_f32(rng.standard_normal((V, H), dtype=np.float32) * np.float32(w_std))
    h = bf16_bits_from_f32(rng.standard_normal((M, H), dtype=np.float32))
    t = _targets(rng, M, V, targets, zipf_a)
    m = _mask(rng, M, mask, mask_frac)
    return dict(w=w, h=h, targets=t, mask=m, M=M, H=H, V=V, softcap=float(softcap), dense=True)


def make_custom(M, H, V, bits, seed, softcap=0.0, scale_lo=None, scale_hi=None,
                targets="uniform", mask="none", mask_frac=0.0, h_scale=1.0,
                boost_rows=0, boost=1.0, group=GROUP, sb_dtype="f32", bias="symmetric",
                w_std=0.02, row_mean_std=0.02) -> dict:
    """A reduced/edge-case workload with the same value distributions."""
    if scale_lo is None:
        scale_lo, scale_hi = (0.005, 0.02) if bits == 4 else (0.0005, 0.002)
    w = Workload("custom", M, H, V, bits, scale_lo, scale_hi, softcap=softcap,
                 targets=targets, mask=mask, mask_frac=mask_frac,
                 boost_rows=boost_rows, boost=boost, group=group, sb_dtype=sb_dtype,
                 bias=bias, w_std=w_std, row_mean_std=row_mean_std)
    d = make_inputs(w, seed)
    if h_scale != 1.0:
        d["h"] = bf16_bits_from_f32(f32_from_bf16_bits(d["h"]) * np.float32(h_scale))
    return d
