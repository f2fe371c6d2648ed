"""Accuracy study: microscaling (MX) number formats for Q and K, against the
INT8 and INT4-valued schemes the library builds.

SageAttention2 ("4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级",
the snippet on the "INT4量化" search page) multiplies 4-bit Q and K.  gfx950
has no INT4 matrix core; its narrow matrix-core formats are the OCP
microscaling ones, which v_mfma_scale_f32_*_f8f6f4 multiplies at twice the
INT8 rate for 4- and 6-bit elements: FP4 E2M1, FP6 E2M3 and E3M2, FP8 E4M3,
each block of 32 consecutive elements along the reduction axis (here d)
sharing one power-of-two E8M0 scale.  This module measures what those formats
do to attention accuracy, so the choice not to build that route rests on
numbers.

Definitions used (the OCP Microscaling Formats specification, v1.0):
- an element format with e exponent and m mantissa bits has bias
  2^(e-1) - 1, subnormals below 2^(1-bias), no infinities or NaNs in the
  FP4/FP6 formats, and largest normal 6 (E2M1), 7.5 (E2M3), 28 (E3M2) or
  448 (E4M3);
- a block's shared scale is X = 2^(floor(log2 amax) - emax), emax the
  exponent of the element format's largest normal (2, 2, 4, 8); each element
  is x / X rounded to nearest-even in the element format, saturating at the
  largest normal.

Only Q and K are quantized here (K after the SageAttention smoothing, the
channel mean over the keys subtracted, which leaves the softmax unchanged);
the softmax and P.V are exact float64, so the numbers isolate the Q.K^T
format.  The inputs are the seeded workload recipes at B = 1, two heads, N =
1024 keys.  Run this file as a script to print the table.
"""
from __future__ import annotations

import itertools
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

# name: (exponent bits, mantissa bits, largest normal, its exponent)
FORMATS = {
    "e2m1": (2, 1, 6.0, 2),
    "e2m3": (2, 3, 7.5, 2),
    "e3m2": (3, 2, 28.0, 4),
    "e4m3": (4, 3, 448.0, 8),
}
MX_BLOCK = 32


def quantize_fp(x, ebits: int, mbits: int, maxval: float) -> np.ndarray:
    """x (float64) rounded to nearest-even in the element format, saturating
    at +-maxval: within a binade [2^e, 2^(e+1)) the step is 2^(e - mbits);
    below the smallest normal exponent 1 - bias the step stays at its value
    there (subnormals)."""
    x = np.asarray(x, dtype=np.float64)
    bias = 2 ** (ebits - 1) - 1
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, 1 - bias)
    step = np.exp2(e - mbits)
    q = np.minimum(np.rint(a / step) * step, maxval)
    return np.copysign(q, x)


def element_grid(ebits: int, mbits: int, maxval: float) -> np.ndarray:
    """Every non-negative value the element format encodes, read off its bit
    fields (exponent field 0: subnormal m / 2^mbits * 2^(1-bias); else
    (1 + m / 2^mbits) * 2^(field - bias)), cut at the largest normal (E4M3
    gives its top code to NaN)."""
    bias = 2 ** (ebits - 1) - 1
    vals = []
    for ef, m in itertools.product(range(2 ** ebits), range(2 ** mbits)):
        if ef == 0:
            v = m / 2 ** mbits * 2.0 ** (1 - bias)
        else:
            v = (1 + m / 2 ** mbits) * 2.0 ** (ef - bias)
        if v <= maxval:
            vals.append(v)
    return np.unique(np.array(vals))


def mx_quantize(x, fmt: str) -> np.ndarray:
    """x [..., d] through the MX format: one E8M0 scale per 32 consecutive
    elements of the last axis; returns the dequantized values."""
    eb, mb, mx, emax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    s = x.shape
    xb = x.reshape(*s[:-1], s[-1] // MX_BLOCK, MX_BLOCK)
    amax = np.abs(xb).max(-1, keepdims=True)
    scale = np.exp2(np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - emax)
    return (quantize_fp(xb / scale, eb, mb, mx) * scale).reshape(s)


def int_quantize(x, group: int, qmax: int) -> np.ndarray:
    """x [..., n, d] with one scale absmax / qmax per `group` consecutive rows
    and codes rint(x / scale) clamped to +-qmax; returns the dequantized
    values (the scheme of the library's per-block, thread-level and token
    scale groups, with qmax 127 for INT8 and 7 for INT4-valued codes)."""
    x = np.asarray(x, dtype=np.float64)
    s = x.shape
    xb = x.reshape(*s[:-2], s[-2] // group, group, s[-1])
    am = np.abs(xb).max(axis=(-2, -1), keepdims=True)
    sc = np.where(am > 0, am / qmax, 1.0)
    return (np.clip(np.rint(xb / sc), -qmax, qmax) * sc).reshape(s)


def attention(q, k, v, causal: bool, sm_scale: float) -> np.ndarray:
    s = q @ np.swapaxes(k, -1, -2) * sm_scale
    if causal:
        n = s.shape[-1]
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    return (p @ v) / p.sum(-1, keepdims=True)


def accuracy(out, ref):
    o, r = out.ravel(), ref.ravel()
    return (float(o @ r / (np.linalg.norm(o) * np.linalg.norm(r))),
            float(np.abs(o - r).sum() / np.abs(r).sum()))


SCHEMES = {
    # name: (Q quantizer, K quantizer), applied to Q and smoothed K
    "int8 per-block": (lambda q: int_quantize(q, 128, 127), lambda k: int_quantize(k, 64, 127)),
    "int8 token": (lambda q: int_quantize(q, 1, 127), lambda k: int_quantize(k, 1, 127)),
    "int4 thread": (lambda q: int_quantize(q, 1, 7), lambda k: int_quantize(k, 32, 7)),
    "mxfp8 e4m3": (lambda q: mx_quantize(q, "e4m3"), lambda k: mx_quantize(k, "e4m3")),
    "mxfp6 e2m3": (lambda q: mx_quantize(q, "e2m3"), lambda k: mx_quantize(k, "e2m3")),
    "mxfp6 e3m2": (lambda q: mx_quantize(q, "e3m2"), lambda k: mx_quantize(k, "e3m2")),
    "mxfp4 e2m1": (lambda q: mx_quantize(q, "e2m1"), lambda k: mx_quantize(k, "e2m1")),
}


def study(n: int = 1024):
    """{workload name: {scheme: (cos, rel-L1)}} over the five recipes."""
    table = {}
    for wi, w0 in sorted(workloads.WORKLOADS.items()):
        w = w0.resized(B=1, Hq=2, Hkv=1 if w0.Hq != w0.Hkv else 2, N=n)
        q, k, v = (t.double().numpy() for t in workloads.generate(w))
        if w.Hkv != w.Hq:
            k = np.repeat(k, w.Hq // w.Hkv, axis=1)
            v = np.repeat(v, w.Hq // w.Hkv, axis=1)
        ref = attention(q, k, v, w.causal, w.sm_scale)
        ks = k - k.mean(axis=-2, keepdims=True)
        table[w0.name] = {name: accuracy(attention(fq(q), fk(ks), v, w.causal, w.sm_scale), ref)
                          for name, (fq, fk) in SCHEMES.items()}
    return table


# ------------------------------------------------------------------ pins

@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_element_grid_sizes_and_extremes(fmt):
    eb, mb, mx, _ = FORMATS[fmt]
    g = element_grid(eb, mb, mx)
    # FP4 and FP6 use every code (2^(e+m) magnitudes); E4M3 loses its NaN code
    assert len(g) == 2 ** (eb + mb) - (1 if fmt == "e4m3" else 0)
    assert g[0] == 0.0 and g[-1] == mx
    if fmt == "e2m1":
        assert list(g) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_rounding_is_nearest_even_on_the_grid(fmt):
    """Brute force: each x goes to the nearest grid value; on a tie, to the
    one whose code is even (the grid index of non-negative codes ordered by
    value has the code's parity); beyond the largest normal, to it."""
    eb, mb, mx, _ = FORMATS[fmt]
    g = element_grid(eb, mb, mx)
    rng = np.random.Generator(np.random.PCG64(11))
    mids = (g[1:] + g[:-1]) / 2
    x = np.concatenate([rng.uniform(-1.2 * mx, 1.2 * mx, 4000), g, -g, mids, -mids, [1.5 * mx, -3 * mx]])
    got = quantize_fp(x, eb, mb, mx)
    a = np.minimum(np.abs(x), mx)
    dist = np.abs(a[:, None] - g[None, :])
    best = dist.min(axis=1, keepdims=True)
    idx = []
    for c in dist == best:
        hits = np.flatnonzero(c)
        # a tie has two neighbours: take the even one
        idx.append(hits[0] if len(hits) == 1 or hits[0] % 2 == 0 else hits[1])
    want = np.copysign(g[np.array(idx)], x)
    assert np.array_equal(got, want)


def test_e4m3_elements_match_the_oracle_codec():
    """The generic quantizer at E4M3 equals the oracle's own E4M3 codec (the
    one P and V use) on values inside the format's range."""
    from oracle import e4m3_decode, e4m3_encode
    rng = np.random.Generator(np.random.PCG64(12))
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 5000),
                        rng.normal(0, 1e-3, 2000)])
    eb, mb, mx, _ = FORMATS["e4m3"]
    assert np.array_equal(quantize_fp(x, eb, mb, mx), e4m3_decode(e4m3_encode(x)))


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_mx_block_scale_rule(fmt):
    """The shared scale puts each block's largest magnitude in the binade of
    the element format's largest normal, and is a power of two."""
    eb, mb, mx, emax = FORMATS[fmt]
    rng = np.random.Generator(np.random.PCG64(13))
    x = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    xb = x.reshape(64, 4, 32)
    amax = np.abs(xb).max(-1)
    scale = np.exp2(np.floor(np.log2(amax)) - emax)
    assert np.all((amax / scale >= 2.0 ** emax) & (amax / scale < 2.0 ** (emax + 1)))
    y = mx_quantize(x, fmt).reshape(64, 4, 32)
    # every element is an element-format value times the block's scale
    g = element_grid(eb, mb, mx)
    e = np.abs(y / scale[..., None])
    assert np.all(np.isin(e, g))


def test_int_quantize_is_the_library_scheme():
    """Per-block INT8 here equals the oracle's quantize_q codes times scales."""
    import torch

    from oracle import quantize_q
    rng = np.random.Generator(np.random.PCG64(14))
    q = torch.from_numpy(rng.standard_normal((1, 2, 256, 64)).astype(np.float32)).half()
    z = quantize_q(q, 128)
    deq = z["q_i8"].astype(np.float64).reshape(1, 2, -1, 64)[:, :, :256] * \
        np.repeat(z["q_scale"].astype(np.float64).reshape(1, 2, -1), 128, axis=-1)[:, :, :256, None]
    got = int_quantize(q.double().numpy(), 128, 127)
    # the oracle divides in float32; allow one code step where a product sits on a tie
    assert np.abs(got - deq).max() <= z["q_scale"].max() * 1.0001


def test_mx_formats_against_the_int8_schemes():
    """The measured finding: no MX format reaches the accuracy of the INT8
    token scheme on any recipe, nor the per-block one's cosine; MXFP4 is as
    far from the lines as INT4-valued codes; of the formats at twice the INT8
    rate, E2M3 is the most accurate."""
    t = study(1024)
    for name, r in t.items():
        for fmt in ("mxfp8 e4m3", "mxfp6 e2m3", "mxfp6 e3m2", "mxfp4 e2m1"):
            assert r[fmt][1] > r["int8 token"][1] and r[fmt][0] < r["int8 token"][0], (name, fmt)
            assert r[fmt][0] < r["int8 per-block"][0], (name, fmt)
        assert r["mxfp4 e2m1"][1] > 0.15, name
        assert 0.6 < r["mxfp4 e2m1"][1] / r["int4 thread"][1] < 1.4, name
        assert r["mxfp6 e2m3"][1] < min(r["mxfp6 e3m2"][1], r["mxfp4 e2m1"][1]), name


if __name__ == "__main__":
    table = study(1024)
    schemes = list(SCHEMES)
    print("| workload (B=1, 2 heads, N=1024) | " + " | ".join(schemes) + " |")
    print("|---|" + "---:|" * len(schemes))
    for name, r in table.items():
        print(f"| {name} | " + " | ".join(f"{r[s][0]:.4f} / {r[s][1]:.4f}" for s in schemes) + " |")
