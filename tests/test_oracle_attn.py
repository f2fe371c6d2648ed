"""Pins of the oracle's attention (full-precision and quantized) against facts
that do not come from the oracle: torch's scaled_dot_product_attention in
float64, the softmax invariance the SageAttention page states for K smoothing,
closed forms, an independently written online-softmax recurrence on tiny
inputs, and the E4M3 error bound."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads


def _sdpa64(q, k, v, causal, scale):
    q, k, v = (x.to(torch.float64) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    return o.reshape(-1, q.shape[-1]).numpy()


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [
    (1, 2, 2, 256, 64, False), (2, 4, 1, 77, 128, True), (1, 8, 2, 300, 64, True),
    (1, 1, 1, 1, 64, False), (1, 1, 1, 1, 128, True)])
def test_f64_attention_matches_torch_sdpa(orc, B, Hq, Hkv, N, d, causal):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, "f16", seed=N, scale=2.0)
    out = orc.attn_f64(q, k, v, causal, 1 / math.sqrt(d))
    np.testing.assert_allclose(out, _sdpa64(q, k, v, causal, 1 / math.sqrt(d)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("recipe", [1, 2, 3, 4, 5])
def test_k_smoothing_leaves_softmax_unchanged(orc, recipe):
    """softmax(QK^T) = softmax(Q(K - mean K)^T): the invariance the SageAttention
    page states for K smoothing, in float64 to 1e-12 (with and without the
    causal mask, since the subtracted term is constant along each row)."""
    w0 = workloads.WORKLOADS[recipe]
    w = w0.resized(B=1, Hq=w0.Hq // w0.Hkv * 2, Hkv=2, N=257)
    q, k, v = workloads.generate(w, seed=recipe)
    z = orc.quantize(q, k, v)
    k32 = orc.to_f32(k).astype(np.float64)
    ks = k32 - z["k_mean"][:, :, None, :].astype(np.float64)
    for causal in (False, True):
        a = orc.attn_f64(q, k32, v, causal, w.sm_scale)
        b = orc.attn_f64(q, ks, v, causal, w.sm_scale)
        scale = np.abs(a).max()
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, scale)


def _deq_inputs(orc, z):
    N = z["N"]
    sq = np.repeat(z["q_scale"].astype(np.float64), z["bq"], axis=-1)[..., :N, None]
    sk = np.repeat(z["k_scale"].astype(np.float64), z["bk"], axis=-1)[..., :N, None]
    qd = z["q_i8"].astype(np.float64) * sq
    kd = z["k_i8"].astype(np.float64) * sk
    if z["pv"] == "f16":
        vd = z["v_f16"].view(np.float16).astype(np.float64)
    else:
        vd = orc.e4m3_decode(z["v_fp8"]) * z["v_scale"].astype(np.float64)[:, :, None, :]
    return qd, kd, vd


def _max_log2_score(qd, kd, sm_scale):
    """Largest |score| in log2 units over every (query, key) pair of the
    dequantized operands (kv head h // G for query head h)."""
    G = qd.shape[1] // kd.shape[1]
    kr = np.repeat(kd, G, axis=1)
    return float(np.abs(qd @ kr.transpose(0, 1, 3, 2)).max() * sm_scale * math.log2(math.e))


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_dequantized_v(orc, causal, pv):
    """Q = 0: every score is 0, every P code is the block maximum's (448, or 1
    in binary16) and the output is the (prefix) mean of the dequantized V
    rows, exactly (the quantized weights are normalised by their own sum)."""
    N, d = 300, 64
    _, k, v = workloads.random_inputs(1, 2, 2, N, d, "f16", seed=5)
    q = torch.zeros(1, 2, N, d, dtype=torch.float16)
    z = orc.quantize(q, k, v, pv=pv)
    out, lo, hi, fl = orc.attn_q(z, causal, 0.125)
    _, _, vd = _deq_inputs(orc, z)
    vd = vd.reshape(2, N, d)
    if causal:
        ref = np.cumsum(vd, axis=1) / np.arange(1, N + 1)[None, :, None]
    else:
        ref = np.broadcast_to(vd.mean(axis=1, keepdims=True), vd.shape)
    np.testing.assert_allclose(out, ref.reshape(-1, d), rtol=1e-12, atol=1e-14)
    assert fl.sum() == 0


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
def test_one_dominant_key_gives_its_value(orc, pv):
    """A key whose score exceeds every other by > 30 nats (> 43 in log2, past
    binary16's smallest subnormal 2^-24): every other P code is 0, so the
    output is exactly its dequantized V row."""
    N, d = 256, 64
    rng = np.random.Generator(np.random.PCG64(9))
    q = torch.ones(1, 1, N, d, dtype=torch.float16)
    k = torch.from_numpy(rng.normal(0, 0.1, (1, 1, N, d)).astype(np.float32)).half()
    jstar = 77
    k[0, 0, jstar] = 10.0
    v = torch.from_numpy(rng.normal(0, 1, (1, 1, N, d)).astype(np.float32)).half()
    z = orc.quantize(q, k, v, pv=pv)
    out, _, _, _ = orc.attn_q(z, False, 0.125)
    _, _, vd = _deq_inputs(orc, z)
    np.testing.assert_allclose(out, np.broadcast_to(vd[0, 0, jstar], out.shape), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_constant_keys_give_weighted_block_means(orc, causal, pv):
    """Keys equal within every 128-key P block: every P code of a block is the
    block maximum's (448, or 1 in binary16),
    so the output is the softmax over blocks (weights n_t * e^{S_t}) of the
    per-block V means -- checks the second accumulation level and the row
    normalisation against the dequantized scores in float64."""
    N, d, bn = 512 + 37, 64, 128
    rng = np.random.Generator(np.random.PCG64(21))
    nb = -(-N // bn)
    kblk = rng.normal(0, 1.5, (nb, d)).astype(np.float32)
    k = torch.from_numpy(np.repeat(kblk, bn, axis=0)[:N][None, None]).half()
    q = torch.from_numpy(rng.normal(0, 1, (1, 1, N, d)).astype(np.float32)).half()
    v = torch.from_numpy(rng.normal(0, 1, (1, 1, N, d)).astype(np.float32)).half()
    z = orc.quantize(q, k, v, bk=128, pv=pv)
    out, _, _, fl = orc.attn_q(z, causal, 0.125, bn=bn)
    qd, kd, vd = _deq_inputs(orc, z)
    ref = orc.attn_f64(qd, kd, vd, causal, 0.125)
    assert fl.sum() == 0
    # every score of a block is equal, so every code is the block maximum's and
    # the only error left is the float32 evaluation of the log2 block weights:
    # c = f32(f32(s_q f32(sm_scale log2 e)) s_k) and m_t = f32(acc c) carry at
    # most four roundings (relative 2^-24 each), so each m_t, and each
    # difference m_t - M, is off by at most eps = 8 2^-24 max|m|; the block
    # weights are off by factors within 2^(+-eps), which moves a convex
    # combination of the block means by at most 2 (2^eps - 1) max|V|
    m_max = _max_log2_score(qd, kd, 0.125)
    eps = 8 * 2.0 ** -24 * (m_max + 1)
    np.testing.assert_allclose(out, ref, rtol=0, atol=2 * (2.0 ** eps - 1) * np.abs(vd).max() + 1e-12)


# ----------------------------------------------------------------------------
# An independent coding of the quantized attention as the online recurrence
# (running maximum, rescaling of the accumulator), with exact float32 rounding
# done through fractions.  Tiny inputs only.

def _round_f32(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even."""
    f = np.float32(float(x))
    lo = f if Fraction(float(f)) <= x else np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    dl, dh = x - Fraction(float(lo)), Fraction(float(hi)) - x
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (np.array(lo).view(np.uint32) & 1) == 0 else hi


def _fma_f32(a, b, c) -> np.float32:
    return _round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def _online_reference(orc, z, causal, sm_scale, bn):
    """P.V in E4M3 (codes through torch's float8_e4m3fn) or in binary16 (codes
    through numpy's float16), never through the oracle's own encoders."""
    B, Hq, Hkv, N, d = z["B"], z["Hq"], z["Hkv"], z["N"], z["d"]
    G = Hq // Hkv
    f16 = z["pv"] == "f16"
    qk = np.float32(sm_scale * math.log2(math.e))
    l448 = np.float32(0.0) if f16 else np.float32(math.log2(448.0))
    if f16:
        vrow = z["v_f16"].view(np.float16).astype(np.float64)
        vscale = np.ones((B, Hkv, d))

        def p_code(y):
            return float(np.float16(y))
    else:
        vrow = torch.from_numpy(z["v_fp8"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        vscale = z["v_scale"].astype(np.float64)

        def p_code(y):
            return torch.tensor([y], dtype=torch.float64).to(torch.float8_e4m3fn).to(
                torch.float64).item()
    out = np.zeros((B * Hq * N, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                m_run, l_run = -math.inf, 0.0
                o_run = np.zeros(d)
                for t0 in range(0, len(keys), bn):
                    blk = [j for j in keys if t0 <= j < t0 + bn]
                    s_q = np.float32(z["q_scale"][b, h, i // z["bq"]])
                    accs, cs = [], []
                    for j in blk:
                        acc = int(np.dot(z["q_i8"][b, h, i].astype(np.int64),
                                         z["k_i8"][b, g, j].astype(np.int64)))
                        c = np.float32(np.float32(s_q * qk) * z["k_scale"][b, g, j // z["bk"]])
                        accs.append(acc)
                        cs.append(c)
                    # FP32 softmax: the exact integer score times the score
                    # factor, rounded once; the block's largest such value is
                    # the P scale (its code is the format's largest, 448 or 1)
                    mt = max(_round_f32(Fraction(a) * Fraction(float(c))) for a, c in zip(accs, cs))
                    bias = np.float32(l448 - mt)
                    a_blk = np.zeros(d)
                    r_blk = 0.0
                    for j, a, c in zip(blk, accs, cs):
                        y = 2.0 ** float(_fma_f32(np.float32(a), c, bias))
                        p = p_code(y)
                        a_blk += p * vrow[b, g, j]
                        r_blk += p
                    m_new = max(m_run, float(mt))
                    alpha = 2.0 ** (m_run - m_new) if m_run > -math.inf else 0.0
                    wgt = 2.0 ** (float(mt) - m_new)
                    o_run = alpha * o_run + wgt * a_blk
                    l_run = alpha * l_run + wgt * r_blk
                    m_run = m_new
                out[(b * Hq + h) * N + i] = o_run * vscale[b, g] / l_run
    return out


@pytest.mark.parametrize("pv,qk_bits", [("e4m3", 8), ("f16", 8), ("e4m3", 4)])
@pytest.mark.parametrize("N", [1, 2, 3, 5, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,G", [(64, 1), (128, 4)])
def test_closed_form_equals_online_recurrence_tiny(orc, N, causal, d, G, pv, qk_bits):
    """The oracle's closed form over P blocks equals the online recurrence
    (running max, rescaled accumulator) with small blocks so several blocks and
    ragged tails occur (bq=4, bk=2, bn=4)."""
    q, k, v = workloads.random_inputs(1, G, 1, N, d, "bf16", seed=100 + N + d, scale=1.5)
    z = orc.quantize(q, k, v, bq=4, bk=2, pv=pv, qk_bits=qk_bits)
    out, lo, hi, fl = orc.attn_q(z, causal, 1 / math.sqrt(d), bn=4)
    ref = _online_reference(orc, z, causal, 1 / math.sqrt(d), bn=4)
    ok = fl == 0
    np.testing.assert_allclose(out[ok], ref[ok], rtol=1e-12, atol=1e-13)
    assert np.all(lo[~ok] <= ref[~ok] + 1e-12) and np.all(ref[~ok] <= hi[~ok] + 1e-12)


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
@pytest.mark.parametrize("N", [7, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_closed_form_equals_online_recurrence_heavy_tails(orc, N, causal, pv):
    """The same check on the heavy-tail recipe (Student-t(3)), with one
    element of +-50 planted in every Q and K scale block: the large block
    absmax against small typical codes makes the score factor c of every
    block about 0.02-0.03, where the float32 evaluation of each exponent must
    still be the plain one (f32(acc) c plus one rounded bias) for the codes
    and block weights to agree."""
    w = workloads.WORKLOADS[5].resized(B=1, Hq=2, Hkv=1, N=N)
    q, k, v = workloads.generate(w, seed=300 + N)
    rng = np.random.Generator(np.random.PCG64(N))
    for t, r0 in ((q, 4), (k, 2)):
        for h in range(t.shape[1]):
            for r in range(0, N, r0):
                t[0, h, r, int(rng.integers(w.d))] = float(rng.choice([-50.0, 50.0]))
    z = orc.quantize(q, k, v, bq=4, bk=2, pv=pv)
    c = np.outer(z["q_scale"].ravel(), z["k_scale"].ravel()) * w.sm_scale * math.log2(math.e)
    assert c.min() > 0.015
    out, lo, hi, fl = orc.attn_q(z, causal, w.sm_scale, bn=4)
    ref = _online_reference(orc, z, causal, w.sm_scale, bn=4)
    ok = fl == 0
    np.testing.assert_allclose(out[ok], ref[ok], rtol=1e-12, atol=1e-12)
    assert np.all(lo[~ok] <= ref[~ok] + 1e-12) and np.all(ref[~ok] <= hi[~ok] + 1e-12)


@pytest.mark.parametrize("recipe", [1, 2, 3, 4, 5])
def test_quantized_attention_within_p_rounding_of_dequantized_reference(orc, recipe):
    """Against float64 attention on the dequantized Q, K-smoothed and V codes,
    the only remaining error is P's E4M3 rounding: P8_j = y_j (1 + e_j) with
    |e_j| <= 2^-4 in the normal range and |P8_j - y_j| <= 2^-10 below it.  The
    output sum_j P8_j V_j / sum_j P8_j is then within
    2 max|V| (2^-4 / (1 - 2^-4) + n 2^-10 / 448) of the exact weighted mean
    (the row sum is at least 448, the code of the row maximum).  The typical
    error is far smaller (the rounding errors are unbiased)."""
    w0 = workloads.WORKLOADS[recipe]
    w = w0.resized(B=1, Hq=w0.Hq // w0.Hkv * 2, Hkv=2, N=700)
    q, k, v = workloads.generate(w, seed=recipe)
    z = orc.quantize(q, k, v)
    rows = workloads.sample_rows(w, 200)
    out, lo, hi, _ = orc.attn_q(z, w.causal, w.sm_scale, rows=rows)
    qd, kd, vd = _deq_inputs(orc, z)
    ref = orc.attn_f64(qd, kd, vd, w.causal, w.sm_scale, rows=rows)
    vmax = np.abs(vd).max()
    bound = 2 * vmax * (2.0 ** -4 / (1 - 2.0 ** -4) + w.N * 2.0 ** -10 / 448.0)
    assert np.abs(out - ref).max() <= bound
    acc = orc.accuracy(out, ref)
    assert acc["rel_l1"] < 0.04 and acc["cos"] > 0.999
    assert np.all(lo <= out) and np.all(out <= hi)


@pytest.mark.parametrize("recipe", [1, 2, 3, 4, 5])
def test_f16_pv_within_p_rounding_of_dequantized_reference(orc, recipe):
    """The binary16 P.V mode against float64 attention on the dequantized Q,
    K-smoothed and binary16 V.  Two errors remain: P16_j = y_j (1 + e_j) with
    |e_j| <= 2^-11 for y_j >= 2^-14 and |P16_j - y_j| <= 2^-25 below; and the
    float32 evaluation of the log2 weights (the score factor c, the block
    maximum m and the exponent x each carry a few roundings of relative size
    2^-24), which moves each log2 weight by at most eps = 16 2^-24 (max|m| +
    1).  Each weight is thus off by a factor within 1 +- r,
    r = (1 + 2^-11) 2^eps - 1, and (the row sum being at least 1, the code of
    the row maximum) the output is within 2 max|V| (r / (1 - r) + n 2^-25) of
    the exact weighted mean."""
    w0 = workloads.WORKLOADS[recipe]
    w = w0.resized(B=1, Hq=w0.Hq // w0.Hkv * 2, Hkv=2, N=700)
    q, k, v = workloads.generate(w, seed=recipe)
    z = orc.quantize(q, k, v, pv="f16")
    rows = workloads.sample_rows(w, 200)
    out, lo, hi, _ = orc.attn_q(z, w.causal, w.sm_scale, rows=rows)
    qd, kd, vd = _deq_inputs(orc, z)
    ref = orc.attn_f64(qd, kd, vd, w.causal, w.sm_scale, rows=rows)
    vmax = np.abs(vd).max()
    eps = 16 * 2.0 ** -24 * (_max_log2_score(qd, kd, w.sm_scale) + 1)
    r = (1 + 2.0 ** -11) * 2.0 ** eps - 1
    bound = 2 * vmax * (r / (1 - r) + w.N * 2.0 ** -25)
    assert np.abs(out - ref).max() <= bound
    assert np.all(lo <= out) and np.all(out <= hi)


@pytest.mark.parametrize("recipe", [3, 5])
def test_f16_pv_is_closer_to_full_precision_than_e4m3(orc, recipe):
    """The SageAttention2 summary ranks E4M3 as nearly as accurate as FP16
    for P and V: the binary16 mode's error against float64 attention on the
    original inputs is the smaller one, and what remains is the INT8 Q.K^T."""
    w0 = workloads.WORKLOADS[recipe]
    w = w0.resized(B=1, Hq=w0.Hq // w0.Hkv * 2, Hkv=2, N=700)
    q, k, v = workloads.generate(w, seed=recipe)
    rows = workloads.sample_rows(w, 200)
    ref = orc.attn_f64(q, k, v, w.causal, w.sm_scale, rows=rows)
    e8 = orc.accuracy(orc.attn_q(orc.quantize(q, k, v), w.causal, w.sm_scale, rows=rows)[0], ref)
    e16 = orc.accuracy(orc.attn_q(orc.quantize(q, k, v, pv="f16"), w.causal, w.sm_scale,
                                  rows=rows)[0], ref)
    assert e16["rel_l1"] < e8["rel_l1"] and e16["cos"] > e8["cos"]


@pytest.mark.parametrize("recipe", [1, 3, 5])
def test_int4_qk_within_p_rounding_of_dequantized_reference(orc, recipe):
    """The 4-bit Q, K variant changes only the codes: against float64
    attention on its own dequantized Q, K and V, the error is P's E4M3
    rounding, as for INT8."""
    w0 = workloads.WORKLOADS[recipe]
    w = w0.resized(B=1, Hq=w0.Hq // w0.Hkv * 2, Hkv=2, N=500)
    q, k, v = workloads.generate(w, seed=recipe)
    z = orc.quantize(q, k, v, qk_bits=4)
    assert np.abs(z["q_i8"]).max() == 7 and np.abs(z["k_i8"]).max() == 7
    rows = workloads.sample_rows(w, 120)
    out, lo, hi, _ = orc.attn_q(z, w.causal, w.sm_scale, rows=rows)
    qd, kd, vd = _deq_inputs(orc, z)
    ref = orc.attn_f64(qd, kd, vd, w.causal, w.sm_scale, rows=rows)
    bound = 2 * np.abs(vd).max() * (2.0 ** -4 / (1 - 2.0 ** -4) + w.N * 2.0 ** -10 / 448.0)
    assert np.abs(out - ref).max() <= bound
    assert np.all(lo <= out) and np.all(out <= hi)


def test_int4_qk_needs_smoothing_and_fine_scales(orc):
    """The Berkeley brief and the SageAttention2 summary: 4-bit Q, K lose
    accuracy without outlier smoothing and fine-grained scales.  With K
    channel outliers, INT4 without smoothing is worse than with it, per-row /
    32-key scales improve on per-block ones, and INT8 stays far better than
    INT4 (attending with exact V isolates the Q, K part)."""
    w = workloads.WORKLOADS[3].resized(B=1, Hq=2, Hkv=2, N=600)
    q, k, v = workloads.generate(w, seed=3)
    rows = workloads.sample_rows(w, 150)
    ref = orc.attn_f64(q, k, v, w.causal, w.sm_scale, rows=rows)

    def err(**kw):
        z = orc.quantize(q, k, v, **kw)
        qd, kd, _ = _deq_inputs(orc, z)
        kd = kd + (0.0 if kw.get("smooth", True) is False else z["k_mean"][:, :, None, :])
        return orc.accuracy(orc.attn_f64(qd, kd, orc.to_f32(v), w.causal, w.sm_scale, rows=rows),
                            ref)["rel_l1"]

    e4_raw = err(qk_bits=4, smooth=False)
    e4 = err(qk_bits=4)
    e4_fine = err(qk_bits=4, bq=1, bk=32)
    e8 = err(qk_bits=8)
    assert e4_raw > 1.2 * e4 and e4_fine < 0.9 * e4 and e8 < 0.2 * e4_fine


def test_smoothing_helps_when_k_has_channel_outliers(orc):
    """The SageAttention page's motivation for smoothing: with K channel
    outliers, INT8 Q,K without smoothing are much less accurate.  The INT8
    part is isolated by attending with the dequantized Q and K and exact V."""
    w = workloads.WORKLOADS[3].resized(B=1, Hq=2, Hkv=2, N=600)
    q, k, v = workloads.generate(w, seed=4)
    rows = workloads.sample_rows(w, 200)
    ref = orc.attn_f64(q, k, v, False, w.sm_scale, rows=rows)
    errs = {}
    for smooth in (True, False):
        z = orc.quantize(q, k, v, smooth=smooth)
        qd, kd, _ = _deq_inputs(orc, z)
        out = orc.attn_f64(qd, kd, v, False, w.sm_scale, rows=rows)
        errs[smooth] = orc.accuracy(out, ref)["rel_l1"]
    assert errs[True] < 0.75 * errs[False]
