"""GPU parity of the short-query path over a quantized KV cache (through the
C ABI) against the CPU oracle.

The cache (K mean, INT8 K and its scales, V as E4M3 code bytes or binary16)
must be bit-exact against the oracle's K/V half of the prep.  The attention
output must lie within the oracle's interval (see test_gpu_parity.py) up to
max-abs 2e-3 and rel-L1 1e-3.  Cases cover one and several query rows, GQA packing of up to several
32-row tiles, caches that take one key chunk (the kernel writes the output)
and many (the merge kernel does), ragged key counts, both K granularities and
both P.V formats.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L1 = 2e-3, 1e-3


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_02_amd as s
    return s


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_decode(sage, q, k, v, causal, sm_scale, granularity="block", pv="e4m3"):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    cache = sage.KVCache(kd, vd, granularity=granularity, pv=pv)
    out = cache.attend(qd, causal=causal, sm_scale=sm_scale)
    torch.cuda.synchronize()
    B, Hkv, Nk, d = k.shape
    quant = sage.read_kv_cache(cache.z, cache.buf, B, Hkv, Nk, d)
    return out, quant


def oracle_dict(orc, q, k, v, granularity, pv):
    bk = {"block": 64, "thread": 32}[granularity]
    z = orc.quantize_q(q, bq=1)
    z.update(orc.quantize_kv(k, v, bk=bk, pv=pv))
    return z


def check_cache(orc, quant, oz):
    np.testing.assert_array_equal(quant["k_i8"].numpy(), oz["k_i8"])
    np.testing.assert_array_equal(quant["k_mean"].numpy(), oz["k_mean"])
    nkb = oz["k_scale"].shape[-1]
    np.testing.assert_array_equal(quant["k_scale"].numpy()[..., :nkb], oz["k_scale"])
    if oz["pv"] == "f16":
        np.testing.assert_array_equal(quant["v_f16"].numpy().view(np.uint16), oz["v_f16"])
        assert (quant["v_scale"].numpy() == 1.0).all()
    else:
        np.testing.assert_array_equal(quant["v_fp8"].numpy(), oz["v_fp8"])
        np.testing.assert_array_equal(quant["v_scale"].numpy(), oz["v_scale"])
    assert not quant["k_pad"].any() and not quant["v_pad"].any()
    vals = orc.f16_decode(oz["v_f16"]) if oz["pv"] == "f16" else orc.e4m3_decode(oz["v_fp8"])
    np.testing.assert_array_equal(quant["v_half"].to(torch.float64).numpy(), vals)


def check_attn(orc, got, oz, causal, sm_scale, rows=None):
    nom, lo, hi, flagged = orc.attn_q(oz, causal, sm_scale, rows=rows)
    g = got.astype(np.float64)
    assert np.isfinite(g).all()
    dist = orc.interval_distance(g, lo, hi)
    max_abs = float(dist.max())
    rel = float(dist.sum() / np.abs(nom).sum())
    _say(f"   parity: max|dist|={max_abs:.3e} relL1={rel:.3e} "
         f"nominal max={float(np.abs(g - nom).max()):.3e} flagged={int(flagged.sum())}")
    assert max_abs <= MAX_ABS and rel <= REL_L1
    return nom


# (B, Hq, Hkv, Nq, Nk, d): single query rows, speculative-style short
# queries, GQA packing of 1..3 row tiles, one chunk (Nk <= 512) and many
CASES = [
    (1, 4, 4, 1, 1, 64), (1, 8, 2, 1, 100, 128), (2, 8, 2, 1, 128, 64), (1, 4, 1, 2, 129, 64),
    (1, 32, 8, 1, 1000, 128), (2, 8, 8, 5, 4097, 64), (1, 16, 2, 5, 3000, 128),
    (1, 12, 1, 7, 700, 64), (1, 4, 2, 16, 16, 128), (1, 2, 2, 3, 20000, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_decode_parity(sage, orc, case, causal):
    B, Hq, Hkv, Nq, Nk, d = case
    i = CASES.index(case)
    granularity = "thread" if i % 2 else "block"
    pv = "f16" if i % 3 == 1 else "e4m3"
    dtype = "bf16" if i % 2 == 0 else "f16"
    _say(f"case decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} "
         f"granularity={granularity} pv={pv} dtype={dtype}")
    q, _, _ = workloads.random_inputs(B, Hq, Hkv, Nq, d, dtype, seed=100 + i, scale=1.5)
    _, k, v = workloads.random_inputs(B, Hq, Hkv, Nk, d, dtype, seed=200 + i, scale=1.5)
    sm = 1 / math.sqrt(d)
    out, quant = run_decode(sage, q, k, v, causal, sm, granularity, pv)
    oz = oracle_dict(orc, q, k, v, granularity, pv)
    check_cache(orc, quant, oz)
    check_attn(orc, out.reshape(-1, d).cpu().numpy(), oz, causal, sm)


def test_decode_degenerate_inputs(sage, orc):
    """Zero query rows (uniform weights over the allowed keys), identical K
    rows, a zero V channel and a dominant key, in one cache."""
    B, Hq, Hkv, Nq, Nk, d = 1, 8, 2, 3, 777, 64
    q, _, _ = workloads.random_inputs(B, Hq, Hkv, Nq, d, "f16", seed=5)
    _, k, v = workloads.random_inputs(B, Hq, Hkv, Nk, d, "f16", seed=6)
    q[0, 0] = 0.0
    k[0, 1] = k[0, 1, :1].clone()
    v[0, 0, :, 5] = 0.0
    k[0, 0, 400] = 12.0
    q[0, 1] = q[0, 1].abs()
    for causal, pv in ((True, "e4m3"), (False, "f16")):
        _say(f"case decode degenerate causal={causal} pv={pv}")
        out, quant = run_decode(sage, q, k, v, causal, 0.125, "block", pv)
        oz = oracle_dict(orc, q, k, v, "block", pv)
        check_cache(orc, quant, oz)
        check_attn(orc, out.reshape(-1, d).cpu().numpy(), oz, causal, 0.125)


def test_cache_on_a_used_buffer(sage, orc):
    """sage_kv_quantize clears its own arrival counters: a cache buffer filled
    with 0xFF bytes gives the same cache as a fresh one."""
    B, Hkv, Nk, d = 2, 2, 1500, 128
    _, k, v = workloads.random_inputs(B, 4, Hkv, Nk, d, "bf16", seed=31, scale=2.0)
    kd, vd = k.cuda(), v.cuda()
    a = sage.KVCache(kd, vd)
    b = sage.KVCache(kd, vd)
    b.buf.fill_(0xFF)
    sage.sage_kv_quantize(kd, vd, b.z)
    torch.cuda.synchronize()
    qa = sage.read_kv_cache(a.z, a.buf, B, Hkv, Nk, d)
    qb = sage.read_kv_cache(b.z, b.buf, B, Hkv, Nk, d)
    for key in ("k_i8", "v_half", "k_mean", "v_scale", "k_scale"):
        assert torch.equal(qa[key], qb[key]), key


@pytest.mark.parametrize("index,granularity,pv", [(6, "block", "e4m3"), (7, "block", "e4m3"),
                                                  (6, "thread", "f16")])
def test_decode_full_size_workloads(sage, orc, index, granularity, pv):
    """The decode workloads at their full size, as the benchmark runs them:
    cache bit-exact, every query row against the oracle, and the method's
    accuracy against float64 reported."""
    w = workloads.DECODE_WORKLOADS[index]
    _say(f"case full-size decode workload {index} {w.name} granularity={granularity} pv={pv}")
    q, k, v = workloads.generate(w)
    out, quant = run_decode(sage, q, k, v, w.causal, w.sm_scale, granularity, pv)
    oz = oracle_dict(orc, q, k, v, granularity, pv)
    check_cache(orc, quant, oz)
    got = out.reshape(-1, w.d).cpu().numpy()
    nom = check_attn(orc, got, oz, w.causal, w.sm_scale)
    ref = orc.attn_f64(q, k, v, w.causal, w.sm_scale)
    a_gpu, a_orc = orc.accuracy(got, ref), orc.accuracy(nom, ref)
    _say(f"   vs float64: gpu cos={a_gpu['cos']:.6f} relL1={a_gpu['rel_l1']:.4f}; "
         f"oracle cos={a_orc['cos']:.6f} relL1={a_orc['rel_l1']:.4f}")
