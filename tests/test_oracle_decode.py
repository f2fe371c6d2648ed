"""Pins of the oracle's short-query form (Nq query rows at the last Nq of Nk
positions, against a KV cache quantized once): against the self-attention
form it generalises (pinned in test_oracle_attn.py), torch's float64
attention with an explicit bottom-right mask, and closed forms."""
import math

import numpy as np
import pytest
import torch

import workloads


def _decode_dict(orc, q, k, v, bk=64, pv="e4m3"):
    z = orc.quantize_q(q, bq=1)
    z.update(orc.quantize_kv(k, v, bk=bk, pv=pv))
    return z


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
@pytest.mark.parametrize("bk", [64, 32])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(1, 300), (4, 300), (16, 129), (1, 1), (7, 7)])
def test_short_query_rows_equal_the_last_rows_of_self_attention(orc, Nq, Nk, causal, bk, pv):
    """With one Q scale per row, the codes of a row do not depend on the other
    rows, and the K/V half is the same: the short-query rows must equal, bit for
    bit, the last Nq rows of self-attention over the whole sequence (the
    bottom-right causal mask is the self-attention mask restricted to those
    rows).  GQA with G = 4."""
    G = 4
    q, k, v = workloads.random_inputs(2, 2 * G, 2, Nk, 64, "bf16", seed=Nq * 31 + Nk, scale=1.5)
    full = orc.quantize(q, k, v, bq=1, bk=bk, pv=pv)
    q_tail = q[:, :, Nk - Nq:].contiguous()
    short = _decode_dict(orc, q_tail, k, v, bk, pv)
    np.testing.assert_array_equal(short["q_i8"], full["q_i8"][:, :, Nk - Nq:])
    out_s, lo_s, hi_s, fl_s = orc.attn_q(short, causal, 0.125)
    rows = np.array([bh * Nk + Nk - Nq + i for bh in range(2 * 2 * G) for i in range(Nq)])
    out_f, lo_f, hi_f, fl_f = orc.attn_q(full, causal, 0.125, rows=rows)
    np.testing.assert_array_equal(out_s, out_f)
    np.testing.assert_array_equal(lo_s, lo_f)
    np.testing.assert_array_equal(hi_s, hi_f)
    np.testing.assert_array_equal(fl_s, fl_f)
    # and the float64 reference the same way
    ref_s = orc.attn_f64(q_tail, k, v, causal, 0.125)
    ref_f = orc.attn_f64(q, k, v, causal, 0.125, rows=rows)
    np.testing.assert_array_equal(ref_s, ref_f)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,G", [(1, 257, 1), (5, 300, 4), (3, 3, 2)])
def test_short_query_f64_matches_torch_with_bottom_right_mask(orc, Nq, Nk, G, causal):
    q, _, _ = workloads.random_inputs(1, 2 * G, 2, Nq, 64, "f16", seed=Nq + Nk, scale=2.0)
    _, k, v = workloads.random_inputs(1, 2 * G, 2, Nk, 64, "f16", seed=Nk, scale=2.0)
    out = orc.attn_f64(q, k, v, causal, 0.125)
    q64, k64, v64 = (x.to(torch.float64) for x in (q, k, v))
    k64 = k64.repeat_interleave(G, dim=1)
    v64 = v64.repeat_interleave(G, dim=1)
    mask = None
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = j <= i + (Nk - Nq)
    ref = torch.nn.functional.scaled_dot_product_attention(q64, k64, v64, attn_mask=mask, scale=0.125)
    np.testing.assert_allclose(out, ref.reshape(-1, 64).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
def test_short_zero_query_gives_prefix_means(orc, pv):
    """Q = 0 against the cache: every P code is the block maximum's, so row i
    gets the mean of the dequantized V over keys 0 .. Nk - Nq + i (causal),
    or over all keys."""
    Nq, Nk, d = 4, 300, 64
    _, k, v = workloads.random_inputs(1, 2, 2, Nk, d, "f16", seed=9)
    q = torch.zeros(1, 2, Nq, d, dtype=torch.float16)
    z = _decode_dict(orc, q, k, v, pv=pv)
    if pv == "f16":
        vd = z["v_f16"].view(np.float16).astype(np.float64)
    else:
        vd = orc.e4m3_decode(z["v_fp8"]) * z["v_scale"].astype(np.float64)[:, :, None, :]
    vd = vd.reshape(2, Nk, d)
    for causal in (False, True):
        out, _, _, fl = orc.attn_q(z, causal, 0.125)
        out = out.reshape(2, Nq, d)
        for i in range(Nq):
            n = Nk - Nq + i + 1 if causal else Nk
            np.testing.assert_allclose(out[:, i], vd[:, :n].mean(axis=1), rtol=1e-12, atol=1e-14)
        assert fl.sum() == 0


def test_decode_workloads_are_short_queries():
    for w in workloads.DECODE_WORKLOADS.values():
        q, k, v = workloads.generate(w.resized(N=300, B=1))
        assert q.shape[2] == w.Nq and k.shape[2] == 300 and v.shape == k.shape
        # ops: Nq rows, each seeing Nk - Nq + i + 1 keys
        pairs = sum(300 - w.Nq + i + 1 for i in range(w.Nq))
        assert w.resized(N=300, B=1).ops == 4.0 * w.Hq * pairs * w.d
