"""The oracle against the regression lock in tests/golden/ (written from the
oracle alone by tests/golden/make_golden.py): the same fp16 inputs must give
the same codes, scales and outputs, byte for byte.  Two closed forms on the
stored case are checked too: with the causal mask the first query sees only
the first key, so its full-precision output is that key's V row and its
quantized output is that row's dequantized E4M3 codes."""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_small_case.json")


def _arr(hexstr, dtype, shape=None):
    a = np.frombuffer(bytes.fromhex(hexstr), dtype=dtype)
    return a.reshape(shape) if shape is not None else a


def _case():
    with open(GOLDEN) as f:
        g = json.load(f)
    s = g["shape"]
    B, Hq, Hkv, N, d = s["B"], s["Hq"], s["Hkv"], s["N"], s["d"]
    q = torch.from_numpy(_arr(g["q_f16"], "<f2", (B, Hq, N, d)).copy())
    k = torch.from_numpy(_arr(g["k_f16"], "<f2", (B, Hkv, N, d)).copy())
    v = torch.from_numpy(_arr(g["v_f16"], "<f2", (B, Hkv, N, d)).copy())
    return g, q, k, v


def test_oracle_reproduces_the_locked_case(orc):
    g, q, k, v = _case()
    oz = orc.quantize(q, k, v, bq=g["q_block"], bk=g["k_block"], pv=g["pv"])
    for key in ("q_i8", "k_i8", "v_fp8"):
        assert np.ascontiguousarray(oz[key]).view(np.uint8).tobytes().hex() == g[key], key
    for key in ("q_scale", "k_scale", "k_mean", "v_scale"):
        assert np.asarray(oz[key], "<f4").tobytes().hex() == g[key], key
    for causal, tag in ((False, "full"), (True, "causal")):
        out = orc.attn_q(oz, causal, g["sm_scale"])[0]
        assert np.asarray(out, "<f8").tobytes().hex() == g[f"attn_q_{tag}"], tag
        ref = orc.attn_f64(q, k, v, causal, g["sm_scale"])
        assert np.asarray(ref, "<f8").tobytes().hex() == g[f"attn_f64_{tag}"], tag


def test_locked_case_first_causal_row_is_the_first_value_row(orc):
    g, q, k, v = _case()
    s = g["shape"]
    Hq, N, d = s["Hq"], s["N"], s["d"]
    f64 = _arr(g["attn_f64_causal"], "<f8", (Hq, N, d))
    qq = _arr(g["attn_q_causal"], "<f8", (Hq, N, d))
    v0 = v[0, 0, 0].double().numpy()
    codes = _arr(g["v_fp8"], np.uint8, (1, 1, N, d))[0, 0, 0]
    v0_q = orc.e4m3_decode(codes).astype(np.float64) * _arr(g["v_scale"], "<f4").astype(np.float64)
    for h in range(Hq):  # both q heads share the one kv head
        np.testing.assert_allclose(f64[h, 0], v0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(qq[h, 0], v0_q, rtol=1e-12, atol=1e-12)
