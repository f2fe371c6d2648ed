"""Writes oracle_small_case.json: a regression lock on the CPU oracle.

The pages print no worked example of the method (the accuracy tables of the
SageAttention article did not survive extraction), so this fixture holds no
value of theirs.  It records the oracle's own results on one tiny seeded case
(B = 1, Hq = 2, Hkv = 1, N = 3, d = 64, fp16, four K channels offset by 8 so
that smoothing matters) so that an unintended change to the oracle's
arithmetic shows up as a failing test (tests/test_oracle_golden.py).  The
oracle's correctness is pinned elsewhere (tests/test_oracle_*.py); this file
only keeps it from drifting.  Every array is stored as its little-endian bytes
in hex: inputs as fp16, codes as int8 / E4M3 bytes, scales and the mean as
float32, outputs as float64, so the comparison is exact.

Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_case.json")
SHAPE = dict(B=1, Hq=2, Hkv=1, N=3, d=64)
SM_SCALE = 0.125


def inputs():
    rng = np.random.Generator(np.random.PCG64(20261203))
    B, Hq, Hkv, N, d = (SHAPE[x] for x in ("B", "Hq", "Hkv", "N", "d"))
    q = rng.standard_normal((B, Hq, N, d)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    k[..., :4] += 8.0
    v = (rng.standard_normal((B, Hkv, N, d)) * 2.0).astype(np.float16)
    return q, k.astype(np.float16), v


def hexbytes(a) -> str:
    return np.ascontiguousarray(a).view(np.uint8).tobytes().hex()


def hexf32(a) -> str:
    return hexbytes(np.asarray(a, dtype="<f4"))


def hexf64(a) -> str:
    return hexbytes(np.asarray(a, dtype="<f8"))


def results(q, k, v) -> dict:
    oracle.build()
    oz = oracle.quantize(q, k, v, bq=128, bk=64, pv="e4m3")
    r = dict(q_i8=hexbytes(oz["q_i8"]), k_i8=hexbytes(oz["k_i8"]), v_fp8=hexbytes(oz["v_fp8"]),
             q_scale=hexf32(oz["q_scale"]), k_scale=hexf32(oz["k_scale"]),
             k_mean=hexf32(oz["k_mean"]), v_scale=hexf32(oz["v_scale"]))
    for causal in (False, True):
        tag = "causal" if causal else "full"
        r[f"attn_q_{tag}"] = hexf64(oracle.attn_q(oz, causal, SM_SCALE)[0])
        r[f"attn_f64_{tag}"] = hexf64(oracle.attn_f64(q, k, v, causal, SM_SCALE))
    return r


def main():
    q, k, v = inputs()
    doc = dict(what="oracle regression lock; written by tests/golden/make_golden.py from oracle/ only",
               shape=SHAPE, sm_scale=SM_SCALE, q_block=128, k_block=64, pv="e4m3",
               q_f16=hexbytes(q), k_f16=hexbytes(k), v_f16=hexbytes(v), **results(q, k, v))
    with open(OUT, "w") as f:  # one key per line
        f.write("{\n" + ",\n".join(f"{json.dumps(key)}: {json.dumps(val)}" for key, val in doc.items())
                + "\n}\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
