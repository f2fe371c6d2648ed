"""The decode entry point that allocates nothing (sage_attn_decode_noalloc),
through the C ABI, against the workspace-taking sage_attn_decode on the same
cache and query: the outputs must be identical (same kernels, same partial
layout; the scratch is the library's own per-GPU array).  Two calls in a row,
the second with a smaller input, then the first shape again, so that what an
earlier call left in the shared array cannot leak into a later result; each
output is also checked against the CPU oracle's interval."""
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


def _inputs(B, Hq, Hkv, Nq, Nk, d, seed):
    w = workloads.WORKLOADS[4].resized(B=B, Hq=Hq, Hkv=Hkv, N=Nk, d=d, Nq=Nq)
    q, k, v = workloads.generate(w, seed=seed)
    return w, q, k, v


def _one(sage, orc, B, Hq, Hkv, Nq, Nk, d, seed, granularity="block", pv="e4m3"):
    _say(f"case no-alloc decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {granularity} {pv}")
    w, q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, seed)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    cache = sage.KVCache(kd, vd, granularity=granularity, pv=pv)
    sm = 1 / math.sqrt(d)
    ref = cache.attend(qd, causal=True, sm_scale=sm)
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32, device="cuda")
    sage.sage_attn_decode_noalloc(qd, cache.z, out, Hkv, Nk, True, sm)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    bk = {"block": 64, "thread": 32}[granularity]
    oz = orc.quantize_q(q, bq=1)
    oz.update(orc.quantize_kv(k, v, bk=bk, pv=pv))
    nom, lo, hi, _ = orc.attn_q(oz, True, sm)
    g = out.reshape(-1, d).cpu().numpy().astype(np.float64)
    dist = orc.interval_distance(g, lo, hi)
    _say(f"   max|dist|={dist.max():.3e} relL1={dist.sum() / np.abs(nom).sum():.3e}")
    assert dist.max() <= MAX_ABS and dist.sum() / np.abs(nom).sum() <= REL_L1


def test_noalloc_decode_equals_workspace_decode(sage, orc):
    # many key chunks (the scratch holds their partials) ...
    _one(sage, orc, 1, 32, 8, 1, 32768, 128, seed=41)
    # ... then a smaller input on the same array (fewer chunks, other layout)
    _one(sage, orc, 2, 8, 2, 3, 5000, 64, seed=42, granularity="thread", pv="f16")
    # one chunk: the kernel writes the output, the array is not touched
    _one(sage, orc, 1, 4, 4, 2, 200, 64, seed=43)
    # the first shape again
    _one(sage, orc, 1, 32, 8, 1, 32768, 128, seed=44)
