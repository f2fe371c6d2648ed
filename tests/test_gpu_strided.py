"""Inputs read through their strides (sage_quantize_strided, sage_attn_fwd_strided):
the operands of a model's attention often come as [B, N, H, d] tensors or as
views into one packed QKV tensor.  Read where they lie, they must give the
workspace bytes and the output bits of the same values copied into
contiguous [B, H, N, d] first.
"""
import math
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_02_amd as s
    return s


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bnhd_view(t):
    """The same values as a [B, H, N, d] view of a [B, N, H, d] tensor."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _quantized(sage, q, k, v, granularity, pv):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    ws = sage.workspace_for(q, k)
    z = sage.sage_workspace_carve(ws, ws.numel(), B, Hq, Hkv, N, d, granularity=granularity, pv=pv)
    sage.sage_quantize(q, k, v, z)
    return sage.read_quantized(z, ws, B, Hq, Hkv, N, d)


@pytest.mark.parametrize("N,d,causal,granularity,pv", [
    (700, 64, False, "block", "e4m3"), (700, 128, True, "block", "e4m3"), (129, 64, True, "thread", "f16"),
    (1, 128, False, "token", "e4m3"), (513, 128, False, "thread", "e4m3"), (300, 64, True, "token", "f16")])
def test_bnhd_views_give_the_contiguous_result(sage, N, d, causal, granularity, pv):
    B, Hq, Hkv = 2, 8, 2
    _say(f"case BNHD views: shape={(B, Hq, Hkv, N, d)} causal={causal} granularity={granularity} pv={pv}")
    q, k, v = (t.cuda() for t in workloads.random_inputs(B, Hq, Hkv, N, d, "f16" if d == 64 else "bf16",
                                                         seed=N + d, scale=1.5))
    qv, kv, vv = _bnhd_view(q), _bnhd_view(k), _bnhd_view(v)
    # (with N = 1 torch counts the view as contiguous, and so does the binding)
    assert N == 1 or (not qv.is_contiguous() and qv.stride() == (N * Hq * d, d, Hq * d, 1))
    a = _quantized(sage, q, k, v, granularity, pv)
    b = _quantized(sage, qv, kv, vv, granularity, pv)
    for name in a:
        assert torch.equal(a[name], b[name]), name
    sm = 1 / math.sqrt(d)
    ref = sage.attn(q, k, v, causal, sm, granularity=granularity, pv=pv)
    out = sage.attn(qv, kv, vv, causal, sm, granularity=granularity, pv=pv)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_packed_qkv_views(sage, d, causal):
    """Q, K, V as slices of one [B, N, 3, H, d] tensor (MHA), and a GQA layout
    where K is [B, N, Hkv, d] and V stays contiguous."""
    B, H, N = 2, 4, 333
    _say(f"case packed QKV: B={B} H={H} N={N} d={d} causal={causal}")
    g = torch.Generator().manual_seed(d)
    dt = torch.float16 if d == 64 else torch.bfloat16
    qkv = (torch.randn(B, N, 3, H, d, generator=g) * 1.5).to(dt).cuda()
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    assert q.stride() == (N * 3 * H * d, d, 3 * H * d, 1)
    sm = 1 / math.sqrt(d)
    ref = sage.attn(q.contiguous(), k.contiguous(), v.contiguous(), causal, sm)
    out = sage.attn(q, k, v, causal, sm)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # GQA: 8 q heads over 2 kv heads, K read as [B, N, Hkv, d], Q and V contiguous
    q2, k2, v2 = (t.cuda() for t in workloads.random_inputs(B, 8, 2, N, d, "f16" if d == 64 else "bf16",
                                                            seed=5 + d, scale=1.5))
    ref2 = sage.attn(q2, k2, v2, causal, sm, granularity="thread")
    out2 = sage.attn(q2, _bnhd_view(k2), v2, causal, sm, granularity="thread")
    torch.cuda.synchronize()
    assert torch.equal(out2, ref2)


def test_workload_shape_through_views(sage):
    """The LLM-prefill workload's recipe at N = 1024 with [B, N, H, d] inputs,
    through sage_attn_fwd_ex on a side stream as a model would call it."""
    w = workloads.WORKLOADS[2].resized(N=1024)
    _say(f"case workload-2 recipe N=1024 as BNHD views, shape={(w.B, w.Hq, w.Hkv, w.N, w.d)}")
    q, k, v = (t.cuda() for t in workloads.generate(w, seed=77))
    qv, kv, vv = _bnhd_view(q), _bnhd_view(k), _bnhd_view(v)
    opts = sage.options("block", "e4m3", 8)
    ws = sage.workspace_for(q, k)
    ref = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    sage.sage_attn_fwd_ex(q, k, v, ref, w.causal, w.sm_scale, opts, ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ws2 = sage.workspace_for(q, k)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        sage.sage_attn_fwd_ex(qv, kv, vv, out, w.causal, w.sm_scale, opts, ws2)
    side.synchronize()
    assert torch.equal(out, ref)


def test_kv_cache_from_views(sage):
    """A KV cache built from [B, Nk, Hkv, d] views holds the bytes of one built
    from contiguous copies, and short queries against both agree bit for bit."""
    B, Hq, Hkv, Nk, Nq, d = 2, 8, 2, 3000, 3, 128
    _say(f"case KV cache from views: B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} Nq={Nq} d={d}")
    q, k, v = (t.cuda() for t in workloads.random_inputs(B, Hq, Hkv, Nk, d, "bf16", seed=91, scale=1.5))
    q = q[:, :, -Nq:].contiguous()
    a = sage.KVCache(k, v)
    b = sage.KVCache(_bnhd_view(k), _bnhd_view(v))
    torch.cuda.synchronize()
    Np = -(-Nk // sage.SAGE_NPAD) * sage.SAGE_NPAD

    def region(c, name, nbytes):  # one carved array of the cache, as bytes
        off = getattr(c.z, name) - c.buf.data_ptr()
        return c.buf[off:off + nbytes]
    for name, nbytes in (("k_i8", B * Hkv * Np * d), ("k_scale", B * Hkv * (Np // 64) * 4),
                         ("k_mean", B * Hkv * d * 4), ("v", B * Hkv * Np * d), ("v_scale", B * Hkv * d * 4)):
        assert torch.equal(region(a, name, nbytes), region(b, name, nbytes)), name
    sm = 1 / math.sqrt(d)
    oa = a.attend(q, causal=True, sm_scale=sm)
    ob = b.attend(q, causal=True, sm_scale=sm)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
