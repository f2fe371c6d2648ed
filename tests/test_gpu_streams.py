"""Stream semantics and determinism of the boundary: every call runs on the stream it is given
(torch's current stream by default), in that stream's order, and can be
captured into a graph.

- A side stream gives the bytes the default stream gives.
- Two problems launched back to back on two streams, each with its own
  workspace, give the bytes each gives alone.
- The whole path (prep + attention) and the no-allocation decode, captured
  into a graph, give on every replay the bytes of an eager call on the inputs
  the replay reads; between replays the program does eager work of its own
  and synchronizes, and the static inputs are rewritten in place.
- Repeated calls on the same inputs give the same bytes.
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


def _problem(index, N, seed, **kw):
    w = workloads.WORKLOADS[index].resized(N=N, **kw)
    q, k, v = workloads.generate(w, seed=seed)
    return w, q.cuda(), k.cuda(), v.cuda()


def _attn(sage, w, q, k, v, ws, opts, stream=None):
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    sage.sage_attn_fwd_ex(q, k, v, out, w.causal, w.sm_scale, opts, ws, stream=stream)
    return out


@pytest.mark.parametrize("index", [3, 4])
def test_side_stream_gives_the_default_stream_bytes(sage, index):
    w, q, k, v = _problem(index, 700, 31 + index, B=1, Hq=4, Hkv=4 if index == 3 else 1)
    _say(f"case side stream workload-{index} recipe N=700")
    opts = sage.options("block", "e4m3", 8)
    ws = sage.workspace_for(q, k)
    ref = _attn(sage, w, q, k, v, ws, opts)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ws2 = sage.workspace_for(q, k)
        out = _attn(sage, w, q, k, v, ws2, opts)
    side.synchronize()
    assert torch.equal(out, ref)


def test_two_streams_back_to_back(sage):
    wa, qa, ka, va = _problem(3, 900, 41, B=1, Hq=4, Hkv=4)
    wb, qb, kb, vb = _problem(4, 1300, 42, B=1, Hq=8, Hkv=2)
    _say("case two streams: workload-3 recipe N=900 and workload-4 recipe N=1300")
    oa_opts = sage.options("block", "e4m3", 8)
    ob_opts = sage.options("token", "f16", 8)
    wsa, wsb = sage.workspace_for(qa, ka), sage.workspace_for(qb, kb)
    ref_a = _attn(sage, wa, qa, ka, va, wsa, oa_opts)
    ref_b = _attn(sage, wb, qb, kb, vb, wsb, ob_opts)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        wsa2 = sage.workspace_for(qa, ka)
        out_a = torch.full(qa.shape, float("nan"), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s2):
        wsb2 = sage.workspace_for(qb, kb)
        out_b = torch.full(qb.shape, float("nan"), dtype=torch.float32, device="cuda")
    for _ in range(3):
        sage.sage_attn_fwd_ex(qa, ka, va, out_a, wa.causal, wa.sm_scale, oa_opts, wsa2, stream=s1)
        sage.sage_attn_fwd_ex(qb, kb, vb, out_b, wb.causal, wb.sm_scale, ob_opts, wsb2, stream=s2)
    s1.synchronize()
    s2.synchronize()
    assert torch.equal(out_a, ref_a)
    assert torch.equal(out_b, ref_b)


def test_graph_replays_of_the_whole_path(sage):
    w, q, k, v = _problem(4, 1000, 51, B=1, Hq=8, Hkv=2)
    _say("case graph of sage_attn_fwd_ex: workload-4 recipe N=1000, causal, GQA")
    opts = sage.options("block", "e4m3", 8)
    sq, sk, sv = q.clone(), k.clone(), v.clone()  # the graph's static inputs
    ws = sage.workspace_for(sq, sk)
    out = torch.full(sq.shape, float("nan"), dtype=torch.float32, device="cuda")
    # eager first: the library settles its launch facts outside the capture
    sage.sage_attn_fwd_ex(sq, sk, sv, out, w.causal, w.sm_scale, opts, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sage.sage_attn_fwd_ex(sq, sk, sv, out, w.causal, w.sm_scale, opts, ws)
    torch.cuda.synchronize()
    eager_ws = sage.workspace_for(sq, sk)
    for rep in range(4):
        _, q2, k2, v2 = _problem(4, 1000, 60 + rep, B=1, Hq=8, Hkv=2)
        sq.copy_(q2)
        sk.copy_(k2)
        sv.copy_(v2)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = _attn(sage, w, q2, k2, v2, eager_ws, opts)  # eager work between replays
        torch.cuda.synchronize()
        _say(f"   replay {rep}")
        assert torch.equal(out, ref)


def test_graph_replays_of_the_no_allocation_decode(sage):
    w, q, k, v = _problem(4, 3000, 71, B=2, Hq=8, Hkv=2, Nq=3)
    _say("case graph of sage_attn_decode_noalloc: Nq=3 against 3000 cached keys, GQA")
    cache = sage.KVCache(k, v)
    sm = 1 / math.sqrt(w.d)
    sq = q.clone()
    out = torch.full(sq.shape, float("nan"), dtype=torch.float32, device="cuda")
    sage.sage_attn_decode_noalloc(sq, cache.z, out, w.Hkv, w.N, True, sm)  # eager first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sage.sage_attn_decode_noalloc(sq, cache.z, out, w.Hkv, w.N, True, sm)
    torch.cuda.synchronize()
    for rep in range(4):
        _, q2, _, _ = _problem(4, 3000, 80 + rep, B=2, Hq=8, Hkv=2, Nq=3)
        sq.copy_(q2)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = cache.attend(q2, causal=True, sm_scale=sm)  # eager work between replays
        torch.cuda.synchronize()
        _say(f"   replay {rep}")
        assert torch.equal(out, ref)


@pytest.mark.parametrize("index,granularity,pv", [(3, "block", "e4m3"), (4, "block", "e4m3"),
                                                  (5, "thread", "f16"), (4, "token", "e4m3")])
def test_repeated_calls_give_identical_bytes(sage, index, granularity, pv):
    """Five calls on the same inputs return the same bytes: with double-buffered
    LDS tiles, cross-work-group statistics and split tail tiles, a race would
    show up as run-to-run differences."""
    # 48 heads of 17 tiles at d = 64: more tiles than the chip holds at once,
    # so the leftover round is split along the keys
    H = 48 if index == 3 else 4
    w, q, k, v = _problem(index, 2100, 91 + index, B=1, Hq=H, Hkv=H if index != 4 else 1)
    _say(f"case determinism workload-{index} recipe N=2100 Hq={H} {granularity} {pv}")
    opts = sage.options(granularity, pv, 8)
    ws = sage.workspace_for(q, k)
    first = _attn(sage, w, q, k, v, ws, opts)
    for _ in range(4):
        again = _attn(sage, w, q, k, v, ws, opts)
        torch.cuda.synchronize()
        assert torch.equal(again, first)


def test_repeated_decode_gives_identical_bytes(sage):
    w, q, k, v = _problem(4, 20000, 99, B=2, Hq=8, Hkv=2, Nq=2)
    _say("case determinism decode: Nq=2 against 20000 cached keys")
    cache = sage.KVCache(k, v)
    sm = 1 / math.sqrt(w.d)
    first = cache.attend(q, causal=True, sm_scale=sm)
    for _ in range(4):
        again = cache.attend(q, causal=True, sm_scale=sm)
        torch.cuda.synchronize()
        assert torch.equal(again, first)
