"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Prep outputs (codes, scales, K mean) must be bit-exact.  The attention output
must lie within the oracle's interval (the set of outputs reachable by the P
codes that sit within 2^-20 of an E4M3 or binary16 rounding midpoint, where
the hardware exp2 may round either way) up to max-abs 2e-3 and rel-L1 1e-3.
Both P.V formats (E4M3 and binary16), both quantization granularities and
both Q, K code widths (INT8 and the INT4 values of the 4-bit variant) are
covered.
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


def run_gpu(sage, q, k, v, causal, sm_scale, granularity="block", pv="e4m3", qk_bits=8):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    ws = sage.workspace_for(qd, kd)
    z = sage.sage_workspace_carve(ws, ws.numel(), B, Hq, Hkv, N, d, granularity=granularity, pv=pv,
                                  qk_bits=qk_bits)
    sage.sage_quantize(qd, kd, vd, z)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    sage.sage_attn_fwd_quantized(z, out, B, Hq, Hkv, N, d, causal, sm_scale)
    torch.cuda.synchronize()
    quant = sage.read_quantized(z, ws, B, Hq, Hkv, N, d)
    return out, quant


def check_prep(orc, quant, oz):
    np.testing.assert_array_equal(quant["q_i8"].numpy(), oz["q_i8"])
    np.testing.assert_array_equal(quant["k_i8"].numpy(), oz["k_i8"])
    np.testing.assert_array_equal(quant["k_mean"].numpy(), oz["k_mean"])
    if oz["pv"] == "f16":
        # V's binary16 rounding, bit for bit, and no V scale
        np.testing.assert_array_equal(quant["v_f16"].numpy().view(np.uint16), oz["v_f16"])
        assert (quant["v_scale"].numpy() == 1.0).all()
    else:
        np.testing.assert_array_equal(quant["v_fp8"].numpy(), oz["v_fp8"])
        np.testing.assert_array_equal(quant["v_scale"].numpy(), oz["v_scale"])
    nqb, nkb = oz["q_scale"].shape[-1], oz["k_scale"].shape[-1]
    np.testing.assert_array_equal(quant["q_scale"].numpy()[..., :nqb], oz["q_scale"])
    np.testing.assert_array_equal(quant["k_scale"].numpy()[..., :nkb], oz["k_scale"])
    assert not quant["q_pad"].any() and not quant["k_pad"].any() and not quant["v_pad"].any()
    # the binary16 V operand denotes exactly the values of the codes
    vals = orc.f16_decode(oz["v_f16"]) if oz["pv"] == "f16" else orc.e4m3_decode(oz["v_fp8"])
    np.testing.assert_array_equal(quant["v_half"].to(torch.float64).numpy(), vals)


def check_attn(orc, out_rows, oz, causal, sm_scale, rows):
    nom, lo, hi, flagged = orc.attn_q(oz, causal, sm_scale, rows=rows)
    g = out_rows.astype(np.float64)
    assert np.isfinite(g).all()
    dist = orc.interval_distance(g, lo, hi)
    max_abs = float(dist.max())
    rel = float(dist.sum() / np.abs(nom).sum())
    nominal = float(np.abs(g - nom).max())
    _say(f"   parity: max|dist|={max_abs:.3e} relL1={rel:.3e} nominal max={nominal:.3e} "
         f"flagged={int(flagged.sum())}")
    assert max_abs <= MAX_ABS and rel <= REL_L1
    return nom


def _rows_of(out, rows, d):
    return out.reshape(-1, d).cpu().numpy()[rows]


def quantize_as(orc, q, k, v, granularity, pv="e4m3", qk_bits=8):
    bq, bk = {"block": (128, 64), "thread": (1, 32), "token": (1, 1)}[granularity]
    return orc.quantize(q, k, v, bq=bq, bk=bk, pv=pv, qk_bits=qk_bits)


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
@pytest.mark.parametrize("granularity", ["block", "thread", "token"])
@pytest.mark.parametrize("recipe", [1, 2, 3, 4, 5])
def test_parity_reduced_workloads(sage, orc, recipe, granularity, pv):
    """Each workload's recipe at a size the oracle covers in full: several
    128-row tiles and a ragged tail (N = 700)."""
    w0 = workloads.WORKLOADS[recipe]
    w = w0.resized(B=2, Hq=2 * (w0.Hq // w0.Hkv), Hkv=2, N=700)
    _say(f"case recipe={recipe} shape={(w.B, w.Hq, w.Hkv, w.N, w.d)} causal={w.causal} "
         f"granularity={granularity} pv={pv}")
    q, k, v = workloads.generate(w, seed=1000 + recipe)
    out, quant = run_gpu(sage, q, k, v, w.causal, w.sm_scale, granularity, pv)
    oz = quantize_as(orc, q, k, v, granularity, pv)
    check_prep(orc, quant, oz)
    rows = np.arange(w.B * w.Hq * w.N)
    check_attn(orc, out.reshape(-1, w.d).cpu().numpy(), oz, w.causal, w.sm_scale, rows)


@pytest.mark.parametrize("granularity", ["block", "thread"])
@pytest.mark.parametrize("recipe", [1, 2, 3, 4, 5])
def test_parity_int4_qk(sage, orc, recipe, granularity):
    """The 4-bit (INT4) Q, K variant on every recipe at N = 700: codes in
    [-7, 7] bit-exact, scores taken exactly as for INT8."""
    w0 = workloads.WORKLOADS[recipe]
    w = w0.resized(B=2, Hq=2 * (w0.Hq // w0.Hkv), Hkv=2, N=700)
    pv = "f16" if recipe == 2 else "e4m3"
    _say(f"case int4 recipe={recipe} shape={(w.B, w.Hq, w.Hkv, w.N, w.d)} causal={w.causal} "
         f"granularity={granularity} pv={pv}")
    q, k, v = workloads.generate(w, seed=2000 + recipe)
    out, quant = run_gpu(sage, q, k, v, w.causal, w.sm_scale, granularity, pv, 4)
    oz = quantize_as(orc, q, k, v, granularity, pv, 4)
    assert np.abs(oz["q_i8"]).max() == 7
    check_prep(orc, quant, oz)
    rows = np.arange(w.B * w.Hq * w.N)
    check_attn(orc, out.reshape(-1, w.d).cpu().numpy(), oz, w.causal, w.sm_scale, rows)


@pytest.mark.parametrize("N", [1, 2, 17, 64, 127, 128, 129, 255, 256, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_parity_edge_lengths(sage, orc, N, d, causal):
    granularity = "thread" if N in (17, 129, 300) else ("token" if N in (2, 127, 255) else "block")
    pv = "f16" if N in (2, 64, 129, 256) else "e4m3"
    qk_bits = 4 if N in (1, 127, 129) else 8
    _say(f"case N={N} d={d} causal={causal} granularity={granularity} pv={pv} qk_bits={qk_bits}")
    q, k, v = workloads.random_inputs(1, 4, 2, N, d, "f16" if d == 64 else "bf16",
                                      seed=N * 7 + d + causal, scale=1.5)
    out, quant = run_gpu(sage, q, k, v, causal, 1 / math.sqrt(d), granularity, pv, qk_bits)
    oz = quantize_as(orc, q, k, v, granularity, pv, qk_bits)
    check_prep(orc, quant, oz)
    check_attn(orc, out.reshape(-1, d).cpu().numpy(), oz, causal, 1 / math.sqrt(d), None)


def _sweep_cases():
    rng = np.random.default_rng(20261204)
    cases = []
    for i in range(24):
        G = int(rng.choice([1, 2, 3, 8, 16]))
        Hkv = int(rng.integers(1, 3)) if G < 8 else 1
        cases.append((i, int(rng.integers(1, 4)), G * Hkv, Hkv, int(rng.integers(1, 640)),
                      int(rng.choice([64, 128])), bool(rng.integers(0, 2)),
                      str(rng.choice(["block", "thread", "token"])), str(rng.choice(["e4m3", "f16"]))))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"s{c[0]}")
def test_parity_shape_sweep(sage, orc, case):
    """Seeded random shapes: 1, 2, 3, 8 or 16 q heads per kv head, one to three
    batches, any N below 640, both head sizes and masks, every granularity and
    P.V format.  Their small tile counts are rarely multiples of the eight
    XCDs, so the work-group numbering's uneven ranges are exercised."""
    i, B, Hq, Hkv, N, d, causal, granularity, pv = case
    dtype = "f16" if i % 2 else "bf16"
    _say(f"case sweep {i}: shape={(B, Hq, Hkv, N, d)} causal={causal} granularity={granularity} "
         f"pv={pv} dtype={dtype}")
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, dtype, seed=3000 + i, scale=1.5)
    sm = 1 / math.sqrt(d)
    out, quant = run_gpu(sage, q, k, v, causal, sm, granularity, pv)
    oz = quantize_as(orc, q, k, v, granularity, pv)
    check_prep(orc, quant, oz)
    check_attn(orc, out.reshape(-1, d).cpu().numpy(), oz, causal, sm, None)


@pytest.mark.parametrize("kind", ["scale100", "planted_outliers"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pv", ["e4m3", "f16"])
def test_parity_large_score_factors(sage, orc, kind, d, causal, pv):
    """Scores whose float32 evaluation is delicate: |Q|, |K| around 100
    (every row dominated by a few keys, scores in the thousands), and
    heavy-tail inputs with a +-50 element planted in every Q and K scale
    block (score factor c of every block about 0.02-0.03 against small
    typical codes).  Checked against the plain FP32 exponent of the oracle."""
    N = 700
    if kind == "scale100":
        q, k, v = workloads.random_inputs(1, 4, 2, N, d, "bf16", seed=900 + d + causal, scale=100.0)
    else:
        w = workloads.WORKLOADS[5].resized(B=1, Hq=4, Hkv=2, N=N, d=d)
        q, k, v = workloads.generate(w, seed=910 + d + causal)
        rng = np.random.Generator(np.random.PCG64(920 + d))
        for t, r0 in ((q, 128), (k, 64)):
            for h in range(t.shape[1]):
                for r in range(0, N, r0):
                    t[0, h, r, int(rng.integers(d))] = float(rng.choice([-50.0, 50.0]))
    _say(f"case large scores kind={kind} d={d} causal={causal} pv={pv}")
    out, quant = run_gpu(sage, q, k, v, causal, 1 / math.sqrt(d), "block", pv)
    oz = quantize_as(orc, q, k, v, "block", pv)
    check_prep(orc, quant, oz)
    check_attn(orc, out.reshape(-1, d).cpu().numpy(), oz, causal, 1 / math.sqrt(d), None)


def test_degenerate_inputs(sage, orc):
    """Zero Q (uniform weights), identical K rows (zero smoothed K), a zero V
    channel and a dominant key."""
    N, d = 333, 64
    q, k, v = workloads.random_inputs(1, 2, 2, N, d, "f16", seed=5)
    q[0, 0] = 0.0
    k[0, 1] = k[0, 1, :1].clone()  # identical rows
    v[0, 0, :, 3] = 0.0
    k[0, 0, 100] = 12.0
    q[0, 1, :, :] = q[0, 1, :, :].abs()
    for causal, granularity, pv in ((False, "block", "e4m3"), (True, "block", "e4m3"),
                                    (True, "thread", "e4m3"), (False, "block", "f16"),
                                    (True, "thread", "f16")):
        _say(f"case degenerate causal={causal} granularity={granularity} pv={pv}")
        out, quant = run_gpu(sage, q, k, v, causal, 0.125, granularity, pv)
        oz = quantize_as(orc, q, k, v, granularity, pv)
        check_prep(orc, quant, oz)
        check_attn(orc, out.reshape(-1, d).cpu().numpy(), oz, causal, 0.125, None)


@pytest.mark.parametrize("d", [64, 128])
def test_prep_on_a_used_workspace(sage, orc, d):
    """The prep step clears its own arrival counters: a workspace filled with
    0xFF bytes, and one already used by a call on other inputs, give the same
    bytes as a fresh one."""
    N = 1100
    B, Hq, Hkv = 2, 4, 2
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, "bf16" if d == 64 else "f16",
                                      seed=77 + d, scale=2.0)
    q2, k2, v2 = workloads.random_inputs(B, Hq, Hkv, N, d, "bf16" if d == 64 else "f16",
                                         seed=78 + d, scale=3.0)
    _say(f"case prep on a used workspace d={d} N={N}")
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    ws = sage.workspace_for(qd, kd)
    z = sage.sage_workspace_carve(ws, ws.numel(), B, Hq, Hkv, N, d)
    results = []
    for fill in ("ones", "used"):
        if fill == "ones":
            ws.fill_(0xFF)
        else:
            sage.sage_quantize(q2.cuda(), k2.cuda(), v2.cuda(), z)
        sage.sage_quantize(qd, kd, vd, z)
        torch.cuda.synchronize()
        results.append(sage.read_quantized(z, ws, B, Hq, Hkv, N, d))
    for key in ("q_i8", "k_i8", "v_half", "k_mean", "v_scale", "q_scale", "k_scale"):
        assert torch.equal(results[0][key], results[1][key]), key
    check_prep(orc, results[1], orc.quantize(q, k, v))


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
def test_sage_attn_fwd_matches_two_step_path(sage, pv):
    w = workloads.WORKLOADS[2].resized(B=1, Hq=4, Hkv=4, N=515)
    q, k, v = (t.cuda() for t in workloads.generate(w, seed=3))
    one = sage.attn(q, k, v, causal=True, pv=pv)
    two, _ = run_gpu(sage, q.cpu(), k.cpu(), v.cpu(), True, w.sm_scale, pv=pv)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    if pv == "e4m3":
        ws = sage.workspace_for(q, k)
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        sage.sage_attn_fwd(q, k, v, out, True, w.sm_scale, ws)
        torch.cuda.synchronize()
        assert torch.equal(one, out)


@pytest.mark.parametrize("pv", ["e4m3", "f16"])
def test_parity_split_tail(sage, orc, pv):
    """780 tiles of 128 rows: on a GPU that runs 768 work-groups of this
    kernel at once (256 CUs, three each) the 12 left over after the first
    round are split along the keys into 8 shares each, then merged.  Every
    row of the last head's last 12 tiles is compared with the oracle, with a
    sample of the others."""
    w = workloads.WORKLOADS[3].resized(B=1, Hq=6, Hkv=6, N=16500)
    _say(f"case split tail shape={(w.B, w.Hq, w.Hkv, w.N, w.d)} pv={pv}")
    q, k, v = workloads.generate(w, seed=77)
    out, quant = run_gpu(sage, q, k, v, False, w.sm_scale, "block", pv)
    oz = quantize_as(orc, q, k, v, "block", pv)
    check_prep(orc, quant, oz)
    last = (w.Hq - 1) * w.N
    tail = np.arange(last + (130 - 12) * 128, last + w.N, dtype=np.int64)
    rows = np.unique(np.concatenate([workloads.sample_rows(w, 128, seed=3), tail]))
    check_attn(orc, _rows_of(out, rows, w.d), oz, False, w.sm_scale, rows)


# The method's accuracy against float64 attention on the original inputs, on
# the rows each full-size case checks.  The pages print no accuracy figure
# (their tables did not survive extraction): these floors are the CPU oracle's
# own cos / rel-L1 on exactly these inputs and rows, less a small margin, so a
# kernel or prep change that loses accuracy fails here.  Where the oracle
# meets the lines cos >= 0.999 or rel-L1 <= 0.03, the line itself is the bar.
# (cos at least, rel-L1 at most)
ACCURACY = {
    (1, "block", "e4m3", 8): (0.999, 0.040),     # oracle 0.999256, 0.03845
    (2, "block", "e4m3", 8): (0.999, 0.0425),    # 0.999213, 0.04081
    (3, "block", "e4m3", 8): (0.999, 0.0385),    # 0.999332, 0.03682
    (4, "block", "e4m3", 8): (0.9975, 0.086),    # 0.997717, 0.08292
    (5, "block", "e4m3", 8): (0.9945, 0.073),    # 0.994697, 0.07026
    (3, "thread", "e4m3", 8): (0.999, 0.0375),   # 0.999366, 0.03599
    (4, "thread", "e4m3", 8): (0.9980, 0.0425),  # 0.998173, 0.04102
    (5, "thread", "e4m3", 8): (0.999, 0.038),    # 0.999057, 0.03665
    (2, "block", "f16", 8): (0.999, 0.03),       # 0.999645, 0.02618
    (3, "block", "f16", 8): (0.999, 0.03),       # 0.999920, 0.01263
    (4, "block", "f16", 8): (0.9978, 0.074),     # 0.998049, 0.07137
    (5, "block", "f16", 8): (0.9948, 0.060),     # 0.995004, 0.05737
    (5, "thread", "f16", 8): (0.999, 0.03),      # 0.999373, 0.02152
    (3, "thread", "e4m3", 4): (0.980, 0.20),     # 0.981769, 0.19191
    (4, "thread", "f16", 4): (0.79, 0.32),       # 0.794744, 0.30783
    (4, "token", "e4m3", 8): (0.9983, 0.0405),   # 0.998536, 0.03887
    (4, "token", "f16", 8): (0.9987, 0.03),      # 0.998888, 0.01790
    (5, "token", "f16", 8): (0.999, 0.03),       # 0.999470, 0.01911
    (2, "token", "e4m3", 8): (0.999, 0.0355),    # 0.999422, 0.03391
}


def tile_rows(w, seed=13):
    """One row of every tile of query rows the attention kernel gives a
    work-group (128 rows at d = 64, 256 at d = 128), at a seeded position
    inside the tile (rows past N excluded), as flattened row indices."""
    rows_per_tile = 128 if w.d == 64 else 256
    nt = -(-w.N // rows_per_tile)
    rng = np.random.Generator(np.random.PCG64(seed))
    heads = np.arange(w.B * w.Hq)[:, None]
    start = np.arange(nt)[None, :] * rows_per_tile
    span = np.minimum(rows_per_tile, w.N - start)
    off = (rng.random((w.B * w.Hq, nt)) * span).astype(np.int64)
    return (heads * w.N + start + off).ravel().astype(np.int64)


@pytest.mark.parametrize("index,granularity,pv,qk_bits", list(ACCURACY))
def test_parity_full_size_workloads(sage, orc, index, granularity, pv, qk_bits):
    """Each workload at its full size, through sage_attn_fwd as the benchmark
    times it.  The output is filled with NaN first and must come back finite
    everywhere (every tile and every key share of a split tile wrote its
    rows).  The prep outputs are compared in full (bit-exact), the attention
    output on rows the oracle computes one by one: one row of every
    work-group tile, the first and last row of the first and last head, 256
    seeded rows, rows of the last head's last tiles (where the tail split
    happens), and for the peaked-row recipe some of the x20 rows.  The
    accuracy against float64 attention must stay at the level ACCURACY
    records."""
    w = workloads.WORKLOADS[index]
    _say(f"case full-size workload {index} {w.name} granularity={granularity} pv={pv} qk_bits={qk_bits}")
    q, k, v = workloads.generate(w)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = sage.workspace_for(qd, kd)
    sage.sage_attn_fwd_ex(qd, kd, vd, out, w.causal, w.sm_scale, sage.options(granularity, pv, qk_bits),
                          ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "some output rows were not written"
    z = sage.sage_workspace_carve(ws, ws.numel(), w.B, w.Hq, w.Hkv, w.N, w.d, granularity=granularity,
                                  pv=pv, qk_bits=qk_bits)
    quant = sage.read_quantized(z, ws, w.B, w.Hq, w.Hkv, w.N, w.d)
    del qd, kd, vd
    oz = quantize_as(orc, q, k, v, granularity, pv, qk_bits)
    check_prep(orc, quant, oz)
    rows = np.concatenate([workloads.sample_rows(w, 256, seed=11), tile_rows(w)])
    if not w.causal:
        # rows of the last head's last 100 tiles: where the tiles left over
        # after the last whole round of work-groups are split along the keys
        last = (w.B * w.Hq - 1) * w.N
        lo = max(0, w.N - 100 * 128)
        pick = np.random.Generator(np.random.PCG64(12)).choice(w.N - lo, size=min(32, w.N - lo), replace=False)
        rows = np.concatenate([rows, last + lo + pick, [last + w.N - 1]])
    if w.recipe == 4:
        # rows scaled x20 in the first head: the largest |Q| rows
        qn = q[0, 0].float().abs().amax(dim=-1)
        hot = torch.nonzero(qn > 4 * qn.median()).flatten()[:32].numpy().astype(np.int64)
        rows = np.concatenate([rows, hot])
    rows = np.unique(rows).astype(np.int64)
    got = out.reshape(-1, w.d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    _say(f"   {len(rows)} rows checked")
    nom = check_attn(orc, got, oz, w.causal, w.sm_scale, rows)
    # the method's accuracy against full precision
    ref = orc.attn_f64(q, k, v, w.causal, w.sm_scale, rows=rows)
    a_gpu, a_orc = orc.accuracy(got, ref), orc.accuracy(nom, ref)
    _say(f"   vs float64: gpu cos={a_gpu['cos']:.6f} relL1={a_gpu['rel_l1']:.4f}; "
         f"oracle cos={a_orc['cos']:.6f} relL1={a_orc['rel_l1']:.4f}")
    cos_min, rel_max = ACCURACY[(index, granularity, pv, qk_bits)]
    assert a_gpu["cos"] >= cos_min and a_gpu["rel_l1"] <= rel_max
