#!/usr/bin/env python3
"""Throughput of the 8-bit quantized attention forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the prep kernels (K mean, smoothing, INT8 Q/K, FP8 V)
followed by the fused attention kernel, i.e. one sage_attn_fwd call.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-cpu]
                    [--granularity block|thread|token] [--pv e4m3|f16]

Prints one JSON line.  `value` is TOPS = 4*B*Hq*N^2*d / t (halved for causal)
for the whole step; `roofline` prices the attention kernel alone (its average
duration measured with HIP events on the stream it runs on) against the dense
INT8/FP8 matrix-core peak; `cpu_baseline` times the CPU oracle on a bounded
sample of query rows of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized attention fwd TOPS (4·B·H·N²·d/t) and % of INT8/FP8 MFMA peak, 1 GPU"
PEAK_TOPS = 5000.0        # MI355X dense INT8 = dense FP8 matrix-core peak (ops/s / 1e12)
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default 50; 2000 with --decode, whose 20-30 us steps need that many "
                        "for the timed window to outlast the clock's ramp)")
    p.add_argument("--warmup", type=int, default=None, help="untimed steps first (default 5; 200 with --decode)")
    p.add_argument("--workload", type=int, default=3,
                   help="1..5; 3 is the non-causal N=17550 video-diffusion shape")
    p.add_argument("--granularity", choices=("block", "thread", "token"), default="block",
                   help="Q/K scale granularity: block (128 rows / 64 keys), thread (per row / 32 keys) or "
                        "token (per row / per key; not for the decode cache)")
    p.add_argument("--pv", choices=("e4m3", "f16"), default="e4m3",
                   help="P.V format: e4m3 (FP8 P and V, the default) or f16 (binary16 P and V)")
    p.add_argument("--qk-bits", type=int, choices=(8, 4), default=8,
                   help="Q, K codes: INT8 (the default) or INT4-valued codes on the INT8 matrix core "
                        "(the 4-bit numerics as an accuracy option, at INT8 speed)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-rows", type=int, default=0, help="rows in the CPU sample (0 = auto)")
    p.add_argument("--no-contrast", action="store_true",
                   help="skip the 16-bit contrast: torch's scaled_dot_product_attention (flash backend "
                        "only) in the input dtype on the same inputs, the native attention this path "
                        "replaces, and a naive unfused 16-bit attention of our own (hipBLASLt products)")
    p.add_argument("--prep-flush", action="store_true",
                   help="also time the prep step alone with a 512 MB write between launches, so the "
                        "last-level cache holds none of its inputs")
    p.add_argument("--decode", type=int, default=0, metavar="WORKLOAD",
                   help="instead of the default line, time the short-query path over a quantized KV "
                        "cache on decode workload 6 or 7 (one JSON line of its own, HBM-bound)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="instead of the benchmark, run a plain device-to-device copy of BYTES "
                        "bytes 7 times (2 untimed, 5 timed with HIP events): a known-size reference for "
                        "hardware byte counters and the achievable copy bandwidth")
    return p.parse_args()


KERNEL_SOURCES = [os.path.join(ROOT, "bit_quantized_attention_02_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "attn_block.h", "sage_internal.h")]
DECODE_SOURCES = [os.path.join(ROOT, "bit_quantized_attention_02_amd", "csrc", f)
                  for f in ("attn_decode.hip", "attn_block.h", "sage_internal.h")]


def kernel_digest(paths=KERNEL_SOURCES):
    """SHA-256 over the attention kernel's sources, in order."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(granularity, pv, qk_bits, prefix="attn_fwd", sources=KERNEL_SOURCES,
                     workload=None):
    """(workload, HBM bytes per launch) from a committed byte-counter summary
    (profiles/<prefix>_*_counters.json) taken with this granularity, P.V
    format and Q/K width (and on `workload`, when given), or (None, None)
    when the kernel sources changed since the counters were taken."""
    import glob
    digest = kernel_digest(sources)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"{prefix}_*_counters.json"))):
        with open(path) as f:
            d = json.load(f)
        if (d.get("kernel_source_sha256") == digest and d.get("granularity", "block") == granularity
                and d.get("pv_format", "e4m3") == pv and d.get("qk_bits", 8) == qk_bits
                and (workload is None or d.get("workload") == workload)):
            return d.get("workload"), d.get("traffic_bytes_per_launch")
    return None, None


def timed(fn, iters, torch):
    """Average milliseconds per call of fn() measured with HIP events on the
    current stream (the stream every library call is launched on)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def contrast_sdpa(w, qd, kd, vd, steps, torch):
    """Native attention on the same inputs: torch SDPA restricted to its flash
    backend (it raises rather than falling back to the unfused math path)."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    kw = {"enable_gqa": True} if w.Hq != w.Hkv else {}

    def run():
        return torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=w.causal,
                                                                scale=w.sm_scale, **kw)
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            run()
            torch.cuda.synchronize()
            ms = timed(run, steps, torch)
    except RuntimeError as e:
        return {"kind": "torch sdpa flash", "error": str(e).splitlines()[0][:200]}
    return {"kind": f"torch {torch.__version__} scaled_dot_product_attention, flash backend, "
                    f"{w.dtype} in and out", "ms_per_call": round(ms, 4),
            "TOPS": round(w.ops / (ms * 1e-3) / 1e12, 2)}


def contrast_naive(w, qd, kd, vd, steps, torch):
    """Unfused 16-bit attention of our own, head by head: S = Q K^T on the
    matrix core through torch.matmul (hipBLASLt; K transposed into a
    contiguous operand first), the mask and softmax in FP32, P rounded to the
    input dtype, O = P V through torch.matmul."""
    G = w.Hq // w.Hkv
    kt = kd.transpose(-1, -2).contiguous()  # [B, Hkv, d, N]
    out = torch.empty(qd.shape, dtype=qd.dtype, device=qd.device)
    mask = None
    if w.causal:
        mask = torch.ones(w.N, w.N, dtype=torch.bool, device=qd.device).triu(1)

    def run():
        for b in range(w.B):
            for h in range(w.Hq):
                s = torch.matmul(qd[b, h], kt[b, h // G]).float() * w.sm_scale
                if mask is not None:
                    s.masked_fill_(mask, float("-inf"))
                p = torch.softmax(s, dim=-1).to(qd.dtype)
                out[b, h] = torch.matmul(p, vd[b, h // G])

    try:
        run()
        torch.cuda.synchronize()
        ms = timed(run, max(1, min(steps, 3)), torch)
    except RuntimeError as e:
        return {"kind": "naive 16-bit attention", "error": str(e).splitlines()[0][:200]}
    return {"kind": f"naive attention of our own: torch.matmul (hipBLASLt) for both products, "
                    f"FP32 softmax, {w.dtype} in and out, one head at a time",
            "ms_per_call": round(ms, 4), "TOPS": round(w.ops / (ms * 1e-3) / 1e12, 2)}


def prep_flushed(sage, qd, kd, vd, z, steps, torch):
    """sage_quantize alone, each launch timed on its own after a 512 MB write."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=qd.device)
    times = []
    for i in range(steps):
        flush.fill_(i & 0xFF)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        sage.sage_quantize(qd, kd, vd, z)
        s1.record()
        torch.cuda.synchronize()
        times.append(s0.elapsed_time(s1))
    times.sort()
    return times[len(times) // 2]


def cpu_baseline(w, q, k, v, rows_wanted, bq, bk, pv, qk_bits):
    """The oracle as it stands: its prep over the whole input, pro-rated to the
    sampled rows, plus its attention over the sampled rows."""
    import numpy as np

    import oracle
    import workloads

    oracle.build()
    t0 = time.perf_counter()
    oz = oracle.quantize(q, k, v, bq=bq, bk=bk, pv=pv, qk_bits=qk_bits)
    t_prep = time.perf_counter() - t0
    total_rows = w.B * w.Hq * w.N
    if rows_wanted <= 0:
        # ~15 s of attention work at the box's thread count, measured first on 64 rows
        probe = workloads.sample_rows(w, 64, seed=1)
        t0 = time.perf_counter()
        oracle.attn_q(oz, w.causal, w.sm_scale, rows=probe, interval=False)
        per_row = (time.perf_counter() - t0) / len(probe)
        rows_wanted = int(max(64, min(total_rows, 15.0 / max(per_row, 1e-9))))
    rows = workloads.sample_rows(w, rows_wanted, seed=2)
    t0 = time.perf_counter()
    oracle.attn_q(oz, w.causal, w.sm_scale, rows=rows, interval=False)
    t_attn = time.perf_counter() - t0
    frac = len(rows) / total_rows
    t = t_attn + t_prep * frac
    ops = w.ops * frac  # causal rows are sampled uniformly, so the average row cost matches
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{len(rows)} of {total_rows} query rows (uniform, seeded) of the same workload; "
                      f"oracle prep over the full input pro-rated by that fraction "
                      f"(prep {t_prep:.2f} s, attention {t_attn:.2f} s)"}


def accuracy_vs_f64(w, q, k, v, out, torch, count=256):
    """Cosine similarity and relative L1 of the GPU output against full-precision
    attention, softmax(Q K^T sm_scale) V in float64 on the CPU (plain torch, not
    the oracle), on a seeded sample of query rows (for the peaked-row recipe,
    plus some of its x20 rows)."""
    import numpy as np

    import workloads

    rows = workloads.sample_rows(w, count, seed=5)
    if w.recipe == 4:
        qn = q[0, 0].float().abs().amax(dim=-1)
        hot = torch.nonzero(qn > 4 * qn.median()).flatten()[:32].numpy().astype(np.int64)
        rows = np.unique(np.concatenate([rows, hot]))
    n, G = w.q_rows, w.Hq // w.Hkv
    got = out.reshape(-1, w.d)[torch.from_numpy(rows).to(out.device)].double().cpu()
    ref = torch.empty_like(got)
    bh, i = rows // n, rows % n
    for key in np.unique(bh // w.Hq * w.Hkv + (bh % w.Hq) // G):
        sel = np.nonzero(bh // w.Hq * w.Hkv + (bh % w.Hq) // G == key)[0]
        b, g = divmod(int(key), w.Hkv)
        qr = q.reshape(w.B * w.Hq, n, w.d)[torch.from_numpy(bh[sel]), torch.from_numpy(i[sel])].double()
        s = (qr @ k[b, g].double().T) * w.sm_scale
        if w.causal:
            pos = torch.from_numpy(i[sel] + (w.N - n))[:, None]
            s.masked_fill_(torch.arange(w.N)[None, :] > pos, float("-inf"))
        ref[torch.from_numpy(sel)] = torch.softmax(s, dim=-1) @ v[b, g].double()
    a, r = got.flatten(), ref.flatten()
    return {"cos": round(float(a @ r / (a.norm() * r.norm())), 6),
            "rel_l1": round(float((a - r).abs().sum() / r.abs().sum()), 5), "rows": int(len(rows)),
            "reference": "float64 softmax(QK^T sm_scale)V on the CPU (torch), same inputs",
            "lines": {"cos_min": 0.999, "rel_l1_max": 0.03}}


def decode_bytes(w, k_block, pv):
    """Bytes one short-query launch must move with this cache format: INT8 K
    (1 B), V as E4M3 codes (1 B) or binary16 (2 B), the K scales and V scales
    of the cache; the query in and the FP32 output."""
    kv = w.B * w.Hkv * w.N * w.d
    return ((2 if pv == "e4m3" else 3) * kv + w.B * w.Hkv * (-(-w.N // k_block)) * 4
            + w.B * w.Hkv * w.d * 4 + w.B * w.Hq * w.q_rows * w.d * (2 + 4))


def cpu_baseline_decode(w, q, k, v, bk, pv):
    """The oracle's short-query attention over every query row, its K/V
    quantization not counted (the cache is built once)."""
    import oracle

    oracle.build()
    z = oracle.quantize_q(q, bq=1)
    z.update(oracle.quantize_kv(k, v, bk=bk, pv=pv))
    oracle.attn_q(z, w.causal, w.sm_scale, interval=False)  # warm: threads, first touch
    t0 = time.perf_counter()
    oracle.attn_q(z, w.causal, w.sm_scale, interval=False)
    one = time.perf_counter() - t0
    # repeat the whole pass for about 10 s of CPU work
    reps = max(1, min(5000, int(10.0 / max(one, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.attn_q(z, w.causal, w.sm_scale, interval=False)
    t = (time.perf_counter() - t0) / reps
    return {"value": decode_bytes(w, bk, pv) / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"all {w.B * w.Hq * w.q_rows} query rows of the workload, "
                                        f"{reps} passes, {t * 1e3:.2f} ms each (the cache "
                                        f"quantization is not timed)"}


def bench_decode(args, sage, workloads, torch):
    w = workloads.DECODE_WORKLOADS[args.decode]
    q, k, v = workloads.generate(w)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    cache = sage.KVCache(kd, vd, granularity=args.granularity, pv=args.pv)
    nbytes = sage.sage_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.q_rows, w.N, w.d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(qd.shape, dtype=torch.float32, device="cuda")

    def step():
        sage.sage_attn_decode(qd, cache.z, out, w.Hkv, w.N, w.causal, w.sm_scale, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = timed(step, args.steps, torch)
    wall = time.perf_counter() - t0
    ms_cache = timed(lambda: sage.sage_kv_quantize(kd, vd, cache.z), max(3, args.steps // 10), torch)
    kb = cache.z.k_block
    nb = decode_bytes(w, kb, args.pv)
    gbs = nb / (ms * 1e-3) / 1e9
    fp16_kv = 2 * 2 * w.B * w.Hkv * w.N * w.d
    _, traffic = measured_traffic(args.granularity, args.pv, 8, "attn_decode", DECODE_SOURCES, w.name)
    line = {
        "metric": "short-query attention over a quantized KV cache, GB/s of cache read (1 GPU)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"i8 (QK^T, i32 acc) + {args.pv} values (P.V, f32 acc)", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.q_rows, "Nk": w.N,
                   "d": w.d, "causal": w.causal, "input_dtype": w.dtype, "k_block": kb,
                   "pv_format": args.pv, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "attn_decode (+ decode_merge)", "bytes_per_launch": nb},
        "cache": {"bytes": int(cache.buf.numel()), "fp16_kv_bytes": fp16_kv,
                  "ratio": round(cache.buf.numel() / fp16_kv, 4),
                  "quantize_ms": round(ms_cache, 4)},
        "tops": round(w.ops / (ms * 1e-3) / 1e12, 2),
        "timed_wall_s": round(wall, 3),
    }
    line["accuracy"] = accuracy_vs_f64(w, q, k, v, out, torch)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_decode(w, q, k, v, kb, args.pv)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.steps is None:
        args.steps = 2000 if args.decode else 50
    if args.warmup is None:
        args.warmup = 200 if args.decode else 5
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_quantized_attention_02_amd as sage
    import workloads

    if args.decode:
        bench_decode(args, sage, workloads, torch)
        return
    if args.copy_probe:
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        ms = timed(lambda: dst.copy_(src), 5, torch)
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "launches": 7, "ms_per_copy": round(ms, 4),
                          "copy_TBps": round(2 * args.copy_probe / (ms * 1e-3) / 1e12, 3)}), flush=True)
        return

    w = workloads.WORKLOADS[args.workload]
    q, k, v = workloads.generate(w)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    ws = sage.workspace_for(qd, kd)
    z = sage.sage_workspace_carve(ws, ws.numel(), w.B, w.Hq, w.Hkv, w.N, w.d,
                                  granularity=args.granularity, pv=args.pv, qk_bits=args.qk_bits)
    opts = sage.options(args.granularity, args.pv, args.qk_bits)
    qb, kb = opts.q_block, opts.k_block

    def step():
        sage.sage_attn_fwd_ex(qd, kd, vd, out, w.causal, w.sm_scale, opts, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = timed(step, args.steps, torch)
    wall = time.perf_counter() - t0

    # per-kernel averages on the same stream
    ms_prep = timed(lambda: sage.sage_quantize(qd, kd, vd, z), args.steps, torch)
    ms_attn = timed(lambda: sage.sage_attn_fwd_quantized(z, out, w.B, w.Hq, w.Hkv, w.N, w.d,
                                                         w.causal, w.sm_scale), args.steps, torch)
    _, traffic = measured_traffic(args.granularity, args.pv, args.qk_bits, workload=w.name)
    tops = w.ops / (ms_step * 1e-3) / 1e12
    attn_tops = w.ops / (ms_attn * 1e-3) / 1e12
    elems = (w.B * w.Hq + 2 * w.B * w.Hkv) * w.N * w.d
    prep_gbs = 3.0 * elems / (ms_prep * 1e-3) / 1e9

    line = {
        "metric": METRIC, "value": round(tops, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{'i8' if args.qk_bits == 8 else 'i4 values in i8'} (QK^T, i32 acc) + {args.pv} values "
                 f"(P.V, f32 acc)", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "input_dtype": w.dtype, "sm_scale": w.sm_scale,
                   "q_block": qb, "k_block": kb, "pv_format": args.pv, "qk_bits": args.qk_bits,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(attn_tops, 2), "peak": PEAK_TOPS,
                     "unit": "TOPS", "frac": round(attn_tops / PEAK_TOPS, 4), "traffic": traffic,
                     "kernel": "attn_fwd (+ attn_tail_merge)", "ms_per_launch": round(ms_attn, 4)},
        "prep": {"ms_per_launch": round(ms_prep, 4), "alg_GBps": round(prep_gbs, 1),
                 "frac_hbm": round(prep_gbs / HBM_PEAK_GBS, 4)},
        "timed_wall_s": round(wall, 3),
    }
    line["accuracy"] = accuracy_vs_f64(w, q, k, v, out, torch)
    if args.prep_flush:
        ms_pf = prep_flushed(sage, qd, kd, vd, z, max(args.steps, 20), torch)
        line["prep"]["flushed_median_ms"] = round(ms_pf, 4)
        line["prep"]["flushed_alg_GBps"] = round(3.0 * elems / (ms_pf * 1e-3) / 1e9, 1)
    if not args.no_contrast:
        line["contrast"] = contrast_sdpa(w, qd, kd, vd, args.steps, torch)
        line["contrast_naive"] = contrast_naive(w, qd, kd, vd, args.steps, torch)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_rows, qb, kb, args.pv, args.qk_bits)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
