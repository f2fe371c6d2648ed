"""Seeded synthetic attention inputs shaped like the workloads the SageAttention
pages evaluate on (LLM prefill, image generation, video diffusion).

This module only draws random numbers; it holds none of the quantized-attention
arithmetic, so both the CPU oracle and the HIP path can take their inputs from
here without sharing any of the method's code.

Notation of the recipes: N(0, s) is a normal with variance s; LogNormal(0, sig)
is numpy's ``lognormal(0, sig)``; a per-channel offset is one draw per
(batch, kv head, channel) added to every token; channel subsets are drawn per
(batch, kv head) without replacement.  Everything is drawn in float32 from
``numpy.random.Generator(PCG64(seed))`` in the order Q, K, V and then rounded
once to the input dtype (fp16 or bf16).

The K channel outliers imitate what the SageAttention page reports for video
and image models (strong channel-wise outliers in K); the Q row scaling and
heavy tails stress the per-block scales.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

SEED_BASE = 20261203


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int          # 1-based workload number
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    recipe: int         # which distribution recipe (1..5)
    Nq: int = 0         # query rows per head against N keys (0: N, self-attention)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def q_rows(self) -> int:
        """Query rows per head (N for self-attention)."""
        return self.Nq if self.Nq else self.N

    @property
    def ops(self) -> float:
        """Algorithmic operation count of the two contractions: 4*d per allowed
        (query, key) pair, i.e. 4*B*Hq*N^2*d halved for causal self-attention.
        Query row i of a short query sits at position N - Nq + i."""
        if not self.Nq:
            o = 4.0 * self.B * self.Hq * self.N * self.N * self.d
            return o / 2 if self.causal else o
        nq, nk = self.Nq, self.N
        pairs = nq * nk - nq * (nq - 1) / 2 if self.causal else nq * nk
        return 4.0 * self.B * self.Hq * pairs * self.d

    def resized(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "selfattn_b1_h2_n256_d64_f16", 1, 2, 2, 256, 64, "f16", False, 1),
    2: Workload(2, "llm_prefill_causal_b4_h32_n4096_d128_bf16", 4, 32, 32, 4096, 128, "bf16", True, 2),
    3: Workload(3, "video_diffusion_b2_h30_n17550_d64_f16", 2, 30, 30, 17550, 64, "f16", False, 3),
    4: Workload(4, "long_context_gqa_causal_b1_hq32_hkv8_n32768_d128_bf16", 1, 32, 8, 32768, 128, "bf16", True, 4),
    5: Workload(5, "image_gen_heavy_tail_b8_h24_n4096_d64_f16", 8, 24, 24, 4096, 64, "f16", False, 5),
}


# Short queries against a long KV cache (decode): N is the number of cached
# keys, Nq the query rows per head (at the last Nq positions).
DECODE_WORKLOADS = {
    6: Workload(6, "long_context_gqa_decode_b1_hq32_hkv8_nq1_nk32768_d128_bf16", 1, 32, 8, 32768, 128,
                "bf16", True, 4, Nq=1),
    7: Workload(7, "llm_decode_gqa_b8_hq32_hkv8_nq1_nk8192_d128_bf16", 8, 32, 8, 8192, 128, "bf16",
                True, 2, Nq=1),
}


def _torch_dtype(name: str) -> torch.dtype:
    return {"f16": torch.float16, "bf16": torch.bfloat16}[name]


def _channel_offsets(rng, B, H, d, count, var):
    """One offset per (b, h, channel) on `count` channels chosen per (b, h)."""
    off = np.zeros((B, H, 1, d), np.float32)
    for b in range(B):
        for h in range(H):
            ch = rng.choice(d, size=count, replace=False)
            off[b, h, 0, ch] = rng.normal(0.0, math.sqrt(var), size=count).astype(np.float32)
    return off


def _bias_all_plus_outliers(rng, B, H, d):
    """Bias ~N(0,2) on every channel, and 3 channels per (b, h) that take a
    bias ~N(0,10) instead."""
    off = rng.normal(0.0, math.sqrt(2.0), size=(B, H, 1, d)).astype(np.float32)
    for b in range(B):
        for h in range(H):
            ch = rng.choice(d, size=3, replace=False)
            off[b, h, 0, ch] = rng.normal(0.0, math.sqrt(10.0), size=3).astype(np.float32)
    return off


def _t3(rng, shape):
    x = rng.standard_t(3.0, size=shape).astype(np.float32)
    return np.clip(x, -60.0, 60.0)


def generate(w: Workload, seed: int | None = None):
    """Return (q, k, v) as contiguous CPU torch tensors of the workload dtype,
    laid out [B, H, rows, d]: q has w.q_rows rows per head, k and v w.N."""
    if seed is None:
        seed = SEED_BASE + w.index
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hq, Hkv, N, d = w.B, w.Hq, w.Hkv, w.N, w.d
    Nq = w.q_rows
    qs, ks = (B, Hq, Nq, d), (B, Hkv, N, d)
    r = w.recipe
    if r == 1:
        q = rng.standard_normal(qs, dtype=np.float32)
        k = rng.standard_normal(ks, dtype=np.float32)
        k += _channel_offsets(rng, B, Hkv, d, 4, 4.0)
        v = rng.standard_normal(ks, dtype=np.float32)
    elif r == 2:
        q = rng.standard_normal(qs, dtype=np.float32)
        q *= rng.lognormal(0.0, 0.5, size=(B, Hq, Nq, 1)).astype(np.float32)
        k = rng.standard_normal(ks, dtype=np.float32)
        k += _bias_all_plus_outliers(rng, B, Hkv, d)
        v = rng.standard_normal(ks, dtype=np.float32)
    elif r == 3:
        q = rng.standard_normal(qs, dtype=np.float32)
        k = rng.standard_normal(ks, dtype=np.float32)
        k += _channel_offsets(rng, B, Hkv, d, min(8, d), 8.0)
        v = rng.standard_normal(ks, dtype=np.float32)
        v *= rng.lognormal(0.0, 1.0, size=(B, Hkv, 1, d)).astype(np.float32)
    elif r == 4:
        q = rng.standard_normal(qs, dtype=np.float32)
        n_hot = int(round(0.01 * Nq))
        for b in range(B):
            for h in range(Hq):
                rows = rng.choice(Nq, size=n_hot, replace=False)
                q[b, h, rows, :] *= 20.0
        k = rng.standard_normal(ks, dtype=np.float32)
        k += _bias_all_plus_outliers(rng, B, Hkv, d)
        v = rng.standard_normal(ks, dtype=np.float32)
    elif r == 5:
        q = _t3(rng, qs)
        k = _t3(rng, ks)
        k += rng.normal(0.0, math.sqrt(6.0), size=(B, Hkv, 1, d)).astype(np.float32)
        v = _t3(rng, ks)
    else:
        raise ValueError(f"unknown recipe {r}")
    dt = _torch_dtype(w.dtype)
    return (torch.from_numpy(q).to(dt).contiguous(),
            torch.from_numpy(k).to(dt).contiguous(),
            torch.from_numpy(v).to(dt).contiguous())


def random_inputs(B, Hq, Hkv, N, d, dtype="f16", seed=0, scale=1.0):
    """Plain N(0, scale^2) inputs of any shape, for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = _torch_dtype(dtype)
    q = (rng.standard_normal((B, Hq, N, d), dtype=np.float32) * scale)
    k = (rng.standard_normal((B, Hkv, N, d), dtype=np.float32) * scale)
    v = (rng.standard_normal((B, Hkv, N, d), dtype=np.float32) * scale)
    return (torch.from_numpy(q).to(dt).contiguous(),
            torch.from_numpy(k).to(dt).contiguous(),
            torch.from_numpy(v).to(dt).contiguous())


def sample_rows(w: Workload, count: int, seed: int = 7):
    """A deterministic sample of flattened query-row indices (b*Hq + h)*rows + i
    (rows = w.q_rows),
    always including the first and last row of every head touched and, for
    recipe 4, some of the x20 rows (found by the caller from the data)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = w.q_rows
    total = w.B * w.Hq * n
    rows = set(int(x) for x in rng.choice(total, size=min(count, total), replace=False))
    for bh in (0, w.B * w.Hq - 1):
        rows.add(bh * n)
        rows.add(bh * n + n - 1)
    return np.array(sorted(rows), dtype=np.int64)
