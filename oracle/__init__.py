"""CPU oracle for 8-bit quantized attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its
binding) never does.  The arithmetic lives in ``oracle.c`` (plain loops, float64
except where a quantisation decision is defined on float32), built here with
gcc and loaded with ctypes.  Nothing in this package is shared with the HIP
path.

Every function follows the method as the SageAttention pages describe it
(K smoothing, per-block INT8 Q/K, FP8 E4M3 P and V with two-level
accumulation); the readings taken where the pages are silent are listed in the
header of ``oracle.c``.  All functions here are pinned by ``tests/test_oracle_*``
against facts fixed by the mathematics or by independent libraries.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# Block parameters of the spec (one INT8 scale per BQ query rows and per BK
# keys; one P scale per row per BN keys).
BQ, BK, BN = 128, 64, 128
# Relative distance to an E4M3 rounding midpoint within which both codes of P
# count as correct: the HIP path evaluates 2^x with a hardware exp2 whose error
# is about one float32 ulp (2^-23); 2^-20 leaves a factor 8 of margin.
TAU = 2.0 ** -20

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


# A sanitizer build of oracle.c (tests/test_host_sanitizers.py) is loaded in
# place of liboracle.so when this variable names its file.
SANITIZED_LIB_ENV = "SAGE_ORACLE_SANITIZED_LIB"


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get(SANITIZED_LIB_ENV)
        if not path:
            path = build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i, f, dd, l = ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_long
        lib.oracle_e4m3_decode.restype = dd
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [dd]
        lib.oracle_e4m3_encode_array.argtypes = [P, l, P]
        lib.oracle_e4m3_decode_array.argtypes = [P, l, P]
        lib.oracle_f16_decode.restype = dd
        lib.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_encode.restype = ctypes.c_uint16
        lib.oracle_f16_encode.argtypes = [dd]
        lib.oracle_f16_encode_array.argtypes = [P, l, P]
        lib.oracle_f16_decode_array.argtypes = [P, l, P]
        lib.oracle_quantize.argtypes = [P, P, P, i, i, i, i, i, i, i, i, i, P, P, P, P, P, P, P]
        lib.oracle_quantize_q.argtypes = [P, i, i, i, i, i, i, P, P]
        lib.oracle_quantize_kv.argtypes = [P, P, i, i, i, i, i, i, i, P, P, P, P, P]
        lib.oracle_attn_q.argtypes = [P, P, P, P, P, P, i, i, i, i, i, i, i, i, i, i, i, f,
                                      dd, P, l, P, P, P, P]
        lib.oracle_attn_f64.argtypes = [P, P, P, i, i, i, i, i, i, i, dd, P, l, P]
        lib.oracle_num_threads.restype = i
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def num_threads() -> int:
    return _load().oracle_num_threads()


def to_f32(t) -> np.ndarray:
    """Exact up-conversion of an fp16/bf16 tensor to a float32 numpy array."""
    if isinstance(t, torch.Tensor):
        return np.ascontiguousarray(t.detach().cpu().to(torch.float32).numpy())
    return np.ascontiguousarray(np.asarray(t, dtype=np.float32))


def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(c, dtype=np.uint8))
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def f16_encode(x) -> np.ndarray:
    """binary16 codes (uint16), round to nearest even, saturating at +-65504."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f16_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(c, dtype=np.uint16))
    out = np.empty(c.shape, np.float64)
    _load().oracle_f16_decode_array(_ptr(c), c.size, _ptr(out))
    return out


# P.V formats: P and V as E4M3 (per-block P scale, per-channel V scale), or as
# binary16 (SageAttention's own P.V, accumulated in FP32 here)
PV_FORMATS = ("e4m3", "f16")


# largest integer code of the Q, K formats: INT8, and the INT4 of the 4-bit variant
QK_MAX = {8: 127, 4: 7}


def quantize_q(q, bq: int = BQ, qk_bits: int = 8) -> dict:
    """The Q half of the prep step on [B,Hq,Nq,d]: integer codes (INT8, or
    INT4 values with qk_bits=4) and one scale per bq rows (see
    oracle_quantize_q in oracle.c)."""
    q = to_f32(q)
    B, Hq, Nq, d = q.shape
    r = dict(q_i8=np.empty((B, Hq, Nq, d), np.int8),
             q_scale=np.empty((B, Hq, -(-Nq // bq)), np.float32))
    _load().oracle_quantize_q(_ptr(q), B, Hq, Nq, d, bq, QK_MAX[qk_bits], _ptr(r["q_i8"]),
                              _ptr(r["q_scale"]))
    r.update(B=B, Hq=Hq, Nq=Nq, d=d, bq=bq, qk_bits=qk_bits)
    return r


def quantize_kv(k, v, bk: int = BK, smooth: bool = True, pv: str = "e4m3", qk_bits: int = 8) -> dict:
    """The K/V half of the prep step on [B,Hkv,Nk,d] (a quantized KV cache):
    K mean, smoothed INT8 K with one scale per bk keys, and V as E4M3 codes
    with per-channel scales, or with pv="f16" also v_f16, the binary16 codes
    of V, which attn_q then uses (no V scale)."""
    if pv not in PV_FORMATS:
        raise ValueError(f"pv must be one of {PV_FORMATS}")
    k, v = to_f32(k), to_f32(v)
    B, Hkv, Nk, d = k.shape
    r = dict(k_i8=np.empty((B, Hkv, Nk, d), np.int8),
             k_scale=np.empty((B, Hkv, -(-Nk // bk)), np.float32),
             k_mean=np.empty((B, Hkv, d), np.float32), v_fp8=np.empty((B, Hkv, Nk, d), np.uint8),
             v_scale=np.empty((B, Hkv, d), np.float32))
    _load().oracle_quantize_kv(_ptr(k), _ptr(v), B, Hkv, Nk, d, bk, QK_MAX[qk_bits], int(smooth),
                               _ptr(r["k_i8"]),
                               _ptr(r["k_scale"]), _ptr(r["k_mean"]), _ptr(r["v_fp8"]),
                               _ptr(r["v_scale"]))
    if pv == "f16":
        r["v_f16"] = f16_encode(v)
    r.update(B=B, Hkv=Hkv, Nk=Nk, d=d, bk=bk, pv=pv, qk_bits=qk_bits)
    return r


def quantize(q, k, v, bq: int = BQ, bk: int = BK, smooth: bool = True, pv: str = "e4m3",
             qk_bits: int = 8) -> dict:
    """The prep step on [B,H,N,d] inputs (both halves, same N).  Returns codes
    in the plain logical layout [B,H,N,d] and the scales (see oracle_quantize
    in oracle.c)."""
    r = quantize_q(q, bq, qk_bits)
    r.update(quantize_kv(k, v, bk, smooth, pv, qk_bits))
    r["N"] = r["Nk"]
    return r


def attn_q(qz: dict, causal: bool, sm_scale: float, rows=None, bn: int = BN,
           tau: float = TAU, interval: bool = True):
    """Quantized attention from the prep outputs `qz` (quantize, or the merged
    dicts of quantize_q and quantize_kv: Nq query rows at the last Nq of Nk
    positions) for the given flattened rows (None = all), in the P.V format
    qz["pv"] was made for.  Returns (out, lo, hi, flagged), float64 [nrows, d]."""
    f16 = qz.get("pv", "e4m3") == "f16"
    v_codes = qz["v_f16"] if f16 else qz["v_fp8"]
    v_scale = None if f16 else qz["v_scale"]
    B, Hq, Hkv, Nq, Nk, d = qz["B"], qz["Hq"], qz["Hkv"], qz["Nq"], qz["Nk"], qz["d"]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows.size
    else:
        nrows = B * Hq * Nq
    out = np.empty((nrows, d), np.float64)
    lo = np.empty((nrows, d), np.float64) if interval else None
    hi = np.empty((nrows, d), np.float64) if interval else None
    flagged = np.empty(nrows, np.int64) if interval else None
    _load().oracle_attn_q(_ptr(qz["q_i8"]), _ptr(qz["q_scale"]), _ptr(qz["k_i8"]),
                          _ptr(qz["k_scale"]), _ptr(v_codes), _ptr(v_scale), int(f16),
                          B, Hq, Hkv, Nq, Nk, d, qz["bq"], qz["bk"], bn, int(causal),
                          float(sm_scale), float(tau), _ptr(rows), nrows,
                          _ptr(out), _ptr(lo), _ptr(hi), _ptr(flagged))
    return out, lo, hi, flagged


def attn_f64(q, k, v, causal: bool, sm_scale: float, rows=None) -> np.ndarray:
    """Full-precision softmax(QK^T*sm_scale)V in float64 for the given rows;
    q [B,Hq,Nq,d] sits at the last Nq of the Nk positions of k, v."""
    q = np.ascontiguousarray(np.asarray(to_f32(q) if isinstance(q, torch.Tensor) else q,
                                        dtype=np.float64))
    k = np.ascontiguousarray(np.asarray(to_f32(k) if isinstance(k, torch.Tensor) else k,
                                        dtype=np.float64))
    v = np.ascontiguousarray(np.asarray(to_f32(v) if isinstance(v, torch.Tensor) else v,
                                        dtype=np.float64))
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk")
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows.size
    else:
        nrows = B * Hq * Nq
    out = np.empty((nrows, d), np.float64)
    _load().oracle_attn_f64(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Nq, Nk, d, int(causal),
                            float(sm_scale), _ptr(rows), nrows, _ptr(out))
    return out


def accuracy(out, ref) -> dict:
    """Cosine similarity and relative L1 of `out` against `ref`."""
    a = np.asarray(out, np.float64).ravel()
    b = np.asarray(ref, np.float64).ravel()
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    rel_l1 = float(np.abs(a - b).sum() / np.abs(b).sum())
    return {"cos": cos, "rel_l1": rel_l1}


def interval_distance(gpu, lo, hi) -> np.ndarray:
    """Distance of each GPU value from the oracle interval [lo, hi]."""
    g = np.asarray(gpu, np.float64)
    return np.maximum(0.0, np.maximum(lo - g, g - hi))
