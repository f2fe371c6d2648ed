"""How gfx950's FP8 matrix-core instructions sum their products, against the
binary16 instruction the P.V product runs on.

The per-block P.V of the quantized attention multiplies E4M3 P by E4M3 V and
adds the products in FP32 (the two-level accumulation of the SageAttention
pages: "两级累加" in the Berkeley brief's checklist, and SageAttention2's P, V
item on the "INT4量化" search page).  The library feeds the exact E4M3 values
to v_mfma_f32_32x32x16_f16 instead of the FP8 instructions; this test records
why.  A probe (tests/probes/fp8_mfma_probe.hip) runs one instruction on
operands whose every output element is one dot product sum_k a[k] b[k]; with
one large product and many small ones, the exact sum is a float32 integer, so
any deviation is the instruction's, not float32 rounding's.
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "probes", "libprobe.so")

pytestmark = pytest.mark.gpu

E4M3_448 = 0x7E   # 1.75 * 2^8
E4M3_ONE = 0x38   # 1.0
KDIM = {0: 16, 1: 64, 2: 16}


def _lib():
    if not os.path.exists(PROBE):
        sys.path.insert(0, os.path.join(ROOT, "tests", "probes"))
        import build as probe_build
        probe_build.build()
    lib = ctypes.CDLL(PROBE)
    lib.fp8_mfma_probe.restype = ctypes.c_int
    lib.fp8_mfma_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return lib


def _run(lib, kind, a, b):
    """a, b: K values as E4M3 code bytes (kinds 0, 1) or floats (kind 2)."""
    if kind == 2:
        ab = np.zeros(32, np.float16)
        bb = np.zeros(32, np.float16)
        ab[:16], bb[:16] = a, b
    else:
        ab = np.zeros(64, np.uint8)
        bb = np.zeros(64, np.uint8)
        ab[:KDIM[kind]], bb[:KDIM[kind]] = a, b
    out = np.zeros(1024, np.float32)
    rc = lib.fp8_mfma_probe(ab.ctypes.data, bb.ctypes.data, kind, out.ctypes.data)
    assert rc == 0, f"probe failed with HIP error {rc}"
    # every lane and accumulator holds the same dot product
    assert np.all(out == out[0]), "operands with equal rows and columns gave unequal outputs"
    return float(out[0])


def test_fp8_instructions_drop_small_products_next_to_a_large_one(orc):
    import torch
    assert torch.cuda.is_available()
    lib = _lib()
    print()
    worst = {}
    for kind, name in ((0, "v_mfma_f32_32x32x16_fp8_fp8"), (1, "v_mfma_scale_f32_32x32x64_f8f6f4")):
        K = KDIM[kind]
        # control: products of equal size are summed exactly
        assert _run(lib, kind, [E4M3_ONE] * K, [E4M3_ONE] * K) == K
        # one product 448^2 and K - 1 products of size x (x an E4M3 value)
        worst[name] = (0.0, 0.0)
        for code in (0x38, 0x40, 0x48, 0x50, 0x58):       # 1, 2, 4, 8, 16
            x = float(orc.e4m3_decode(np.array([code], np.uint8))[0])
            got = _run(lib, kind, [E4M3_448] + [code] * (K - 1), [E4M3_448] + [E4M3_ONE] * (K - 1))
            exact = 448.0 * 448.0 + (K - 1) * x
            err = abs(got - exact)
            # a float32 sum of K terms is off by at most K half-ulps of its size
            fp32_bound = K * float(np.spacing(np.float32(exact))) / 2
            worst[name] = max(worst[name], (err / fp32_bound, err / (448.0 * 448.0)))
            print(f"{name}: 448^2 + {K - 1} x {x:g}: got {got:.1f}, exact {exact:.1f}, error "
                  f"{err:g} = {err / fp32_bound:.1f} x the float32 bound = {err / 448.0 ** 2:.2e} of the "
                  f"largest product", flush=True)
    for name, (vs_fp32, vs_max) in worst.items():
        assert vs_fp32 > 10, name     # far beyond float32 accumulation
        assert vs_max < 1e-3, name    # a truncation of the low-order bits, not a wrong sum


def test_f16_instruction_sums_the_same_values_exactly():
    import torch
    assert torch.cuda.is_available()
    lib = _lib()
    for x in (1.0, 2.0, 4.0, 8.0, 16.0):
        got = _run(lib, 2, [448.0] + [x] * 15, [448.0] + [1.0] * 15)
        assert got == 448.0 * 448.0 + 15 * x
