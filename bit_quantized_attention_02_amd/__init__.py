"""Python binding of libsage, the MI355X (gfx950) 8-bit quantized attention
library declared in include/sage.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current
stream.  The functions keep the C names; tensors replace raw pointers.  If the
library is not built, importing this package raises (there is no fallback).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsage.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python bit_quantized_attention_02_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

SAGE_OK, SAGE_ERR_INVALID_ARG, SAGE_ERR_UNSUPPORTED, SAGE_ERR_WORKSPACE, SAGE_ERR_HIP = 0, -1, -2, -3, -4
SAGE_F16, SAGE_BF16 = 0, 1
SAGE_BQ, SAGE_BK, SAGE_BN, SAGE_NPAD = 128, 64, 128, 256
SAGE_MAX_N = 1 << 20  # longest sequence (N, Nk, Nq) the library accepts
SAGE_DECODE_SCRATCH_BYTES = 17039360  # the library's own decode scratch, per GPU
SAGE_BQ_THREAD, SAGE_BK_THREAD, SAGE_BK_TOKEN = 1, 32, 1
SAGE_PV_E4M3, SAGE_PV_F16 = 0, 1
SAGE_QK_INT8, SAGE_QK_INT4 = 8, 4
# (q_block, k_block) of the quantization granularities
GRANULARITY = {"block": (SAGE_BQ, SAGE_BK), "thread": (SAGE_BQ_THREAD, SAGE_BK_THREAD),
               "token": (SAGE_BQ_THREAD, SAGE_BK_TOKEN)}
# P.V formats: FP8 E4M3 P and V, or binary16 P and V (both accumulated in FP32)
PV_FORMAT = {"e4m3": SAGE_PV_E4M3, "f16": SAGE_PV_F16}


class sage_config(ctypes.Structure):
    _fields_ = [("bq", ctypes.c_int), ("bk", ctypes.c_int), ("bn", ctypes.c_int),
                ("fp8_max", ctypes.c_int), ("version", ctypes.c_int)]


class sage_qkv_quant(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v16", "v_scale", "v_inv",
                 "k_part", "v_part", "sync")] + [("q_block", ctypes.c_int32), ("k_block", ctypes.c_int32),
                                                 ("pv_format", ctypes.c_int32), ("qk_bits", ctypes.c_int32),
                                                 ("tail_part", ctypes.c_void_p), ("tail_rows", ctypes.c_int64)] + \
               [(n, ctypes.c_int32) for n in ("B", "Hq", "Hkv", "N", "d")]


class sage_kv_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("k_i8", "k_scale", "k_mean", "v", "v_scale", "v_inv", "k_part", "v_part", "sync")] + \
               [(n, ctypes.c_int32) for n in ("k_block", "pv_format", "B", "Hkv", "Nk", "d")]


class sage_options(ctypes.Structure):
    _fields_ = [("q_block", ctypes.c_int32), ("k_block", ctypes.c_int32), ("pv_format", ctypes.c_int32),
                ("qk_bits", ctypes.c_int32)]


class sage_strides(ctypes.Structure):
    """Element strides (batch, head, token) of a [B, H, N, d] input whose d
    elements are contiguous."""
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_lib.sage_workspace_bytes.restype = _S
_lib.sage_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.sage_workspace_carve.argtypes = [_P, _S, _I, _I, _I, _I, _I, ctypes.POINTER(sage_qkv_quant)]
_lib.sage_quantize.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.POINTER(sage_qkv_quant), _P]
_lib.sage_attn_fwd_quantized.argtypes = [ctypes.POINTER(sage_qkv_quant), _P, _I, _I, _I, _I, _I, _I,
                                         _F, _P]
_lib.sage_attn_fwd.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _S, _P]
_lib.sage_attn_fwd_granular.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P,
                                        _S, _P]
_lib.sage_attn_fwd_ex.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                                  ctypes.POINTER(sage_options), _P, _S, _P]
_SP = ctypes.POINTER(sage_strides)
_lib.sage_quantize_strided.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _SP, _SP, _SP,
                                       ctypes.POINTER(sage_qkv_quant), _P]
_lib.sage_attn_fwd_strided.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                                       ctypes.POINTER(sage_options), _SP, _SP, _SP, _P, _S, _P]
_lib.sage_kv_cache_bytes.restype = _S
_lib.sage_kv_cache_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.sage_kv_cache_carve.argtypes = [_P, _S, _I, _I, _I, _I, _I, _I, ctypes.POINTER(sage_kv_cache)]
_lib.sage_kv_quantize.argtypes = [_P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(sage_kv_cache), _P]
_lib.sage_kv_quantize_strided.argtypes = [_P, _P, _I, _I, _I, _I, _I, _SP, _SP, ctypes.POINTER(sage_kv_cache),
                                          _P]
_lib.sage_decode_workspace_bytes.restype = _S
_lib.sage_decode_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
_lib.sage_attn_decode.argtypes = [_P, _I, ctypes.POINTER(sage_kv_cache), _P, _I, _I, _I, _I, _I, _I,
                                  _I, _F, _P, _S, _P]
_lib.sage_attn_decode_noalloc.argtypes = [_P, _I, ctypes.POINTER(sage_kv_cache), _P, _I, _I, _I, _I, _I,
                                          _I, _I, _F, _P]
_lib.sage_get_config.argtypes = [ctypes.POINTER(sage_config)]
_lib.sage_v_key_position.argtypes = [_I]
_lib.sage_status_string.restype = ctypes.c_char_p
_lib.sage_status_string.argtypes = [_I]

EXPORTED = ["sage_workspace_bytes", "sage_workspace_carve", "sage_quantize",
            "sage_attn_fwd_quantized", "sage_attn_fwd", "sage_attn_fwd_granular", "sage_attn_fwd_ex",
            "sage_quantize_strided", "sage_attn_fwd_strided",
            "sage_kv_cache_bytes", "sage_kv_cache_carve", "sage_kv_quantize", "sage_kv_quantize_strided",
            "sage_decode_workspace_bytes", "sage_attn_decode", "sage_attn_decode_noalloc", "sage_get_config",
            "sage_v_key_position", "sage_status_string"]


class SageError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"sage status {status}: {sage_status_string(status)}")
        self.status = status


def _check(rc: int) -> None:
    if rc != SAGE_OK:
        raise SageError(rc)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return SAGE_F16
    if t.dtype == torch.bfloat16:
        return SAGE_BF16
    raise TypeError(f"Q, K, V must be float16 or bfloat16, got {t.dtype}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _shape(q: torch.Tensor, k: torch.Tensor):
    B, Hq, N, d = q.shape
    return B, Hq, k.shape[1], N, d


# The C calls take every size from the integers they are passed and read or
# write each buffer by those sizes; the checks below keep a tensor of another
# shape, element type or device from being read or written out of bounds.

def _check_device(ref: torch.Tensor, *ts) -> None:
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or t.device != ref.device or not t.is_contiguous():
            raise ValueError(f"tensors must be contiguous and on {ref.device}")


def _strides(t: torch.Tensor):
    """None for a contiguous [B, H, N, d] tensor; else its element strides as
    sage_strides, when its d elements are contiguous and every row starts
    16 bytes apart in multiples (strides of 8 elements), as the library
    requires of inputs read through strides."""
    if t.is_contiguous():
        return None
    st = t.stride()
    if st[3] != 1 and t.shape[3] > 1:
        raise ValueError(f"the last dimension (d) must be contiguous; strides {st}")
    if any(x < 0 or x % 8 for x in st[:3]) or t.data_ptr() % 16:
        raise ValueError(f"strides {st[:3]} must be non-negative multiples of 8 elements, "
                         "from a 16-byte aligned start")
    return sage_strides(st[0], st[1], st[2])


def _check_inputs(ref: torch.Tensor, *ts) -> None:
    """Q, K, V: on ref's GPU, contiguous or readable through their strides."""
    for t in ts:
        if not t.is_cuda or t.device != ref.device:
            raise ValueError(f"tensors must be on {ref.device}")
        _strides(t)


def _check_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out=None, strided: bool = False) -> None:
    """Q [B, Hq, N, d], K and V [B, Hkv, N, d] of one dtype, out FP32 of Q's
    shape, all contiguous on one GPU; with `strided`, Q, K and V may instead
    have their d elements contiguous and row strides of 8 elements (the calls
    that read them through their strides)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("Q, K, V must be 4-D [B, H, N, d]")
    if k.shape != v.shape or (k.shape[0], k.shape[2], k.shape[3]) != (q.shape[0], q.shape[2], q.shape[3]):
        raise ValueError(f"K and V must be [B, Hkv, N, d] for Q of shape {tuple(q.shape)}; "
                         f"got {tuple(k.shape)} and {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"Q, K, V must share one dtype; got {q.dtype}, {k.dtype}, {v.dtype}")
    if out is not None and (out.shape != q.shape or out.dtype != torch.float32):
        raise ValueError(f"out must be float32 of shape {tuple(q.shape)}")
    if strided:
        _check_inputs(q, q, k, v)
        _check_device(q, out)
    else:
        _check_device(q, k, v, out)


def _check_out(ref: torch.Tensor, out: torch.Tensor, shape) -> None:
    if tuple(out.shape) != tuple(shape) or out.dtype != torch.float32:
        raise ValueError(f"out must be float32 of shape {tuple(shape)}")
    _check_device(ref, out)


# ------------------------------------------------------------------ C names

def sage_status_string(status: int) -> str:
    return _lib.sage_status_string(int(status)).decode()


def sage_get_config() -> dict:
    c = sage_config()
    _check(_lib.sage_get_config(ctypes.byref(c)))
    return {f: getattr(c, f) for f, _ in sage_config._fields_}


def sage_v_key_position(j: int) -> int:
    return _lib.sage_v_key_position(int(j))


def sage_workspace_bytes(B: int, Hq: int, Hkv: int, N: int, d: int) -> int:
    return int(_lib.sage_workspace_bytes(B, Hq, Hkv, N, d))


def sage_workspace_carve(workspace: torch.Tensor | int | None, ws_bytes: int, B: int, Hq: int,
                         Hkv: int, N: int, d: int, granularity: str = "block",
                         pv: str = "e4m3", qk_bits: int = 8) -> sage_qkv_quant:
    """The C call, then (q_block, k_block), pv_format and qk_bits set to the
    chosen granularity, P.V format and Q, K code width."""
    z = sage_qkv_quant()
    ptr = workspace.data_ptr() if isinstance(workspace, torch.Tensor) else workspace
    _check(_lib.sage_workspace_carve(ptr, ws_bytes, B, Hq, Hkv, N, d, ctypes.byref(z)))
    z.q_block, z.k_block = GRANULARITY[granularity]
    z.pv_format = PV_FORMAT[pv]
    z.qk_bits = qk_bits
    return z


def sage_quantize(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dst: sage_qkv_quant,
                  stream=None) -> None:
    _check_qkv(q, k, v, strided=True)
    B, Hq, Hkv, N, d = _shape(q, k)
    st = [_strides(t) for t in (q, k, v)]
    if all(x is None for x in st):
        _check(_lib.sage_quantize(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, N, d,
                                  ctypes.byref(dst), _stream(stream)))
    else:
        _check(_lib.sage_quantize_strided(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, N, d,
                                          *(None if x is None else ctypes.byref(x) for x in st),
                                          ctypes.byref(dst), _stream(stream)))


def sage_attn_fwd_quantized(src: sage_qkv_quant, out: torch.Tensor, B: int, Hq: int, Hkv: int,
                            N: int, d: int, causal: bool, sm_scale: float, stream=None) -> None:
    _check_out(out, out, (B, Hq, N, d))
    _check(_lib.sage_attn_fwd_quantized(ctypes.byref(src), _ptr(out), B, Hq, Hkv, N, d,
                                        int(causal), float(sm_scale), _stream(stream)))


def sage_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                  causal: bool, sm_scale: float, workspace: torch.Tensor, stream=None) -> None:
    _check_qkv(q, k, v, out)
    _check_device(q, workspace)
    B, Hq, Hkv, N, d = _shape(q, k)
    _check(_lib.sage_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, N, d, int(causal),
                              float(sm_scale), _dtype_code(q), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)))


def sage_attn_fwd_granular(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                           causal: bool, sm_scale: float, q_block: int, k_block: int,
                           workspace: torch.Tensor, stream=None) -> None:
    _check_qkv(q, k, v, out)
    _check_device(q, workspace)
    B, Hq, Hkv, N, d = _shape(q, k)
    _check(_lib.sage_attn_fwd_granular(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, N, d,
                                       int(causal), float(sm_scale), _dtype_code(q), int(q_block),
                                       int(k_block), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))


def sage_attn_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                     causal: bool, sm_scale: float, opts: sage_options, workspace: torch.Tensor,
                     stream=None) -> None:
    _check_qkv(q, k, v, out, strided=True)
    _check_device(q, workspace)
    B, Hq, Hkv, N, d = _shape(q, k)
    st = [_strides(t) for t in (q, k, v)]
    if all(x is None for x in st):
        _check(_lib.sage_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, N, d, int(causal),
                                     float(sm_scale), _dtype_code(q), ctypes.byref(opts), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    else:
        _check(_lib.sage_attn_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, N, d, int(causal),
                                          float(sm_scale), _dtype_code(q), ctypes.byref(opts),
                                          *(None if x is None else ctypes.byref(x) for x in st),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)))


def sage_kv_cache_bytes(B: int, Hkv: int, Nk: int, d: int, pv: str = "e4m3") -> int:
    return int(_lib.sage_kv_cache_bytes(B, Hkv, Nk, d, PV_FORMAT[pv]))


def sage_kv_cache_carve(buf: torch.Tensor | int | None, nbytes: int, B: int, Hkv: int, Nk: int,
                        d: int, granularity: str = "block", pv: str = "e4m3") -> sage_kv_cache:
    """The C call with the K granularity ("block": 64 keys per scale,
    "thread": 32) and the P.V format by name."""
    z = sage_kv_cache()
    ptr = buf.data_ptr() if isinstance(buf, torch.Tensor) else buf
    _check(_lib.sage_kv_cache_carve(ptr, nbytes, B, Hkv, Nk, d, GRANULARITY[granularity][1],
                                    PV_FORMAT[pv], ctypes.byref(z)))
    return z


def sage_kv_quantize(k: torch.Tensor, v: torch.Tensor, cache: sage_kv_cache, stream=None) -> None:
    """K and V contiguous, or views read through their strides (e.g. a
    [B, Nk, Hkv, d] cache seen as [B, Hkv, Nk, d])."""
    if k.dim() != 4 or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("K and V must be [B, Hkv, Nk, d] of one shape and dtype")
    _check_inputs(k, k, v)
    B, Hkv, Nk, d = k.shape
    st = [_strides(t) for t in (k, v)]
    if all(x is None for x in st):
        _check(_lib.sage_kv_quantize(_ptr(k), _ptr(v), _dtype_code(k), B, Hkv, Nk, d, ctypes.byref(cache),
                                     _stream(stream)))
    else:
        _check(_lib.sage_kv_quantize_strided(_ptr(k), _ptr(v), _dtype_code(k), B, Hkv, Nk, d,
                                             *(None if x is None else ctypes.byref(x) for x in st),
                                             ctypes.byref(cache), _stream(stream)))


def sage_decode_workspace_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(_lib.sage_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d))


def sage_attn_decode(q: torch.Tensor, cache: sage_kv_cache, out: torch.Tensor, Hkv: int, Nk: int,
                     causal: bool, sm_scale: float, workspace: torch.Tensor, stream=None) -> None:
    if q.dim() != 4:
        raise ValueError("Q must be 4-D [B, Hq, Nq, d]")
    _check_out(q, out, q.shape)
    _check_device(q, q, workspace)
    B, Hq, Nq, d = q.shape
    _check(_lib.sage_attn_decode(_ptr(q), _dtype_code(q), ctypes.byref(cache), _ptr(out), B, Hq, Hkv,
                                 Nq, Nk, d, int(causal), float(sm_scale), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def sage_attn_decode_noalloc(q: torch.Tensor, cache: sage_kv_cache, out: torch.Tensor, Hkv: int, Nk: int,
                             causal: bool, sm_scale: float, stream=None) -> None:
    """sage_attn_decode without a workspace: the library's own per-GPU
    scratch holds the key split's partials (no allocation; calls that overlap
    on one GPU race)."""
    if q.dim() != 4:
        raise ValueError("Q must be 4-D [B, Hq, Nq, d]")
    _check_out(q, out, q.shape)
    _check_device(q, q)
    B, Hq, Nq, d = q.shape
    _check(_lib.sage_attn_decode_noalloc(_ptr(q), _dtype_code(q), ctypes.byref(cache), _ptr(out), B, Hq,
                                         Hkv, Nq, Nk, d, int(causal), float(sm_scale), _stream(stream)))


# ------------------------------------------------------------------ helpers

def options(granularity: str = "block", pv: str = "e4m3", qk_bits: int = 8) -> sage_options:
    """sage_options from the names of a granularity and a P.V format, and the
    Q, K code width (8, or 4 for INT4-valued codes: an accuracy option at INT8 speed)."""
    qb, kb = GRANULARITY[granularity]
    return sage_options(qb, kb, PV_FORMAT[pv], qk_bits)


def workspace_for(q: torch.Tensor, k: torch.Tensor) -> torch.Tensor:
    """Allocate a workspace (torch-owned device bytes) for these shapes."""
    B, Hq, Hkv, N, d = _shape(q, k)
    nbytes = sage_workspace_bytes(B, Hq, Hkv, N, d)
    if nbytes == 0:
        raise SageError(SAGE_ERR_UNSUPPORTED)
    return torch.empty(nbytes, dtype=torch.uint8, device=q.device)


def attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
         sm_scale: float | None = None, workspace: torch.Tensor | None = None,
         granularity: str = "block", pv: str = "e4m3", qk_bits: int = 8) -> torch.Tensor:
    """Drop-in attention: [B,Hq,N,d] fp16/bf16 Q and [B,Hkv,N,d] K,V on the GPU
    -> FP32 [B,Hq,N,d], on the current stream.  Q, K and V may be views, e.g.
    the transpose(1, 2) of [B,N,H,d] tensors: they are read through their
    strides, not copied.  granularity: "block" (one Q
    scale per 128 rows, one K scale per 64 keys), "thread" (per row, per 32
    keys) or "token" (per row, per key); pv: "e4m3" (FP8 P and V) or "f16" (binary16 P and V); qk_bits: 8
    (INT8 Q, K) or 4 (INT4-valued codes on the INT8 matrix core, an accuracy option)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    _check_qkv(q, k, v, strided=True)
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, k)
    sage_attn_fwd_ex(q, k, v, out, causal, sm_scale, options(granularity, pv, qk_bits), workspace)
    return out


class KVCache:
    """A quantized KV cache in torch-owned device memory: the K/V half of the
    prep step over [B, Hkv, Nk, d] fp16/bf16 K and V, quantized once."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, granularity: str = "block",
                 pv: str = "e4m3", stream=None):
        if k.dim() != 4 or k.shape != v.shape or k.dtype != v.dtype:
            raise ValueError("K and V must be [B, Hkv, Nk, d] of one shape and dtype")
        _check_inputs(k, k, v)
        self.B, self.Hkv, self.Nk, self.d = k.shape
        nbytes = sage_kv_cache_bytes(self.B, self.Hkv, self.Nk, self.d, pv)
        if nbytes == 0:
            raise SageError(SAGE_ERR_UNSUPPORTED)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=k.device)
        self.z = sage_kv_cache_carve(self.buf, nbytes, self.B, self.Hkv, self.Nk, self.d,
                                     granularity, pv)
        sage_kv_quantize(k, v, self.z, stream)

    def attend(self, q: torch.Tensor, causal: bool = True, sm_scale: float | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """softmax(Q K^T sm_scale) V for q [B, Hq, Nq, d] at the last Nq of the
        Nk positions -> FP32 [B, Hq, Nq, d]."""
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(q.shape[-1])
        if q.dim() != 4 or q.shape[0] != self.B or q.shape[3] != self.d:
            raise ValueError(f"Q must be [{self.B}, Hq, Nq, {self.d}] for this cache")
        _check_device(self.buf, q)
        B, Hq, Nq, d = q.shape
        if workspace is None:
            nbytes = sage_decode_workspace_bytes(B, Hq, self.Hkv, Nq, self.Nk, d)
            if nbytes == 0:
                raise SageError(SAGE_ERR_UNSUPPORTED)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        sage_attn_decode(q, self.z, out, self.Hkv, self.Nk, causal, sm_scale, workspace, stream)
        return out


def _host_view(buf: torch.Tensor, addr: int, shape, dtype) -> torch.Tensor:
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    off = addr - buf.data_ptr()
    return buf[off:off + nbytes].cpu().view(dtype).reshape(shape)


def _unpermute_v(vb: torch.Tensor, B: int, H: int, Np: int, d: int) -> torch.Tensor:
    """[B, H, Np/128, d, 128] blocks with keys in sage_v_key_position order ->
    [B, H, Np, d]."""
    perm = torch.tensor([sage_v_key_position(j) for j in range(SAGE_BN)], dtype=torch.long)
    return vb[..., perm].permute(0, 1, 2, 4, 3).reshape(B, H, Np, d)


def read_kv_cache(c: sage_kv_cache, buf: torch.Tensor, B: int, Hkv: int, Nk: int, d: int) -> dict:
    """Copy a KV cache (carved from `buf`) to host tensors in the plain
    [B,Hkv,Nk,d] layout: K codes, scales and mean, and V as E4M3 code bytes
    (v_fp8) or binary16 bit patterns (v_f16), plus the values (v_half).
    Layout only; `*_pad` hold rows Nk..N_p-1."""
    Np = -(-Nk // SAGE_NPAD) * SAGE_NPAD
    torch.cuda.synchronize()
    k_full = _host_view(buf, c.k_i8, (B, Hkv, Np, d), torch.int8)
    f16 = c.pv_format == SAGE_PV_F16
    vb = _host_view(buf, c.v, (B, Hkv, Np // SAGE_BN, d, SAGE_BN), torch.int16 if f16 else torch.uint8)
    v_full = _unpermute_v(vb, B, Hkv, Np, d)
    if f16:
        codes = dict(v_f16=v_full[:, :, :Nk].contiguous())
        v_half = v_full.view(torch.float16)
    else:
        codes = dict(v_fp8=v_full[:, :, :Nk].contiguous())
        v_half = v_full.view(torch.float8_e4m3fn).to(torch.float16)
    return dict(
        **codes, k_i8=k_full[:, :, :Nk].contiguous(), v_half=v_half[:, :, :Nk].contiguous(),
        k_pad=k_full[:, :, Nk:].contiguous(), v_pad=v_full[:, :, Nk:].contiguous(),
        k_scale=_host_view(buf, c.k_scale, (B, Hkv, Np // c.k_block), torch.float32),
        k_mean=_host_view(buf, c.k_mean, (B, Hkv, d), torch.float32),
        v_scale=_host_view(buf, c.v_scale, (B, Hkv, d), torch.float32))


def read_quantized(z: sage_qkv_quant, workspace: torch.Tensor, B: int, Hq: int, Hkv: int,
                   N: int, d: int) -> dict:
    """Copy the quantized operands out of `workspace` (carved into `z`) to host
    tensors in the plain [B,H,N,d] layout, the V block permutation undone.  V
    comes back as its binary16 values (v_half) and as codes: E4M3 codes
    (v_fp8; the binary16 values convert back exactly) or, for the binary16
    P.V format, the binary16 bit patterns (v_f16).  Layout only; `*_pad` hold
    rows N..N_p-1."""
    Np = -(-N // SAGE_NPAD) * SAGE_NPAD
    torch.cuda.synchronize()

    def host(addr, shape, dtype):
        return _host_view(workspace, addr, shape, dtype)

    k_full = host(z.k_i8, (B, Hkv, Np, d), torch.int8)
    vb = host(z.v16, (B, Hkv, Np // SAGE_BN, d, SAGE_BN), torch.float16)
    v_half = _unpermute_v(vb, B, Hkv, Np, d)
    if z.pv_format == SAGE_PV_F16:
        v_codes = dict(v_f16=v_half.view(torch.int16)[:, :, :N].contiguous())
    else:
        v_codes = dict(v_fp8=v_half.to(torch.float8_e4m3fn).view(torch.uint8)[:, :, :N].contiguous())
    q_full = host(z.q_i8, (B, Hq, Np, d), torch.int8)
    return dict(
        **v_codes, q_i8=q_full[:, :, :N].contiguous(), k_i8=k_full[:, :, :N].contiguous(),
        v_half=v_half[:, :, :N].contiguous(),
        q_pad=q_full[:, :, N:].contiguous(), k_pad=k_full[:, :, N:].contiguous(),
        v_pad=v_half[:, :, N:].contiguous(),
        q_scale=host(z.q_scale, (B, Hq, Np // z.q_block), torch.float32),
        k_scale=host(z.k_scale, (B, Hkv, Np // z.k_block), torch.float32),
        k_mean=host(z.k_mean, (B, Hkv, d), torch.float32),
        v_scale=host(z.v_scale, (B, Hkv, d), torch.float32))
