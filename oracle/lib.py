"""ctypes wrapper around orc.c (test infrastructure only).

Builds liborc.so with gcc on first use when it is missing.  Arrays are numpy; every
function returns fresh output arrays plus the status bits the C code reports.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

ORC_NONFINITE = 1
ORC_SCALE_OVF = 2
ORC_F16_OVF = 4
ORC_BAD_AWQ = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "orc.c")
_LIB = os.path.join(_HERE, "liborc.so")
# ORC_LIB names another build of orc.c to load instead (the tests' mutation and sanitizer runs);
# it is used as given, never rebuilt.
_LIB_OVERRIDE = os.environ.get("ORC_LIB")
_lock = threading.Lock()
_lib = None

# Strict IEEE binary32: no contraction into FMA, no fast-math, SSE scalar (x86-64 default).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-strict-aliasing", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile orc.c into liborc.so (gcc)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32


def load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                lib = ctypes.CDLL(_LIB_OVERRIDE)
            else:
                build(force=False)
                lib = ctypes.CDLL(_LIB)
            lib.orc_f32_to_f16_n.argtypes = [_P, _P, _I64]
            lib.orc_f32_to_bf16_n.argtypes = [_P, _P, _I64]
            lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
            lib.orc_f16_to_f32.restype = ctypes.c_float
            lib.orc_percentile_rank.argtypes = [_I64, _U32, _U32]
            lib.orc_percentile_rank.restype = _I64
            lib.orc_quantize_rows.argtypes = [_P, _I64, _I64, _I64, _I32, _U32, _U32, _P, _P, _P, _P, _P, _P]
            lib.orc_quantize_rows.restype = _U32
            lib.orc_quantize_tensor.argtypes = [_P, _I64, _I64, _I64, _I32, _U32, _U32, _P, _P, _P, _P]
            lib.orc_quantize_tensor.restype = _U32
            lib.orc_pack6_rows.argtypes = [_P, _I64, _I64, _P]
            lib.orc_pack6_rows.restype = None
            lib.orc_unpack6_rows.argtypes = [_P, _I64, _I64, _P]
            lib.orc_unpack6_rows.restype = None
            lib.orc_dequant_rows.argtypes = [_P, _I64, _I64, _P, _I32, _P, _P]
            lib.orc_dequant_rows.restype = None
            lib.orc_qgemm_bf16.argtypes = [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _P]
            lib.orc_qgemm_bf16.restype = None
            lib.orc_awq_multipliers.argtypes = [_P, _I64, _P]
            lib.orc_awq_multipliers.restype = _U32
            lib.orc_fakequant_rows.argtypes = [_P, _I64, _I64, _I64, _I32, _U32, _U32, _P, _P, _P, _P, _P, _P]
            lib.orc_fakequant_rows.restype = _U32
            lib.orc_f16_passthrough.argtypes = [_P, _I64, _P]
            lib.orc_f16_passthrough.restype = _U32
            lib.orc_sqwa_update.argtypes = [_P, _P, _I64, _I32]
            lib.orc_sqwa_update.restype = None
            lib.orc_ema_update.argtypes = [_P, _P, _I64, ctypes.c_float, _I32]
            lib.orc_ema_update.restype = _U32
            lib.orc_swa_update.argtypes = [_P, _P, _I64, _I32]
            lib.orc_swa_update.restype = _U32
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def f32_to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    load().orc_f32_to_f16_n(_ptr(x), _ptr(y), x.size)
    return y


def f32_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    load().orc_f32_to_bf16_n(_ptr(x), _ptr(y), x.size)
    return y


_F16_TABLE = None


def f16_to_f32(h) -> np.ndarray:
    """Exact binary16 -> binary32 through a 65536-entry table filled by orc_f16_to_f32."""
    global _F16_TABLE
    if _F16_TABLE is None:
        lib = load()
        _F16_TABLE = np.array([lib.orc_f16_to_f32(i) for i in range(65536)], dtype=np.float32)
    return _F16_TABLE[np.ascontiguousarray(h, dtype=np.uint16)]


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def percentile_rank(n: int, num: int, den: int) -> int:
    return int(load().orc_percentile_rank(n, num, den))


def quantize_rows(w, Q: int, num: int = 1, den: int = 1, awq=None, want_t: bool = False,
                  want_clip: bool = False):
    """Per-row quantization of a 2-D float32 array (rows x cols).

    Returns dict(codes int8 [rows, cols], scales uint16 [rows], dq float32 [rows, cols],
    status, and t / clip when asked)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.ndim == 2
    rows, cols = w.shape
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty(rows, dtype=np.uint16)
    dq = np.empty((rows, cols), dtype=np.float32)
    t = np.empty((rows, cols), dtype=np.float32) if want_t else None
    clip = np.empty(rows, dtype=np.float32) if want_clip else None
    a = None if awq is None else np.ascontiguousarray(awq, dtype=np.uint16)
    if a is not None:
        assert a.shape == (cols,)
    st = load().orc_quantize_rows(_ptr(w), rows, cols, cols, Q, num, den, _ptr(a), _ptr(codes),
                                  _ptr(scales), _ptr(dq), _ptr(t), _ptr(clip))
    out = dict(codes=codes, scales=scales, dq=dq, status=int(st))
    if want_t:
        out["t"] = t
    if want_clip:
        out["clip"] = clip
    return out


def quantize_tensor(w, Q: int, num: int = 1, den: int = 1) -> dict:
    """Per-tensor quantization of a 2-D float32 array: one fp16 scale for all rows * cols.

    Returns dict(codes int8 [rows, cols], scale uint16 [1], dq float32 [rows, cols], clip
    float32, status)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.ndim == 2 and w.size > 0
    rows, cols = w.shape
    codes = np.empty((rows, cols), dtype=np.int8)
    scale = np.empty(1, dtype=np.uint16)
    dq = np.empty((rows, cols), dtype=np.float32)
    clip = np.empty(1, dtype=np.float32)
    st = load().orc_quantize_tensor(_ptr(w), rows, cols, cols, Q, num, den, _ptr(codes), _ptr(scale), _ptr(dq),
                                    _ptr(clip))
    return dict(codes=codes, scale=scale, dq=dq, clip=float(clip[0]), status=int(st))


def awq_multipliers(s):
    s = np.ascontiguousarray(s, dtype=np.float32)
    a = np.empty(s.shape, dtype=np.uint16)
    st = load().orc_awq_multipliers(_ptr(s), s.size, _ptr(a))
    return a, int(st)


def fakequant_rows(w_bf16, Q: int = 31, num: int = 1, den: int = 1, g_bf16=None):
    """STE fake quantization of a 2-D bfloat16 (uint16 bits) array."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    rows, cols = w.shape
    mb = (cols + 7) // 8
    dq = np.empty((rows, cols), dtype=np.uint16)
    scales = np.empty(rows, dtype=np.uint16)
    mask = np.empty((rows, mb), dtype=np.uint8)
    codes = np.empty((rows, cols), dtype=np.int8)
    g = None if g_bf16 is None else np.ascontiguousarray(g_bf16, dtype=np.uint16)
    g_out = None if g is None else np.empty((rows, cols), dtype=np.uint16)
    st = load().orc_fakequant_rows(_ptr(w), rows, cols, cols, Q, num, den, _ptr(dq), _ptr(scales),
                                   _ptr(mask), _ptr(g), _ptr(g_out), _ptr(codes))
    return dict(dq=dq, scales=scales, mask=mask, codes=codes, g_out=g_out, status=int(st))


def f16_passthrough(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    st = load().orc_f16_passthrough(_ptr(x), x.size, _ptr(y))
    return y, int(st)


def sqwa_update(mean: np.ndarray, xhat, k: int) -> np.ndarray:
    """In-place running-mean update of a contiguous float32 array; returns it."""
    assert mean.dtype == np.float32 and mean.flags.c_contiguous
    xhat = np.ascontiguousarray(xhat, dtype=np.float32)
    assert xhat.size == mean.size
    load().orc_sqwa_update(_ptr(mean), _ptr(xhat), mean.size, k)
    return mean


def ema_update(e: np.ndarray, w, decay: float, init: bool = False) -> int:
    """In-place EMA update of a contiguous float32 array e with weights w; returns the status."""
    assert e.dtype == np.float32 and e.flags.c_contiguous
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.size == e.size
    return int(load().orc_ema_update(_ptr(e), _ptr(w), e.size, float(np.float32(decay)), 1 if init else 0))


def swa_update(mean: np.ndarray, w, k: int) -> int:
    """In-place running-mean (SWA) update with checkpoint k (1-based); returns the status."""
    assert mean.dtype == np.float32 and mean.flags.c_contiguous
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.size == mean.size
    return int(load().orc_swa_update(_ptr(mean), _ptr(w), mean.size, k))


def pack6_row_bytes(cols: int) -> int:
    return 3 * ((cols + 3) // 4)


def pack6(codes) -> np.ndarray:
    """int8 codes [rows, cols] in [-32, 31] -> packed bytes [rows, 3 * ceil(cols / 4)]."""
    c = np.ascontiguousarray(codes, dtype=np.int8)
    assert c.ndim == 2
    rows, cols = c.shape
    out = np.empty((rows, pack6_row_bytes(cols)), dtype=np.uint8)
    load().orc_pack6_rows(_ptr(c), rows, cols, _ptr(out))
    return out


def unpack6(packed, cols: int) -> np.ndarray:
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = p.shape[0]
    assert p.shape == (rows, pack6_row_bytes(cols))
    out = np.empty((rows, cols), dtype=np.int8)
    load().orc_unpack6_rows(_ptr(p), rows, cols, _ptr(out))
    return out


def dequant(codes, scales, per_tensor: bool = False, awq=None) -> np.ndarray:
    """x = code * s (/ a_j) for int8 codes [rows, cols] with fp16 scales (bit patterns)."""
    c = np.ascontiguousarray(codes, dtype=np.int8)
    rows, cols = c.shape
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    a = None if awq is None else np.ascontiguousarray(awq, dtype=np.uint16)
    out = np.empty((rows, cols), dtype=np.float32)
    load().orc_dequant_rows(_ptr(c), rows, cols, _ptr(s), 1 if per_tensor else 0, _ptr(a), _ptr(out))
    return out


def qgemm_bf16(x_bf16, codes, scales):
    """Y = X What^T in double, What = bf16(code * s) per row; returns (y, sum |x What|)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    c = np.ascontiguousarray(codes, dtype=np.int8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    M, K = x.shape
    N = c.shape[0]
    assert c.shape == (N, K) and s.shape == (N,)
    y = np.empty((M, N), dtype=np.float64)
    b = np.empty((M, N), dtype=np.float64)
    load().orc_qgemm_bf16(_ptr(x), M, K, K, _ptr(c), K, _ptr(s), N, _ptr(y), _ptr(b))
    return y, b
