"""ctypes binding of libpgq (include/pgq.h): same names, argument marshalling only.

Every pgq_* function here takes plain integers for device pointers (e.g. a torch
tensor's data_ptr()) and for the HIP stream handle, and returns the pgq_status integer.
All computation happens in the HIP library; if it is not built or cannot be loaded,
importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpgq.so")

PGQ_OK = 0
PGQ_ERR_NULL = 1
PGQ_ERR_SHAPE = 2
PGQ_ERR_DTYPE = 3
PGQ_ERR_PARAM = 4
PGQ_ERR_ALIGN = 5
PGQ_ERR_WORKSPACE = 6
PGQ_ERR_HIP = 7

PGQ_DEV_NONFINITE = 1
PGQ_DEV_SCALE_OVF = 2
PGQ_DEV_F16_OVF = 4
PGQ_DEV_BAD_AWQ = 8
PGQ_DEV_STALE_TABLE = 16

PGQ_F32 = 0
PGQ_BF16 = 1
PGQ_F16 = 2
PGQ_KIND_F16 = 16
PGQ_TABLE_RESIDENT = 1

PGQ_FQ_FWD = 1
PGQ_FQ_BWD = 2
PGQ_FQ_FWD_BWD = 3


class PgqError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        detail = f" [{pgq_last_error()}]" if status == PGQ_ERR_HIP else ""
        super().__init__(f"{what}: {pgq_status_str(status)} (status {status}){detail}")


class pgq_qparams(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("pct_num", ctypes.c_uint32), ("pct_den", ctypes.c_uint32)]


class pgq_fq_tensor(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("dq", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("mask", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("grad_out", ctypes.c_void_p),
                ("codes", ctypes.c_void_p)]


class pgq_tensor_in(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("w", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("awq_s", ctypes.c_void_p)]


class pgq_policy(ctypes.Structure):
    _fields_ = [("int8_patterns", ctypes.POINTER(ctypes.c_char_p)), ("n_patterns", ctypes.c_int32),
                ("per_tensor", ctypes.c_int32), ("passthrough_below", ctypes.c_int64),
                ("q_default", pgq_qparams), ("q_sensitive", pgq_qparams), ("pack6", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class pgq_tensor_plan(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("has_awq", ctypes.c_int32), ("qp", pgq_qparams),
                ("per_tensor", ctypes.c_int32), ("codes_off", ctypes.c_int64), ("scales_off", ctypes.c_int64),
                ("f16_off", ctypes.c_int64), ("awq_off", ctypes.c_int64), ("packed", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "pgq_quantize_rows": (_I32, [_P, _I32, _I64, _I64, _I64, pgq_qparams, _P, _P, _P, _P, _P, _I32, _P, _P]),
    "pgq_fakequant_workspace": (_I32, [ctypes.POINTER(pgq_fq_tensor), _I32, ctypes.POINTER(_SZ)]),
    "pgq_fakequant_fwd_bwd": (_I32, [_I32, ctypes.POINTER(pgq_fq_tensor), _I32, pgq_qparams, _P, _SZ, _U32, _P, _P]),
    "pgq_export_plan": (_I32, [ctypes.POINTER(pgq_tensor_in), _I32, ctypes.POINTER(pgq_policy),
                               ctypes.POINTER(pgq_tensor_plan), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "pgq_export_model": (_I32, [ctypes.POINTER(pgq_tensor_in), _I32, ctypes.POINTER(pgq_tensor_plan), _P,
                                ctypes.POINTER(_P), _P, _SZ, _U32, _P, _P]),
    "pgq_export_model_noalloc": (_I32, [ctypes.POINTER(pgq_tensor_in), _I32, ctypes.POINTER(pgq_tensor_plan), _P,
                                        ctypes.POINTER(_P), _U32, _P, _P]),
    "pgq_sqwa_accumulate": (_I32, [ctypes.POINTER(pgq_tensor_in), _I32, ctypes.POINTER(pgq_tensor_plan),
                                   ctypes.POINTER(_P), _I32, _P, _SZ, _U32, _P, _P]),
    "pgq_dequant_codes": (_I32, [_P, _I32, _I64, _I64, _P, _I32, _P, _P, _P, _P]),
    "pgq_qgemm_bf16": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P]),
    "pgq_qgemm_bf16_ybf16": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P]),
    "pgq_dequant_model": (_I32, [ctypes.POINTER(pgq_tensor_in), _I32, ctypes.POINTER(pgq_tensor_plan), _P,
                                 ctypes.POINTER(_P), _P, _SZ, _U32, _P, _P]),
    "pgq_average_workspace": (_I32, [ctypes.POINTER(pgq_tensor_in), _I32, ctypes.POINTER(_SZ)]),
    "pgq_ema_update": (_I32, [ctypes.POINTER(pgq_tensor_in), _I32, ctypes.POINTER(_P), ctypes.c_float, _I32, _P,
                              _SZ, _U32, _P, _P]),
    "pgq_swa_accumulate": (_I32, [ctypes.POINTER(pgq_tensor_in), _I32, ctypes.POINTER(_P), _I32, _P, _SZ, _U32,
                                  _P, _P]),
    "pgq_time_next_launch": (_I32, [_P, _P]),
    "pgq_status_str": (ctypes.c_char_p, [_I32]),
    "pgq_version": (ctypes.c_char_p, []),
    "pgq_last_error": (ctypes.c_char_p, []),
}


def _load():
    # One HIP runtime per process: PyTorch-ROCm ships its own libamdhip64 (soname
    # libamdhip64.so.7) and loads it by file name, so if libpgq were loaded first it would pull
    # in the system runtime and PyTorch a second copy, which then disagree about the device.
    # Loading PyTorch first lets libpgq's dependency resolve to the runtime already mapped.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libpgq.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                          f"python -m int6_weight_export_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def pgq_quantize_rows(w, w_dtype, rows, cols, ld, qp, awq_s, awq_mult, codes, scales, dq, dq_dtype,
                      dev_status, stream):
    return _lib.pgq_quantize_rows(w, w_dtype, rows, cols, ld, qp, awq_s, awq_mult, codes, scales, dq,
                                  dq_dtype, dev_status, stream)


def pgq_fakequant_workspace(t, n, workspace_bytes):
    return _lib.pgq_fakequant_workspace(t, n, workspace_bytes)


def pgq_fakequant_fwd_bwd(mode, t, n, qp, workspace, workspace_bytes, flags, dev_status, stream):
    return _lib.pgq_fakequant_fwd_bwd(mode, t, n, qp, workspace, workspace_bytes, flags, dev_status, stream)


def pgq_export_plan(t, n, pol, plan, arena_bytes, workspace_bytes):
    return _lib.pgq_export_plan(t, n, pol, plan, arena_bytes, workspace_bytes)


def pgq_export_model(t, n, plan, arena, dq_out, workspace, workspace_bytes, flags, dev_status, stream):
    return _lib.pgq_export_model(t, n, plan, arena, dq_out, workspace, workspace_bytes, flags, dev_status,
                                 stream)


def pgq_export_model_noalloc(t, n, plan, arena, dq_out, flags, dev_status, stream):
    return _lib.pgq_export_model_noalloc(t, n, plan, arena, dq_out, flags, dev_status, stream)


def pgq_sqwa_accumulate(snap, n, plan, mean, k, workspace, workspace_bytes, flags, dev_status, stream):
    return _lib.pgq_sqwa_accumulate(snap, n, plan, mean, k, workspace, workspace_bytes, flags, dev_status,
                                    stream)


def pgq_qgemm_bf16(x, M, K, ldx, codes, ldc, scales, N, y, ldy, stream):
    return _lib.pgq_qgemm_bf16(x, M, K, ldx, codes, ldc, scales, N, y, ldy, stream)


def pgq_qgemm_bf16_ybf16(x, M, K, ldx, codes, ldc, scales, N, y, ldy, stream):
    return _lib.pgq_qgemm_bf16_ybf16(x, M, K, ldx, codes, ldc, scales, N, y, ldy, stream)


def pgq_dequant_codes(codes, packed, rows, cols, scales, per_tensor, awq_mult, out, dev_status, stream):
    return _lib.pgq_dequant_codes(codes, packed, rows, cols, scales, per_tensor, awq_mult, out, dev_status, stream)


def pgq_dequant_model(t, n, plan, arena, out, workspace, workspace_bytes, flags, dev_status, stream):
    return _lib.pgq_dequant_model(t, n, plan, arena, out, workspace, workspace_bytes, flags, dev_status, stream)


def pgq_average_workspace(w, n, workspace_bytes):
    return _lib.pgq_average_workspace(w, n, workspace_bytes)


def pgq_ema_update(w, n, ema, decay, init, workspace, workspace_bytes, flags, dev_status, stream):
    return _lib.pgq_ema_update(w, n, ema, decay, init, workspace, workspace_bytes, flags, dev_status, stream)


def pgq_swa_accumulate(w, n, mean, k, workspace, workspace_bytes, flags, dev_status, stream):
    return _lib.pgq_swa_accumulate(w, n, mean, k, workspace, workspace_bytes, flags, dev_status, stream)


def pgq_time_next_launch(start_event, stop_event):
    return _lib.pgq_time_next_launch(start_event, stop_event)


def pgq_status_str(s: int) -> str:
    return _lib.pgq_status_str(s).decode()


def pgq_version() -> str:
    return _lib.pgq_version().decode()


def pgq_last_error() -> str:
    return _lib.pgq_last_error().decode()


def check(status: int, what: str = "pgq") -> None:
    if status != PGQ_OK:
        raise PgqError(status, what)
