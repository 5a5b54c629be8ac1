"""torch-facing helpers over the libpgq C ABI.

torch provides device memory and the current HIP stream; every step of the quantizer
runs in libpgq's kernels.  Outputs that are fp16 / bf16 bit patterns are returned as
int16 tensors (reinterpret with .view(torch.float16) / .view(torch.bfloat16)).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import pgq

DEFAULT_INT8_PATTERNS = ("tok_emb.weight", "lm_head.weight")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return pgq.PGQ_F32
    if dt == torch.bfloat16:
        return pgq.PGQ_BF16
    if dt == torch.float16:
        return pgq.PGQ_F16
    raise TypeError(f"unsupported dtype {dt}")


def _rows_view(t: torch.Tensor) -> Tuple[int, int, int]:
    """(rows, cols, ld) of a tensor seen as [shape0, prod(rest)] (1-D: one row)."""
    if t.dim() == 0:
        return 1, 1, 1
    if t.dim() == 1:
        assert t.stride(0) == 1 or t.numel() <= 1, "1-D tensors must be contiguous"
        return 1, t.numel(), t.numel()
    if t.dim() > 2:
        t = t.reshape(t.shape[0], -1)
    assert t.stride(1) == 1 or t.shape[1] <= 1, "rows must be contiguous"
    return t.shape[0], t.shape[1], (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def new_status(device=None) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device or "cuda")


def qparams(bits: int, pct: Tuple[int, int] = (1, 1)) -> pgq.pgq_qparams:
    return pgq.pgq_qparams(bits, pct[0], pct[1])


def quantize_rows(w: torch.Tensor, bits: int = 6, pct: Tuple[int, int] = (1, 1),
                  awq_s: Optional[torch.Tensor] = None, want_codes: bool = True,
                  dq_dtype: Optional[torch.dtype] = torch.float32,
                  status: Optional[torch.Tensor] = None, out: Optional[dict] = None) -> dict:
    """Per-row quantization of one matrix (fp32, bf16 or fp16, rows contiguous)."""
    rows, cols, ld = _rows_view(w)
    dev = w.device
    if out is None:
        out = {}
        out["scales"] = torch.empty(rows, dtype=torch.int16, device=dev)
        if want_codes:
            out["codes"] = torch.empty(rows, cols, dtype=torch.int8, device=dev)
        if dq_dtype is not None:
            out["dq"] = torch.empty(rows, cols, dtype=dq_dtype, device=dev)
        if awq_s is not None:
            out["awq"] = torch.empty(cols, dtype=torch.int16, device=dev)
    st = status if status is not None else new_status(dev)
    dq = out.get("dq")
    rc = pgq.pgq_quantize_rows(_p(w), _dtype_code(w.dtype), rows, cols, ld, qparams(bits, pct), _p(awq_s),
                               _p(out.get("awq")), _p(out.get("codes")), _p(out["scales"]), _p(dq),
                               _dtype_code(dq.dtype) if dq is not None else pgq.PGQ_F32, _p(st), _stream())
    pgq.check(rc, "pgq_quantize_rows")
    out["status"] = st
    return out


class FakeQuant:
    """STE fake quantization of a fixed list of bf16 weight matrices (grouped launches).

    Buffers for dq, scales, mask and grad_out are allocated once; each call re-runs the
    kernels on the same buffers, reusing the uploaded descriptor table."""

    def __init__(self, weights: Sequence[torch.Tensor], bits: int = 6, pct: Tuple[int, int] = (1, 1),
                 want_codes: bool = False):
        self.weights = list(weights)
        self.qp = qparams(bits, pct)
        dev = self.weights[0].device
        self.dq, self.scales, self.mask, self.codes, self.grad_out = [], [], [], [], []
        for w in self.weights:
            assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1
            r, c = w.shape
            self.dq.append(torch.empty(r, c, dtype=torch.bfloat16, device=dev))
            self.scales.append(torch.empty(r, dtype=torch.int16, device=dev))
            self.mask.append(torch.empty(r, (c + 7) // 8, dtype=torch.uint8, device=dev))
            self.codes.append(torch.empty(r, c, dtype=torch.int8, device=dev) if want_codes else None)
            self.grad_out.append(torch.empty(r, c, dtype=torch.bfloat16, device=dev))
        self.status = new_status(dev)
        self._tables = {}

    def _descs(self, grads):
        n = len(self.weights)
        arr = (pgq.pgq_fq_tensor * n)()
        for i, w in enumerate(self.weights):
            g = None if grads is None else grads[i]
            if g is not None:
                assert g.shape == w.shape and g.dtype == torch.bfloat16 and g.is_contiguous()
            arr[i] = pgq.pgq_fq_tensor(w.data_ptr(), w.shape[0], w.shape[1], w.stride(0),
                                       self.dq[i].data_ptr(), self.scales[i].data_ptr(), self.mask[i].data_ptr(),
                                       0 if g is None else g.data_ptr(), self.grad_out[i].data_ptr(),
                                       0 if self.codes[i] is None else self.codes[i].data_ptr())
        return arr

    def run(self, mode: int, grads: Optional[Sequence[torch.Tensor]] = None, reuse_table: bool = True):
        """Enqueue one grouped launch.  The descriptor array and the workspace holding its
        uploaded table are kept per (mode, gradient buffers), so repeated steps over the same
        buffers only re-enqueue the kernel."""
        n = len(self.weights)
        key = (mode, tuple(0 if grads is None else g.data_ptr() for g in (grads or [])))
        cached = self._tables.get(key)
        flags = 0
        if cached is not None and reuse_table:
            arr, ws = cached
            flags = pgq.PGQ_TABLE_RESIDENT
        else:
            arr = self._descs(grads)
            need = ctypes.c_size_t(0)
            pgq.check(pgq.pgq_fakequant_workspace(arr, n, ctypes.byref(need)), "pgq_fakequant_workspace")
            ws = torch.empty(max(need.value, 64), dtype=torch.uint8, device=self.weights[0].device)
            self._tables[key] = (arr, ws)
        rc = pgq.pgq_fakequant_fwd_bwd(mode, arr, n, self.qp, _p(ws), ws.numel(), flags, _p(self.status), _stream())
        pgq.check(rc, "pgq_fakequant_fwd_bwd")


@dataclass
class ExportTensor:
    name: str
    w: torch.Tensor
    awq_s: Optional[torch.Tensor] = None


def _tensor_in_array(tensors: Sequence[ExportTensor]):
    n = len(tensors)
    arr = (pgq.pgq_tensor_in * n)()
    keep = []
    for i, t in enumerate(tensors):
        rows, cols, ld = _rows_view(t.w)
        nm = t.name.encode()
        keep.append(nm)
        arr[i] = pgq.pgq_tensor_in(nm, t.w.data_ptr() if t.w.numel() else 0, _dtype_code(t.w.dtype), 0,
                                   rows, cols, ld, 0 if t.awq_s is None else t.awq_s.data_ptr())
    return arr, keep


def make_policy(int8_patterns=DEFAULT_INT8_PATTERNS, passthrough_below: int = 65536,
                q_default=(6, 9999, 10000), q_sensitive=(8, 1, 1), per_tensor: bool = False,
                pack6: bool = False):
    pats = [p.encode() for p in int8_patterns]
    parr = (ctypes.c_char_p * max(1, len(pats)))(*pats)
    pol = pgq.pgq_policy(ctypes.cast(parr, ctypes.POINTER(ctypes.c_char_p)), len(pats), 1 if per_tensor else 0,
                         passthrough_below,
                         pgq.pgq_qparams(*q_default), pgq.pgq_qparams(*q_sensitive), 1 if pack6 else 0, 0)
    pol._keep = (pats, parr)
    return pol


class Exporter:
    """Whole-model export: plan once, then one grouped launch per call."""

    def __init__(self, tensors: Sequence[ExportTensor], policy=None, want_dq: bool = False):
        self.tensors = list(tensors)
        self.policy = policy if policy is not None else make_policy()
        n = len(self.tensors)
        self.n = n
        self.arr, self._keep = _tensor_in_array(self.tensors)
        self.plan = (pgq.pgq_tensor_plan * max(n, 1))()
        ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
        pgq.check(pgq.pgq_export_plan(self.arr, n, ctypes.byref(self.policy), self.plan, ctypes.byref(ab),
                                      ctypes.byref(wb)), "pgq_export_plan")
        dev = self.tensors[0].w.device
        self.arena = torch.empty(ab.value, dtype=torch.uint8, device=dev)
        self.workspace = torch.empty(max(wb.value, 64), dtype=torch.uint8, device=dev)
        self.dq = None
        self.dq_ptrs = None
        if want_dq:
            self.dq = [torch.empty(t.w.shape, dtype=torch.float32, device=dev) for t in self.tensors]
            self.dq_ptrs = (ctypes.c_void_p * n)(*[d.data_ptr() for d in self.dq])
        self.status = new_status(dev)
        self._uploaded = False

    def run(self, reuse_table: bool = True):
        flags = pgq.PGQ_TABLE_RESIDENT if (reuse_table and self._uploaded) else 0
        rc = pgq.pgq_export_model(self.arr, self.n, self.plan, _p(self.arena), self.dq_ptrs, _p(self.workspace),
                                  self.workspace.numel(), flags, _p(self.status), _stream())
        pgq.check(rc, "pgq_export_model")
        self._uploaded = True

    def decode(self, out: Optional[List[torch.Tensor]] = None, reuse_table: bool = True) -> List[torch.Tensor]:
        """fp32 weights from the arena (the stored artifact), every tensor in one launch."""
        dev = self.arena.device
        if out is None:
            out = [torch.empty(t.w.shape, dtype=torch.float32, device=dev) for t in self.tensors]
        key = tuple(o.data_ptr() for o in out)
        cached = getattr(self, "_decode_table", None)
        flags = 0
        if cached is not None and cached[0] == key and reuse_table:
            ptrs, ws = cached[1], cached[2]
            flags = pgq.PGQ_TABLE_RESIDENT
        else:
            ptrs = (ctypes.c_void_p * self.n)(*[o.data_ptr() for o in out])
            ws = torch.empty(self.workspace.numel(), dtype=torch.uint8, device=dev)
            self._decode_table = (key, ptrs, ws)
        rc = pgq.pgq_dequant_model(self.arr, self.n, self.plan, _p(self.arena), ptrs, _p(ws), ws.numel(), flags,
                                   _p(self.status), _stream())
        pgq.check(rc, "pgq_dequant_model")
        return out

    def kinds(self) -> List[int]:
        return [self.plan[i].kind for i in range(self.n)]

    def outputs(self) -> List[dict]:
        """Per-tensor views into the arena: codes [rows, cols] int8, scales [rows] int16,
        f16 [shape] int16, awq [cols] int16."""
        res = []
        for i, t in enumerate(self.tensors):
            p = self.plan[i]
            rows, cols, _ = _rows_view(t.w)
            rec = {"name": t.name, "kind": p.kind}
            if p.kind == pgq.PGQ_KIND_F16:
                rec["f16"] = self.arena[p.f16_off:p.f16_off + 2 * rows * cols].view(torch.int16).view(t.w.shape)
            else:
                if p.packed:
                    rb = 3 * ((cols + 3) // 4)
                    rec["packed"] = self.arena[p.codes_off:p.codes_off + rows * rb].view(rows, rb)
                else:
                    rec["codes"] = self.arena[p.codes_off:p.codes_off + rows * cols].view(torch.int8).view(rows, cols)
                ns = 1 if p.per_tensor else rows
                rec["scales"] = self.arena[p.scales_off:p.scales_off + 2 * ns].view(torch.int16)
                if p.has_awq:
                    rec["awq"] = self.arena[p.awq_off:p.awq_off + 2 * cols].view(torch.int16)
            if self.dq is not None:
                rec["dq"] = self.dq[i]
            res.append(rec)
        return res


class Sqwa:
    """Running mean of quantize-dequantize snapshots, then export of the mean."""

    def __init__(self, tensors: Sequence[ExportTensor], policy=None):
        self.policy = policy if policy is not None else make_policy(int8_patterns=())
        self.exporter_template = list(tensors)
        dev = tensors[0].w.device
        self.means = [torch.empty(t.w.shape, dtype=torch.float32, device=dev) for t in tensors]
        self.mean_ptrs = (ctypes.c_void_p * len(tensors))(*[m.data_ptr() for m in self.means])
        self.n = len(tensors)
        arr, keep = _tensor_in_array(tensors)
        self.plan = (pgq.pgq_tensor_plan * max(self.n, 1))()
        ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
        pgq.check(pgq.pgq_export_plan(arr, self.n, ctypes.byref(self.policy), self.plan, ctypes.byref(ab),
                                      ctypes.byref(wb)), "pgq_export_plan")
        self.workspace_bytes = max(wb.value, 64)
        self.status = new_status(dev)
        self._tables: Dict[tuple, tuple] = {}

    def accumulate(self, snapshot: Sequence[torch.Tensor], k: int, reuse_table: bool = True):
        """Fold snapshot k (1-based) into the means.  The tensor array and the workspace with
        its uploaded table are kept per snapshot buffer set (k is a kernel argument, not part
        of the table), so repeated runs over resident snapshots only re-enqueue the kernel."""
        key = tuple(w.data_ptr() for w in snapshot)
        cached = self._tables.get(key)
        flags = 0
        if cached is not None and reuse_table:
            arr, keep, ws = cached
            flags = pgq.PGQ_TABLE_RESIDENT
        else:
            tensors = [ExportTensor(t.name, w, t.awq_s) for t, w in zip(self.exporter_template, snapshot)]
            arr, keep = _tensor_in_array(tensors)
            ws = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.means[0].device)
            self._tables[key] = (arr, keep, ws)
        rc = pgq.pgq_sqwa_accumulate(arr, self.n, self.plan, self.mean_ptrs, k, _p(ws), ws.numel(), flags,
                                     _p(self.status), _stream())
        pgq.check(rc, "pgq_sqwa_accumulate")

    def exporter(self, want_dq: bool = False) -> Exporter:
        return Exporter([ExportTensor(t.name, m, t.awq_s) for t, m in zip(self.exporter_template, self.means)],
                        self.policy, want_dq=want_dq)


class _Averager:
    """fp32 averages of a fixed list of weight tensors (fp32, bf16 or fp16, rows contiguous), updated
    in place by one grouped launch per call.  The tensor array and the workspace holding the
    uploaded descriptor table are kept per weight buffer set, so calls over resident weights
    only re-enqueue the kernel."""

    def __init__(self, like: Sequence[torch.Tensor]):
        like = list(like)
        self.n = len(like)
        dev = like[0].device
        self.avg = [torch.empty(w.shape, dtype=torch.float32, device=dev) for w in like]
        self.avg_ptrs = (ctypes.c_void_p * self.n)(*[a.data_ptr() for a in self.avg])
        self.status = new_status(dev)
        self._tables: Dict[tuple, tuple] = {}

    def _table(self, weights: Sequence[torch.Tensor], reuse_table: bool):
        key = tuple(w.data_ptr() for w in weights)
        cached = self._tables.get(key)
        if cached is not None and reuse_table:
            return cached + (pgq.PGQ_TABLE_RESIDENT,)
        assert len(weights) == self.n
        arr, keep = _tensor_in_array([ExportTensor("", w) for w in weights])
        wb = ctypes.c_size_t(0)
        pgq.check(pgq.pgq_average_workspace(arr, self.n, ctypes.byref(wb)), "pgq_average_workspace")
        ws = torch.empty(max(wb.value, 64), dtype=torch.uint8, device=self.avg[0].device)
        self._tables[key] = (arr, keep, ws)
        return arr, keep, ws, 0


class Ema(_Averager):
    """Exponential moving average of the weights (decay 0.997 by default)."""

    def __init__(self, like: Sequence[torch.Tensor], decay: float = 0.997):
        super().__init__(like)
        self.decay = decay

    def update(self, weights: Sequence[torch.Tensor], init: bool = False, reuse_table: bool = True):
        arr, _, ws, flags = self._table(weights, reuse_table)
        rc = pgq.pgq_ema_update(arr, self.n, self.avg_ptrs, self.decay, 1 if init else 0, _p(ws), ws.numel(),
                                flags, _p(self.status), _stream())
        pgq.check(rc, "pgq_ema_update")


class Swa(_Averager):
    """Running mean of weight checkpoints k = 1, 2, ... (stochastic weight averaging)."""

    def accumulate(self, weights: Sequence[torch.Tensor], k: int, reuse_table: bool = True):
        arr, _, ws, flags = self._table(weights, reuse_table)
        rc = pgq.pgq_swa_accumulate(arr, self.n, self.avg_ptrs, k, _p(ws), ws.numel(), flags, _p(self.status),
                                    _stream())
        pgq.check(rc, "pgq_swa_accumulate")


def dequant_codes(codes: torch.Tensor, scales: torch.Tensor, cols: int, packed: bool = False,
                  per_tensor: bool = False, awq: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 weights from stored codes (int8 [rows, cols], or packed uint8 [rows, 3 ceil(cols/4)])
    and fp16 scales (int16 bit patterns); awq: cols fp16 multipliers (int16 bit patterns)."""
    rows = codes.shape[0]
    assert codes.is_contiguous() and scales.is_contiguous()
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.float32, device=codes.device)
    rc = pgq.pgq_dequant_codes(_p(codes), 1 if packed else 0, rows, cols, _p(scales), 1 if per_tensor else 0,
                               _p(awq), _p(out), None, _stream())
    pgq.check(rc, "pgq_dequant_codes")
    return out


def qgemm(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None,
          out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Y = X What^T with What = bf16(code * s) formed inside the GEMM.  x: bf16 [M, K] (rows
    contiguous), codes: int8 [N, K], scales: fp16 bit patterns [N] (int16); returns Y [M, N] in
    out_dtype: fp32, or bf16 (each element bf16 of the fp32 result, the same accumulation)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    assert codes.dtype == torch.int8 and codes.dim() == 2 and codes.stride(1) == 1
    assert out_dtype in (torch.float32, torch.bfloat16)
    M, K = x.shape
    N = codes.shape[0]
    assert codes.shape[1] == K and scales.numel() == N and scales.is_contiguous()
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=x.device)
    assert out.dtype == out_dtype and out.dim() == 2 and out.shape == (M, N) and out.stride(1) == 1
    fn, name = ((pgq.pgq_qgemm_bf16, "pgq_qgemm_bf16") if out_dtype == torch.float32
                else (pgq.pgq_qgemm_bf16_ybf16, "pgq_qgemm_bf16_ybf16"))
    rc = fn(_p(x), M, K, x.stride(0) if M > 1 else K, _p(codes), codes.stride(0) if N > 1 else K,
            _p(scales), N, _p(out), out.stride(0) if M > 1 else N, _stream())
    pgq.check(rc, name)
    return out
