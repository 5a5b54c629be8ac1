"""Per-tensor export policy and snapshot averaging, written plainly over orc.c.

Sources (Parameter Golf submission pages):
  * "Swiglu gating ... 10min/16MB Track" (PR #2159), Key Explored Modifications:
    per-row quantization, percentile clipping for export, small-tensor FP16 passthrough.
  * "12L 24min Vocab1792 ... Int6AWQ MixedBits" (PR #1495), Submission summary: mixed-bit
    int6 AWQ export; Mixed-bit quantization details: the export stays int6 for most
    tensors and tensors named by QUANT_INT8_NAME_PATTERNS (default tok_emb.weight,
    lm_head.weight) are promoted to int8.
  * "Discriminative TTT + SLOT-24" card (PR #1414), Novel Contributions: SQWA averages
    quantize-dequantize snapshots; section Quantization: int6 with scope "all".

Readings where the pages are silent: a tensor with fewer than `passthrough_below`
elements (65,536) is stored as fp16; otherwise a name that contains any int8 pattern
as a substring is int8 (absmax); everything else is int6 with the policy's percentile.
The passthrough test comes first.  A 2-D [out, in] tensor is quantized per row; a
1-D tensor is one row; higher ranks flatten to [shape[0], prod(shape[1:])].  AWQ
multipliers apply to int6 tensors only.  The running mean of SQWA uses the same
policy for the per-snapshot quantize-dequantize, and the final mean is exported
with it.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import lib

KIND_F16 = 16
KIND_INT6 = 6
KIND_INT8 = 8

DEFAULT_INT8_PATTERNS = ("tok_emb.weight", "lm_head.weight")


@dataclass
class Policy:
    int8_patterns: Tuple[str, ...] = DEFAULT_INT8_PATTERNS
    passthrough_below: int = 65536
    q6: Tuple[int, int, int] = (6, 9999, 10000)   # (bits, pct_num, pct_den)
    q8: Tuple[int, int, int] = (8, 1, 1)
    per_tensor: bool = False                      # one scale per integer-kind tensor
    pack6: bool = False                           # int6 codes stored 4 per 3 bytes


def qmax(bits: int) -> int:
    return (1 << (bits - 1)) - 1


def tensor_kind(name: str, numel: int, pol: Policy) -> int:
    if numel < pol.passthrough_below:
        return KIND_F16
    for p in pol.int8_patterns:
        if p and p in name:
            return KIND_INT8
    return KIND_INT6


def as_rows(shape: Sequence[int]) -> Tuple[int, int]:
    if len(shape) == 0:
        return 1, 1
    if len(shape) == 1:
        return 1, int(shape[0])
    return int(shape[0]), int(np.prod(shape[1:]))


def _qparams(kind: int, pol: Policy):
    bits, num, den = pol.q8 if kind == KIND_INT8 else pol.q6
    return qmax(bits), num, den


def export(tensors, pol: Policy, awq: Optional[Dict[str, np.ndarray]] = None) -> List[dict]:
    """tensors: sequence of (name, float32 array).  awq: name -> per-column s_j.

    Returns one dict per tensor: kind, and codes/scales (int kinds), f16 (passthrough),
    awq (binary16 multipliers, AWQ tensors), dq (float32, the value the export decodes
    to), status."""
    out = []
    for name, w in tensors:
        w = np.asarray(w, dtype=np.float32)
        kind = tensor_kind(name, w.size, pol)
        rec = dict(name=name, kind=kind, shape=w.shape)
        if kind == KIND_F16:
            h, st = lib.f16_passthrough(w.reshape(-1))
            rec.update(f16=h, dq=lib.f16_to_f32(h).reshape(w.shape), status=st)
        else:
            rows, cols = as_rows(w.shape)
            Q, num, den = _qparams(kind, pol)
            a = None
            st = 0
            s = None if awq is None else awq.get(name)
            if s is not None and kind == KIND_INT6:
                a, st = lib.awq_multipliers(s)
                rec["awq"] = a
            if pol.per_tensor:
                if a is not None:
                    raise ValueError("AWQ and per-tensor scales do not combine")
                r = lib.quantize_tensor(w.reshape(rows, cols), Q, num, den)
                r["scales"] = r["scale"]
            else:
                r = lib.quantize_rows(w.reshape(rows, cols), Q, num, den, awq=a)
            rec.update(codes=r["codes"], scales=r["scales"], dq=r["dq"].reshape(w.shape),
                       status=st | r["status"])
            if pol.pack6 and kind == KIND_INT6:
                rec["packed"] = lib.pack6(r["codes"])
        out.append(rec)
    return out


def qdq_tensor(name: str, w: np.ndarray, pol: Policy) -> np.ndarray:
    """The value a tensor decodes to after one export: fp16 round trip or per-row QDQ."""
    return export([(name, w)], pol)[0]["dq"]


def sqwa_run(snapshots, pol: Policy, k0: int = 1, means: Optional[List[np.ndarray]] = None):
    """Fold snapshots k0, k0+1, ... (each a list of (name, array)) into running means.

    Returns the list of float32 means (one per tensor).  `means` resumes a run."""
    k = k0
    for snap in snapshots:
        if means is None:
            means = [np.empty(np.asarray(w).shape, dtype=np.float32) for _, w in snap]
        for i, (name, w) in enumerate(snap):
            xhat = qdq_tensor(name, np.asarray(w, dtype=np.float32), pol)
            lib.sqwa_update(means[i], xhat, k)
        k += 1
    return means


def ema_run(steps, decay: float, states: Optional[List[np.ndarray]] = None):
    """EMA over a sequence of weight sets (each a list of arrays, one per tensor).  With no
    `states` the first set initialises the averages.  Returns (float32 states, status OR)."""
    st = 0
    for ws in steps:
        init = states is None
        if init:
            states = [np.empty(np.asarray(w).shape, dtype=np.float32) for w in ws]
        for e, w in zip(states, ws):
            st |= lib.ema_update(e, np.asarray(w, dtype=np.float32), decay, init)
    return states, st


def swa_run(checkpoints, k0: int = 1, means: Optional[List[np.ndarray]] = None):
    """SWA running means over checkpoints k0, k0+1, ... (each a list of arrays).
    Returns (float32 means, status OR); `means` resumes a run."""
    st = 0
    k = k0
    for ws in checkpoints:
        if means is None:
            means = [np.empty(np.asarray(w).shape, dtype=np.float32) for w in ws]
        for m, w in zip(means, ws):
            st |= lib.swa_update(m, np.asarray(w, dtype=np.float32), k)
        k += 1
    return means, st
