"""Throughput of the per-row weight quantizer on one MI355X.

Default step (--mode export) = one whole-model export of the 9-layer d=512 GPT weight set (21,767,168 fp32
parameters in 73 tensors): int6 per-row codes with the clip at the 99.99th percentile of
|w| per row, int8 absmax for tok_emb.weight, fp16 passthrough for the 18 vectors, fp16
row scales and the fp32 dequantized weights.  That is every step of the path in one
grouped launch (load, clip, scale, round, clamp, dequant, export dispatch).

Inputs are seeded synthetic N(0, 0.02^2) weights, resident in HBM before timing.  Several
independent copies of the inputs and outputs are used in rotation, so that no step finds
its data in the 256 MiB Infinity Cache.  `value` comes from K plain steps; the roofline's
kernel time from K further steps whose launches each carry dispatch timing events.  Prints
one JSON line.  --mode selects the other
workloads of the path (AWQ export, a 128-matrix batch, a percentile-select stress set, the STE
forward + backward step, a whole SQWA run, and the EMA / SWA weight-averaging updates), each
reported the same way.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "quantizer GB/s (bytes in+out) and % of MI355X HBM peak, int6 per-row"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0          # dense bf16 matrix-core peak of the MI355X
KERNEL_SOURCES = ["int6_weight_export_amd/csrc/pgq_kernels.hip", "int6_weight_export_amd/csrc/pgq_api.hip",
                  "int6_weight_export_amd/csrc/pgq_desc.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_export_gpt9.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def algorithmic_bytes(tensors, want_dq: bool, per_tensor: bool = False) -> dict:
    """Bytes each launch must move at least once: inputs read, outputs written."""
    import oracle

    pol = oracle.Policy(per_tensor=per_tensor)
    b_in = b_codes = b_scales = b_f16 = b_dq = 0
    rows_total = 0
    for t in tensors:
        kind = oracle.tensor_kind(t.name, t.numel, pol)
        rows, cols = oracle.as_rows(t.shape)
        b_in += 4 * t.numel
        if kind == oracle.KIND_F16:
            b_f16 += 2 * t.numel
        else:
            b_codes += t.numel
            b_scales += 2 * (1 if per_tensor else rows)
            rows_total += rows
        if want_dq:
            b_dq += 4 * t.numel
    total = b_in + b_codes + b_scales + b_f16 + b_dq
    return dict(total=total, read=b_in, write=total - b_in, rows=rows_total)


def cpu_baseline(tensors, min_seconds: float = 10.0, max_passes: int = 30) -> dict:
    """The oracle (single-threaded C) on the same weight set, whole export passes."""
    import oracle

    pol = oracle.Policy()
    data = [(t.name, t.data) for t in tensors]
    nbytes = algorithmic_bytes(tensors, want_dq=True)["total"]
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.export(data, pol)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or passes >= max_passes:
            break
    return {"value": round(nbytes * passes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} full export pass(es) of the same 9-layer weight set with fp32 dequant "
                      f"({el:.1f} s, single thread)"}


class Workload:
    """One bench workload: `step(i)` enqueues one step on input set i % copies."""

    def __init__(self, name, desc, nbytes, rows, step, statuses, config, kernel, launches=1, timed_calls=(),
                 flops=None):
        self.name, self.desc, self.nbytes, self.rows = name, desc, nbytes, rows
        self.step, self.statuses, self.config, self.kernel = step, statuses, config, kernel
        self.launches, self.timed_calls = launches, list(timed_calls)   # library calls per step
        self.flops = flops                       # a contraction: roofline against the MFMA peak


def _dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _bf16_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def workload_export(copies, torch, ops):
    tensors = synth.config2()
    ab = algorithmic_bytes(tensors, want_dq=True)
    sets = []
    for _ in range(copies):
        ex = ops.Exporter([ops.ExportTensor(t.name, _dev(t.data, torch)) for t in tensors], want_dq=True)
        ex.run()                                  # uploads the descriptor table once
        sets.append(ex)
    cfg = {"workload": "whole-model export of the 9-layer d=512 GPT weight set: int6 per-row codes with "
                       "99.99th-percentile clip, int8 tok_emb.weight, fp16 passthrough vectors, fp16 row "
                       "scales, fp32 dequantized weights",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    return Workload("export", cfg["workload"], ab["total"], ab["rows"], lambda i: sets[i % len(sets)].run(),
                    lambda: [int(s.status.item()) for s in sets], cfg, "pgq_table_kernel<0, 5u>"), tensors


def workload_awq(copies, torch, ops):
    tensors = synth.config4()
    pol = ops.make_policy(q_default=(6, 1, 1))
    nbytes = rows = 0
    for t in tensors:
        r, c = t.shape
        nbytes += 9 * t.numel + 2 * r
        rows += r
        if t.awq_s is not None:
            nbytes += 4 * c + 2 * c               # activation scales in, fp16 multipliers out
    sets = []
    for _ in range(copies):
        ex = ops.Exporter([ops.ExportTensor(t.name, _dev(t.data, torch), None if t.awq_s is None else _dev(t.awq_s, torch))
                           for t in tensors], pol, want_dq=True)
        ex.run()
        sets.append(ex)
    cfg = {"workload": "mixed-bit AWQ export of the 12-layer d=512 vocab-1792 GPT weight set: int6 per-row "
                       "absmax on w * fp16(sqrt(s_j)), int8 tok_emb/lm_head, fp16 scales and multipliers, fp32 "
                       "dequant", "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    return Workload("awq", cfg["workload"], nbytes, rows, lambda i: sets[i % len(sets)].run(),
                    lambda: [int(s.status.item()) for s in sets], cfg, "pgq_table_kernel<0, 13u>"), None


def workload_batch(copies, torch, ops):
    mats = synth.config1_batch(128)
    pol = ops.make_policy(int8_patterns=(), passthrough_below=0, q_default=(6, 1, 1))
    sets = []
    for _ in range(max(2, copies // 3)):
        ex = ops.Exporter([ops.ExportTensor(m.name, _dev(m.data, torch)) for m in mats], pol, want_dq=True)
        ex.run()
        sets.append(ex)
    nbytes = 128 * (1536 * 512 * 9 + 1536 * 2)
    cfg = {"workload": "128 independent 1536x512 fp32 matrices, int6 per-row absmax, codes + fp16 scales + fp32 "
                       "dequant, one grouped launch", "tensors": 128, "params": 128 * 1536 * 512}
    return Workload("batch", cfg["workload"], nbytes, 128 * 1536, lambda i: sets[i % len(sets)].run(),
                    lambda: [int(s.status.item()) for s in sets], cfg, "pgq_table_kernel<0, 5u>"), None


def workload_select(copies, torch, ops):
    tensors = synth.stress_s1()
    ab = algorithmic_bytes(tensors, want_dq=True)
    pol = ops.make_policy(q_default=(6, 99, 100))
    sets = []
    for _ in range(copies):
        ex = ops.Exporter([ops.ExportTensor(t.name, _dev(t.data, torch)) for t in tensors], pol, want_dq=True)
        ex.run()
        sets.append(ex)
    cfg = {"workload": "export of heavy-tailed (0.02 * Student-t(3)) 9-layer d=512 weights with the clip at the "
                       "99th percentile per row (exact select), int8 tok_emb, fp16 vectors, fp32 dequant",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    return Workload("select", cfg["workload"], ab["total"], ab["rows"], lambda i: sets[i % len(sets)].run(),
                    lambda: [int(s.status.item()) for s in sets], cfg, "pgq_table_kernel<0, 21u>"), None


def workload_fakequant(copies, torch, ops, pgq):
    ws = synth.config3_weights()
    nbytes = rows = 0
    for t in ws:
        r, c = t.shape
        nbytes += 8 * t.numel + r * ((c + 7) // 8) + 2 * r
        rows += r
    sets = []
    for k in range(copies):
        fq = ops.FakeQuant([_bf16_dev(t.data, torch) for t in ws])
        grads = [_bf16_dev(g.data, torch) for g in synth.config3_grads(k)]
        fq.run(pgq.PGQ_FQ_FWD_BWD, grads)
        sets.append((fq, grads))
    cfg = {"workload": "STE fake-quant forward + backward of the 11-layer d=528 model (unified QKV 1584x528, Wo "
                       "528x528, MLP 1584x528 / 528x1584, bf16), int6 absmax: bf16 dequant, fp16 scales, mask bits, "
                       "masked bf16 gradients; a fresh gradient set per step in rotation",
           "tensors": len(ws), "params": int(sum(t.numel for t in ws))}
    return Workload("fakequant", cfg["workload"], nbytes, rows,
                    lambda i: sets[i % len(sets)][0].run(pgq.PGQ_FQ_FWD_BWD, sets[i % len(sets)][1]),
                    lambda: [int(s[0].status.item()) for s in sets], cfg, "pgq_table_kernel<2, 2u>"), None


def workload_sqwa(copies, torch, ops):
    base = synth.config5_base()
    snaps = [[_dev(t.data, torch) for t in synth.config5_snapshot(k, base)] for k in range(1, 17)]
    sq = ops.Sqwa([ops.ExportTensor(t.name, s) for t, s in zip(base, snaps[0])], ops.make_policy(int8_patterns=()))
    for k in range(1, 17):
        sq.accumulate(snaps[k - 1], k)
    ex = sq.exporter(want_dq=False)
    ex.run()
    numel = sum(t.numel for t in base)
    nvec = sum(t.numel for t in base if t.numel < 65536)
    rows = sum(t.shape[0] for t in base if t.numel >= 65536)
    nbytes = 8 * numel + 15 * 12 * numel + (4 * numel + (numel - nvec) + 2 * rows + 2 * nvec)

    def step(i):
        for k in range(1, 17):
            sq.accumulate(snaps[k - 1], k)
        ex.run()

    cfg = {"workload": "SQWA over 16 snapshots of the 9-layer d=512 weight set (snapshot k = base + N(0, "
                       "(0.002k)^2)): int6 99.99th-percentile QDQ of every matrix, fp16 round trip of vectors, "
                       "fp32 running mean, then int6 codes + scales of the mean; 17 launches per step",
           "tensors": len(base), "params": int(numel), "snapshots": 16}
    return Workload("sqwa", cfg["workload"], nbytes, 17 * rows, step,
                    lambda: [int(sq.status.item()), int(ex.status.item())], cfg, "pgq_table_kernel<1, 5u>",
                    launches=17, timed_calls=[(ops.Sqwa, "accumulate"), (ops.Exporter, "run")]), None


def algorithmic_bytes_pack6(tensors) -> int:
    """Export with 6-bit int6 codes: as algorithmic_bytes, with 3/4 byte per int6 code."""
    import oracle

    pol = oracle.Policy(pack6=True)
    total = algorithmic_bytes(tensors, want_dq=True)["total"]
    for t in tensors:
        if oracle.tensor_kind(t.name, t.numel, pol) == oracle.KIND_INT6:
            rows, cols = oracle.as_rows(t.shape)
            total += rows * 3 * ((cols + 3) // 4) - t.numel
    return total


def workload_pack6(copies, torch, ops):
    """The whole-model export with int6 codes stored four per three bytes."""
    tensors = synth.config2()
    sets = []
    for _ in range(copies):
        ex = ops.Exporter([ops.ExportTensor(t.name, _dev(t.data, torch)) for t in tensors],
                          ops.make_policy(pack6=True), want_dq=True)
        ex.run()
        sets.append(ex)
    cfg = {"workload": "whole-model export of the 9-layer d=512 GPT weight set with int6 codes stored four per "
                       "three bytes (99.99th-percentile clip), int8 tok_emb.weight, fp16 vectors, fp32 dequant",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    rows = algorithmic_bytes(tensors, want_dq=True)["rows"]
    return Workload("pack6", cfg["workload"], algorithmic_bytes_pack6(tensors), rows,
                    lambda i: sets[i % len(sets)].run(), lambda: [int(s.status.item()) for s in sets], cfg,
                    "pgq_table_kernel<7, 5u>"), tensors


def workload_decode(copies, torch, ops):
    """Decode of the exported 9-layer artifact (6-bit int6 codes, int8 tok_emb, fp16 row scales,
    fp16 vectors) back to fp32 weights: one grouped pgq_dequant_model launch per step."""
    tensors = synth.config2()
    sets = []
    for _ in range(copies):
        ex = ops.Exporter([ops.ExportTensor(t.name, _dev(t.data, torch)) for t in tensors],
                          ops.make_policy(pack6=True), want_dq=False)
        ex.run()
        outs = ex.decode()
        sets.append((ex, outs))
    import oracle

    pol = oracle.Policy(pack6=True)
    nbytes = rows = 0
    for t in tensors:
        r, c = oracle.as_rows(t.shape)
        kind = oracle.tensor_kind(t.name, t.numel, pol)
        nbytes += 4 * t.numel
        if kind == oracle.KIND_F16:
            nbytes += 2 * t.numel
        else:
            nbytes += (r * 3 * ((c + 3) // 4) if kind == oracle.KIND_INT6 else t.numel) + 2 * r
            rows += r
    cfg = {"workload": "decode of the exported 9-layer d=512 artifact (int6 codes four per three bytes, int8 "
                       "tok_emb.weight, fp16 row scales, fp16 vectors) to fp32 weights, one launch",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    return Workload("decode", cfg["workload"], nbytes, rows, lambda i: sets[i % len(sets)][0].decode(sets[i % len(sets)][1]),
                    lambda: [int(s[0].status.item()) for s in sets], cfg, "pgq_table_kernel<8, 1u>"), None


def workload_qgemm(copies, torch, ops):
    """The QAT forward's consumer GEMM with the STE dequantization fused in: 16384 tokens through
    the d=528 unified Q/K/V projection (What 1584 x 528 from int8 codes + fp16 row scales),
    bf16 MFMA with fp32 accumulation."""
    import oracle

    M, N, K = 16384, 1584, 528
    rng = np.random.default_rng(0)
    w = oracle.f32_to_bf16((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    fq = oracle.fakequant_rows(w, 31)
    codes = torch.from_numpy(fq["codes"]).cuda()
    scales = torch.from_numpy(fq["scales"].view(np.int16)).cuda()
    sets = []
    for k in range(copies):
        x = torch.randn(M, K, generator=torch.Generator().manual_seed(k)).to(torch.bfloat16).cuda()
        sets.append((x, torch.empty(M, N, dtype=torch.float32, device="cuda")))
    nbytes = 2 * M * K + N * K + 2 * N + 4 * M * N
    cfg = {"workload": "fused-dequant GEMM of the QAT forward: Y[16384 x 1584] = X[16384 x 528] (bf16) times "
                       "bf16(code * s)^T from int8 codes and fp16 row scales, fp32 accumulation on MFMA",
           "M": M, "N": N, "K": K}
    return Workload("qgemm", cfg["workload"], nbytes, M,
                    lambda i: ops.qgemm(sets[i % len(sets)][0], codes, scales, out=sets[i % len(sets)][1]),
                    lambda: [0], cfg, "pgq_qgemm_kernel", flops=2 * M * N * K), None


def workload_tensor(copies, torch, ops):
    """Per-tensor scales: the 9-layer export with one scale per integer tensor, the clip at the
    99.99th percentile of |w| over the whole tensor (int8 tok_emb: absmax).  A step is the
    call's five launches (four radix select passes, then the quantize pass)."""
    tensors = synth.config2()
    ab = algorithmic_bytes(tensors, want_dq=True, per_tensor=True)
    sets = []
    for _ in range(copies):
        ex = ops.Exporter([ops.ExportTensor(t.name, _dev(t.data, torch)) for t in tensors],
                          ops.make_policy(per_tensor=True), want_dq=True)
        ex.run()
        sets.append(ex)
    cfg = {"workload": "per-tensor export of the 9-layer d=512 GPT weight set: one fp16 scale per tensor, "
                       "int6 with the clip at the 99.99th percentile of |w| over the tensor (exact multi-"
                       "workgroup radix select), int8 absmax tok_emb.weight, fp16 vectors, fp32 dequant",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    return Workload("tensor", cfg["workload"], ab["total"], ab["rows"], lambda i: sets[i % len(sets)].run(),
                    lambda: [int(s.status.item()) for s in sets], cfg,
                    "pgq_table_kernel<6, 1u> x4 + pgq_table_kernel<0, 5u>"), tensors


def _workload_average(kind, copies, torch, ops):
    """One EMA update (decay 0.997) or one SWA checkpoint fold (k >= 2) of the 9-layer d=512 fp32
    weight set per step: read the weights and the fp32 average, write the average."""
    base = synth.config5_base()
    numel = sum(t.numel for t in base)
    rows = sum(t.shape[0] if len(t.shape) == 2 else 1 for t in base)
    sets = []
    for k in range(copies):
        ws = [_dev(t.data, torch) for t in synth.config5_snapshot(k + 1, base)]
        if kind == "ema":
            av = ops.Ema(ws, decay=0.997)
            av.update(ws, init=True)
        else:
            av = ops.Swa(ws)
            av.accumulate(ws, 1)
        sets.append((av, ws))
    if kind == "ema":
        step = lambda i: sets[i % copies][0].update(sets[i % copies][1])  # noqa: E731
        what = "EMA update (decay 0.997)"
        kernel = "pgq_table_kernel<4, 1u>"
    else:
        step = lambda i: sets[i % copies][0].accumulate(sets[i % copies][1], 2 + i % 15)  # noqa: E731
        what = "SWA checkpoint fold (running mean, k = 2..16)"
        kernel = "pgq_table_kernel<5, 1u>"
    cfg = {"workload": f"{what} of the 9-layer d=512 GPT weight set, fp32 weights and fp32 averages",
           "tensors": len(base), "params": int(numel)}
    return Workload(kind, cfg["workload"], 12 * numel, rows, step,
                    lambda: [int(s[0].status.item()) for s in sets], cfg, kernel), None


def workload_ema(copies, torch, ops):
    return _workload_average("ema", copies, torch, ops)


def workload_swa(copies, torch, ops):
    return _workload_average("swa", copies, torch, ops)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 1000; 50 for --mode sqwa)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 50; 3 for --mode sqwa)")
    ap.add_argument("--mode", default="export", choices=["export", "awq", "batch", "select", "fakequant", "sqwa", "ema", "swa", "tensor",
                                                    "pack6", "decode", "qgemm"],
                    help="export (default): the 9-layer whole-model export; the others time the remaining "
                         "rows of the path")
    ap.add_argument("--copies", type=int, default=6, help="input/output sets used in rotation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="N",
                    help="after the timed steps, run N plain device copies of 256 MiB (torch copy_) so "
                         "that hardware byte counters can be scaled against a copy of known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the quantizer is "
              f"row-parallel within a GPU and this build runs no collectives)", file=sys.stderr)
        return 2
    steps = args.steps if args.steps is not None else {"sqwa": 50}.get(args.mode, 1000)
    warmup = args.warmup if args.warmup is not None else (3 if args.mode == "sqwa" else 50)

    import torch

    from int6_weight_export_amd import ops, pgq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    make = {"export": workload_export, "awq": workload_awq, "batch": workload_batch, "select": workload_select,
            "ema": workload_ema, "swa": workload_swa, "tensor": workload_tensor, "pack6": workload_pack6,
            "decode": workload_decode, "qgemm": workload_qgemm,
            "sqwa": workload_sqwa}
    if args.mode == "fakequant":
        wl, tensors = workload_fakequant(args.copies, torch, ops, pgq)
    else:
        wl, tensors = make[args.mode](args.copies, torch, ops)
    torch.cuda.synchronize()
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()

    # Throughput: K plain steps, nothing but the library calls between the two synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Kernel time: K more steps in which every launch records its own start / stop events from
    # its dispatch (pgq_time_next_launch), so a pair times one kernel alone, on the stream it
    # runs on.  Recording them costs host time per launch, which is why the throughput steps
    # above run without them.
    launches = wl.launches
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps * launches)]
    for a, b in ev:                              # create the underlying HIP events
        a.record()
        b.record()
    handles = [(ctypes.c_void_p(a.cuda_event), ctypes.c_void_p(b.cuda_event)) for a, b in ev]
    torch.cuda.synchronize()
    if launches > 1:
        # every library call of a step gets its own event pair
        it = iter(handles)
        saved = [(obj, name, getattr(obj, name)) for obj, name in wl.timed_calls]

        def timed(fn):
            def call(*a, **k):
                pgq.pgq_time_next_launch(*next(it))
                return fn(*a, **k)
            return call
        for obj, name, fn in saved:
            setattr(obj, name, timed(fn))
        try:
            for i in range(steps):
                wl.step(i)
        finally:
            for obj, name, fn in saved:
                setattr(obj, name, fn)
    else:
        for i in range(steps):
            pgq.pgq_time_next_launch(*handles[i])
            wl.step(i)
    torch.cuda.synchronize()
    kern_ms = np.array([a.elapsed_time(b) for a, b in ev])
    status = wl.statuses()
    assert all(x == 0 for x in status), status

    ms_per_step = wall / steps * 1e3
    value = wl.nbytes / (wall / steps) / 1e9
    k_step_s = float(kern_ms.sum()) / steps / 1e3       # kernel time per step
    achieved = wl.nbytes / k_step_s / 1e9

    traffic = None
    if args.mode == "export" and os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256") == kernel_source_hash():
            traffic = tr.get("hbm_bytes_per_launch")

    config = dict(wl.config)
    config.update({"bytes_per_step": wl.nbytes, "rows_per_step": wl.rows, "input_copies_in_rotation":
                   (1 if args.mode == "sqwa" else args.copies if args.mode != "batch" else max(2, args.copies // 3))})
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.mode in ("fakequant", "qgemm") else "f32",
        "data": "synthetic",
        "config": config,
        "roofline": ({
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        } if wl.flops is None else {
            "bound": "mfma",
            "achieved": round(wl.flops / k_step_s / 1e12, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(wl.flops / k_step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
        }),
        "kernel": wl.kernel,
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernel_us_per_step": round(k_step_s * 1e6, 3),
        "kernel_us_p10_p90_per_launch": [round(float(np.percentile(kern_ms, 10)) * 1e3, 3),
                                         round(float(np.percentile(kern_ms, 90)) * 1e3, 3)],
        "rows_per_s": round(wl.rows / (wall / steps), 1),
    }
    if args.mode == "export" and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(tensors)
    if args.copy_calibration:
        n = (256 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.copy_calibration):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = {"read": 4 * n, "write": 4 * n, "launches": args.copy_calibration}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
