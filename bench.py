"""Throughput of the per-row weight quantizer on one MI355X.

Default step (--mode export) = one whole-model export of the 9-layer d=512 GPT weight set (21,767,168 fp32
parameters in 73 tensors): int6 per-row codes with the clip at the 99.99th percentile of
|w| per row, int8 absmax for tok_emb.weight, fp16 passthrough for the 18 vectors, fp16
row scales and the fp32 dequantized weights.  That is every step of the path in one
grouped launch (load, clip, scale, round, clamp, dequant, export dispatch).

Inputs are seeded synthetic weights, resident in HBM before timing.  Several independent
copies of the inputs and outputs are used in rotation, so that no step finds its data in the
256 MiB Infinity Cache.  `value` comes from K plain steps; the roofline's kernel time from K
further steps whose launches each carry dispatch timing events.  Algorithmic bytes are counted
from the library's own export plan (each tensor's kind and output regions).

The default run also times the other whole-workload configurations and reports them in the
`configs` field of the same JSON line: 128 independent 1536x512 matrices in one launch, the
STE forward + backward step of the 11-layer d=528 model, the mixed-bit AWQ export of the
12-layer vocab-1792 model, and one SQWA run over 16 snapshots.  --mode runs any single
workload (those, plus a percentile-select stress set, EMA / SWA updates, per-tensor scales,
6-bit code storage, the artifact decode and the fused-dequant GEMM) as the main line.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
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
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # 312.5
KERNEL_SOURCES = sorted(os.path.relpath(p, ROOT) for p in glob.glob(os.path.join(ROOT, "int6_weight_export_amd", "csrc", "*"))
                        if p.endswith((".hip", ".h")))
GEMM_SOURCE = os.path.join("int6_weight_export_amd", "csrc", "pgq_gemm.hip")
PROFILES = os.path.join(ROOT, "profiles")
HOST_WORKERS = 16                       # host threads for input generation and the CPU leg
CONFIG_MODES = ("batch", "fakequant", "awq", "sqwa")   # timed beside the export in the default run


def kernel_sources(mode: str) -> list:
    """The sources a mode's kernels are built from: the GEMM file for qgemm, every other kernel
    source for the rest (the host API, the shared descriptor and the header for both)."""
    if mode in ("qgemm", "qgemm16"):
        return [f for f in KERNEL_SOURCES if f == GEMM_SOURCE or f.endswith(("pgq_api.hip", "pgq_desc.h"))]
    return [f for f in KERNEL_SOURCES if f != GEMM_SOURCE]


def kernel_source_hash(mode: str = "export") -> str:
    h = hashlib.sha256()
    for f in kernel_sources(mode):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(mode: str):
    """HBM bytes per step (per launch, for the single-launch modes) from the committed counter
    summary of this mode, or None when there is none or the kernel sources changed since the
    counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{mode}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_source_sha256") != kernel_source_hash(mode):
        return None
    return tr.get("hbm_bytes_per_step")


# ---- counter summaries (no GPU needed) ------------------------------------------------------
# A profile directory holds three rocprofv3 runs of one `bench.py --mode M` command line:
#   trace/       --kernel-trace --stats        (log: trace.log)
#   FETCH_SIZE/  --pmc FETCH_SIZE, with --copy-calibration 6   (log: FETCH_SIZE.log)
#   WRITE_SIZE/  --pmc WRITE_SIZE, with --copy-calibration 6   (log: WRITE_SIZE.log)
# and commands.txt, one "pass: command" line per run.  The bench's launches are the last
# (warmup + 2 * steps) * dispatches_per_step dispatches of the library's kernels; the counter
# scale comes from the six 256 MiB device copies appended by --copy-calibration.
COPY_CAL_BYTES = 256 << 20


def _bench_line(log_path: str) -> dict:
    with open(log_path) as f:
        for ln in f:
            if ln.startswith('{"metric"'):
                return json.loads(ln)
    raise ValueError(f"no bench line in {log_path}")


def _csv_rows(path: str):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _step_dispatches(rows, line, key="Dispatch_Id"):
    lib = sorted((r for r in rows if "pgq_" in r["Kernel_Name"]), key=lambda r: int(r[key]))
    n = (line["warmup"] + 2 * line["steps"]) * line.get("dispatches_per_step", line["launches_per_step"])
    return lib[-n:], line["warmup"] + 2 * line["steps"]


def _short(name: str) -> str:
    name = name.replace("pgq::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def profile_summary(d: str) -> None:
    tl = _bench_line(os.path.join(d, "trace.log"))
    mode = tl["mode"]
    cmds = {}
    with open(os.path.join(d, "commands.txt")) as f:
        for ln in f:
            if ":" in ln:
                k, v = ln.split(":", 1)
                cmds[k.strip()] = v.strip()
    # kernel trace: durations of the step dispatches per kernel
    tr, nsteps = _step_dispatches(_csv_rows(os.path.join(d, "trace", "run_kernel_trace.csv")), tl)
    per = {}
    for r in tr:
        per.setdefault(_short(r["Kernel_Name"]), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    dom = max(per, key=lambda k: sum(per[k]))
    kern = {k: {"launches_per_step": round(len(v) / nsteps, 3), "mean_us": round(float(np.mean(v)), 3),
                "min_us": round(float(np.min(v)), 3), "max_us": round(float(np.max(v)), 3)} for k, v in per.items()}
    step_us = sum(float(np.mean(v)) * len(v) / nsteps for v in per.values())
    # counters: scale from the calibration copies, then bytes per step over the step dispatches
    res = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cl = _bench_line(os.path.join(d, f"{c}.log"))
        rows = _csv_rows(os.path.join(d, c, "run_counter_collection.csv"))
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        gmax = max(int(r["Grid_Size"]) for r in copies)
        cal = [float(r["Counter_Value"]) for r in copies if int(r["Grid_Size"]) == gmax]
        scale = COPY_CAL_BYTES / (float(np.mean(cal)) * 1024)
        sd, ns = _step_dispatches(rows, cl)
        by = {}
        for r in sd:
            by.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]) * 1024 * scale)
        res[c] = {"scale": scale, "cal_kib": float(np.mean(cal)), "per_step": sum(sum(v) for v in by.values()) / ns,
                  "per_kernel": {k: float(np.mean(v)) for k, v in by.items()}}
    for k in kern:
        kern[k]["fetch_bytes_per_launch"] = round(res["FETCH_SIZE"]["per_kernel"].get(k, 0.0))
        kern[k]["write_bytes_per_launch"] = round(res["WRITE_SIZE"]["per_kernel"].get(k, 0.0))
    alg = tl["config"]["bytes_per_step"]
    hbm = res["FETCH_SIZE"]["per_step"] + res["WRITE_SIZE"]["per_step"]
    out = {
        "mode": mode, "workload": tl["config"]["workload"], "dominant_kernel": dom,
        "kernel_source_sha256": kernel_source_hash(mode),
        "kernel_sources": kernel_sources(mode),
        "kernels": kern,
        "kernel_us_per_step": round(step_us, 3),
        "hbm_read_bytes_per_step": round(res["FETCH_SIZE"]["per_step"]),
        "hbm_write_bytes_per_step": round(res["WRITE_SIZE"]["per_step"]),
        "hbm_bytes_per_step": round(hbm),
        "algorithmic_bytes_per_step": alg,
        "traffic_over_algorithmic": round(hbm / alg, 4),
        "copy_calibration": {"bytes_per_copy": COPY_CAL_BYTES,
                             "fetch_kib": round(res["FETCH_SIZE"]["cal_kib"], 1),
                             "write_kib": round(res["WRITE_SIZE"]["cal_kib"], 1),
                             "fetch_scale": round(res["FETCH_SIZE"]["scale"], 4),
                             "write_scale": round(res["WRITE_SIZE"]["scale"], 4)},
        "commands": cmds,
    }
    with open(os.path.join(PROFILES, f"traffic_{mode}.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    md = [f"# {mode}: rocprofv3 kernel trace and HBM traffic", "",
          f"Workload: {tl['config']['workload']}.", "",
          "Commands (each a separate run; `<dir>` is the output directory):", "", "```"]
    md += [f"{k}: {v}" for k, v in cmds.items()]
    md += ["```", "",
           f"Step launches only: the last (warmup + 2 x steps) x {tl.get('dispatches_per_step', tl['launches_per_step'])} dispatches of the "
           "library's kernels.  Counter KiB are scaled by the readings of six 256 MiB device copies "
           f"(FETCH_SIZE x {res['FETCH_SIZE']['scale']:.4f}, WRITE_SIZE x {res['WRITE_SIZE']['scale']:.4f}).", "",
           "| kernel | launches / step | mean us | min us | max us | read B / launch | written B / launch |",
           "|---|---|---|---|---|---|---|"]
    for k, v in sorted(kern.items(), key=lambda kv: -kv[1]["mean_us"] * kv[1]["launches_per_step"]):
        md.append(f"| `{k}` | {v['launches_per_step']} | {v['mean_us']} | {v['min_us']} | {v['max_us']} | "
                  f"{v['fetch_bytes_per_launch']:,} | {v['write_bytes_per_launch']:,} |")
    md += ["", f"Kernel time per step {step_us:.3f} us.  HBM traffic per step {round(hbm):,} B "
           f"(read {round(res['FETCH_SIZE']['per_step']):,}, written {round(res['WRITE_SIZE']['per_step']):,}) "
           f"against {alg:,} algorithmic bytes: ratio {hbm / alg:.4f}.", "",
           f"Kernel sources ({', '.join(os.path.basename(f) for f in kernel_sources(mode))}) sha256: "
           f"`{kernel_source_hash(mode)}`.", ""]
    with open(os.path.join(PROFILES, f"{mode}_kernel_trace.md"), "w") as f:
        f.write("\n".join(md))
    print(json.dumps({"mode": mode, "kernel_us_per_step": round(step_us, 3), "traffic_over_algorithmic": round(hbm / alg, 4)}))


def plan_bytes(ex, want_dq: bool) -> dict:
    """Algorithmic bytes of one export launch, from the library's plan: every input read once,
    every output region written once."""
    from int6_weight_export_amd import pgq

    total = rows_total = 0
    for i, t in enumerate(ex.tensors):
        p = ex.plan[i]
        n = t.w.numel()
        rows = t.w.shape[0] if t.w.dim() >= 2 else 1
        cols = n // rows
        total += n * t.w.element_size()
        if p.kind == pgq.PGQ_KIND_F16:
            total += 2 * n
        else:
            total += rows * 3 * ((cols + 3) // 4) if p.packed else n
            total += 2 * (1 if p.per_tensor else rows)
            rows_total += rows
            if p.has_awq:
                total += 4 * cols + 2 * cols      # activation scales in, fp16 multipliers out
        if want_dq:
            total += 4 * n
    return dict(total=total, rows=rows_total)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(tensors, nbytes: int, min_seconds: float = 10.0, max_passes: int = 30) -> dict:
    """The oracle on the same weight set: whole export passes on one pinned core, then the same
    oracle functions on host threads over disjoint row ranges."""
    import threading
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    pol = oracle.Policy()
    data = [(t.name, t.data) for t in tensors]
    avail = sorted(os.sched_getaffinity(0))
    pinned = avail[-1]
    old = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {pinned})          # this thread only
    try:
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle.export(data, pol)
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or passes >= max_passes:
                break
    finally:
        os.sched_setaffinity(0, old)

    # threads over disjoint row ranges: per-row quantization of each range, fp16 passthrough of
    # each vector (the oracle's own functions; per-row results do not depend on other rows)
    threads = max(1, min(HOST_WORKERS, len(avail)))
    items = []
    for name, w in data:
        kind = oracle.tensor_kind(name, w.size, pol)
        if kind == oracle.KIND_F16:
            items.append((kind, w.reshape(-1), 0, 0))
            continue
        rows, cols = oracle.as_rows(w.shape)
        w2 = w.reshape(rows, cols)
        step = max(1, rows // (2 * threads))
        for r0 in range(0, rows, step):
            items.append((kind, w2, r0, min(rows, r0 + step)))

    def run(item):
        kind, w, r0, r1 = item
        if kind == oracle.KIND_F16:
            h, _ = oracle.f16_passthrough(w)
            oracle.f16_to_f32(h)
        else:
            bits, num, den = pol.q8 if kind == oracle.KIND_INT8 else pol.q6
            oracle.quantize_rows(w[r0:r1], (1 << (bits - 1)) - 1, num, den)

    oracle.f16_to_f32(np.zeros(1, dtype=np.uint16))    # build the decode table outside the timing
    lock = threading.Lock()
    with ThreadPoolExecutor(threads) as pool:
        passes_t, t0 = 0, time.perf_counter()
        while True:
            list(pool.map(run, items))
            passes_t += 1
            el_t = time.perf_counter() - t0
            if el_t >= min_seconds / 3 or passes_t >= max_passes:
                break
    del lock
    return {"value": round(nbytes * passes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} full export pass(es) of the same 9-layer weight set with fp32 dequant "
                      f"({el:.1f} s, one thread pinned to core {pinned})",
            "cpu": cpu_model(), "nproc": len(avail), "pinned_core": pinned,
            "threads_leg": {"value": round(nbytes * passes_t / el_t / 1e9, 4), "unit": "GB/s", "cores": threads,
                            "sample": f"{passes_t} pass(es) of the same export, the oracle's per-row quantizer "
                                      f"and fp16 passthrough on {threads} host threads over {len(items)} disjoint "
                                      f"row ranges ({el_t:.1f} s)"}}


class Workload:
    """One bench workload: `step(i)` enqueues one step on input set i % copies."""

    def __init__(self, name, nbytes, rows, step, statuses, config, kernel, launches=1, timed_calls=(),
                 flops=None, copies=1, tensors=None, dispatches=None):
        self.name, self.nbytes, self.rows = name, nbytes, rows
        self.step, self.statuses, self.config, self.kernel = step, statuses, config, kernel
        self.launches, self.timed_calls = launches, list(timed_calls)   # library calls per step
        self.dispatches = dispatches if dispatches is not None else launches   # kernel dispatches per step
        self.flops = flops                       # a contraction: flops per step
        self.copies = copies
        self.tensors = tensors                   # host weight set (for the CPU baseline)


def _dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _bf16_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def _exporters(tensors, copies, torch, ops, policy=None, want_dq=True, awq=False):
    sets = []
    for _ in range(copies):
        ex = ops.Exporter([ops.ExportTensor(t.name, _dev(t.data, torch),
                                            _dev(t.awq_s, torch) if (awq and t.awq_s is not None) else None)
                           for t in tensors], policy, want_dq=want_dq)
        ex.run()                                  # uploads the descriptor table once
        sets.append(ex)
    return sets


def _export_workload(name, sets, cfg, kernel, want_dq=True, tensors=None, dispatches=1):
    ab = plan_bytes(sets[0], want_dq)
    return Workload(name, ab["total"], ab["rows"], lambda i: sets[i % len(sets)].run(),
                    lambda: [int(s.status.item()) for s in sets], cfg, kernel, copies=len(sets), tensors=tensors,
                    dispatches=dispatches)


def workload_export(copies, torch, ops):
    tensors = synth.config2()
    cfg = {"workload": "whole-model export of the 9-layer d=512 GPT weight set: int6 per-row codes with "
                       "99.99th-percentile clip, int8 tok_emb.weight, fp16 passthrough vectors, fp16 row "
                       "scales, fp32 dequantized weights",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    return _export_workload("export", _exporters(tensors, copies, torch, ops), cfg, "pgq_table_kernel<0, 5u>",
                            tensors=tensors)


def workload_awq(copies, torch, ops):
    tensors = synth.config4()
    cfg = {"workload": "mixed-bit AWQ export of the 12-layer d=512 vocab-1792 GPT weight set: int6 per-row "
                       "absmax on w * fp16(sqrt(s_j)), int8 tok_emb/lm_head, fp16 scales and multipliers, fp32 "
                       "dequant", "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    sets = _exporters(tensors, copies, torch, ops, ops.make_policy(q_default=(6, 1, 1)), awq=True)
    return _export_workload("awq", sets, cfg, "pgq_table_kernel<0, 13u>")


def workload_batch(copies, torch, ops):
    mats = synth.config1_batch(128, workers=HOST_WORKERS)
    pol = ops.make_policy(int8_patterns=(), passthrough_below=0, q_default=(6, 1, 1))
    cfg = {"workload": "128 independent 1536x512 fp32 matrices, int6 per-row absmax, codes + fp16 scales + fp32 "
                       "dequant, one grouped launch", "tensors": 128, "params": 128 * 1536 * 512}
    return _export_workload("batch", _exporters(mats, max(2, copies // 3), torch, ops, pol), cfg,
                            "pgq_table_kernel<0, 5u>")


def workload_select(copies, torch, ops):
    tensors = synth.stress_s1()
    cfg = {"workload": "export of heavy-tailed (0.02 * Student-t(3)) 9-layer d=512 weights with the clip at the "
                       "99th percentile per row (exact select), int8 tok_emb, fp16 vectors, fp32 dequant",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    sets = _exporters(tensors, copies, torch, ops, ops.make_policy(q_default=(6, 99, 100)))
    return _export_workload("select", sets, cfg, "pgq_table_kernel<0, 21u>")


def workload_pack6(copies, torch, ops):
    """The whole-model export with int6 codes stored four per three bytes."""
    tensors = synth.config2()
    cfg = {"workload": "whole-model export of the 9-layer d=512 GPT weight set with int6 codes stored four per "
                       "three bytes (99.99th-percentile clip), int8 tok_emb.weight, fp16 vectors, fp32 dequant",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    sets = _exporters(tensors, copies, torch, ops, ops.make_policy(pack6=True))
    return _export_workload("pack6", sets, cfg, "pgq_table_kernel<7, 5u>")


def workload_tensor(copies, torch, ops):
    """Per-tensor scales: the 9-layer export with one scale per integer tensor, the clip at the
    99.99th percentile of |w| over the whole tensor (int8 tok_emb: absmax)."""
    tensors = synth.config2()
    cfg = {"workload": "per-tensor export of the 9-layer d=512 GPT weight set: one fp16 scale per tensor, "
                       "int6 with the clip at the 99.99th percentile of |w| over the tensor (exact: candidate "
                       "keys from one read of the tensor, one pick per tensor), int8 absmax tok_emb.weight, fp16 "
                       "vectors, fp32 dequant",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    sets = _exporters(tensors, copies, torch, ops, ops.make_policy(per_tensor=True))
    # one call = the candidate pass, the pick and the export (every clip here has rank <= 256)
    return _export_workload("tensor", sets, cfg, "pgq_table_kernel<9, 1u> + pgq_tensor_pick_kernel + "
                                                 "pgq_table_kernel<0, 5u>",
                            dispatches=3)


def workload_fakequant(copies, torch, ops):
    from int6_weight_export_amd import pgq

    ws = synth.config3_weights()
    nbytes = rows = 0
    for t in ws:
        r, c = t.shape
        nbytes += 8 * t.numel + r * ((c + 7) // 8) + 2 * r
        rows += r
    sets = []
    for k in range(copies):
        fq = ops.FakeQuant([_bf16_dev(t.data, torch) for t in ws])
        g = torch.Generator(device="cuda").manual_seed(1000 + k)
        grads = [(torch.randn(t.shape, generator=g, device="cuda") * 1e-4).to(torch.bfloat16) for t in ws]
        fq.run(pgq.PGQ_FQ_FWD_BWD, grads)
        sets.append((fq, grads))
    cfg = {"workload": "STE fake-quant forward + backward of the 11-layer d=528 model (unified QKV 1584x528, Wo "
                       "528x528, MLP 1584x528 / 528x1584, bf16), int6 absmax: bf16 dequant, fp16 scales, mask bits, "
                       "masked bf16 gradients; N(0, 1e-4^2) bf16 gradient sets in rotation",
           "tensors": len(ws), "params": int(sum(t.numel for t in ws))}
    return Workload("fakequant", nbytes, rows,
                    lambda i: sets[i % len(sets)][0].run(pgq.PGQ_FQ_FWD_BWD, sets[i % len(sets)][1]),
                    lambda: [int(s[0].status.item()) for s in sets], cfg, "pgq_table_kernel<2, 2u>", copies=copies)


def workload_sqwa(copies, torch, ops):
    base = synth.config5_base()
    snaps = [[_dev(t.data, torch) for t in s] for s in synth.config5_snapshots(range(1, 17), base, workers=HOST_WORKERS)]
    sq = ops.Sqwa([ops.ExportTensor(t.name, s) for t, s in zip(base, snaps[0])], ops.make_policy(int8_patterns=()))
    for k in range(1, 17):
        sq.accumulate(snaps[k - 1], k)
    ex = sq.exporter(want_dq=False)
    ex.run()
    # the snapshot fold of k > 1 reads the snapshot and the mean and writes the mean; k = 1 writes only
    numel = sum(t.numel for t in base)
    fold = 8 * numel + 15 * 12 * numel
    final = plan_bytes(ex, want_dq=False)
    nbytes = fold + final["total"]

    def step(i):
        for k in range(1, 17):
            sq.accumulate(snaps[k - 1], k)
        ex.run()

    cfg = {"workload": "SQWA over 16 snapshots of the 9-layer d=512 weight set (snapshot k = base + N(0, "
                       "(0.002k)^2)): int6 99.99th-percentile QDQ of every matrix, fp16 round trip of vectors, "
                       "fp32 running mean, then int6 codes + scales of the mean; 17 launches per step",
           "tensors": len(base), "params": int(numel), "snapshots": 16}
    return Workload("sqwa", nbytes, 17 * final["rows"], step,
                    lambda: [int(sq.status.item()), int(ex.status.item())], cfg, "pgq_table_kernel<1, 5u>",
                    launches=17, timed_calls=[(ops.Sqwa, "accumulate"), (ops.Exporter, "run")])


def workload_decode(copies, torch, ops):
    """Decode of the exported 9-layer artifact (6-bit int6 codes, int8 tok_emb, fp16 row scales,
    fp16 vectors) back to fp32 weights: one grouped pgq_dequant_model launch per step."""
    from int6_weight_export_amd import pgq

    tensors = synth.config2()
    sets = []
    for ex in _exporters(tensors, copies, torch, ops, ops.make_policy(pack6=True), want_dq=False):
        sets.append((ex, ex.decode()))
    ex = sets[0][0]
    nbytes = rows = 0
    for i, t in enumerate(ex.tensors):
        p = ex.plan[i]
        n = t.w.numel()
        r = t.w.shape[0] if t.w.dim() >= 2 else 1
        c = n // r
        nbytes += 4 * n
        if p.kind == pgq.PGQ_KIND_F16:
            nbytes += 2 * n
        else:
            nbytes += (r * 3 * ((c + 3) // 4) if p.packed else n) + 2 * r
            rows += r
    cfg = {"workload": "decode of the exported 9-layer d=512 artifact (int6 codes four per three bytes, int8 "
                       "tok_emb.weight, fp16 row scales, fp16 vectors) to fp32 weights, one launch",
           "tensors": len(tensors), "params": int(sum(t.numel for t in tensors))}
    return Workload("decode", nbytes, rows, lambda i: sets[i % len(sets)][0].decode(sets[i % len(sets)][1]),
                    lambda: [int(s[0].status.item()) for s in sets], cfg, "pgq_table_kernel<8, 1u>", copies=copies)


def _workload_qgemm(copies, torch, ops, ybf16):
    """The QAT forward's consumer GEMM with the STE dequantization fused in: 16384 tokens through
    the d=528 unified Q/K/V projection (What 1584 x 528 from int8 codes + fp16 row scales, both
    from the library's own fake-quant forward), bf16 MFMA with fp32 accumulation; Y fp32, or bf16
    (the QAT forward's activation type) with ybf16."""
    from int6_weight_export_amd import pgq

    M, N, K = 16384, 1584, 528
    g = torch.Generator(device="cuda").manual_seed(0)
    w = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    fq = ops.FakeQuant([w], want_codes=True)
    fq.run(pgq.PGQ_FQ_FWD)
    codes, scales = fq.codes[0], fq.scales[0]
    ydt = torch.bfloat16 if ybf16 else torch.float32
    sets = []
    for k in range(copies):
        gk = torch.Generator(device="cuda").manual_seed(1 + k)
        x = torch.randn(M, K, generator=gk, device="cuda").to(torch.bfloat16)
        sets.append((x, torch.empty(M, N, dtype=ydt, device="cuda")))
    ysz = 2 if ybf16 else 4
    nbytes = 2 * M * K + N * K + 2 * N + ysz * M * N
    cfg = {"workload": "fused-dequant GEMM of the QAT forward: Y[16384 x 1584] = X[16384 x 528] (bf16) times "
                       "bf16(code * s)^T from int8 codes and fp16 row scales, fp32 accumulation on MFMA, "
                       + ("bf16 Y (round to nearest even of the fp32 result)" if ybf16 else "fp32 Y"),
           "M": M, "N": N, "K": K}
    return Workload("qgemm16" if ybf16 else "qgemm", nbytes, M,
                    lambda i: ops.qgemm(sets[i % len(sets)][0], codes, scales, out=sets[i % len(sets)][1],
                                        out_dtype=ydt),
                    lambda: [int(fq.status.item())], cfg,
                    "pgq_qgemm_kernel<unsigned short>" if ybf16 else "pgq_qgemm_kernel<float>",
                    flops=2 * M * N * K, copies=copies)


def workload_qgemm(copies, torch, ops):
    return _workload_qgemm(copies, torch, ops, False)


def workload_qgemm16(copies, torch, ops):
    return _workload_qgemm(copies, torch, ops, True)


def _workload_average(kind, copies, torch, ops):
    """One EMA update (decay 0.997) or one SWA checkpoint fold (k >= 2) of the 9-layer d=512 fp32
    weight set per step: read the weights and the fp32 average, write the average."""
    base = synth.config5_base()
    numel = sum(t.numel for t in base)
    rows = sum(t.shape[0] if len(t.shape) == 2 else 1 for t in base)
    sets = []
    for snap in synth.config5_snapshots(range(1, copies + 1), base, workers=HOST_WORKERS):
        ws = [_dev(t.data, torch) for t in snap]
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
    return Workload(kind, 12 * numel, rows, step, lambda: [int(s[0].status.item()) for s in sets], cfg, kernel,
                    copies=copies)


def workload_ema(copies, torch, ops):
    return _workload_average("ema", copies, torch, ops)


def workload_swa(copies, torch, ops):
    return _workload_average("swa", copies, torch, ops)


MAKERS = {"export": workload_export, "awq": workload_awq, "batch": workload_batch, "select": workload_select,
          "fakequant": workload_fakequant, "sqwa": workload_sqwa, "ema": workload_ema, "swa": workload_swa,
          "tensor": workload_tensor, "pack6": workload_pack6, "decode": workload_decode, "qgemm": workload_qgemm,
          "qgemm16": workload_qgemm16}
DEFAULT_STEPS = {"sqwa": 50}
DEFAULT_WARMUP = {"sqwa": 3}
CONFIG_STEPS = {"batch": 50, "fakequant": 100, "awq": 100, "sqwa": 5}     # steps of each `configs` entry


def measure(wl, steps: int, warmup: int, torch) -> dict:
    """Wall-clock throughput over `steps` plain steps, then kernel time per step from `steps`
    further steps whose library calls record dispatch events."""
    from int6_weight_export_amd import pgq

    torch.cuda.synchronize()
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()

    # Throughput: K plain steps, nothing but the library calls between the two synchronisations.
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Kernel time: every launch records its own start / stop events from its dispatch
    # (pgq_time_next_launch), so a pair times the call's kernels alone, on the stream they run on.
    # Recording them costs host time per launch, which is why the throughput steps run without.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps * wl.launches)]
    for a, b in ev:                              # create the underlying HIP events
        a.record()
        b.record()
    handles = [(ctypes.c_void_p(a.cuda_event), ctypes.c_void_p(b.cuda_event)) for a, b in ev]
    torch.cuda.synchronize()
    if wl.launches > 1:
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
    k_step_s = float(kern_ms.sum()) / steps / 1e3
    return dict(wall=wall, steps=steps, k_step_s=k_step_s, kern_ms=kern_ms)


def roofline(wl, m) -> dict:
    """The dominant kernel against its bound: HBM unless a contraction's arithmetic intensity
    exceeds the bf16 MFMA ridge point (peak flops / peak bandwidth)."""
    achieved_gbs = wl.nbytes / m["k_step_s"] / 1e9
    traffic = traffic_for(wl.name)
    if wl.flops is None:
        return {"bound": "hbm", "achieved": round(achieved_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    ai = wl.flops / wl.nbytes
    tflops = wl.flops / m["k_step_s"] / 1e12
    extra = {"flop_per_byte": round(ai, 1), "ridge_flop_per_byte": round(RIDGE_FLOP_PER_BYTE, 1),
             "tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    if ai < RIDGE_FLOP_PER_BYTE:
        return {"bound": "hbm", "achieved": round(achieved_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, **extra}
    return {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic, **extra}


def config_entry(wl, m) -> dict:
    rf = roofline(wl, m)
    return {"workload": wl.config["workload"], "bytes_per_step": wl.nbytes, "steps": m["steps"],
            "value": round(wl.nbytes / (m["wall"] / m["steps"]) / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(m["wall"] / m["steps"] * 1e3, 5), "kernel": wl.kernel,
            "kernel_us_per_step": round(m["k_step_s"] * 1e6, 3), "launches_per_step": wl.launches,
            "frac": rf["frac"], "achieved": rf["achieved"], "traffic": rf["traffic"]}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 1000; 50 for --mode sqwa)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 50; 3 for --mode sqwa)")
    ap.add_argument("--mode", default="export", choices=sorted(MAKERS),
                    help="export (default): the 9-layer whole-model export; the others time the remaining "
                         "rows of the path")
    ap.add_argument("--copies", type=int, default=6, help="input/output sets used in rotation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other whole-workload configurations of the default run")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="N",
                    help="after the timed steps, run N plain device copies of 256 MiB (torch copy_) so "
                         "that hardware byte counters can be scaled against a copy of known size")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="write profiles/traffic_<mode>.json and profiles/<mode>_kernel_trace.md from the "
                         "rocprofv3 runs in DIR (no GPU needed) and exit")
    args = ap.parse_args()
    if args.profile_summary:
        profile_summary(args.profile_summary)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the quantizer is "
              f"row-parallel within a GPU; sharding over GPUs is not implemented)", file=sys.stderr)
        return 2
    steps = args.steps if args.steps is not None else DEFAULT_STEPS.get(args.mode, 1000)
    warmup = args.warmup if args.warmup is not None else DEFAULT_WARMUP.get(args.mode, 50)

    import torch

    from int6_weight_export_amd import ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = MAKERS[args.mode](args.copies, torch, ops)
    m = measure(wl, steps, warmup, torch)
    wall, kern_ms = m["wall"], m["kern_ms"]

    config = dict(wl.config)
    config.update({"bytes_per_step": wl.nbytes, "rows_per_step": wl.rows, "input_copies_in_rotation": wl.copies})
    line = {
        "metric": METRIC,
        "value": round(wl.nbytes / (wall / steps) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.mode in ("fakequant", "qgemm", "qgemm16") else "f32",
        "data": "synthetic",
        "config": config,
        "roofline": roofline(wl, m),
        "kernel": wl.kernel,
        "mode": args.mode,
        "launches_per_step": wl.launches,
        "dispatches_per_step": wl.dispatches,
        "pct_of_hbm_peak": round(100 * wl.nbytes / (wall / steps) / 1e9 / HBM_PEAK_GBS, 2),
        "kernel_us_per_step": round(m["k_step_s"] * 1e6, 3),
        "kernel_us_p10_p90_per_launch": [round(float(np.percentile(kern_ms, 10)) * 1e3, 3),
                                         round(float(np.percentile(kern_ms, 90)) * 1e3, 3)],
        "rows_per_s": round(wl.rows / (wall / steps), 1),
    }
    host_tensors = wl.tensors
    main_bytes = wl.nbytes
    if args.copy_calibration:
        n = (256 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.copy_calibration):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = {"read": 4 * n, "write": 4 * n, "launches": args.copy_calibration}
        del src, dst
    if args.mode == "export" and not args.no_configs:
        del wl
        torch.cuda.empty_cache()
        cfgs = {}
        for name in CONFIG_MODES:
            w2 = MAKERS[name](args.copies, torch, ops)
            cfgs[name] = config_entry(w2, measure(w2, CONFIG_STEPS[name], 2, torch))
            del w2
            torch.cuda.empty_cache()
        line["configs"] = cfgs
    if args.mode == "export" and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(host_tensors, main_bytes)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
