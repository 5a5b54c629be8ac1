"""C-ABI checks that need no GPU: the library loads, exports every function include/pgq.h
declares, rejects bad arguments synchronously, and plans exports like the oracle's policy.
No call here reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pgq.h")

pgq = pytest.importorskip("int6_weight_export_amd.pgq")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(pgq_[a-z_0-9]+)\s*\(", txt, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 8, names
    lib = ctypes.CDLL(pgq.LIB_PATH)
    for nm in names:
        assert hasattr(lib, nm), nm
        assert nm in pgq.SIGNATURES, nm
    assert set(pgq.SIGNATURES) == set(names)


def test_version_and_status_strings():
    assert "gfx950" in pgq.pgq_version()
    for s in range(8):
        assert pgq.pgq_status_str(s)


FAKE = 0x10000      # a non-null, aligned address never dereferenced (validation fails or no launch)


def q(bits=6, num=1, den=1):
    return pgq.pgq_qparams(bits, num, den)


@pytest.mark.parametrize("args,want", [
    (dict(rows=-1), pgq.PGQ_ERR_SHAPE),
    (dict(ld=100, cols=200), pgq.PGQ_ERR_SHAPE),
    (dict(cols=0), pgq.PGQ_ERR_SHAPE),
    (dict(qp=q(9)), pgq.PGQ_ERR_PARAM),
    (dict(qp=q(1)), pgq.PGQ_ERR_PARAM),
    (dict(qp=q(6, 1, 0)), pgq.PGQ_ERR_PARAM),
    (dict(qp=q(6, 3, 2)), pgq.PGQ_ERR_PARAM),
    (dict(w_dtype=5), pgq.PGQ_ERR_DTYPE),
    (dict(dq=FAKE, dq_dtype=9), pgq.PGQ_ERR_DTYPE),
    (dict(dq=FAKE, dq_dtype=pgq.PGQ_F16), pgq.PGQ_ERR_DTYPE),     # fp16 is a weight type, not an output
    (dict(w_dtype=pgq.PGQ_F16, rows=0), pgq.PGQ_OK),                # fp16 weights pass validation
    (dict(w_dtype=pgq.PGQ_F16, w=FAKE + 1), pgq.PGQ_ERR_ALIGN),
    (dict(scales=None), pgq.PGQ_ERR_NULL),
    (dict(w=None), pgq.PGQ_ERR_NULL),
    (dict(awq_mult=FAKE), pgq.PGQ_ERR_NULL),
    (dict(w=FAKE + 2), pgq.PGQ_ERR_ALIGN),
    (dict(scales=FAKE + 1), pgq.PGQ_ERR_ALIGN),
])
def test_quantize_rows_argument_errors(args, want):
    a = dict(w=FAKE, w_dtype=pgq.PGQ_F32, rows=4, cols=200, ld=200, qp=q(), awq_s=None, awq_mult=None,
             codes=FAKE, scales=FAKE, dq=None, dq_dtype=pgq.PGQ_F32, dev_status=None, stream=None)
    a.update(args)
    if "ld" not in args:
        a["ld"] = a["cols"]
    assert pgq.pgq_quantize_rows(**a) == want


def test_fakequant_argument_errors():
    t = (pgq.pgq_fq_tensor * 1)()
    t[0] = pgq.pgq_fq_tensor(FAKE, 4, 16, 16, FAKE, FAKE, FAKE, 0, 0, 0)
    assert pgq.pgq_fakequant_fwd_bwd(0, t, 1, q(), None, 0, 0, None, None) == pgq.PGQ_ERR_PARAM
    assert pgq.pgq_fakequant_fwd_bwd(pgq.PGQ_FQ_FWD, t, -1, q(), None, 0, 0, None, None) == pgq.PGQ_ERR_SHAPE
    assert pgq.pgq_fakequant_fwd_bwd(pgq.PGQ_FQ_BWD, t, 1, q(), None, 0, 0, None, None) == pgq.PGQ_ERR_NULL
    assert pgq.pgq_fakequant_fwd_bwd(pgq.PGQ_FQ_FWD_BWD, t, 1, q(), None, 0, 0, None, None) == pgq.PGQ_ERR_NULL
    t[0].dq = 0
    assert pgq.pgq_fakequant_fwd_bwd(pgq.PGQ_FQ_FWD, t, 1, q(), None, 0, 0, None, None) == pgq.PGQ_ERR_NULL
    t[0].dq = FAKE
    t2 = (pgq.pgq_fq_tensor * 2)(t[0], t[0])
    assert pgq.pgq_fakequant_fwd_bwd(pgq.PGQ_FQ_FWD, t2, 2, q(), None, 0, 0, None, None) == pgq.PGQ_ERR_WORKSPACE
    need = ctypes.c_size_t(0)
    assert pgq.pgq_fakequant_workspace(t2, 2, ctypes.byref(need)) == pgq.PGQ_OK and need.value > 0
    assert pgq.pgq_fakequant_fwd_bwd(pgq.PGQ_FQ_FWD, t2, 2, q(), FAKE, 64, 0, None, None) == pgq.PGQ_ERR_WORKSPACE


def _tensor_array(ts, awq=False):
    arr = (pgq.pgq_tensor_in * len(ts))()
    keep = []
    for i, t in enumerate(ts):
        rows, cols = oracle.as_rows(t.shape)
        nm = t.name.encode()
        keep.append(nm)
        arr[i] = pgq.pgq_tensor_in(nm, FAKE, pgq.PGQ_F32, 0, rows, cols, cols,
                                   FAKE if (awq and t.awq_s is not None) else 0)
    return arr, keep


def _policy(patterns=oracle.DEFAULT_INT8_PATTERNS, below=65536, q6=(6, 9999, 10000), q8=(8, 1, 1)):
    pats = [p.encode() for p in patterns]
    parr = (ctypes.c_char_p * max(1, len(pats)))(*pats)
    pol = pgq.pgq_policy(ctypes.cast(parr, ctypes.POINTER(ctypes.c_char_p)), len(pats), 0, below,
                         pgq.pgq_qparams(*q6), pgq.pgq_qparams(*q8))
    return pol, (pats, parr)


@pytest.mark.parametrize("cfg", ["gpt9", "gpt12", "gpt9_all_int6"])
def test_export_plan_matches_oracle_policy(cfg):
    if cfg == "gpt12":
        ts = synth.config4()
        pol, keep = _policy(q6=(6, 1, 1))
        opol = oracle.Policy(q6=(6, 1, 1))
    elif cfg == "gpt9":
        ts = synth.config2()
        pol, keep = _policy()
        opol = oracle.Policy()
    else:
        ts = synth.config2()
        pol, keep = _policy(patterns=())
        opol = oracle.Policy(int8_patterns=())
    arr, k2 = _tensor_array(ts, awq=True)
    plan = (pgq.pgq_tensor_plan * len(ts))()
    ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pgq.pgq_export_plan(arr, len(ts), ctypes.byref(pol), plan, ctypes.byref(ab), ctypes.byref(wb)) == 0
    regions = []
    for i, t in enumerate(ts):
        kind = oracle.tensor_kind(t.name, t.numel, opol)
        p = plan[i]
        assert p.kind == kind, t.name
        rows, cols = oracle.as_rows(t.shape)
        if kind == oracle.KIND_F16:
            regions.append((p.f16_off, 2 * t.numel))
            assert p.codes_off == -1 and p.scales_off == -1
        else:
            want_q = opol.q8 if kind == oracle.KIND_INT8 else opol.q6
            assert (p.qp.bits, p.qp.pct_num, p.qp.pct_den) == want_q
            regions += [(p.codes_off, rows * cols), (p.scales_off, 2 * rows)]
            assert p.has_awq == int(t.awq_s is not None and kind == oracle.KIND_INT6)
            if p.has_awq:
                regions.append((p.awq_off, 2 * cols))
    # regions are 256-byte aligned, disjoint and inside the arena
    regions.sort()
    for (o1, n1), (o2, n2) in zip(regions, regions[1:]):
        assert o1 % 256 == 0 and o1 + n1 <= o2
    assert regions[-1][0] + regions[-1][1] <= ab.value
    assert wb.value > 0


def test_export_and_sqwa_argument_errors():
    ts = synth.config2()[:3]
    arr, keep = _tensor_array(ts)
    pol, k2 = _policy()
    plan = (pgq.pgq_tensor_plan * 3)()
    ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pgq.pgq_export_plan(arr, 3, ctypes.byref(pol), plan, ctypes.byref(ab), ctypes.byref(wb)) == 0
    assert pgq.pgq_export_plan(arr, 3, None, plan, ctypes.byref(ab), ctypes.byref(wb)) == pgq.PGQ_ERR_NULL
    bad, k3 = _policy(q6=(6, 2, 1))
    assert pgq.pgq_export_plan(arr, 3, ctypes.byref(bad), plan, ctypes.byref(ab),
                               ctypes.byref(wb)) == pgq.PGQ_ERR_PARAM
    assert pgq.pgq_export_model(arr, 3, plan, None, None, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_NULL
    assert pgq.pgq_export_model(arr, 3, plan, FAKE + 64, None, FAKE, wb.value, 0, None,
                                None) == pgq.PGQ_ERR_ALIGN
    assert pgq.pgq_export_model(arr, 3, plan, FAKE, None, FAKE, 64, 0, None, None) == pgq.PGQ_ERR_WORKSPACE
    assert pgq.pgq_export_model(arr, 3, plan, FAKE, None, None, 0, 0, None, None) == pgq.PGQ_ERR_WORKSPACE
    plan[0].kind = 5  # bits 5 without matching qparams
    assert pgq.pgq_export_model(arr, 3, plan, FAKE, None, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_PARAM
    means = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    assert pgq.pgq_sqwa_accumulate(arr, 3, plan, means, 0, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_PARAM
    arr[1].dtype = 4
    assert pgq.pgq_export_plan(arr, 3, ctypes.byref(pol), plan, ctypes.byref(ab),
                               ctypes.byref(wb)) == pgq.PGQ_ERR_DTYPE


def test_average_argument_errors():
    ts = synth.config2()[:4]
    arr, keep = _tensor_array(ts)
    wb = ctypes.c_size_t(0)
    assert pgq.pgq_average_workspace(arr, 4, ctypes.byref(wb)) == 0 and wb.value > 64
    assert pgq.pgq_average_workspace(arr, 4, None) == pgq.PGQ_ERR_NULL
    assert pgq.pgq_average_workspace(arr, -1, ctypes.byref(wb)) == pgq.PGQ_ERR_SHAPE
    st = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    ema, swa = pgq.pgq_ema_update, pgq.pgq_swa_accumulate
    assert ema(arr, 0, st, 0.997, 0, None, 0, 0, None, None) == pgq.PGQ_OK        # nothing to do
    for bad in (-0.5, 1.5, float("nan")):
        assert ema(arr, 4, st, bad, 0, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_PARAM
    assert ema(arr, 4, None, 0.997, 0, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_NULL
    assert ema(arr, -2, st, 0.997, 0, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_SHAPE
    assert ema(arr, 4, st, 0.997, 0, FAKE, 64, 0, None, None) == pgq.PGQ_ERR_WORKSPACE
    assert ema(arr, 4, st, 0.997, 0, FAKE + 4, wb.value, 0, None, None) == pgq.PGQ_ERR_ALIGN
    for k in (0, -1, (1 << 24) + 1):
        assert swa(arr, 4, st, k, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_PARAM
    assert swa(arr, 4, st, 2, FAKE, 64, 0, None, None) == pgq.PGQ_ERR_WORKSPACE
    st[2] = FAKE + 2                                                                # misaligned average
    assert swa(arr, 4, st, 2, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_ALIGN
    st[2] = None
    assert swa(arr, 4, st, 2, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_NULL
    st[2] = FAKE
    arr[1].awq_s = FAKE                                                             # no AWQ here
    assert ema(arr, 4, st, 0.997, 0, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_PARAM
    arr[1].awq_s = 0
    arr[3].dtype = 9
    assert swa(arr, 4, st, 2, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_DTYPE


def test_constants_match_the_header(tmp_path):
    """The binding's copies of the header's #defines (element types, kinds, flags, status bits)."""
    import subprocess
    names = [n for n in dir(pgq) if n.startswith(("PGQ_F", "PGQ_BF", "PGQ_KIND", "PGQ_TABLE", "PGQ_DEV_", "PGQ_FQ_"))
             and isinstance(getattr(pgq, n), int)]
    assert {"PGQ_F32", "PGQ_BF16", "PGQ_F16"} <= set(names)
    lines = ['#include <stdio.h>', f'#include "{HEADER}"', 'int main(void) {']
    lines += [f'printf("{n} %lld\\n", (long long)({n}));' for n in names]
    lines.append("return 0; }")
    src, exe = tmp_path / "consts.c", tmp_path / "consts"
    src.write_text("\n".join(lines))
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    for line in filter(None, out):
        n, v = line.split()
        assert getattr(pgq, n) == int(v), line


def test_struct_layouts_match_the_header(tmp_path):
    """ctypes mirrors of the header's structs have the C sizes and field offsets."""
    import subprocess
    structs = {"pgq_qparams": pgq.pgq_qparams, "pgq_fq_tensor": pgq.pgq_fq_tensor,
               "pgq_tensor_in": pgq.pgq_tensor_in, "pgq_policy": pgq.pgq_policy,
               "pgq_tensor_plan": pgq.pgq_tensor_plan}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', 'int main(void) {']
    for name, cls in structs.items():
        lines.append(f'printf("{name} size %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines.append("return 0; }")
    src, exe = tmp_path / "layout.c", tmp_path / "layout"
    src.write_text("\n".join(lines))
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    for line in filter(None, out):
        name, field, val = line.split()
        cls = structs[name]
        got = ctypes.sizeof(cls) if field == "size" else getattr(cls, field).offset
        assert got == int(val), line


def test_per_tensor_plan():
    ts = synth.config2()[:8]
    arr, keep = _tensor_array(ts)
    pol, k2 = _policy()
    pol.per_tensor = 1
    plan = (pgq.pgq_tensor_plan * 8)()
    ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pgq.pgq_export_plan(arr, 8, ctypes.byref(pol), plan, ctypes.byref(ab), ctypes.byref(wb)) == 0
    opol = oracle.Policy(per_tensor=True)
    for i, t in enumerate(ts):
        kind = oracle.tensor_kind(t.name, t.numel, opol)
        if kind == oracle.KIND_F16:
            assert plan[i].kind == pgq.PGQ_KIND_F16
            continue
        assert plan[i].kind == kind and plan[i].per_tensor == 1
        assert plan[i].scales_off % 256 == 0
        # the scales region holds one fp16: the next region starts 256 bytes later
        nxt = [plan[j].codes_off for j in range(i + 1, 8) if plan[j].codes_off >= 0] + \
              [plan[j].f16_off for j in range(i + 1, 8) if plan[j].f16_off >= 0]
        if nxt:
            assert min(nxt) == plan[i].scales_off + 256
    # per-tensor scales do not combine with AWQ; the flag is 0 or 1; SQWA takes per-row plans only
    arr_awq, keep2 = _tensor_array(synth.config4()[1:3], awq=True)
    plan2 = (pgq.pgq_tensor_plan * 2)()
    assert pgq.pgq_export_plan(arr_awq, 2, ctypes.byref(pol), plan2, ctypes.byref(ab),
                               ctypes.byref(wb)) == pgq.PGQ_ERR_PARAM
    pol.per_tensor = 2
    assert pgq.pgq_export_plan(arr, 8, ctypes.byref(pol), plan, ctypes.byref(ab),
                               ctypes.byref(wb)) == pgq.PGQ_ERR_PARAM
    pol.per_tensor = 1
    assert pgq.pgq_export_plan(arr, 8, ctypes.byref(pol), plan, ctypes.byref(ab), ctypes.byref(wb)) == 0
    means = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    assert pgq.pgq_sqwa_accumulate(arr, 8, plan, means, 1, FAKE, wb.value, 0, None,
                                   None) == pgq.PGQ_ERR_PARAM


def test_pack6_plan_and_decode_argument_errors():
    ts = synth.config2()[:8]
    arr, keep = _tensor_array(ts)
    pol, k2 = _policy()
    pol.pack6 = 1
    plan = (pgq.pgq_tensor_plan * 8)()
    ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pgq.pgq_export_plan(arr, 8, ctypes.byref(pol), plan, ctypes.byref(ab), ctypes.byref(wb)) == 0
    for i, t in enumerate(ts):
        if plan[i].kind == 6:
            rows, cols = oracle.as_rows(t.shape)
            assert plan[i].packed == 1
            assert plan[i].scales_off - plan[i].codes_off == -(-rows * 3 * ((cols + 3) // 4) // 256) * 256
        else:
            assert plan[i].packed == 0                 # int8 and fp16 tensors are not packed
    pol.pack6 = 3
    assert pgq.pgq_export_plan(arr, 8, ctypes.byref(pol), plan, ctypes.byref(ab),
                               ctypes.byref(wb)) == pgq.PGQ_ERR_PARAM
    dq = pgq.pgq_dequant_codes
    assert dq(FAKE, 1, 0, 512, FAKE, 0, None, FAKE, None, None) == pgq.PGQ_OK           # empty
    assert dq(FAKE, 1, -1, 512, FAKE, 0, None, FAKE, None, None) == pgq.PGQ_ERR_SHAPE
    assert dq(FAKE, 2, 4, 512, FAKE, 0, None, FAKE, None, None) == pgq.PGQ_ERR_PARAM
    assert dq(FAKE, 1, 4, 512, FAKE, 5, None, FAKE, None, None) == pgq.PGQ_ERR_PARAM
    assert dq(None, 1, 4, 512, FAKE, 0, None, FAKE, None, None) == pgq.PGQ_ERR_NULL
    assert dq(FAKE, 1, 4, 512, FAKE + 1, 0, None, FAKE, None, None) == pgq.PGQ_ERR_ALIGN
    assert dq(FAKE, 1, 4, 512, FAKE, 0, None, FAKE + 2, None, None) == pgq.PGQ_ERR_ALIGN


def test_dequant_model_argument_errors():
    ts = synth.config2()[:4]
    arr, keep = _tensor_array(ts)
    pol, k2 = _policy()
    plan = (pgq.pgq_tensor_plan * 4)()
    ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pgq.pgq_export_plan(arr, 4, ctypes.byref(pol), plan, ctypes.byref(ab), ctypes.byref(wb)) == 0
    outs = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    dm = pgq.pgq_dequant_model
    assert dm(arr, 0, plan, None, None, None, 0, 0, None, None) == pgq.PGQ_OK
    assert dm(arr, 4, plan, None, outs, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_NULL
    assert dm(arr, 4, plan, FAKE + 64, outs, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_ALIGN
    assert dm(arr, 4, plan, FAKE, outs, FAKE, 64, 0, None, None) == pgq.PGQ_ERR_WORKSPACE
    outs[1] = FAKE + 2
    assert dm(arr, 4, plan, FAKE, outs, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_ALIGN
    outs[1] = FAKE
    plan[0].kind = 9
    assert dm(arr, 4, plan, FAKE, outs, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_PARAM


@pytest.mark.parametrize("entry,ysize", [("pgq_qgemm_bf16", 4), ("pgq_qgemm_bf16_ybf16", 2)])
def test_qgemm_argument_errors(entry, ysize):
    g = getattr(pgq, entry)
    # (x, M, K, ldx, codes, ldc, scales, N, y, ldy, stream)
    ok = dict(x=FAKE, M=4, K=32, ldx=32, codes=FAKE, ldc=32, scales=FAKE, N=8, y=FAKE, ldy=8)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return g(a["x"], a["M"], a["K"], a["ldx"], a["codes"], a["ldc"], a["scales"], a["N"], a["y"], a["ldy"], None)

    assert call(M=-1) == pgq.PGQ_ERR_SHAPE
    assert call(N=-1) == pgq.PGQ_ERR_SHAPE
    assert call(K=-1) == pgq.PGQ_ERR_SHAPE
    assert call(ldx=31) == pgq.PGQ_ERR_SHAPE
    assert call(ldc=31) == pgq.PGQ_ERR_SHAPE
    assert call(ldy=7) == pgq.PGQ_ERR_SHAPE
    assert call(M=0) == pgq.PGQ_OK                     # nothing to do, nothing enqueued
    assert call(N=0) == pgq.PGQ_OK
    assert call(y=None) == pgq.PGQ_ERR_NULL
    assert call(x=None) == pgq.PGQ_ERR_NULL
    assert call(codes=None) == pgq.PGQ_ERR_NULL
    assert call(scales=None) == pgq.PGQ_ERR_NULL
    assert call(x=FAKE + 1) == pgq.PGQ_ERR_ALIGN
    assert call(scales=FAKE + 1) == pgq.PGQ_ERR_ALIGN
    assert call(y=FAKE + ysize // 2) == pgq.PGQ_ERR_ALIGN   # y must hold whole elements


def test_per_tensor_export_without_weights_is_refused():
    """A per-tensor export descriptor must carry its weights (the whole-tensor select reads them):
    the host refuses a NULL weight pointer before anything is enqueued."""
    ts = synth.config2()[:9]
    arr, keep = _tensor_array(ts)
    pol, k2 = _policy()
    pol.per_tensor = 1
    plan = (pgq.pgq_tensor_plan * 9)()
    ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pgq.pgq_export_plan(arr, 9, ctypes.byref(pol), plan, ctypes.byref(ab), ctypes.byref(wb)) == 0
    assert any(plan[i].per_tensor for i in range(9))
    i = next(i for i in range(9) if plan[i].per_tensor)
    arr[i].w = None
    assert pgq.pgq_export_model(arr, 9, plan, FAKE, None, FAKE, wb.value, 0, None, None) == pgq.PGQ_ERR_NULL
