"""Planted mistakes in the oracle must fail its pins (CPU).

Each case copies oracle/orc.c to a temporary directory, makes one plausible mistake in the copy
(a wrong tie rule, an off-by-one rank, a dropped term, a swapped operand, a wrong bit order, a
fused multiply-add where the pages' reading rounds twice, ...), builds it, and runs the pins that
cover that step in a subprocess with ORC_LIB pointing at the mutant.  The case passes when those
pins fail (pytest exit status 1, i.e. assertion failures, not a crash).  The oracle itself is
never modified.  Its stored output hashes (test_oracle_regression) are not used: they would
catch every change trivially without saying anything about the pins.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "orc.c")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing"]

CONVERT = ["tests/test_oracle_convert.py"]
F16 = ["tests/test_oracle_convert.py::test_f16_decode_all", "tests/test_oracle_convert.py::test_f32_to_f16_numpy_sample"]
BF16 = ["tests/test_oracle_convert.py::test_f32_to_bf16_exhaustive"]
RANK = ["tests/test_oracle_convert.py::test_percentile_rank"]
STATUS = ["tests/test_oracle_invariants.py::test_status_bits"]
EXACT = ["tests/test_oracle_exact.py"]
INVAR = ["tests/test_oracle_invariants.py"]
AVG = ["tests/test_oracle_average.py"]
PACK = ["tests/test_oracle_pack.py"]
QGEMM = ["tests/test_oracle_qgemm.py"]
TENSOR = ["tests/test_oracle_tensor.py"]

# (name, text in orc.c, replacement, pins expected to catch it)
MUTANTS = [
    ("f16 ties away from zero", "if (rem > half || (rem == half && (q & 1))) q += 1;", "if (rem >= half) q += 1;",
     F16),
    ("f16 subnormal scale", "uint64_t n = shift_rne(m, -(e + 1));", "uint64_t n = shift_rne(m, -(e + 2));", F16),
    ("f16 overflow threshold", "if (ee > 15) return sign | 0x7C00u;", "if (ee > 16) return sign | 0x7C00u;", F16),
    ("f16 decode subnormal", "float v = (float)fr * 0x1p-24f;", "float v = (float)fr * 0x1p-25f;", F16),
    ("bf16 ties down", "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;", "if (lo > 0x8000u) hi += 1;",
     BF16),
    ("percentile rank floor", "int64_t k = (int64_t)((p + den - 1) / den);", "int64_t k = (int64_t)(p / den);",
     RANK + EXACT),
    ("clip one rank off", "float clip = mag[k - 1];", "float clip = mag[k < n ? k : n - 1];", EXACT + INVAR),
    ("scale divides by Q + 1", "float s32 = clip / (float)Q;", "float s32 = clip / (float)(Q + 1);", EXACT + INVAR),
    ("zero scale kept", "if ((s16 & 0x7FFFu) == 0) s16 = 0x3C00u;", "", EXACT + INVAR),
    ("scale overflow not reported", "if ((s16 & 0x7FFFu) == 0x7C00u) st |= ORC_SCALE_OVF;", "", STATUS),
    ("codes round half away", "float r = rintf(t);", "float r = roundf(t);", EXACT + INVAR),
    ("codes clamp to -Q-1", "else if (r < (float)(-Q)) q = -Q;", "else if (r < (float)(-Q - 1)) q = -Q - 1;",
     EXACT + INVAR),
    ("AWQ dequant multiplies", "if (awq) d = d / orc_f16_to_f32(awq[j]);\n            dq[j] = d;",
     "if (awq) d = d * orc_f16_to_f32(awq[j]);\n            dq[j] = d;", EXACT + INVAR),
    ("AWQ applied as a divide", "if (awq) v = v * orc_f16_to_f32(awq[j]);", "if (awq) v = v / orc_f16_to_f32(awq[j]);",
     EXACT + INVAR),
    ("AWQ multiplier without sqrt", "a[j] = orc_f32_to_f16(sqrtf(v));", "a[j] = orc_f32_to_f16(v);", EXACT + INVAR),
    ("STE mask strict", "int keep = fabsf(t[j]) <= lim;", "int keep = fabsf(t[j]) < lim;", EXACT),
    ("STE mask at Q", "float lim = (float)Q + 0.5f;", "float lim = (float)Q;", EXACT),
    ("STE backward inverted", "keep ? g[r * cols + j] : (uint16_t)0", "keep ? (uint16_t)0 : g[r * cols + j]",
     EXACT + INVAR),
    ("STE mask bit order", "(uint8_t)(1u << (j % 8))", "(uint8_t)(0x80u >> (j % 8))", EXACT + INVAR),
    ("STE dequant truncated to bf16", "if (dq) dq[r * cols + j] = orc_f32_to_bf16(d[j]);",
     "if (dq) dq[r * cols + j] = (uint16_t)(bits_of(d[j]) >> 16);", EXACT + INVAR),
    ("pack6 field order", "word |= ((uint32_t)c & 0x3Fu) << (6 * t);", "word |= ((uint32_t)c & 0x3Fu) << (6 * (3 - t));",
     PACK),
    ("unpack6 without sign", "codes[r * cols + j] = (int8_t)(f >= 32 ? f - 64 : f);", "codes[r * cols + j] = (int8_t)f;",
     PACK),
    ("per-tensor clip from the first row", "uint32_t st = orc_quantize_row(flat, n, Q, num, den, NULL, codes, scale, dq, NULL, clip);",
     "uint32_t st = orc_quantize_row(flat, cols, Q, num, den, NULL, codes, scale, dq, NULL, clip);\n"
     "    for (int64_t i = cols; i < n; ++i) { codes[i] = 0; if (dq) dq[i] = 0.0f; }", TENSOR),
    ("GEMM weights not rounded to bf16", "wq[n * K + k] = orc_bf16_to_f32(orc_f32_to_bf16(d));", "wq[n * K + k] = d;",
     QGEMM),
    ("GEMM drops the row scale", "float d = (float)codes[n * ldc + k] * s;\n            wq",
     "float d = (float)codes[n * ldc + k];\n            wq", QGEMM),
    ("EMA weight factor is the decay", "const float c = 1.0f - decay;", "const float c = decay;", AVG + EXACT),
    ("EMA fused multiply-add", "e[j] = kept + added;", "e[j] = fmaf(decay, e[j], added); (void)kept;", EXACT),
    ("EMA without its first copy", "if (init) {", "if (0) {", AVG),
    ("SQWA divides by k + 1", "float step = diff / kf;", "float step = diff / (kf + 1.0f);", EXACT + INVAR + AVG),
    ("SQWA step subtracted", "mean[j] = mean[j] + step;", "mean[j] = mean[j] - step;", EXACT + INVAR + AVG),
    ("fp16 passthrough overflow not reported", "else if ((y[j] & 0x7FFFu) == 0x7C00u) st |= ORC_F16_OVF;", "",
     STATUS),
]


def _run(mutant, tmp):
    name, old, new, tests = mutant
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"{name}: text not found once in orc.c"
    d = tempfile.mkdtemp(dir=tmp)
    c = os.path.join(d, "orc.c")
    with open(c, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(d, "liborc.so")
    subprocess.check_call(["gcc", *CFLAGS, "-o", so, c, "-lm"])
    env = dict(os.environ, ORC_LIB=so, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return name, r.returncode, (r.stdout + r.stderr)[-1500:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    # control: the same machinery with no change passes every selection used below, so a failure of a
    # mutant is the mutation's
    sel = []
    for m in MUTANTS:
        sel += [t for t in m[3] if t not in sel]
    first = MUTANTS[0]
    control = ("unchanged", first[1], first[1], sel)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda m: _run(m, str(tmp_path)), [control] + MUTANTS))
    name, rc, out = results[0]
    assert rc == 0, f"the unchanged build fails its pins: exit {rc}\n{out}"
    survived = [(n, rc, out) for n, rc, out in results[1:] if rc != 1]
    assert not survived, "\n\n".join(f"{n}: exit {rc}\n{out}" for n, rc, out in survived)
