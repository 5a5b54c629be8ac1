"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

orc.c is built with -fsanitize=address,undefined (every report fatal) into a temporary
directory and the pins that exercise it run in a subprocess that loads that build (ORC_LIB) with
the ASan runtime preloaded into the Python interpreter.  Any out-of-bounds access, use after
free, signed overflow, misaligned access or invalid shift in the oracle ends that run with a
report and fails this test.  Leak checking is off: the interpreter itself does not free
everything at exit.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "orc.c")
# three groups of pins, run side by side
PINS = [["tests/test_oracle_exact.py", "tests/test_oracle_pack.py", "tests/test_oracle_qgemm.py"],
        ["tests/test_oracle_invariants.py"],
        ["tests/test_oracle_tensor.py", "tests/test_oracle_average.py",
         "tests/test_oracle_convert.py::test_percentile_rank", "tests/test_oracle_convert.py::test_f16_decode_all",
         "tests/test_oracle_convert.py::test_f32_to_f16_numpy_sample"]]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None,
                    reason="gcc with the ASan runtime is required")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "liborc_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                           "-fno-strict-aliasing", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-o", so, SRC, "-lm"])
    logs = str(tmp_path / "san")

    def run(group):
        env = dict(os.environ, ORC_LIB=so, PYTHONDONTWRITEBYTECODE="1", LD_PRELOAD=_runtime("libasan.so"),
                   ASAN_OPTIONS=f"detect_leaks=0:verify_asan_link_order=0:exitcode=86:log_path={logs}",
                   UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:exitcode=87:log_path={logs}")
        return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                               *group], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)

    with cf.ThreadPoolExecutor(max_workers=len(PINS)) as ex:
        results = list(ex.map(run, PINS))
    reports = ""
    for f in sorted(os.listdir(tmp_path)):
        if f.startswith("san"):
            with open(tmp_path / f) as fh:
                reports += fh.read()[-3000:]
    for r in results:
        out = r.stdout + r.stderr
        assert r.returncode == 0, (reports or out)[-4000:]
        assert " passed" in out, out[-2000:]
    assert not reports, reports
