"""bench.py on the CPU: the single-GPU refusal, and committed counter summaries that still describe
the current kernel sources (a stale summary would silently turn roofline.traffic into null)."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("mode", sorted(_bench().MAKERS))
def test_every_mode_has_a_counter_summary_of_the_current_sources(mode):
    b = _bench()
    path = os.path.join(ROOT, "profiles", f"traffic_{mode}.json")
    assert os.path.exists(path), f"no counter summary for --mode {mode}"
    with open(path) as f:
        tr = json.load(f)
    assert tr["mode"] == mode
    assert tr["kernel_source_sha256"] == b.kernel_source_hash(mode), \
        f"profiles/traffic_{mode}.json was taken from other kernel sources: profile the mode again"
    assert b.traffic_for(mode) == tr["hbm_bytes_per_step"]
    assert os.path.exists(os.path.join(ROOT, "profiles", f"{mode}_kernel_trace.md"))
    # the counters see the algorithmic bytes, give or take re-reads (the per-tensor mode reads
    # its weights twice by design)
    assert 1.0 <= tr["traffic_over_algorithmic"] < (1.6 if mode == "tensor" else 1.3)


def test_modes_table_lists_every_mode():
    with open(os.path.join(ROOT, "profiles", "modes.md")) as f:
        text = f.read()
    for mode in _bench().MAKERS:
        assert f"| {mode} |" in text, mode
