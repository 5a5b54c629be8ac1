"""The allocation-free export entry point (pgq_export_model_noalloc) against the workspace entry
point (pgq_export_model) through the C ABI: identical arenas and dequantized outputs, bit for
bit, on two calls in a row (the second with a smaller weight set), for per-row and per-tensor
scales; and the size limit of its scratch array refused before anything is enqueued."""
import ctypes
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
import synth  # noqa: E402
from int6_weight_export_amd import ops, pgq  # noqa: E402
from tests.gpu_util import dev  # noqa: E402


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _run_both(tensors, policy):
    """Export the set with both entry points; return (arena, dq list) of each and the plan."""
    devs = [ops.ExportTensor(t.name, dev(t.data)) for t in tensors]
    arr, keep = ops._tensor_in_array(devs)
    n = len(devs)
    plan = (pgq.pgq_tensor_plan * n)()
    ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    pgq.check(pgq.pgq_export_plan(arr, n, ctypes.byref(policy), plan, ctypes.byref(ab), ctypes.byref(wb)),
              "pgq_export_plan")
    outs = []
    for which in ("workspace", "noalloc"):
        arena = torch.full((ab.value,), 0x5A, dtype=torch.uint8, device="cuda")
        dq = [torch.full(t.data.shape, float("nan"), dtype=torch.float32, device="cuda") for t in tensors]
        ptrs = (ctypes.c_void_p * n)(*[d.data_ptr() for d in dq])
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        if which == "workspace":
            ws = torch.empty(max(wb.value, 64), dtype=torch.uint8, device="cuda")
            rc = pgq.pgq_export_model(arr, n, plan, arena.data_ptr(), ptrs, ws.data_ptr(), ws.numel(), 0,
                                      status.data_ptr(), _stream())
        else:
            rc = pgq.pgq_export_model_noalloc(arr, n, plan, arena.data_ptr(), ptrs, 0, status.data_ptr(), _stream())
        assert rc == pgq.PGQ_OK, (which, rc)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, which
        outs.append((arena.cpu().numpy(), [d.cpu().numpy() for d in dq]))
    return outs, plan


def _compare(outs, tensors, plan, pol, what):
    (a0, d0), (a1, d1) = outs
    # every byte of the arena that the plan assigns (the gaps between regions are not written)
    for i, t in enumerate(tensors):
        p = plan[i]
        rows, cols = oracle.as_rows(t.shape)
        regions = []
        if p.kind == pgq.PGQ_KIND_F16:
            regions.append((p.f16_off, 2 * rows * cols))
        else:
            regions.append((p.codes_off, rows * cols))
            regions.append((p.scales_off, 2 * (1 if p.per_tensor else rows)))
        for off, nb in regions:
            assert np.array_equal(a0[off:off + nb], a1[off:off + nb]), f"{what}: arena of {t.name}"
        assert np.array_equal(d0[i].view(np.uint32), d1[i].view(np.uint32)), f"{what}: dq of {t.name}"
    # and the workspace entry point's result is the oracle's
    ref = oracle.export([(t.name, t.data) for t in tensors], pol)
    for i, r in enumerate(ref):
        assert np.array_equal(d0[i].reshape(-1).view(np.uint32), r["dq"].reshape(-1).view(np.uint32)), \
            f"{what}: oracle dq of {tensors[i].name}"


@pytest.mark.parametrize("per_tensor", [False, True])
def test_noalloc_matches_workspace_call_twice(per_tensor):
    pol_c = ops.make_policy(per_tensor=per_tensor)
    pol_o = oracle.Policy(per_tensor=per_tensor)
    big = synth.config2()                      # 73 tensors: the whole 9-layer set
    small = synth.config2()[:9]                # then a smaller call on the same (reused) array
    for what, ts in (("first call, 73 tensors", big), ("second call, 9 tensors", small)):
        say(f"noalloc per_tensor={per_tensor}: {what}")
        outs, plan = _run_both(ts, pol_c)
        _compare(outs, ts, plan, pol_o, f"per_tensor={per_tensor} {what}")


def test_noalloc_refuses_a_table_beyond_its_array():
    """1,100 per-tensor tensors need more select state than the 4 MiB array holds: the call returns
    PGQ_ERR_WORKSPACE before enqueueing anything (the device pointers are never read)."""
    say("noalloc size limit")
    n = 1100
    fake = 0x10000
    arr = (pgq.pgq_tensor_in * n)()
    names = [f"blocks.{i}.w".encode() for i in range(n)]
    for i in range(n):
        arr[i] = pgq.pgq_tensor_in(names[i], fake, pgq.PGQ_F32, 0, 128, 512, 512, 0)
    pol = ops.make_policy(per_tensor=True)
    plan = (pgq.pgq_tensor_plan * n)()
    ab, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert pgq.pgq_export_plan(arr, n, ctypes.byref(pol), plan, ctypes.byref(ab), ctypes.byref(wb)) == pgq.PGQ_OK
    assert wb.value > (4 << 20)
    rc = pgq.pgq_export_model_noalloc(arr, n, plan, fake, None, 0, None, _stream())
    assert rc == pgq.PGQ_ERR_WORKSPACE
