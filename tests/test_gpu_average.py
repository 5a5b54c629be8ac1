"""GPU parity of the weight-averaging kernels (EMA, SWA) against the CPU oracle, bit for bit.

EMA: decay 0.997 (Weight Averaging sections of the PR #1414 / PR #1202 cards); SWA: running mean
of checkpoints (PR #69 card).  Cases: the 9-layer d=512 weight set over several steps (fp32),
bf16 weights of the d=528 shapes, ragged / padded / misaligned / 1-D tensors, the copy cases
(init, k = 1, decay 0 and 1), resume, and the non-finite status bit.
"""
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
from tests.gpu_util import bf16_dev, dev, f16_dev, f32_bits_equal  # noqa: E402


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _check(avg, ref, what):
    for i, (g, r) in enumerate(zip(avg, ref)):
        f32_bits_equal(g.cpu().numpy(), r, f"{what} tensor {i}")


def test_ema_nine_layer_set_over_steps():
    say("EMA 9-layer set, init + 3 steps")
    base = synth.config5_base()
    steps = [[t.data for t in synth.config5_snapshot(k, base)] for k in range(1, 5)]
    ema = ops.Ema([dev(w) for w in steps[0]])
    for s, ws in enumerate(steps):
        ema.update([dev(w) for w in ws], init=(s == 0), reuse_table=False)
    torch.cuda.synchronize()
    ref, st = oracle.ema_run(steps, 0.997)
    assert int(ema.status.item()) == st == 0
    _check(ema.avg, ref, "ema")


def test_ema_resident_table_and_bf16_weights():
    say("EMA bf16 d=528 weights, resident table")
    from synth.weights import config3_shapes
    shapes = [s for _, s in config3_shapes(2)]
    rng = np.random.default_rng(5)
    sets = [[oracle.f32_to_bf16((rng.standard_normal(s) * 0.02).astype(np.float32)) for s in shapes]
            for _ in range(3)]
    bufs = [bf16_dev(b) for b in sets[0]]
    ema = ops.Ema(bufs, decay=0.997)
    for s, ws in enumerate(sets):
        for buf, b in zip(bufs, ws):
            buf.copy_(bf16_dev(b))
        ema.update(bufs, init=(s == 0))            # same buffers: the table stays resident
    torch.cuda.synchronize()
    ref, _ = oracle.ema_run([[oracle.bf16_to_f32(b) for b in ws] for ws in sets], 0.997)
    _check(ema.avg, ref, "ema bf16")


def test_ema_and_swa_fp16_weights():
    """fp16 weights (widened exactly): EMA over three steps and SWA over three checkpoints, with a
    ragged and an odd-width tensor beside 528-wide ones."""
    say("EMA / SWA fp16 weights")
    shapes = [(528, 528), (70, 1000), (9, 37)]
    rng = np.random.default_rng(6)
    sets = [[oracle.f32_to_f16((rng.standard_normal(s) * 0.02).astype(np.float32)) for s in shapes]
            for _ in range(3)]
    ema = ops.Ema([f16_dev(h) for h in sets[0]], decay=0.997)
    for s, ws in enumerate(sets):
        ema.update([f16_dev(h) for h in ws], init=(s == 0), reuse_table=False)
    torch.cuda.synchronize()
    ref, st = oracle.ema_run([[oracle.f16_to_f32(h) for h in ws] for ws in sets], 0.997)
    assert int(ema.status.item()) == st == 0
    _check(ema.avg, ref, "ema f16")
    swa = ops.Swa([f16_dev(h) for h in sets[0]])
    means = [np.empty(s, dtype=np.float32) for s in shapes]
    for k, ws in enumerate(sets, start=1):
        swa.accumulate([f16_dev(h) for h in ws], k, reuse_table=False)
        for m, h in zip(means, ws):
            oracle.swa_update(m.reshape(-1), oracle.f16_to_f32(h).reshape(-1), k)
    torch.cuda.synchronize()
    _check(swa.avg, means, "swa f16")


@pytest.mark.parametrize("layout", ["dense", "ld_pad", "misaligned"])
def test_average_ragged_shapes(layout):
    say(f"EMA/SWA ragged {layout}")
    rng = np.random.default_rng(11)
    shapes = [(1, 1), (3, 5), (7, 129), (2, 513), (5, 1024), (1, 700), (33, 8)]
    sets = [[(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes] for _ in range(3)]

    def place(a):
        if layout == "dense":
            return dev(a)
        r, c = a.shape
        if layout == "ld_pad":
            big = torch.zeros(r, c + 3, dtype=torch.float32, device="cuda")
            big[:, :c] = dev(a)
            return big[:, :c]
        flat = torch.zeros(r * c + 1, dtype=torch.float32, device="cuda")
        v = flat[1:].view(r, c)
        v.copy_(dev(a))
        return v

    ws = [[place(a) for a in s] for s in sets]
    ema = ops.Ema(ws[0], decay=0.9)
    swa = ops.Swa(ws[0])
    for s in range(3):
        ema.update(ws[s], init=(s == 0))
        swa.accumulate(ws[s], s + 1)
    torch.cuda.synchronize()
    ref_e, _ = oracle.ema_run(sets, 0.9)
    ref_s, _ = oracle.swa_run(sets)
    _check(ema.avg, ref_e, f"ema {layout}")
    _check(swa.avg, ref_s, f"swa {layout}")


def test_ema_special_decays_and_vectors():
    say("EMA decay 0 and 1, 1-D tensors")
    rng = np.random.default_rng(12)
    a = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in [(512,), (64, 512)]]
    b = [(rng.standard_normal(x.shape) * 0.02).astype(np.float32) for x in a]
    for decay in (0.0, 1.0):
        ema = ops.Ema([dev(x) for x in a], decay=decay)
        ema.update([dev(x) for x in a], init=True)
        ema.update([dev(x) for x in b])
        torch.cuda.synchronize()
        ref, _ = oracle.ema_run([a, b], decay)
        _check(ema.avg, ref, f"decay {decay}")
        _check(ema.avg, b if decay == 0.0 else a, f"decay {decay} closed form")


def test_swa_sixteen_checkpoints_and_resume():
    say("SWA 16 checkpoints of the 9-layer set, split in two runs")
    base = synth.config5_base()
    like = [dev(t.data) for t in base]
    swa = ops.Swa(like)
    means = None
    for k in range(1, 17):
        ws = [t.data for t in synth.config5_snapshot(k, base)]
        for buf, w in zip(like, ws):
            buf.copy_(dev(w))
        swa.accumulate(like, k)
        means, _ = oracle.swa_run([ws], k0=k, means=means)
        if k in (1, 8, 16):
            torch.cuda.synchronize()
            _check(swa.avg, means, f"swa k={k}")


def test_average_nonfinite_status():
    say("EMA / SWA non-finite status")
    w = (np.random.default_rng(13).standard_normal((4, 256)) * 0.02).astype(np.float32)
    w[2, 17] = np.inf
    ema = ops.Ema([dev(w)])
    ema.update([dev(w)], init=True)
    swa = ops.Swa([dev(w)])
    swa.accumulate([dev(w)], 1)
    torch.cuda.synchronize()
    assert int(ema.status.item()) & pgq.PGQ_DEV_NONFINITE
    assert int(swa.status.item()) & pgq.PGQ_DEV_NONFINITE
    ok = ops.Ema([dev(np.abs(w[:1]) * 0 + 1)])
    ok.update([dev(np.ones((1, 256), np.float32))], init=True)
    torch.cuda.synchronize()
    assert int(ok.status.item()) == 0
