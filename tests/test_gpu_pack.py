"""GPU parity of 6-bit code storage and of the decode of stored codes, bit for bit.

Layout (our reading of the int6 artifact savings of the PR #69 card): per row, four 6-bit
two's-complement codes per three bytes.  Cases: the 9-layer set exported packed (int8 tok_emb
stays one byte per code), ragged / padded / misaligned rows (the element-wise path packs across
lanes), bf16 rows, AWQ and per-tensor tensors, and the decode of every stored form back to the
export's own dequantized values.
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
from int6_weight_export_amd import ops  # noqa: E402
from tests.gpu_util import bf16_dev, dev, f32, f32_bits_equal, same_bits, u16  # noqa: E402


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _export(named, pol_kwargs, place=dev, awq=None):
    ex = ops.Exporter([ops.ExportTensor(nm, place(w), None if awq is None or nm not in awq else dev(awq[nm]))
                       for nm, w in named], ops.make_policy(pack6=True, **pol_kwargs), want_dq=True)
    ex.run()
    torch.cuda.synchronize()
    return ex


def _check(ex, named, opol, awq=None, decode=True):
    outs = ex.outputs()
    ref = oracle.export(named, opol, awq=awq)
    for o, r, (nm, w) in zip(outs, ref, named):
        if r["kind"] == oracle.KIND_F16:
            continue
        rows, cols = oracle.as_rows(np.asarray(w).shape)
        same_bits(u16(o["scales"]), r["scales"], nm + " scales")
        if "packed" in r:
            assert "packed" in o, nm
            same_bits(o["packed"].cpu().numpy(), r["packed"], nm + " packed")
        else:
            same_bits(o["codes"].cpu().numpy(), r["codes"], nm + " codes")
        f32_bits_equal(f32(o["dq"]).reshape(-1), r["dq"].reshape(-1), nm + " dq")
        if decode:
            codes = o["packed"] if "packed" in o else o["codes"]
            got = ops.dequant_codes(codes, o["scales"], cols, packed="packed" in o,
                                    per_tensor=opol.per_tensor, awq=o.get("awq"))
            torch.cuda.synchronize()
            f32_bits_equal(f32(got).reshape(-1), r["dq"].reshape(-1), nm + " decode")


def test_nine_layer_set_packed_and_decoded():
    say("9-layer set exported with 6-bit codes, then decoded")
    named = [(t.name, t.data) for t in synth.config2()]
    ex = _export(named, {})
    assert int(ex.status.item()) == 0
    _check(ex, named, oracle.Policy(pack6=True))


@pytest.mark.parametrize("layout", ["dense", "ld_pad", "misaligned"])
def test_ragged_rows_packed(layout):
    say(f"packed ragged rows, {layout}")
    rng = np.random.default_rng(31)
    shapes = [(260, 257), (129, 515), (64, 1027), (33, 3000), (300, 260)]
    named = [(f"blocks.{i}.w", (rng.standard_normal(s) * 0.02).astype(np.float32)) for i, s in enumerate(shapes)]

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

    for pct in [(1, 1), (99, 100)]:
        ex = _export(named, {"q_default": (6,) + pct}, place=place)
        _check(ex, named, oracle.Policy(q6=(6,) + pct, pack6=True))


def test_bf16_rows_packed():
    say("packed bf16 rows")
    rng = np.random.default_rng(32)
    bits = [oracle.f32_to_bf16((rng.standard_normal(s) * 0.02).astype(np.float32))
            for s in [(528, 528), (300, 1584), (129, 1032)]]
    named = [(f"blocks.{i}.w", b) for i, b in enumerate(bits)]
    ex = ops.Exporter([ops.ExportTensor(nm, bf16_dev(b)) for nm, b in named],
                      ops.make_policy(pack6=True), want_dq=True)
    ex.run()
    torch.cuda.synchronize()
    _check(ex, [(nm, oracle.bf16_to_f32(b)) for nm, b in named], oracle.Policy(pack6=True))


def test_awq_and_per_tensor_packed():
    say("packed AWQ tensors and packed per-tensor tensors, decoded")
    ts = synth.config4()[:8]
    awq = {t.name: t.awq_s for t in ts if t.awq_s is not None}
    named = [(t.name, t.data) for t in ts]
    ex = _export(named, {"q_default": (6, 1, 1)}, awq=awq)
    _check(ex, named, oracle.Policy(q6=(6, 1, 1), pack6=True), awq=awq)
    named2 = [(t.name, t.data) for t in synth.stress_s1()[:8]]
    ex2 = _export(named2, {"q_default": (6, 99, 100), "per_tensor": True})
    _check(ex2, named2, oracle.Policy(q6=(6, 99, 100), pack6=True, per_tensor=True))


@pytest.mark.parametrize("pol_kwargs,opol_kwargs", [
    ({}, {}),
    ({"pack6": True}, {"pack6": True}),
    ({"pack6": True, "per_tensor": True, "q_default": (6, 99, 100)},
     {"pack6": True, "per_tensor": True, "q6": (6, 99, 100)}),
])
def test_whole_model_decode(pol_kwargs, opol_kwargs):
    say(f"whole-model decode {pol_kwargs}")
    named = [(t.name, t.data) for t in synth.config2()]
    ex = ops.Exporter([ops.ExportTensor(nm, dev(w)) for nm, w in named], ops.make_policy(**pol_kwargs),
                      want_dq=False)
    ex.run()
    ref = oracle.export(named, oracle.Policy(**opol_kwargs))
    for rep in range(2):                               # second call on the resident table
        outs = ex.decode()
        torch.cuda.synchronize()
        for o, r, (nm, _) in zip(outs, ref, named):
            f32_bits_equal(f32(o).reshape(-1), r["dq"].reshape(-1), f"{nm} decode {rep}")


def test_whole_model_decode_awq():
    say("whole-model decode of an AWQ export")
    ts = synth.config4()[:10]
    awq = {t.name: t.awq_s for t in ts if t.awq_s is not None}
    named = [(t.name, t.data) for t in ts]
    ex = ops.Exporter([ops.ExportTensor(nm, dev(w), None if nm not in awq else dev(awq[nm])) for nm, w in named],
                      ops.make_policy(q_default=(6, 1, 1), pack6=True), want_dq=False)
    ex.run()
    outs = ex.decode()
    torch.cuda.synchronize()
    ref = oracle.export(named, oracle.Policy(q6=(6, 1, 1), pack6=True), awq=awq)
    for o, r, (nm, _) in zip(outs, ref, named):
        f32_bits_equal(f32(o).reshape(-1), r["dq"].reshape(-1), f"{nm} decode")
