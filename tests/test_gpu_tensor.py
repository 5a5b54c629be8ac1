"""GPU parity of per-tensor scales (one fp16 scale per tensor, clip = the percentile of |w| over
the whole tensor; PR #2159 Key Explored Modifications) against the CPU oracle, bit for bit.

The clip comes from one read of the tensor for ranks up to 256 from the top (every workgroup
appends its candidate keys, one workgroup per tensor ranks them), else from a multi-workgroup
radix select (one launch per digit); then the export pass quantizes with it.  Cases: the 9-layer
set (int8 absmax tok_emb next to int6 99.99th-percentile matrices), heavy tails at several
percentiles (candidate and radix tensors in one call), repeated calls on a resident table (the
select state must return to its start), bf16 / ragged / padded / misaligned / long-row tensors,
ranks 256 and 257 (either side of the switch), tied keys that overflow a tile's candidate
space and the pick's LDS buffer, a tensor with one outsized row, and the non-finite status bit.
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


def _check(ex, named, opol, what):
    outs = ex.outputs()
    ref = oracle.export(named, opol)
    for o, r, (nm, _) in zip(outs, ref, named):
        assert o["kind"] == r["kind"], (nm, o["kind"], r["kind"])
        if r["kind"] == oracle.KIND_F16:
            same_bits(u16(o["f16"]).reshape(-1), r["f16"].reshape(-1), f"{what} {nm} f16")
        else:
            same_bits(u16(o["scales"]), r["scales"], f"{what} {nm} scale")
            same_bits(o["codes"].cpu().numpy().reshape(r["codes"].shape), r["codes"], f"{what} {nm} codes")
        f32_bits_equal(f32(o["dq"]).reshape(-1), r["dq"].reshape(-1), f"{what} {nm} dq")


def _export(named, q_default, reps=1, place=dev):
    ex = ops.Exporter([ops.ExportTensor(nm, place(w)) for nm, w in named],
                      ops.make_policy(q_default=q_default, per_tensor=True), want_dq=True)
    for r in range(reps):
        ex.run(reuse_table=r > 0)
    torch.cuda.synchronize()
    return ex


def test_nine_layer_set_per_tensor():
    say("per-tensor export of the 9-layer set, 99.99th percentile (int8 tok_emb absmax)")
    named = [(t.name, t.data) for t in synth.config2()]
    ex = _export(named, (6, 9999, 10000))
    assert int(ex.status.item()) == 0
    _check(ex, named, oracle.Policy(per_tensor=True), "cfg2")


@pytest.mark.parametrize("pct", [(1, 1), (99, 100), (999, 1000), (1, 2), (1, 1000)])
def test_heavy_tails_per_tensor_percentiles(pct):
    say(f"per-tensor heavy tails, percentile {pct}")
    named = [(t.name, t.data) for t in synth.stress_s1()[:14]]
    ex = _export(named, (6,) + pct)
    _check(ex, named, oracle.Policy(q6=(6,) + pct, per_tensor=True), f"s1 {pct}")


def test_resident_table_repeats_exactly():
    say("per-tensor export, four calls on a resident table")
    named = [(t.name, t.data) for t in synth.stress_s1()[:10]]
    ex = _export(named, (6, 99, 100), reps=4)
    _check(ex, named, oracle.Policy(q6=(6, 99, 100), per_tensor=True), "resident x4")


@pytest.mark.parametrize("layout", ["dense", "ld_pad", "misaligned"])
def test_ragged_and_long_tensors(layout):
    say(f"per-tensor ragged / long tensors, {layout}")
    rng = np.random.default_rng(21)
    shapes = [(300, 257), (129, 513), (40, 3000), (1, 70000), (257, 260)]
    named = [(f"blocks.{i}.w", (rng.standard_t(3, s) * 0.02).astype(np.float32)) for i, s in enumerate(shapes)]

    def place(a):
        if layout == "dense":
            return dev(a)
        r, c = a.shape
        if layout == "ld_pad":
            big = torch.zeros(r, c + 5, dtype=torch.float32, device="cuda")
            big[:, :c] = dev(a)
            return big[:, :c]
        flat = torch.zeros(r * c + 1, dtype=torch.float32, device="cuda")
        v = flat[1:].view(r, c)
        v.copy_(dev(a))
        return v

    for pct in [(99, 100), (1, 1)]:
        ex = _export(named, (6,) + pct, place=place)
        _check(ex, named, oracle.Policy(q6=(6,) + pct, per_tensor=True), f"{layout} {pct}")


def test_bf16_weights_per_tensor():
    say("per-tensor export of bf16 weights")
    rng = np.random.default_rng(22)
    bits = [oracle.f32_to_bf16((rng.standard_normal(s) * 0.02).astype(np.float32))
            for s in [(528, 528), (1584, 528), (96, 1000)]]
    named = [(f"blocks.{i}.w", b) for i, b in enumerate(bits)]
    ex = ops.Exporter([ops.ExportTensor(nm, bf16_dev(b)) for nm, b in named],
                      ops.make_policy(q_default=(6, 9999, 10000), per_tensor=True), want_dq=True)
    ex.run()
    torch.cuda.synchronize()
    _check(ex, [(nm, oracle.bf16_to_f32(b)) for nm, b in named], oracle.Policy(per_tensor=True), "bf16")


def test_nonfinite_per_tensor_status():
    say("per-tensor export with an infinity")
    w = (np.random.default_rng(23).standard_normal((300, 512)) * 0.02).astype(np.float32)
    w[17, 5] = np.inf
    ex = _export([("blocks.0.w", w)], (6, 99, 100))
    assert int(ex.status.item()) & 1


def test_rank_boundary_candidate_and_radix():
    """Ranks 256 (candidate select, the largest it takes) and 257 (radix select) on one tensor."""
    w = (np.random.default_rng(31).standard_t(3, (256, 512)) * 0.02).astype(np.float32)
    n = w.size
    for rank in (256, 257):
        say(f"per-tensor rank {rank} from the top")
        pct = (n - rank + 1, n)                       # k = n - rank + 1 exactly
        named = [("blocks.0.w", w)]
        ex = _export(named, (6,) + pct)
        _check(ex, named, oracle.Policy(q6=(6,) + pct, per_tensor=True), f"rank {rank}")


def test_tied_keys_overflow_tile_candidates():
    """5,000 entries equal to the tensor's maximum: tiles holding many of them have more keys at or
    above their bound than candidate space, so they append their exact top-R instead."""
    say("per-tensor tied maxima (tile fallback)")
    rng = np.random.default_rng(32)
    w = (rng.standard_normal((512, 512)) * 0.02).astype(np.float32)
    idx = rng.choice(w.size, 5000, replace=False)
    w.reshape(-1)[idx] = np.float32(0.25) * np.where(rng.random(5000) < 0.5, -1, 1).astype(np.float32)
    named = [("blocks.0.w", w)]
    ex = _export(named, (6, 9999, 10000))
    _check(ex, named, oracle.Policy(per_tensor=True), "tied maxima")


def test_tied_keys_overflow_pick_buffer():
    """3,000 equal maxima with rank 200: more candidates at the pick's bound than its LDS buffer
    holds (the pick's radix fallback)."""
    say("per-tensor tied maxima (pick fallback)")
    rng = np.random.default_rng(33)
    w = (rng.standard_normal((512, 1536)) * 0.02).astype(np.float32)
    idx = rng.choice(w.size, 3000, replace=False)
    w.reshape(-1)[idx] = np.float32(0.5)
    n = w.size
    pct = (n - 199, n)                                 # rank 200 from the top
    named = [("blocks.0.w", w)]
    ex = _export(named, (6,) + pct)
    _check(ex, named, oracle.Policy(q6=(6,) + pct, per_tensor=True), "pick fallback")


def test_one_outsized_row():
    """One row 100x larger than the rest: every key of that row passes its tile's bound."""
    say("per-tensor outsized row")
    rng = np.random.default_rng(34)
    w = (rng.standard_normal((1536, 512)) * 0.02).astype(np.float32)
    w[777] *= 100.0
    named = [("blocks.0.mlp.up.weight", w), ("blocks.0.attn.wq.weight", w[:512].copy())]
    ex = _export(named, (6, 9999, 10000))
    _check(ex, named, oracle.Policy(per_tensor=True), "outsized row")


def test_mixed_dtypes_one_call():
    say("per-tensor fp32 and bf16 tensors in one call")
    rng = np.random.default_rng(35)
    a = (rng.standard_normal((300, 512)) * 0.02).astype(np.float32)
    b = oracle.f32_to_bf16((rng.standard_normal((70, 1000)) * 0.02).astype(np.float32))
    ex = ops.Exporter([ops.ExportTensor("blocks.0.a", dev(a)), ops.ExportTensor("blocks.0.b", bf16_dev(b))],
                      ops.make_policy(q_default=(6, 9999, 10000), per_tensor=True), want_dq=True)
    ex.run()
    ex.run()
    torch.cuda.synchronize()
    _check(ex, [("blocks.0.a", a), ("blocks.0.b", oracle.bf16_to_f32(b))], oracle.Policy(per_tensor=True), "mixed")
