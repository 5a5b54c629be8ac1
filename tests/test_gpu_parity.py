"""GPU parity: libpgq (HIP, gfx950) against the CPU oracle, element by element.

Codes, scales, masks, fp16/bf16 outputs and fp32 dequant/mean values must be bit-identical,
sign of zero included.  Cases: the five workloads at full size (the
oracle checks every output, or sampled tensors where the oracle would take minutes), ragged
and misaligned shapes, heavy-tailed and long rows, edge rows and status bits.
"""
import os
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
from tests.gpu_util import bf16_dev, dev, f16_dev, f32, f32_bits_equal, same_bits, u16  # noqa: E402


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _check_rows(w_np, out, Q, num, den, what, awq_bits=None, dq_bf16=False):
    ref = oracle.quantize_rows(w_np, Q, num, den, awq=awq_bits)
    same_bits(u16(out["scales"]), ref["scales"], what + " scales")
    if "codes" in out:
        same_bits(out["codes"].cpu().numpy(), ref["codes"], what + " codes")
    if "dq" in out:
        if dq_bf16:
            same_bits(u16(out["dq"]), oracle.f32_to_bf16(ref["dq"]), what + " dq bf16")
        else:
            f32_bits_equal(f32(out["dq"]), ref["dq"], what + " dq")
    return ref


# ---------------------------------------------------------------------------------------------
def test_config1_quantize_dequant():
    say("config1 1536x512 fp32 int6 absmax")
    w = synth.config1().data
    out = ops.quantize_rows(dev(w), bits=6)
    torch.cuda.synchronize()
    _check_rows(w, out, 31, 1, 1, "config1")
    assert int(out["status"].item()) == 0


def test_config1_bf16_dq_and_int8():
    w = synth.config1().data
    say("config1 dq bf16")
    out = ops.quantize_rows(dev(w), bits=6, dq_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check_rows(w, out, 31, 1, 1, "config1 bf16", dq_bf16=True)
    say("config1 int8")
    out = ops.quantize_rows(dev(w), bits=8)
    torch.cuda.synchronize()
    _check_rows(w, out, 127, 1, 1, "config1 int8")


SHAPES = [(1, 1), (3, 3), (5, 7), (2, 64), (7, 65), (4, 100), (9, 511), (6, 512), (5, 513), (3, 1536),
          (2, 2047), (3, 2048), (2, 2049), (2, 3000), (3, 4096 + 4), (1, 8192)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("layout", ["dense", "ld_pad", "misaligned"])
def test_ragged_fp32(rows, cols, layout):
    say(f"ragged fp32 {rows}x{cols} {layout}")
    rng = np.random.default_rng(rows * 1000 + cols)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    pad = {"dense": 0, "ld_pad": 5, "misaligned": 0}[layout]
    big = np.zeros((rows, cols + pad + 1), np.float32)
    off = 1 if layout == "misaligned" else 0
    big[:, off:off + cols] = w
    bd = dev(big)
    view = bd[:, off:off + cols]
    for bits, pct in [(6, (1, 1)), (6, (99, 100)), (8, (1, 2)), (6, (9999, 10000))]:
        out = ops.quantize_rows(view, bits=bits, pct=pct)
        torch.cuda.synchronize()
        _check_rows(w, out, (1 << (bits - 1)) - 1, pct[0], pct[1], f"{rows}x{cols} {layout} b{bits} p{pct}")


@pytest.mark.parametrize("rows,cols", [(3, 8), (5, 528), (4, 1584), (3, 100), (2, 2056), (2, 4100)])
def test_ragged_bf16_input(rows, cols):
    say(f"bf16 input {rows}x{cols}")
    rng = np.random.default_rng(cols)
    w32 = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    wb = oracle.f32_to_bf16(w32)
    for pct in [(1, 1), (99, 100)]:
        out = ops.quantize_rows(bf16_dev(wb), bits=6, pct=pct)
        torch.cuda.synchronize()
        _check_rows(oracle.bf16_to_f32(wb), out, 31, pct[0], pct[1], f"bf16 {rows}x{cols} {pct}")


@pytest.mark.parametrize("q", [(6, 9999, 10000), (6, 1, 1)])
def test_export_bf16_flat_runs(q):
    """Dense bf16 rows whose width leaves a partly used wave-wide load per row (528, 600, 1040
    columns) are exported several rows per run; ragged last runs, an int8 tensor, one-row tensors."""
    say(f"bf16 export, flat runs, {q}")
    rng = np.random.default_rng(78)
    shapes = [(1583, 528), (13, 600), (9, 1040), (1, 528), (7, 528), (130, 1040)]
    names = ["blocks.0.attn.qkv.weight", "blocks.0.mlp.fc.weight", "blocks.1.mlp.proj.weight",
             "blocks.2.attn.proj.weight", "blocks.3.attn.proj.weight", "tok_emb.weight"]
    bits = [oracle.f32_to_bf16((rng.standard_t(4, s) * 0.02).astype(np.float32)) for s in shapes]
    ex = ops.Exporter([ops.ExportTensor(nm, bf16_dev(b)) for nm, b in zip(names, bits)],
                      ops.make_policy(q_default=q, passthrough_below=0), want_dq=True)
    ex.run()
    ex.run()
    torch.cuda.synchronize()
    assert int(ex.status.item()) == 0
    outs = ex.outputs()
    ref = oracle.export([(nm, oracle.bf16_to_f32(b)) for nm, b in zip(names, bits)],
                        oracle.Policy(q6=q, passthrough_below=0))
    for o, r, nm in zip(outs, ref, names):
        assert o["kind"] == r["kind"], (nm, o["kind"], r["kind"])
        same_bits(o["codes"].cpu().numpy(), r["codes"], nm + " codes")
        same_bits(u16(o["scales"]), r["scales"], nm + " scales")
        f32_bits_equal(f32(o["dq"]).reshape(-1), r["dq"].reshape(-1), nm + " dq")


def _f16_weights(rng, shape, scale=0.02):
    """fp16 bit patterns of N(0, scale^2) weights with a few edge values: fp16 subnormals, a large
    magnitude and a signed zero."""
    w = (rng.standard_normal(shape) * scale).astype(np.float32)
    flat = w.reshape(-1)
    k = flat.size
    flat[: min(4, k)] = np.float32([3e-7, -5e-8, -0.0, 0.0])[: min(4, k)]
    if k > 9:
        flat[9] = np.float32(-7.25)
    return oracle.f32_to_f16(w)


@pytest.mark.parametrize("rows,cols", [(5, 528), (3, 100), (4, 1584), (2, 4100), (7, 8)])
def test_f16_input_rows(rows, cols):
    """fp16 weights (widened exactly to binary32): vector, element-wise and streamed rows, absmax and
    a percentile clip, fp32 and bf16 dequant."""
    say(f"fp16 input {rows}x{cols}")
    h = _f16_weights(np.random.default_rng(cols + 1), (rows, cols))
    w32 = oracle.f16_to_f32(h)
    for pct in [(1, 1), (99, 100)]:
        out = ops.quantize_rows(f16_dev(h), bits=6, pct=pct)
        torch.cuda.synchronize()
        _check_rows(w32, out, 31, pct[0], pct[1], f"f16 {rows}x{cols} {pct}")
    out = ops.quantize_rows(f16_dev(h), bits=8, dq_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check_rows(w32, out, 127, 1, 1, f"f16 {rows}x{cols} int8 bf16 dq", dq_bf16=True)


@pytest.mark.parametrize("per_tensor", [False, True])
def test_f16_input_export_model(per_tensor):
    """The 9-layer set as fp16 weights: int6 99.99th-percentile rows (or per-tensor clips), int8
    tok_emb, fp16 passthrough of the vectors (an identity on fp16 input), fp32 dequant."""
    say(f"fp16 9-layer export, per_tensor={per_tensor}")
    named = [(t.name, oracle.f32_to_f16(t.data)) for t in synth.config2()]
    ex = ops.Exporter([ops.ExportTensor(nm, f16_dev(h)) for nm, h in named],
                      ops.make_policy(per_tensor=per_tensor), want_dq=True)
    ex.run()
    ex.run()
    torch.cuda.synchronize()
    assert int(ex.status.item()) == 0
    outs = ex.outputs()
    ref = oracle.export([(nm, oracle.f16_to_f32(h)) for nm, h in named], oracle.Policy(per_tensor=per_tensor))
    for o, r, (nm, h) in zip(outs, ref, named):
        assert o["kind"] == r["kind"], (nm, o["kind"], r["kind"])
        if r["kind"] == oracle.KIND_F16:
            same_bits(u16(o["f16"]).reshape(-1), r["f16"].reshape(-1), nm + " f16")
            same_bits(u16(o["f16"]).reshape(-1), np.asarray(h).reshape(-1), nm + " f16 identity")
        else:
            same_bits(o["codes"].cpu().numpy().reshape(r["codes"].shape), r["codes"], nm + " codes")
            same_bits(u16(o["scales"]), r["scales"], nm + " scales")
        f32_bits_equal(f32(o["dq"]).reshape(-1), r["dq"].reshape(-1), nm + " dq")


def test_awq_single_matrix():
    say("awq single matrix")
    ts = synth.config4()
    t = [x for x in ts if x.awq_s is not None][5]
    out = ops.quantize_rows(dev(t.data), bits=6, awq_s=dev(t.awq_s))
    torch.cuda.synchronize()
    a, st = oracle.awq_multipliers(t.awq_s)
    same_bits(u16(out["awq"]), a, "awq multipliers")
    _check_rows(t.data, out, 31, 1, 1, "awq", awq_bits=a)


# ---------------------------------------------------------------------------------------------
def _export_and_check(tensors, pol_kwargs, oracle_pol, awq=None, want_dq=True, check_names=None):
    ex = ops.Exporter([ops.ExportTensor(t.name, dev(t.data), None if t.awq_s is None else dev(t.awq_s))
                       for t in tensors], ops.make_policy(**pol_kwargs), want_dq=want_dq)
    ex.run()
    torch.cuda.synchronize()
    outs = ex.outputs()
    assert int(ex.status.item()) == 0
    sel = [i for i, t in enumerate(tensors) if check_names is None or t.name in check_names]
    ref = oracle.export([(tensors[i].name, tensors[i].data) for i in sel], oracle_pol,
                        awq=awq)
    for i, r in zip(sel, ref):
        o = outs[i]
        assert o["kind"] == r["kind"], (tensors[i].name, o["kind"], r["kind"])
        nm = tensors[i].name
        if r["kind"] == oracle.KIND_F16:
            same_bits(u16(o["f16"]).reshape(-1), r["f16"].reshape(-1), nm + " f16")
        else:
            same_bits(o["codes"].cpu().numpy(), r["codes"], nm + " codes")
            same_bits(u16(o["scales"]), r["scales"], nm + " scales")
            if "awq" in r:
                same_bits(u16(o["awq"]), r["awq"], nm + " awq")
        if want_dq:
            f32_bits_equal(f32(o["dq"]).reshape(-1), r["dq"].reshape(-1), nm + " dq")
    return ex


def test_config2_export_full():
    say("config2 export, every tensor")
    _export_and_check(synth.config2(), {}, oracle.Policy())


def test_config4_awq_export_full():
    say("config4 AWQ mixed-bit export, every tensor")
    ts = synth.config4()
    _export_and_check(ts, {"q_default": (6, 1, 1)}, oracle.Policy(q6=(6, 1, 1)),
                      awq={t.name: t.awq_s for t in ts if t.awq_s is not None})


def test_config1_batch_export_sampled():
    say("config1 x128 grouped quantize+dequant, sampled matrices")
    ts = synth.config1_batch(128)
    pick = {ts[i].name for i in (0, 1, 63, 127)}
    _export_and_check(ts, {"int8_patterns": (), "passthrough_below": 0, "q_default": (6, 1, 1)},
                      oracle.Policy(int8_patterns=(), passthrough_below=0, q6=(6, 1, 1)), check_names=pick)


def test_stress_s1_percentile_export():
    ts = synth.stress_s1()
    for pct in [(99, 100), (999, 1000), (1, 2)]:
        say(f"S1 heavy tails, percentile {pct}")
        _export_and_check(ts, {"q_default": (6,) + pct}, oracle.Policy(q6=(6,) + pct), want_dq=True,
                          check_names={t.name for t in ts[:14]} | {"tok_emb.weight"})


def test_stress_s2_long_rows_sampled():
    ts = synth.stress_s2()
    for pct in [(1, 1), (9999, 10000), (99, 100)]:
        say(f"S2 long rows {pct}")
        for t in ts:
            out = ops.quantize_rows(dev(t.data), bits=6, pct=pct)
            torch.cuda.synchronize()
            rows = [0, 1, t.data.shape[0] // 2, t.data.shape[0] - 1]
            ref = oracle.quantize_rows(t.data[rows], 31, *pct)
            same_bits(u16(out["scales"])[rows], ref["scales"], f"{t.name} scales")
            same_bits(out["codes"].cpu().numpy()[rows], ref["codes"], f"{t.name} codes")
            f32_bits_equal(f32(out["dq"])[rows], ref["dq"], f"{t.name} dq")


# ---------------------------------------------------------------------------------------------
def _fq_check(ws, gs, fq, num, den, what, check_grad=True, idx=None):
    idx = range(len(ws)) if idx is None else idx
    for i in idx:
        ref = oracle.fakequant_rows(ws[i].data, 31, num, den, g_bf16=gs[i].data if gs is not None else None)
        same_bits(u16(fq.dq[i]), ref["dq"], f"{what} {ws[i].name} dq")
        same_bits(u16(fq.scales[i]), ref["scales"], f"{what} {ws[i].name} scales")
        same_bits(fq.mask[i].cpu().numpy(), ref["mask"], f"{what} {ws[i].name} mask")
        if check_grad:
            same_bits(u16(fq.grad_out[i]), ref["g_out"], f"{what} {ws[i].name} grad_out")


def test_config3_fakequant_fwd_bwd():
    say("config3 STE fwd+bwd, 11 layers, steps 0..2")
    ws = synth.config3_weights()
    wd = [bf16_dev(t.data) for t in ws]
    fq = ops.FakeQuant(wd)
    for step in range(3):
        gs = synth.config3_grads(step)
        gd = [bf16_dev(g.data) for g in gs]
        fq.run(pgq.PGQ_FQ_FWD_BWD, gd)
        torch.cuda.synchronize()
        _fq_check(ws, gs, fq, 1, 1, f"step{step}", idx=range(0, len(ws), 1 if step == 0 else 7))
    assert int(fq.status.item()) == 0


def test_config3_fwd_then_bwd():
    say("config3 STE FWD then BWD as separate calls")
    ws = synth.config3_weights(layers=2)
    gs = synth.config3_grads(5, layers=2)
    wd = [bf16_dev(t.data) for t in ws]
    gd = [bf16_dev(g.data) for g in gs]
    fq = ops.FakeQuant(wd)
    fq.run(pgq.PGQ_FQ_FWD)
    fq.run(pgq.PGQ_FQ_BWD, gd)
    torch.cuda.synchronize()
    _fq_check(ws, gs, fq, 1, 1, "fwd/bwd")


def test_stress_s4_fakequant_percentile():
    ws = synth.stress_s4_weights(layers=1)
    gs = synth.config3_grads(9, layers=1)
    wd = [bf16_dev(t.data) for t in ws]
    gd = [bf16_dev(g.data) for g in gs]
    for pct in [(99, 100), (1, 2)]:
        say(f"S4 STE with percentile {pct}")
        fq = ops.FakeQuant(wd, pct=pct)
        fq.run(pgq.PGQ_FQ_FWD_BWD, gd)
        torch.cuda.synchronize()
        _fq_check(ws, gs, fq, pct[0], pct[1], f"S4 {pct}")
        zeros = sum(int((m.cpu().numpy() != 0xFF).sum()) for m in fq.mask)
        assert zeros > 0  # the clip leaves some gradients masked


@pytest.mark.parametrize("rows,cols", [(3, 5), (4, 17), (2, 100), (5, 528), (2, 3001)])
def test_fakequant_ragged(rows, cols):
    say(f"STE ragged {rows}x{cols}")
    rng = np.random.default_rng(cols)
    wb = oracle.f32_to_bf16((rng.standard_normal((rows, cols)) * 0.02).astype(np.float32))
    gb = oracle.f32_to_bf16((rng.standard_normal((rows, cols)) * 1e-4).astype(np.float32))

    class T:
        pass
    w = T(); w.data = wb; w.name = "w"
    g = T(); g.data = gb; g.name = "g"
    fq = ops.FakeQuant([bf16_dev(wb)], pct=(1, 2))
    fq.run(pgq.PGQ_FQ_FWD_BWD, [bf16_dev(gb)])
    torch.cuda.synchronize()
    _fq_check([w], [g], fq, 1, 2, f"{rows}x{cols}")


@pytest.mark.parametrize("rows,cols", [(1583, 528), (7, 528), (1, 528), (13, 600), (9, 1040), (6, 2056)])
@pytest.mark.parametrize("mode", ["fwd_bwd", "fwd_codes"])
def test_fakequant_flat_groups(rows, cols, mode):
    """Dense absmax STE rows of widths that leave a partial chunk instruction per row go through
    the flattened row groups (4 rows of 528 share 5 chunk instructions); ragged last groups."""
    say(f"STE flat groups {rows}x{cols} {mode}")
    rng = np.random.default_rng(rows * 7 + cols)
    wb = oracle.f32_to_bf16((rng.standard_normal((rows, cols)) * 0.02).astype(np.float32))
    gb = oracle.f32_to_bf16((rng.standard_normal((rows, cols)) * 1e-4).astype(np.float32))

    class T:
        pass
    w = T(); w.data = wb; w.name = "w"
    g = T(); g.data = gb; g.name = "g"
    fq = ops.FakeQuant([bf16_dev(wb)], want_codes=(mode == "fwd_codes"))
    if mode == "fwd_bwd":
        fq.run(pgq.PGQ_FQ_FWD_BWD, [bf16_dev(gb)])
    else:
        fq.run(pgq.PGQ_FQ_FWD)
    torch.cuda.synchronize()
    _fq_check([w], [g] if mode == "fwd_bwd" else None, fq, 1, 1, f"flat {rows}x{cols}",
              check_grad=(mode == "fwd_bwd"))
    if mode == "fwd_codes":
        ref = oracle.fakequant_rows(wb, 31)
        same_bits(fq.codes[0].cpu().numpy(), ref["codes"], "flat codes")
    assert int(fq.status.item()) == 0


# ---------------------------------------------------------------------------------------------
def test_config5_sqwa_full_run_sampled():
    say("config5 SQWA, 16 snapshots, final requant")
    base = synth.config5_base()
    pol = oracle.Policy(int8_patterns=(), q6=(6, 9999, 10000))
    sq = ops.Sqwa([ops.ExportTensor(t.name, dev(t.data)) for t in base], ops.make_policy(int8_patterns=()))
    pick = [0, 1, 2, 6, 7, 8, 63]
    ref_means = None
    for k in range(1, 17):
        snap = synth.config5_snapshot(k, base)
        sq.accumulate([dev(t.data) for t in snap], k)
        ref_means = oracle.sqwa_run([[(snap[i].name, snap[i].data) for i in pick]], pol, k0=k, means=ref_means)
    torch.cuda.synchronize()
    assert int(sq.status.item()) == 0
    for j, i in enumerate(pick):
        f32_bits_equal(f32(sq.means[i]), ref_means[j], f"mean {base[i].name}")
    ex = sq.exporter(want_dq=True)
    ex.run()
    torch.cuda.synchronize()
    outs = ex.outputs()
    ref = oracle.export([(base[i].name, ref_means[j]) for j, i in enumerate(pick)], pol)
    for j, i in enumerate(pick):
        r, o = ref[j], outs[i]
        if r["kind"] == oracle.KIND_F16:
            same_bits(u16(o["f16"]).reshape(-1), r["f16"].reshape(-1), "final f16")
        else:
            same_bits(o["codes"].cpu().numpy(), r["codes"], "final codes " + base[i].name)
            same_bits(u16(o["scales"]), r["scales"], "final scales")


def test_sqwa_resume_equals_uninterrupted():
    say("SQWA resume after snapshot 8")
    base = synth.config5_base()[:9]
    tens = [ops.ExportTensor(t.name, dev(t.data)) for t in base]
    pol = ops.make_policy(int8_patterns=())
    full = ops.Sqwa(tens, pol)
    part = ops.Sqwa(tens, pol)
    snaps = [[dev(t.data) for t in synth.config5_snapshot(k, base)] for k in range(1, 12)]
    for k, s in enumerate(snaps, 1):
        full.accumulate(s, k)
        if k <= 8:
            part.accumulate(s, k)
    saved = [m.cpu() for m in part.means]
    for m, sv in zip(part.means, saved):
        m.copy_(sv.to("cuda"))
    for k in range(9, 12):
        part.accumulate(snaps[k - 1], k)
    torch.cuda.synchronize()
    for a, b in zip(full.means, part.means):
        same_bits(f32(a), f32(b), "resume")


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("cols", [700, 1536, 2000, 3000])
def test_select_every_rank_path(cols):
    """Exact order statistics for ranks on both sides of each select strategy (iterated maximum
    up to 8, candidate packing up to 64, radix above), on continuous rows, rows with heavy ties
    (a 7-value alphabet, so more than 64 keys can tie at the bound) and sparse spiky rows."""
    rng = np.random.default_rng(cols)
    cont = (rng.standard_normal((4, cols)) * 0.02).astype(np.float32)
    ties = (rng.integers(-3, 4, (4, cols)) * 0.01).astype(np.float32)
    spiky = np.zeros((4, cols), np.float32)
    for r in range(4):
        idx = rng.choice(cols, 40 + 10 * r, replace=False)
        spiky[r, idx] = (rng.standard_normal(idx.size) * (r + 1)).astype(np.float32)
    w = np.concatenate([cont, ties, spiky])
    for rank in [1, 2, 7, 8, 9, 16, 33, 40, 63, 64, 65, 100]:
        say(f"select {w.shape[0]}x{cols} rank {rank}")
        num, den = cols - rank + 1, cols             # k = n - rank + 1: the rank-th largest |w|
        out = ops.quantize_rows(dev(w), bits=6, pct=(num, den))
        torch.cuda.synchronize()
        _check_rows(w, out, 31, num, den, f"select {cols} rank {rank}")


@pytest.mark.parametrize("cols", [512, 528, 1536, 2000])
def test_select_top_keys_sharing_lanes(cols):
    """Ranks 2-25 from the top, with the largest keys placed where they share a lane: a run of
    consecutive elements (one 16- or 32-byte slot), every 64th element (one lane of the
    element-wise layouts), pairs of keys per slot (two per lane, the most the two-largest
    path accepts), and copies of one value tying at the answer."""
    rng = np.random.default_rng(cols + 7)
    base = (rng.standard_normal((6, cols)) * 0.02).astype(np.float32)
    w = base.copy()
    big = (np.arange(30, 0, -1) * 0.05).astype(np.float32)
    w[0, :8] = big[:8]                               # one run of consecutive elements
    w[1, 0:64 * 6:64] = big[:6]                      # every 64th element
    w[2, 8:16] = -big[:8]                            # a run of negatives
    for k in range(12):                              # two keys per 4-element slot
        w[3, 8 * k] = big[2 * k]
        w[3, 8 * k + 1] = -big[2 * k + 1]
    w[4, 0:64 * 10:64] = 0.75                        # ten copies of one key, one lane
    w[4, 3:3 + 64 * 10:64] = 0.75                    # and ten in another
    w[5, :4] = 0.75                                  # a tie inside one slot, more copies elsewhere
    w[5, 100:1000:100] = 0.75 if cols > 900 else 0.5
    for rank in [2, 3, 4, 5, 6, 9, 12, 16, 20, 24, 25]:
        say(f"select lanes {w.shape[0]}x{cols} rank {rank}")
        num, den = cols - rank + 1, cols
        out = ops.quantize_rows(dev(w), bits=6, pct=(num, den))
        torch.cuda.synchronize()
        _check_rows(w, out, 31, num, den, f"select lanes {cols} rank {rank}")


def test_edge_rows_and_status_bits():
    say("edge rows: zeros, spike, constant, grid, ties, tiny")
    n = 512
    s0 = float(np.array([0x2A3D], np.uint16).view(np.float16)[0])
    rows = [np.zeros(n), np.full(n, -0.0)]
    spike = np.zeros(n); spike[77] = -0.37; rows.append(spike)
    rows.append(np.full(n, 0.25))
    rng = np.random.default_rng(1)
    m = rng.integers(-31, 32, n); m[3] = 31; rows.append(m * s0)
    t = (np.arange(n) % 62 - 31 + 0.5) * s0; t[0] = 31 * s0; rows.append(t)
    tiny = np.zeros(n); tiny[9] = 31 * 2.0 ** -26; rows.append(tiny)
    sub = rng.standard_normal(n) * 1e-6; rows.append(sub)
    w = np.array(rows, dtype=np.float32)
    for pct in [(1, 1), (99, 100)]:
        out = ops.quantize_rows(dev(w), bits=6, pct=pct)
        torch.cuda.synchronize()
        _check_rows(w, out, 31, pct[0], pct[1], f"edge {pct}")
        assert int(out["status"].item()) == 0
    say("status bits: NaN, Inf, scale overflow")
    bad = np.zeros((3, 64), np.float32)
    bad[0, 5] = np.nan
    bad[1, 6] = np.inf
    bad[2, 7] = 2_031_120.0
    for r, bit in [(0, pgq.PGQ_DEV_NONFINITE), (1, pgq.PGQ_DEV_NONFINITE), (2, pgq.PGQ_DEV_SCALE_OVF)]:
        out = ops.quantize_rows(dev(bad[r:r + 1]), bits=6)
        torch.cuda.synchronize()
        assert int(out["status"].item()) & bit
    say("status bits: fp16 passthrough overflow, bad AWQ scale")
    ex = ops.Exporter([ops.ExportTensor("v", dev(np.array([1.0, 7e4], np.float32)))], want_dq=False)
    ex.run()
    torch.cuda.synchronize()
    assert int(ex.status.item()) == pgq.PGQ_DEV_F16_OVF
    s = np.ones(512, np.float32); s[3] = 0.0
    out = ops.quantize_rows(dev(synth.config1().data[:4]), bits=6, awq_s=dev(s))
    torch.cuda.synchronize()
    assert int(out["status"].item()) & pgq.PGQ_DEV_BAD_AWQ


def test_stale_table_is_detected_and_writes_nothing():
    say("stale descriptor table")
    a = synth.config2()[:3]
    b = synth.config2(cfg_id=7)[:3]
    ea = ops.Exporter([ops.ExportTensor(t.name, dev(t.data)) for t in a])
    eb = ops.Exporter([ops.ExportTensor(t.name, dev(t.data)) for t in b])
    ea.run()
    eb.arena.fill_(0x5A)
    eb.workspace = ea.workspace   # eb's table is not in this workspace
    eb._uploaded = True
    eb.run(reuse_table=True)
    torch.cuda.synchronize()
    assert int(eb.status.item()) & pgq.PGQ_DEV_STALE_TABLE
    assert bool((eb.arena == 0x5A).all())


def test_deterministic_repeat():
    say("determinism")
    ts = synth.stress_s1()[:8]
    ex = ops.Exporter([ops.ExportTensor(t.name, dev(t.data)) for t in ts],
                      ops.make_policy(q_default=(6, 99, 100)), want_dq=True)
    ex.run()
    torch.cuda.synchronize()
    first = ex.arena.clone()
    ex.arena.fill_(0)
    ex.run(reuse_table=False)
    ex.run(reuse_table=True)
    torch.cuda.synchronize()
    assert torch.equal(first, ex.arena)


def test_empty_inputs_are_noops():
    say("empty inputs")
    z = torch.empty(0, 512, dtype=torch.float32, device="cuda")
    st = ops.new_status()
    rc = pgq.pgq_quantize_rows(z.data_ptr(), pgq.PGQ_F32, 0, 512, 512, ops.qparams(6), None, None, None,
                               None, None, pgq.PGQ_F32, st.data_ptr(), ops._stream())
    assert rc == pgq.PGQ_OK
    fq = pgq.pgq_fakequant_fwd_bwd(pgq.PGQ_FQ_FWD, None, 0, ops.qparams(6), None, 0, 0, None, ops._stream())
    assert fq == pgq.PGQ_OK


def test_binding_loaded_before_torch():
    """A process that imports the binding before PyTorch still runs one HIP runtime."""
    say("binding imported before torch (subprocess)")
    import subprocess
    code = ("import int6_weight_export_amd.pgq as pgq\n"
            "import torch\n"
            "from int6_weight_export_amd import ops\n"
            "w = torch.randn(64, 512, device='cuda') * 0.02\n"
            "out = ops.quantize_rows(w, bits=6)\n"
            "torch.cuda.synchronize()\n"
            "assert int(out['status'].item()) == 0\n"
            "print('ok')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=100)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]
