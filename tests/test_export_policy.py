"""Export-policy pins against the constants the pages print (tests/golden/pages_constants.json).

The synthetic weight sets must have the pages' shapes; the oracle's export must send the
named sensitive tensors to int8, small tensors to fp16 and everything else to int6, with
the byte counts those shapes imply.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


@pytest.fixture(scope="module")
def pages():
    with open(GOLD) as f:
        return json.load(f)


def test_shapes_follow_pages(pages):
    g9 = pages["gpt9"]
    ts = synth.config2()
    d, hd = g9["dim"], g9["dim"] // g9["heads"]
    by = {t.name: t.shape for t in ts}
    assert by["tok_emb.weight"] == (g9["vocab_size"], d)
    assert "lm_head.weight" not in by            # tied
    layers = {int(n.split(".")[1]) for n in by if n.startswith("blocks.")}
    assert layers == set(range(g9["layers"]))
    assert by["blocks.0.attn.wk.weight"] == (g9["kv_heads"] * hd, d)
    assert by["blocks.3.mlp.up.weight"] == (g9["hidden_dim"], d)
    assert by["blocks.8.mlp.down.weight"] == (d, g9["hidden_dim"])
    u = pages["unified11"]
    shapes3 = [t.shape for t in synth.config3_weights(layers=1)]
    assert shapes3 == [(u["mlp_multiplier"] * u["dim"], u["dim"]), (u["dim"], u["dim"]),
                       (u["mlp_multiplier"] * u["dim"], u["dim"]), (u["dim"], u["mlp_multiplier"] * u["dim"])]
    g12 = pages["gpt12"]
    ts4 = synth.config4()
    by4 = {t.name: t for t in ts4}
    for nm in g12["untied"]:
        assert by4[nm].shape == (g12["vocab_size"], 512)
    assert {int(n.split(".")[1]) for n in by4 if n.startswith("blocks.")} == set(range(g12["layers"]))


def test_default_policy_constants(pages):
    assert tuple(pages["int8_default_patterns"]["value"]) == oracle.DEFAULT_INT8_PATTERNS
    lo, hi = pages["int6_range"]["value"]
    bits = pages["int6_bits"]["value"]
    assert (lo, hi) == (-((1 << (bits - 1)) - 1), (1 << (bits - 1)) - 1)
    assert oracle.Policy().q6[0] == bits
    assert oracle.Policy().q8[0] == pages["int8_bits_embeddings"]["value"]


def test_gpt9_export_bytes(orc, pages):
    want = pages["gpt9_export_derived"]
    ts = synth.config2()
    pol = oracle.Policy()
    kinds = {t.name: oracle.tensor_kind(t.name, t.numel, pol) for t in ts}
    assert sorted(n for n, k in kinds.items() if k == oracle.KIND_INT8) == want["int8_tensors"]
    code_bytes = sum(t.numel for t in ts if kinds[t.name] != oracle.KIND_F16)
    rows = sum(oracle.as_rows(t.shape)[0] for t in ts if kinds[t.name] != oracle.KIND_F16)
    f16 = sum(t.numel for t in ts if kinds[t.name] == oracle.KIND_F16)
    assert (code_bytes, rows, f16) == (want["int_code_bytes"], want["row_scales"], want["fp16_values"])
    out = oracle.export([(t.name, t.data) for t in ts], pol)
    assert sum(r["codes"].size for r in out if "codes" in r) == want["int_code_bytes"]
    assert sum(r["scales"].size for r in out if "scales" in r) == want["row_scales"]
    assert sum(r["f16"].size for r in out if "f16" in r) == want["fp16_values"]
    for r in out:
        lim = 127 if r["kind"] == oracle.KIND_INT8 else 31
        if "codes" in r:
            assert np.abs(r["codes"].astype(np.int32)).max() <= lim
            # the int8 embedding actually uses its wider range
            if r["kind"] == oracle.KIND_INT8:
                assert np.abs(r["codes"].astype(np.int32)).max() == 127
        assert r["status"] == 0


def test_gpt12_awq_export_bytes(orc, pages):
    want = pages["gpt12_export_derived"]
    ts = synth.config4()
    pol = oracle.Policy(q6=(6, 1, 1))
    out = oracle.export([(t.name, t.data) for t in ts], pol,
                        awq={t.name: t.awq_s for t in ts if t.awq_s is not None})
    assert sorted(r["name"] for r in out if r["kind"] == oracle.KIND_INT8) == sorted(want["int8_tensors"])
    assert sum(r["codes"].size for r in out) == want["int_code_bytes"]
    assert sum(r["scales"].size for r in out) == want["row_scales"]
    assert sum(r["awq"].size for r in out if "awq" in r) == want["awq_columns"]
    assert all("awq" not in r for r in out if r["kind"] == oracle.KIND_INT8)


def test_policy_precedence():
    pol = oracle.Policy()
    # passthrough beats the int8 name match; threshold is strict
    assert oracle.tensor_kind("tok_emb.weight", 65535, pol) == oracle.KIND_F16
    assert oracle.tensor_kind("tok_emb.weight", 65536, pol) == oracle.KIND_INT8
    assert oracle.tensor_kind("model.lm_head.weight", 1 << 20, pol) == oracle.KIND_INT8  # substring
    assert oracle.tensor_kind("blocks.0.mlp.up.weight", 65536, pol) == oracle.KIND_INT6
    assert oracle.as_rows((7,)) == (1, 7)
    assert oracle.as_rows((4, 3, 5)) == (4, 15)
