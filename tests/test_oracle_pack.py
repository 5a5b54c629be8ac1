"""Pins of the oracle's 6-bit code storage and its decode.

Layout (the pages give none; our reading of the int6 artifact savings the PR #69 card names):
per row, four 6-bit two's-complement codes per three bytes, least significant bits first.
Checked against a hand-worked group, an independent bit-level unpacking with numpy, exhaustive
round trips, and the decode against the export's own dequantized values and numpy float32.
"""
import numpy as np
import pytest

import oracle


def test_hand_worked_group():
    # codes 1, -1, 31, -31 -> fields 0x01, 0x3F, 0x1F, 0x21 -> 24-bit word 0x85FFC1
    p = oracle.pack6(np.array([[1, -1, 31, -31]], np.int8))
    assert p.tolist() == [[0xC1, 0xFF, 0x85]]
    # a short last group is padded with code 0
    p = oracle.pack6(np.array([[1, -1, 31, -31, -32]], np.int8))
    assert p.tolist() == [[0xC1, 0xFF, 0x85, 0x20, 0x00, 0x00]]


@pytest.mark.parametrize("cols", [1, 2, 3, 4, 5, 7, 8, 9, 527, 528])
def test_round_trip_and_size(cols):
    rng = np.random.default_rng(cols)
    c = rng.integers(-32, 32, (5, cols)).astype(np.int8)
    p = oracle.pack6(c)
    assert p.shape == (5, 3 * ((cols + 3) // 4)) == (5, oracle.pack6_row_bytes(cols))
    assert np.array_equal(oracle.unpack6(p, cols), c)


def test_every_code_in_every_position():
    vals = np.arange(-32, 32, dtype=np.int8)
    for t in range(4):
        c = np.zeros((64, 4), np.int8)
        c[:, t] = vals
        p = oracle.pack6(c)
        # independent reading of the bytes: little-endian bit stream, 6-bit fields
        bits = np.unpackbits(p, axis=1, bitorder="little")
        field = bits[:, 6 * t:6 * t + 6].astype(np.int64) @ (1 << np.arange(6))
        signed = np.where(field >= 32, field - 64, field)
        assert np.array_equal(signed, vals.astype(np.int64))
        others = np.delete(bits.reshape(64, 4, 6), t, axis=1)
        assert not others.any()


def test_decode_matches_the_export_and_numpy():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((40, 300)) * 0.02).astype(np.float32)
    r = oracle.quantize_rows(w, 31, 99, 100)
    d = oracle.dequant(r["codes"], r["scales"])
    assert np.array_equal(d.view(np.uint32), r["dq"].view(np.uint32))
    s = r["scales"].view(np.float16).astype(np.float32)
    assert np.array_equal(d, r["codes"].astype(np.float32) * s[:, None])
    # through the 6-bit storage
    d6 = oracle.dequant(oracle.unpack6(oracle.pack6(r["codes"]), 300), r["scales"])
    assert np.array_equal(d6, d)


def test_decode_awq_and_per_tensor():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    s = np.exp(rng.standard_normal(64) * 0.5).astype(np.float32)
    a, _ = oracle.awq_multipliers(s)
    r = oracle.quantize_rows(w, 31, awq=a)
    d = oracle.dequant(r["codes"], r["scales"], awq=a)
    assert np.array_equal(d.view(np.uint32), r["dq"].view(np.uint32))
    sc = r["scales"].view(np.float16).astype(np.float32)
    ref = (r["codes"].astype(np.float32) * sc[:, None]) / a.view(np.float16).astype(np.float32)[None, :]
    assert np.array_equal(d, ref)
    t = oracle.quantize_tensor(w, 31, 9999, 10000)
    dt = oracle.dequant(t["codes"], t["scale"], per_tensor=True)
    assert np.array_equal(dt.view(np.uint32), t["dq"].view(np.uint32))


def test_policy_packs_int6_only():
    rng = np.random.default_rng(7)
    ts = [("tok_emb.weight", (rng.standard_normal((256, 512)) * 0.02).astype(np.float32)),
          ("blocks.0.mlp.up.weight", (rng.standard_normal((384, 515)) * 0.02).astype(np.float32))]
    out = oracle.export(ts, oracle.Policy(pack6=True))
    assert "packed" not in out[0]                      # int8 stays one byte per code
    assert out[1]["packed"].shape == (384, 3 * 129)
    assert np.array_equal(oracle.unpack6(out[1]["packed"], 515), out[1]["codes"])
