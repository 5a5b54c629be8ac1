"""Pins of the oracle's per-tensor quantization ("Per-row / per-tensor quantization strategy"
and "Percentile clipping for stable int8 export", PR #2159 Key Explored Modifications).

One scale per tensor: the clip is the k-th smallest |w| over the whole tensor (k = ceil(p n)),
s = fp16(fl32(clip / Q)), codes clamp(rne(fl32(w / s))).  Checked against numpy's own
partition, float32 division, float16 rounding and rint, and against closed forms.
"""
import math

import numpy as np
import pytest

import oracle


def _w(seed, shape, dist="normal"):
    rng = np.random.default_rng(seed)
    if dist == "t3":
        return (rng.standard_t(3, shape) * 0.02).astype(np.float32)
    return (rng.standard_normal(shape) * 0.02).astype(np.float32)


@pytest.mark.parametrize("num,den", [(1, 1), (9999, 10000), (99, 100), (1, 2), (1, 1000)])
@pytest.mark.parametrize("shape,dist", [((64, 512), "normal"), ((37, 129), "t3"), ((1, 4096), "normal")])
def test_tensor_clip_scale_and_codes_match_numpy(num, den, shape, dist):
    w = _w(sum(shape) + num, shape, dist)
    Q = 31
    r = oracle.quantize_tensor(w, Q, num, den)
    n = w.size
    k = -(-num * n // den)                                  # ceil in integers
    clip = np.partition(np.abs(w).ravel(), k - 1)[k - 1]
    assert r["clip"] == clip
    s16 = np.float16(np.float32(clip) / np.float32(Q))
    if s16 == 0:
        s16 = np.float16(1.0)
    assert r["scale"][0] == s16.view(np.uint16)
    s = np.float32(s16)
    codes = np.clip(np.rint(w / s), -Q, Q).astype(np.int8)
    assert np.array_equal(r["codes"], codes)
    assert np.array_equal(r["dq"], codes.astype(np.float32) * s)
    # reconstruction error of the entries inside the code range is at most half a step (the
    # fp16 scale may round below clip / Q, so the range ends at Q s rather than at the clip)
    keep = np.abs(w.astype(np.float64)) <= Q * np.float64(s)
    assert np.all(np.abs(w[keep].astype(np.float64) - r["dq"][keep]) <= s / 2 * (1 + 2 ** -20))


def test_identical_rows_give_the_per_row_result():
    row = _w(3, (1, 300))
    w = np.repeat(row, 9, axis=0)
    for num, den in [(1, 1), (99, 100)]:
        t = oracle.quantize_tensor(w, 31, num, den)
        r = oracle.quantize_rows(w, 31, num, den)
        # the k-th of 9 copies of each value is the ceil(k/9)-th of one row: equal for these p
        assert np.all(r["scales"] == t["scale"][0])
        assert np.array_equal(r["codes"], t["codes"])


def test_one_row_tensor_is_the_row_quantizer():
    w = _w(4, (1, 1000), "t3")
    t = oracle.quantize_tensor(w, 127, 999, 1000)
    r = oracle.quantize_rows(w, 127, 999, 1000)
    assert t["scale"][0] == r["scales"][0]
    assert np.array_equal(t["codes"], r["codes"])


def test_tensor_scale_is_shared_and_spike_sets_it():
    w = _w(5, (16, 64))
    w[7, 9] = 3.1
    t = oracle.quantize_tensor(w, 31, 1, 1)
    assert t["scale"][0] == np.float16(np.float32(3.1) / np.float32(31)).view(np.uint16)
    assert t["codes"][7, 9] == 31
    # every other entry is tiny next to the spike: most codes round to zero
    assert np.mean(t["codes"] == 0) > 0.9


def test_policy_per_tensor_export():
    ts = [("tok_emb.weight", _w(6, (256, 512))), ("blocks.0.attn.wq.weight", _w(7, (512, 512))),
          ("blocks.0.attn_scale", _w(8, (512,)))]
    pol = oracle.Policy(per_tensor=True)
    out = oracle.export(ts, pol)
    assert out[0]["kind"] == oracle.KIND_INT8 and out[0]["scales"].shape == (1,)
    assert out[1]["kind"] == oracle.KIND_INT6 and out[1]["scales"].shape == (1,)
    assert out[2]["kind"] == oracle.KIND_F16
    k = math.ceil(0.9999 * 512 * 512)
    clip = np.partition(np.abs(ts[1][1]).ravel(), k - 1)[k - 1]
    assert out[1]["scales"][0] == np.float16(np.float32(clip) / np.float32(31)).view(np.uint16)
    with pytest.raises(ValueError):
        oracle.export(ts[1:2], pol, awq={"blocks.0.attn.wq.weight": np.ones(512, np.float32)})


def test_tensor_nonfinite_status():
    w = _w(9, (8, 32))
    w[3, 3] = np.nan
    assert oracle.quantize_tensor(w, 31)["status"] & oracle.ORC_NONFINITE
