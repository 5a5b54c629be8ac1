"""Brute-force pins of the oracle in exact rational arithmetic on tiny matrices.

For 4 x 8 matrices whose entries come from small alphabets built around a binary16
grid step s0 (grid points, exact ties, their binary32 neighbours, zeros of both signs,
repeated magnitudes, values beyond the clip, binary16-subnormal steps), every output
is recomputed from the definitions with fractions.Fraction:
  * the clip is the k-th smallest |x| by sorting, k = ceil(p n);
  * the scale is the binary16 value nearest to the exact clip / Q (1 when that is 0);
  * the code is found by trying every integer in [-Q, Q];
  * the STE mask is |x| <= (Q + 1/2) s evaluated exactly;
  * AWQ: x' = RN32(w a), dequant = RN32(q s / a);
  * SQWA: mean = RN32(mean + RN32(RN32(xhat - mean) / k));
  * EMA: e = RN32(RN32(d e) + RN32(c w)) with d = RN32(0.997), c = RN32(1 - d), which a fused
    multiply-add or the e + c (w - e) form would not reproduce;
  * SWA: the SQWA running mean on the weights themselves.
A dropped term, a wrong sign, an off-by-one rank or a wrong tie rule in the oracle
changes at least one of these values.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact as ex

PCTS = [(1, 1), (9999, 10000), (7, 8), (1, 2), (1, 8)]


def _alphabet(s0: float, Q: int, rng) -> list:
    vals = [0.0, -0.0, Q * s0, -Q * s0]
    for _ in range(6):
        m = int(rng.integers(0, Q + 1))
        g = np.float32(m * s0)
        tie = np.float32((m + 0.5) * s0)
        vals += [float(g), float(tie), float(np.nextafter(tie, np.float32(np.inf))),
                 float(np.nextafter(tie, np.float32(-np.inf)))]
    vals += [(Q + 0.5) * s0, (Q + 1) * s0, 0.75 * s0, s0 / 1024]
    out = []
    for v in vals:
        f = np.float32(v)
        out += [float(f), float(-f)]
    return out


def _s0_choices():
    # binary16 steps across binades, including subnormal steps and powers of two
    bits = [0x3C00, 0x1E66, 0x2A3D, 0x07FF, 0x0400, 0x1400, 0x3555, 0x4BFF, 0x0123, 0x0001, 0x0200,
            0x2000, 0x1BAD, 0x33C1]
    return [float(np.array([b], dtype=np.uint16).view(np.float16)[0]) for b in bits]


def _matrices(Q: int, count: int, seed: int):
    rng = np.random.default_rng(seed)
    s0s = _s0_choices()
    for i in range(count):
        s0 = s0s[i % len(s0s)]
        alpha = _alphabet(s0, Q, rng)
        m = np.array(rng.choice(alpha, size=(4, 8)), dtype=np.float32)
        if i % 3 == 0:   # force the grid maximum into each row so that ties are exact
            m[:, int(rng.integers(0, 8))] = np.float32(Q * s0) * np.float32(rng.choice([-1, 1]))
        if i % 7 == 0:   # repeated magnitudes
            m[:, 1] = -m[:, 0]
        yield m


def _exact_row(x_row, Q, num, den, a=None):
    xs = [ex.frac(v) for v in x_row]
    if a is not None:
        xs = [ex.rn_f32(x * ex.f16_value(int(aj))) for x, aj in zip(xs, a)]
    k = ex.ceil_rank(len(xs), num, den)
    clip = ex.kth_smallest_abs(xs, k)
    sb = ex.rn_f16_bits(clip / Q)
    if sb & 0x7FFF == 0:
        sb = 0x3C00
    s = ex.f16_value(sb)
    codes = [ex.brute_code(x, s, Q) for x in xs]
    if a is None:
        dq = [ex.rn_f32(q * s) for q in codes]
    else:
        dq = [ex.rn_f32(q * s / ex.f16_value(int(aj))) for q, aj in zip(codes, a)]
    mask = [abs(x) <= (Q + Fraction(1, 2)) * s for x in xs]
    return sb, codes, dq, mask, clip


@pytest.mark.parametrize("Q,count", [(31, 56), (127, 14)])
@pytest.mark.parametrize("num,den", PCTS)
def test_quantize_rows_bruteforce(orc, Q, count, num, den):
    checked = 0
    for m in _matrices(Q, count, seed=Q * 1000 + num % 97):
        r = oracle.quantize_rows(m, Q, num, den, want_clip=True)
        for i in range(m.shape[0]):
            sb, codes, dq, _, clip = _exact_row(m[i], Q, num, den)
            if sb & 0x7C00 == 0x7C00:
                continue
            assert ex.frac(r["clip"][i]) == clip
            assert int(r["scales"][i]) == sb, (m[i], hex(int(r["scales"][i])), hex(sb))
            assert r["codes"][i].tolist() == codes, (m[i], r["codes"][i], codes)
            assert [ex.frac(v) for v in r["dq"][i]] == dq
            checked += 1
    assert checked > 0


def test_fakequant_mask_bruteforce(orc):
    """bfloat16 rows with a percentile clip so that |x/s| reaches Q + 1/2 and beyond.
    Steps s0 are powers of two, so (Q + 1/2) s0 and its bfloat16 neighbours are exact."""
    rng = np.random.default_rng(7)
    Q = 31
    checked_edge = 0
    for e in range(-20, 3):
        s0 = 2.0 ** e
        edge = np.float32(31.5 * s0)
        pool = [0.0, s0 * 31, s0 * 31.5, s0 * 32, s0 * 3.5, s0 * 4.5, s0 * 40, s0 * 0.5]
        bf = oracle.f32_to_bf16(np.array(pool, dtype=np.float32))
        up = bf.copy() + 1
        dn = bf.copy() - 1
        cand = np.concatenate([bf, up[1:], dn[1:], bf | 0x8000]).astype(np.uint16)
        for _ in range(6):
            row = rng.choice(cand, size=(4, 16))
            row[:, 0] = oracle.f32_to_bf16(np.array([31 * s0], dtype=np.float32))[0]
            g = rng.integers(0, 0xFFFF, size=row.shape).astype(np.uint16)
            g &= 0xBFFF  # finite gradients
            for num, den in [(1, 1), (1, 2), (3, 4)]:
                r = oracle.fakequant_rows(row, Q, num, den, g_bf16=g)
                x32 = oracle.bf16_to_f32(row)
                for i in range(row.shape[0]):
                    sb, codes, dq, mask, _ = _exact_row(x32[i], Q, num, den)
                    bits = np.unpackbits(r["mask"][i], bitorder="little")[: row.shape[1]].astype(bool)
                    assert bits.tolist() == mask
                    assert int(r["scales"][i]) == sb
                    assert r["codes"][i].tolist() == codes
                    want_dq = oracle.f32_to_bf16(np.array([float(v) for v in dq], dtype=np.float32))
                    assert np.array_equal(r["dq"][i], want_dq)
                    want_g = np.where(bits, g[i], 0).astype(np.uint16)
                    assert np.array_equal(r["g_out"][i], want_g)
                    checked_edge += int(np.any(np.abs(x32[i]) == edge) and num != 1)
    assert checked_edge > 0


def test_awq_bruteforce(orc):
    rng = np.random.default_rng(11)
    Q = 31
    for it in range(20):
        s = np.exp(rng.normal(0, 0.5, size=8)).astype(np.float32)
        if it % 4 == 0:
            s[:3] = np.float32([1.0, 4.0, 0.25])
        a, st = oracle.awq_multipliers(s)
        assert st == 0
        for j in range(8):
            assert int(a[j]) == ex.rn_f16_bits(ex.rn_sqrt32(ex.frac(s[j])))
        w = (rng.normal(0, 0.02, size=(4, 8))).astype(np.float32)
        r = oracle.quantize_rows(w, Q, 1, 1, awq=a)
        for i in range(4):
            sb, codes, dq, _, _ = _exact_row(w[i], Q, 1, 1, a=a)
            assert int(r["scales"][i]) == sb
            assert r["codes"][i].tolist() == codes
            assert [ex.frac(v) for v in r["dq"][i]] == dq


def test_sqwa_update_exact(orc):
    rng = np.random.default_rng(5)
    n = 64
    mean = np.empty(n, dtype=np.float32)
    ref = [Fraction(0)] * n
    for k in range(1, 17):
        x = (rng.normal(0, 0.02, n) * (1 + k)).astype(np.float32)
        oracle.sqwa_update(mean, x, k)
        xs = [ex.frac(v) for v in x]
        if k == 1:
            ref = xs
        else:
            ref = [ex.rn_f32(m + ex.rn_f32(ex.rn_f32(v - m) / k)) for m, v in zip(ref, xs)]
        assert [ex.frac(v) for v in mean] == ref, k


def test_ema_update_exact(orc):
    """Twelve updates of 64 averages, each element recomputed in exact arithmetic and rounded
    to binary32 after every operation of the update (Weight Averaging, decay 0.997)."""
    rng = np.random.default_rng(6)
    n = 64
    e = rng.normal(0, 0.02, n).astype(np.float32)
    e[:3] = np.float32([0.0, -0.0, 1e-39])
    ref = [ex.frac(v) for v in e]
    d = ex.frac(np.float32(0.997))
    c = ex.rn_f32(1 - d)
    assert c == ex.frac(np.float32(1.0) - np.float32(0.997))
    for step in range(12):
        w = (rng.normal(0, 0.02, n) * (1 + step)).astype(np.float32)
        w[3] = np.float32(-e[3]) if step == 0 else w[3]
        assert oracle.ema_update(e, w, 0.997) == 0
        ref = [ex.rn_f32(ex.rn_f32(d * m) + ex.rn_f32(c * ex.frac(v))) for m, v in zip(ref, w)]
        assert [ex.frac(v) for v in e] == ref, step
    # an FMA-style single rounding differs from the two-product form on some element
    fused = [ex.rn_f32(d * m + ex.rn_f32(c * ex.frac(v))) for m, v in zip(ref, w)]
    assert fused != [ex.rn_f32(ex.rn_f32(d * m) + ex.rn_f32(c * ex.frac(v))) for m, v in zip(ref, w)]


def test_swa_update_exact(orc):
    rng = np.random.default_rng(7)
    n = 64
    mean = np.empty(n, dtype=np.float32)
    ref = []
    for k in range(1, 17):
        w = rng.normal(0, 0.02, n).astype(np.float32)
        assert oracle.swa_update(mean, w, k) == 0
        ws = [ex.frac(v) for v in w]
        ref = ws if k == 1 else [ex.rn_f32(m + ex.rn_f32(ex.rn_f32(v - m) / k)) for m, v in zip(ref, ws)]
        assert [ex.frac(v) for v in mean] == ref, k
