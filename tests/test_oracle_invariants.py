"""Invariant, closed-form and library pins of the oracle on synthetic weight sets.

  P1  |code| <= Q everywhere (int6 range [-31, 31], int8 [-127, 127]).
  P2  |x - code * s| <= s / 2 exactly for |x| <= clip in rows with a normal binary16 scale.
  P3  quantize(dequantize(codes)) returns the same codes and scales (normal-scale rows).
  P4  closed forms: zero row, single spike, constant row, grid-aligned row, tie row.
  P5  library cross-checks: the clip equals numpy's partition of |x| at rank k; codes
      equal numpy's rint of the float32 quotient, clamped.
  --  symmetry: negating a row negates its codes and keeps its scale; permuting a row's
      columns permutes its codes; scaling a row by 2^m scales the binary16 step by 2^m.
  P8  AWQ special cases: s_j = 1 is plain quantization; s_j = 4^m gives a_j = 2^m exactly.
  P9  SQWA special cases: identical snapshots average to the snapshot's QDQ; one snapshot
      is its QDQ; two snapshots are within one binary32 ulp of their exact mean.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import exact as ex


def _f16(b):
    return oracle.f16_to_f32(np.asarray(b, dtype=np.uint16))


def _sets():
    s1 = synth.stress_s1()
    return {
        "cfg1": [synth.config1().data],
        "s1_t3": [t.data for t in s1 if t.data.ndim == 2][:14],
        "cfg2": [t.data for t in synth.config2() if t.data.ndim == 2][:14],
    }


@pytest.fixture(scope="module")
def sets():
    return _sets()


@pytest.mark.parametrize("Q,num,den", [(31, 1, 1), (31, 9999, 10000), (31, 99, 100), (31, 999, 1000),
                                       (127, 1, 1), (31, 1, 2)])
@pytest.mark.parametrize("name", ["cfg1", "s1_t3", "cfg2"])
def test_range_error_idempotence(orc, sets, name, Q, num, den):
    for w in sets[name]:
        r = oracle.quantize_rows(w, Q, num, den, want_clip=True)
        codes, sc, dq, clip = r["codes"], r["scales"], r["dq"], r["clip"]
        assert r["status"] == 0
        # P1
        assert np.abs(codes.astype(np.int32)).max() <= Q
        assert codes.min() >= -Q
        s = _f16(sc).astype(np.float64)
        normal = clip >= Q * 2.0 ** -14
        # P2 (double arithmetic is exact for these differences)
        inside = np.abs(w) <= clip[:, None]
        err = np.abs(w.astype(np.float64) - codes.astype(np.float64) * s[:, None])
        bad = inside & normal[:, None] & (err > s[:, None] / 2)
        assert not bad.any()
        # dequant is exactly code * scale
        assert np.array_equal(dq.astype(np.float64), codes.astype(np.float64) * s[:, None])
        # P3
        r2 = oracle.quantize_rows(dq, Q, num, den)
        assert np.array_equal(r2["codes"][normal], codes[normal])
        assert np.array_equal(r2["scales"][normal], sc[normal])


def test_library_crosscheck(orc, sets):
    """P5: numpy's partition and rint, used as independent library routines."""
    for w in sets["s1_t3"][:6]:
        for (Q, num, den) in [(31, 99, 100), (31, 1, 1), (127, 999, 1000)]:
            r = oracle.quantize_rows(w, Q, num, den, want_clip=True)
            n = w.shape[1]
            k = -((-num * n) // den)
            ref_clip = np.partition(np.abs(w), k - 1, axis=1)[:, k - 1]
            assert np.array_equal(r["clip"], ref_clip)
            s = _f16(r["scales"])
            ref_codes = np.clip(np.rint(w / s[:, None]), -Q, Q).astype(np.int8)
            assert np.array_equal(r["codes"], ref_codes)


def test_symmetries(orc, sets):
    rng = np.random.default_rng(3)
    w = sets["cfg2"][4]
    r = oracle.quantize_rows(w, 31, 9999, 10000)
    rn = oracle.quantize_rows(-w, 31, 9999, 10000)
    assert np.array_equal(rn["codes"], -r["codes"])
    assert np.array_equal(rn["scales"], r["scales"])
    perm = rng.permutation(w.shape[1])
    rp = oracle.quantize_rows(w[:, perm], 31, 9999, 10000)
    assert np.array_equal(rp["codes"], r["codes"][:, perm])
    assert np.array_equal(rp["scales"], r["scales"])
    for m in (-3, 2, 5):
        rs = oracle.quantize_rows(w * np.float32(2.0 ** m), 31, 9999, 10000)
        s0, s1 = _f16(r["scales"]).astype(np.float64), _f16(rs["scales"]).astype(np.float64)
        ok = (s0 * 2.0 ** m >= 2.0 ** -14) & (s0 >= 2.0 ** -14)
        assert np.array_equal(s1[ok], s0[ok] * 2.0 ** m)
        assert np.array_equal(rs["codes"][ok], r["codes"][ok])


def test_closed_forms(orc):
    Q = 31
    n = 64
    # all-zero row: scale 1.0, codes 0, dequant +0
    r = oracle.quantize_rows(np.zeros((1, n), np.float32), Q)
    assert r["scales"][0] == 0x3C00 and not r["codes"].any()
    assert np.array_equal(r["dq"].view(np.uint32), np.zeros((1, n), np.uint32))
    # negative zeros also give +0 dequant
    r = oracle.quantize_rows(np.full((1, n), -0.0, np.float32), Q)
    assert np.array_equal(r["dq"].view(np.uint32), np.zeros((1, n), np.uint32))
    # single spike v: code +-Q at the spike, zeros elsewhere, scale fp16(v / Q)
    for v in (0.037, -1.5, 3.0e-3, 100.0):
        x = np.zeros((1, n), np.float32)
        x[0, 17] = v
        r = oracle.quantize_rows(x, Q)
        assert r["codes"][0, 17] == (Q if v > 0 else -Q)
        assert np.count_nonzero(r["codes"]) == 1
        assert int(r["scales"][0]) == ex.rn_f16_bits(Fraction(abs(float(np.float32(v)))) / Q)
    # constant row: every code is Q
    r = oracle.quantize_rows(np.full((1, n), 0.25, np.float32), Q)
    assert (r["codes"] == Q).all()
    # grid-aligned row x_j = m_j s0 with max |m_j| = Q: the scale is s0, codes m_j, dq == x
    rng = np.random.default_rng(0)
    for s0b in (0x2A3D, 0x1E00, 0x3C00, 0x0400):
        s0 = float(_f16([s0b])[0])
        m = rng.integers(-Q, Q + 1, size=n)
        m[5] = Q
        x = (m * s0).astype(np.float32)[None, :]
        r = oracle.quantize_rows(x, Q)
        assert int(r["scales"][0]) == s0b
        assert np.array_equal(r["codes"][0], m.astype(np.int8))
        assert np.array_equal(r["dq"], x)
    # tie row x_j = (m + 1/2) s0 with the maximum Q s0 present: codes go to the even neighbour
    s0 = float(_f16([0x2A3D])[0])
    m = np.arange(-Q, Q)            # -31 .. 30
    x = np.concatenate([(m + 0.5) * s0, [Q * s0]]).astype(np.float32)[None, :]
    r = oracle.quantize_rows(x, Q)
    want = np.array([int(mm) if mm % 2 == 0 else int(mm) + 1 for mm in m] + [Q], np.int8)
    assert np.array_equal(r["codes"][0], want)
    # underflowing scale: clip > 0 but fp16(clip / Q) == 0 -> scale 1.0, codes 0
    x = np.zeros((1, n), np.float32)
    x[0, 3] = 31 * 2.0 ** -26
    r = oracle.quantize_rows(x, Q)
    assert r["scales"][0] == 0x3C00 and not r["codes"].any()


def test_status_bits(orc):
    x = np.zeros((3, 16), np.float32)
    x[0, 2] = np.nan
    x[1, 5] = 2_031_120.0          # 65,520 * 31: the int6 scale rounds to fp16 infinity
    x[2, 7] = 2_031_100.0          # just below: finite scale
    r = oracle.quantize_rows(x[:1], 31)
    assert r["status"] & oracle.ORC_NONFINITE
    r = oracle.quantize_rows(x[1:2], 31)
    assert r["status"] == oracle.ORC_SCALE_OVF
    r = oracle.quantize_rows(x[2:3], 31)
    assert r["status"] == 0
    _, st = oracle.f16_passthrough(np.array([65519.0, 1.0], np.float32))
    assert st == 0
    _, st = oracle.f16_passthrough(np.array([65520.0], np.float32))
    assert st == oracle.ORC_F16_OVF
    _, st = oracle.awq_multipliers(np.array([1.0, 0.0], np.float32))
    assert st == oracle.ORC_BAD_AWQ


def test_awq_special_cases(orc):
    w = synth.config1().data[:64]
    plain = oracle.quantize_rows(w, 31)
    a, st = oracle.awq_multipliers(np.ones(w.shape[1], np.float32))
    assert st == 0 and (a == 0x3C00).all()
    r = oracle.quantize_rows(w, 31, awq=a)
    for key in ("codes", "scales", "dq"):
        assert np.array_equal(r[key], plain[key])
    for m in (-2, 1, 3):
        a, st = oracle.awq_multipliers(np.full(w.shape[1], 4.0 ** m, np.float32))
        assert (oracle.f16_to_f32(a) == np.float32(2.0 ** m)).all()
        r = oracle.quantize_rows(w, 31, awq=a)
        ref = oracle.quantize_rows(w * np.float32(2.0 ** m), 31)
        assert np.array_equal(r["codes"], ref["codes"])
        assert np.array_equal(r["scales"], ref["scales"])
        assert np.array_equal(r["dq"], ref["dq"] / np.float32(2.0 ** m))


def test_sqwa_special_cases(orc):
    pol = oracle.Policy(int8_patterns=(), passthrough_below=65536, q6=(6, 9999, 10000))
    base = [(t.name, t.data) for t in synth.config2()[:9]]
    qdq = [oracle.qdq_tensor(n, w, pol) for n, w in base]
    # one snapshot: its QDQ
    means = oracle.sqwa_run([base], pol)
    for m, q in zip(means, qdq):
        assert np.array_equal(m.view(np.uint32), q.view(np.uint32))
    # identical snapshots: still the QDQ, bit for bit
    means = oracle.sqwa_run([base] * 5, pol)
    for m, q in zip(means, qdq):
        assert np.array_equal(m.view(np.uint32), q.view(np.uint32))
    # two snapshots: within one binary32 ulp of the exact mean of the two QDQs
    other = [(n, (w * np.float32(1.25)).astype(np.float32)) for n, w in base]
    qdq2 = [oracle.qdq_tensor(n, w, pol) for n, w in other]
    means = oracle.sqwa_run([base, other], pol)
    for m, a, b in zip(means, qdq, qdq2):
        exact = (a.astype(np.float64) + b.astype(np.float64)) / 2
        ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
        assert (np.abs(m.astype(np.float64) - exact) <= ulp).all()
    # resuming after snapshot 1 with the saved mean equals the uninterrupted run
    snaps = [base, other, base]
    full = oracle.sqwa_run(snaps, pol)
    part = oracle.sqwa_run(snaps[:1], pol)
    part = [p.copy() for p in part]
    resumed = oracle.sqwa_run(snaps[1:], pol, k0=2, means=part)
    for f, r in zip(full, resumed):
        assert np.array_equal(f.view(np.uint32), r.view(np.uint32))
