"""Pins of the oracle's weight averaging (EMA with decay 0.997 from the PR #1414 / PR #1202
cards' Weight Averaging sections; SWA over checkpoints from the PR #69 card).

Each check comes from the mathematics, not from the oracle's own formula: special decays that
reduce the update to a copy, error bounds against float64, geometric decay, power-of-two
scaling, and for SWA identical, paired and many checkpoints against exact or float64 means.
"""
import numpy as np
import pytest

import oracle

D = 0.997


def _rand(seed, n=4096, scale=0.02):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)


def _ulp(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def test_ema_init_copies_bits():
    w = _rand(1)
    w[:4] = [0.0, -0.0, np.float32(1e-40), -3.5]
    e = np.full(w.shape, 7.0, np.float32)
    assert oracle.ema_update(e, w, D, init=True) == 0
    assert np.array_equal(e.view(np.uint32), w.view(np.uint32))


def test_ema_decay_zero_is_the_weights_and_decay_one_keeps_the_average():
    e0, w = _rand(2), _rand(3)
    e = e0.copy()
    oracle.ema_update(e, w, 0.0)
    assert np.array_equal(e, w)             # 0 * e + 1 * w
    e = e0.copy()
    oracle.ema_update(e, w, 1.0)
    assert np.array_equal(e, e0)            # 1 * e + 0 * w


def test_ema_within_rounding_of_the_real_update():
    e0, w = _rand(4, 1 << 16), _rand(5, 1 << 16, 0.05)
    e = e0.copy()
    oracle.ema_update(e, w, D)
    d = np.float64(np.float32(D))
    exact = d * e0.astype(np.float64) + (1.0 - d) * w.astype(np.float64)
    c32 = np.float64(np.float32(1.0) - np.float32(D))
    bound = (0.5 * _ulp(d * e0) + 0.5 * _ulp(c32 * w) + np.abs(w) * abs(c32 - (1.0 - d))
             + 0.5 * _ulp(exact) + 1e-45)
    assert np.all(np.abs(e.astype(np.float64) - exact) <= bound)
    # the update is not symmetric in e and w: swapping them is far outside the bound
    swapped = d * w.astype(np.float64) + (1.0 - d) * e0.astype(np.float64)
    assert np.mean(np.abs(e.astype(np.float64) - swapped) > bound) > 0.99


def test_ema_geometric_decay_of_a_zero_signal():
    e = np.ones(8, np.float32)
    z = np.zeros(8, np.float32)
    k = 500
    for _ in range(k):
        oracle.ema_update(e, z, D)
    ref = np.float64(np.float32(D)) ** k
    assert np.all(np.abs(e - ref) <= k * 2.0 ** -24 * ref * 1.01)
    assert np.all(e > 0)


def test_ema_scales_exactly_by_powers_of_two():
    e0, w = _rand(6), _rand(7)
    a, b = e0.copy(), e0 * np.float32(8.0)
    oracle.ema_update(a, w, D)
    oracle.ema_update(b, w * np.float32(8.0), D)
    assert np.array_equal(b, a * np.float32(8.0))


def test_ema_nonfinite_status():
    w = _rand(8, 16)
    w[3] = np.inf
    e = np.zeros(16, np.float32)
    assert oracle.ema_update(e, w, D) & oracle.ORC_NONFINITE
    w[3] = 1.0
    assert oracle.ema_update(np.zeros(16, np.float32), w, D) == 0


def test_ema_run_initialises_then_averages():
    steps = [[_rand(10 + s, 64)] for s in range(3)]
    (e,), st = oracle.ema_run(steps, D)
    assert st == 0
    ref = steps[0][0].astype(np.float64)
    for s in steps[1:]:
        ref = np.float32(D) * ref + (1 - np.float64(np.float32(D))) * s[0]
    assert np.allclose(e, ref, rtol=0, atol=4 * float(np.max(_ulp(ref))))


def test_swa_identical_checkpoints_are_exact():
    w = _rand(20)
    (m,), st = oracle.swa_run([[w]] * 16)
    assert st == 0 and np.array_equal(m, w)


def test_swa_two_checkpoints_is_their_midpoint():
    a, b = _rand(21, 1 << 15), _rand(22, 1 << 15)
    (m,), _ = oracle.swa_run([[a], [b]])
    mid = (a.astype(np.float64) + b.astype(np.float64)) / 2
    # a + fl(b - a)/2: the difference carries at most half an ulp of |b - a| (halved exactly),
    # the sum half an ulp of the result
    bound = 0.25 * _ulp(b.astype(np.float64) - a) + 0.5 * _ulp(mid) + 0.5 * _ulp(m) + 1e-45
    assert np.all(np.abs(m - mid) <= bound)
    # and it is not the plain sum or either endpoint
    assert np.mean(np.abs(m - (a + b)) > bound) > 0.99


def test_swa_sixteen_checkpoints_against_float64_mean():
    base = _rand(23, 1 << 14)
    cks = [[base + _rand(100 + k, 1 << 14, 0.002 * k)] for k in range(1, 17)]
    (m,), _ = oracle.swa_run(cks)
    ref = np.mean([c[0].astype(np.float64) for c in cks], axis=0)
    err = np.abs(m - ref)
    assert np.all(err <= 16 * 2.0 ** -24 * np.max(np.abs(ref)) + 1e-45)
    # a running mean that forgot the 1/k weighting would be the last checkpoint instead
    assert np.mean(np.abs(cks[-1][0] - ref) > 16 * 2.0 ** -24 * np.max(np.abs(ref))) > 0.9


def test_swa_resume_equals_one_run():
    cks = [[_rand(200 + k, 256)] for k in range(6)]
    full, _ = oracle.swa_run(cks)
    half, _ = oracle.swa_run(cks[:3])
    rest, _ = oracle.swa_run(cks[3:], k0=4, means=[half[0].copy()])
    assert np.array_equal(full[0], rest[0])


@pytest.mark.parametrize("k", [1, 2, 3, 7])
def test_swa_first_checkpoint_copies(k):
    w = _rand(300 + k, 32)
    m = np.full(32, 5.0, np.float32)
    oracle.swa_update(m, w, 1)
    assert np.array_equal(m, w)


def test_swa_nonfinite_status():
    w = _rand(400, 16)
    m = np.zeros(16, np.float32)
    assert oracle.swa_update(m, w, 1) == 0
    w[5] = np.nan
    assert oracle.swa_update(m, w, 2) & oracle.ORC_NONFINITE
