"""Pins for the oracle's own format conversions.

The oracle converts binary32 to binary16 and to bfloat16 with code written from the
format definitions.  These tests compare every one of the 2^32 binary32 bit patterns
with torch's CPU casts (round to nearest even), check the binary16 decode against
numpy for all 65,536 patterns, and cross-check a second library (numpy) on a sample.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle

CHUNK = 1 << 25


def _check_chunk(c, conv, tdtype, expo_mask, frac_mask):
    """Compare oracle conversion with torch's cast on bit patterns [c, c + CHUNK).
    Returns None or a description of the first mismatch (NaNs compare by NaN-ness)."""
    u = np.arange(CHUNK, dtype=np.uint32) + np.uint32(c)
    x = u.view(np.float32)
    got = conv(x)
    ref = torch.from_numpy(x).to(tdtype).view(torch.int16).numpy().view(np.uint16)
    eq = got == ref
    if eq.all():
        return None
    gn = ((got & expo_mask) == expo_mask) & ((got & frac_mask) != 0)
    rn = ((ref & expo_mask) == expo_mask) & ((ref & frac_mask) != 0)
    ok = eq | (gn & rn)
    if ok.all():
        return None
    i = int(np.argmin(ok))
    return f"input {int(u[i]):#010x}: oracle {int(got[i]):#06x} torch {int(ref[i]):#06x}"


def _exhaustive(conv, tdtype, expo_mask, frac_mask):
    torch.set_num_threads(1)
    with ThreadPoolExecutor(max_workers=6) as ex:
        res = list(ex.map(lambda c: _check_chunk(c, conv, tdtype, expo_mask, frac_mask),
                          range(0, 1 << 32, CHUNK)))
    bad = [r for r in res if r]
    assert not bad, bad[:5]


def test_f32_to_f16_exhaustive(orc):
    """All 2^32 inputs: oracle binary16 bits == torch's round-to-nearest-even cast."""
    _exhaustive(oracle.f32_to_f16, torch.float16, 0x7C00, 0x3FF)


def test_f32_to_bf16_exhaustive(orc):
    """All 2^32 inputs: oracle bfloat16 bits == torch's round-to-nearest-even cast."""
    _exhaustive(oracle.f32_to_bf16, torch.bfloat16, 0x7F80, 0x7F)


def test_f32_to_f16_numpy_sample(orc):
    """Second library: numpy's cast on every pattern near the binary16 range
    (|x| in [2^-26, 2^17)) with a stride, plus random patterns."""
    lo, hi = 0x32800000, 0x48000000
    u = np.arange(lo, hi, 7, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    x = u.view(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16(x)
    assert np.array_equal(got, ref)


def test_f16_decode_all(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("n,num,den,k", [
    (512, 9999, 10000, 512), (1536, 9999, 10000, 1536), (528, 9999, 10000, 528),
    (9999, 9999, 10000, 9999), (10000, 9999, 10000, 9999), (19999, 9999, 10000, 19998),
    (16384, 9999, 10000, 16383), (65536, 9999, 10000, 65530), (512, 99, 100, 507),
    (1536, 99, 100, 1521), (8, 1, 2, 4), (8, 1, 8, 1), (8, 7, 8, 7), (1, 1, 10000, 1), (3, 0, 1, 1),
])
def test_percentile_rank(orc, n, num, den, k):
    """k = ceil(num * n / den) in exact integers, clamped to [1, n]; the 9,999 and 19,999
    cases are where a float32 ceil of 0.9999 * n would be off by one."""
    assert oracle.percentile_rank(n, num, den) == k
