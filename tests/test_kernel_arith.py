"""Exhaustive host checks of the floating-point identities the HIP kernels rely on.

These do not touch the oracle or the GPU: they prove, over every operand the kernels can meet,
that a cheaper instruction sequence returns the same fp32 result as the operation the method
defines (run in plain C on the host, which rounds like the GPU's IEEE fp32 units).
"""
import subprocess

import pytest

# AWQ dequantisation (PR #1495 "int6 AWQ", Submission summary): dq = fl32((code * s) / a_j).
# The kernel takes y = fl32(1 / a_j) once per column, then q = fl32(n * y),
# r = fma(-q, a_j, n), dq = fma(r, y, q).  n = code * s has at most 7 + 11 significant bits
# (|code| <= 127, s an fp16 value) and a_j is an fp16 value (<= 11 bits); scaling either by a
# power of two scales every intermediate exactly (no under/overflow for fp16-range operands),
# so it suffices to try every odd 18-bit numerator against every odd 11-bit denominator.
MARKSTEIN_C = r"""
#include <math.h>
#include <stdio.h>
#include <stdint.h>
int main(void) {
    volatile float one = 1.0f;
    long bad = 0, plain_bad = 0, n = 0;
    for (uint32_t d = 1; d < 2048; d += 2) {
        const float a = (float)d, y = one / a;
        for (uint32_t m = 1; m < (1u << 18); m += 2) {
            const float num = (float)m, ref = num / a;
            const float q = num * y;
            const float q2 = fmaf(fmaf(-q, a, num), y, q);
            n++;
            bad += q2 != ref;
            plain_bad += q != ref;
        }
    }
    printf("%ld %ld %ld\n", n, bad, plain_bad);
    return 0;
}
"""


def test_awq_dequant_reciprocal_correction_is_exact(tmp_path):
    src = tmp_path / "markstein.c"
    exe = tmp_path / "markstein"
    src.write_text(MARKSTEIN_C)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe), str(src), "-lm"],
                   check=True)
    n, bad, plain_bad = map(int, subprocess.run([str(exe)], check=True, capture_output=True,
                                                text=True).stdout.split())
    assert n == 1024 * (1 << 17)
    assert bad == 0
    # the correction step matters: the bare product misrounds a share of the quotients
    assert plain_bad > 0
