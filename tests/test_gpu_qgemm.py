"""GPU parity of the fused-dequant GEMM (the QAT forward's consumer matmul over STE-dequantized
weights, PR #69 card section Other) against the oracle's double-precision product.

Tolerance (derived from the arithmetic): every product of two bf16 values is exact in binary32;
summing K of them in binary32 in any order errs by at most (K - 1) u sum |x w| with u = 2^-24,
so |y - y_ref| <= (K + 1) 2^-24 sum_k |x_k w_k| is required elementwise.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
from int6_weight_export_amd import ops  # noqa: E402


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = oracle.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    w = oracle.f32_to_bf16((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    fq = oracle.fakequant_rows(w, 31)                  # the STE forward: codes and fp16 scales
    return x, fq["codes"], fq["scales"]


def _check(y, x, codes, scales, rows=None, what=""):
    xs = x if rows is None else x[rows]
    ref, bound = oracle.qgemm_bf16(xs, codes, scales)
    got = y if rows is None else y[rows]
    K = x.shape[1]
    tol = (K + 1) * 2.0 ** -24 * bound + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= tol), f"{what}: max err {err.max()} vs tol {tol[err > tol].min()}"


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 7, 3), (129, 130, 33), (64, 128, 32), (200, 1584, 528),
                                   (300, 528, 1584), (131, 257, 100)])
def test_qgemm_small_and_ragged(M, N, K):
    say(f"qgemm {M}x{N}x{K}")
    x, codes, scales = _inputs(M, N, K, M + N + K)
    y = ops.qgemm(_bf16(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda())
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), x, codes, scales, what=f"{M}x{N}x{K}")


def test_qgemm_strided_operands():
    say("qgemm with padded row strides")
    M, N, K = 77, 150, 96
    x, codes, scales = _inputs(M, N, K, 5)
    xb = torch.zeros(M, K + 8, dtype=torch.bfloat16, device="cuda")
    xb[:, :K] = _bf16(x)
    cb = torch.zeros(N, K + 16, dtype=torch.int8, device="cuda")
    cb[:, :K] = torch.from_numpy(codes).cuda()
    yb = torch.full((M, N + 3), 7.0, dtype=torch.float32, device="cuda")
    ops.qgemm(xb[:, :K], cb[:, :K], torch.from_numpy(scales.view(np.int16)).cuda(), out=yb[:, :N])
    torch.cuda.synchronize()
    _check(yb[:, :N].cpu().numpy(), x, codes, scales, what="strided")
    assert bool((yb[:, N:] == 7.0).all())              # nothing written past N


def test_qgemm_qat_shape_sampled_rows():
    say("qgemm 8192 x 1584 x 528 (the d=528 unified projection), sampled rows")
    M, N, K = 8192, 1584, 528
    x, codes, scales = _inputs(M, N, K, 11)
    y = ops.qgemm(_bf16(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda())
    torch.cuda.synchronize()
    rows = np.r_[0:3, 127:130, 4095:4098, 8189:8192]
    _check(y.cpu().numpy(), x, codes, scales, rows=rows, what="qat")


def test_qgemm_uses_the_fake_quant_outputs_on_device():
    say("qgemm on the codes and scales of the device STE forward")
    rng = np.random.default_rng(13)
    w = oracle.f32_to_bf16((rng.standard_normal((256, 528)) * 0.02).astype(np.float32))
    fq = ops.FakeQuant([_bf16(w)], want_codes=True)
    fq.run(1)                                           # forward only
    x = oracle.f32_to_bf16(rng.standard_normal((96, 528)).astype(np.float32))
    y = ops.qgemm(_bf16(x), fq.codes[0], fq.scales[0])
    torch.cuda.synchronize()
    ref = oracle.fakequant_rows(w, 31)
    _check(y.cpu().numpy(), x, ref["codes"], ref["scales"], what="device fake quant")
