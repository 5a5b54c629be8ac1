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


# K a multiple of 16 with 16-byte rows takes the direct-to-LDS kernel (K % 64 = 0, 16, 32, 48 cover
# its tail stage; K = 16 has no full stage); the others take the generic kernel
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 7, 3), (129, 130, 33), (64, 128, 32), (200, 1584, 528),
                                   (300, 528, 1584), (131, 257, 100), (1, 1, 16), (3, 5, 48), (130, 129, 64),
                                   (257, 300, 80), (520, 390, 1040), (128, 128, 2048), (384, 260, 176)])
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


def test_qgemm_k_zero_writes_zeros_without_reading_operands():
    """K = 0: Y = +0 everywhere, with x, codes and scales NULL (nothing is read)."""
    from int6_weight_export_amd import pgq

    say("qgemm K = 0 with NULL operands")
    M, N = 70, 45
    y = torch.full((M, N + 3), 7.0, dtype=torch.float32, device="cuda")
    rc = pgq.pgq_qgemm_bf16(None, M, 0, 0, None, 0, None, N, y.data_ptr(), N + 3,
                            torch.cuda.current_stream().cuda_stream)
    assert rc == pgq.PGQ_OK
    torch.cuda.synchronize()
    yy = y.cpu().numpy()
    assert np.all(yy[:, :N].view(np.uint32) == 0)        # +0, sign included
    assert np.all(yy[:, N:] == 7.0)


def test_qgemm_bench_shape_sampled_rows_and_repeatable():
    """16384 x 1584 x 528, the timed workload: sampled rows from every region of the output
    (first and last row tiles, the ragged last column tile), and bit-identical on a second run."""
    say("qgemm 16384 x 1584 x 528 sampled rows, repeat")
    M, N, K = 16384, 1584, 528
    x, codes, scales = _inputs(M, N, K, 17)
    xd, cd, sd = _bf16(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda()
    y1 = ops.qgemm(xd, cd, sd)
    y2 = ops.qgemm(xd, cd, sd)
    torch.cuda.synchronize()
    a, b = y1.cpu().numpy(), y2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rows = np.r_[0:2, 126:131, 8000:8002, 16255:16258, 16382:16384]
    _check(a, x, codes, scales, rows=rows, what="bench shape")


# ---- bf16 Y: each element is bf16 (round to nearest even) of the fp32 result of the same GEMM ----

def _ybf16_tol(ref, bound, K):
    """Against the exact product: the fp32 bound plus half a bf16 ulp of the value (bf16 keeps 8
    significant bits, so half an ulp is at most 2^-8 |v|; 2^-133 covers the subnormal steps)."""
    tol32 = (K + 1) * 2.0 ** -24 * bound
    return tol32 + 2.0 ** -8 * (np.abs(ref) + tol32) + 2.0 ** -133


def _bf16_bits_of(y32):
    return oracle.f32_to_bf16(np.ascontiguousarray(y32, dtype=np.float32)).view(np.uint16)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 7, 3), (129, 130, 33), (200, 1584, 528), (131, 257, 100),
                                   (3, 5, 48), (130, 129, 64), (257, 300, 80), (384, 260, 176), (70, 13, 16)])
def test_qgemm_ybf16_is_the_rounded_fp32_result(M, N, K):
    say(f"qgemm bf16 Y {M}x{N}x{K}")
    x, codes, scales = _inputs(M, N, K, 3 * M + N + K)
    xd, cd, sd = _bf16(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda()
    y32 = ops.qgemm(xd, cd, sd)
    y16 = ops.qgemm(xd, cd, sd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a = y32.cpu().numpy()
    b = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(b, _bf16_bits_of(a)), f"{M}x{N}x{K}: bf16 Y differs from bf16 of the fp32 Y"
    ref, bound = oracle.qgemm_bf16(x, codes, scales)
    got = oracle.bf16_to_f32(b).astype(np.float64)
    err = np.abs(got - ref)
    tol = _ybf16_tol(ref, bound, K)
    assert np.all(err <= tol), f"{M}x{N}x{K}: max err {err.max()}"


def test_qgemm_ybf16_strided_and_k_zero():
    from int6_weight_export_amd import pgq

    say("qgemm bf16 Y with a padded row stride; K = 0")
    M, N, K = 77, 150, 96
    x, codes, scales = _inputs(M, N, K, 6)
    yb = torch.full((M, N + 5), 3.0, dtype=torch.bfloat16, device="cuda")
    ops.qgemm(_bf16(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda(),
              out=yb[:, :N], out_dtype=torch.bfloat16)
    y32 = ops.qgemm(_bf16(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda())
    torch.cuda.synchronize()
    b = yb[:, :N].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(b, _bf16_bits_of(y32.cpu().numpy()))
    assert bool((yb[:, N:] == 3.0).all())              # nothing written past N
    y0 = torch.full((M, N + 3), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = pgq.pgq_qgemm_bf16_ybf16(None, M, 0, 0, None, 0, None, N, y0.data_ptr(), N + 3,
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == pgq.PGQ_OK
    torch.cuda.synchronize()
    z = y0.view(torch.int16).cpu().numpy()
    assert np.all(z[:, :N] == 0) and bool((y0[:, N:] == 7.0).all())   # +0, sign included


def test_qgemm_ybf16_bench_shape_sampled_rows():
    say("qgemm bf16 Y 16384 x 1584 x 528 sampled rows")
    M, N, K = 16384, 1584, 528
    x, codes, scales = _inputs(M, N, K, 19)
    xd, cd, sd = _bf16(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda()
    y32 = ops.qgemm(xd, cd, sd)
    y16 = ops.qgemm(xd, cd, sd, out_dtype=torch.bfloat16)
    y16b = ops.qgemm(xd, cd, sd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    b = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(b, y16b.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(b, _bf16_bits_of(y32.cpu().numpy()))
    rows = np.r_[0:2, 126:131, 8000:8002, 16255:16258, 16382:16384]
    ref, bound = oracle.qgemm_bf16(x[rows], codes, scales)
    err = np.abs(oracle.bf16_to_f32(b[rows]).astype(np.float64) - ref)
    assert np.all(err <= _ybf16_tol(ref, bound, K))


def test_qgemm_ybf16_unaligned_rows_take_the_same_kernel():
    """bf16 Y starting 2 bytes into a buffer, row stride odd: no 16-byte stores are possible, the
    element-store path of the same kernel writes it, and it still equals bf16 of the fp32 Y (K a
    multiple of 16 with 16-byte rows: the direct-to-LDS kernel for both)."""
    say("qgemm bf16 Y at a 2-byte offset, odd row stride")
    M, N, K = 300, 203, 160
    x, codes, scales = _inputs(M, N, K, 23)
    xd, cd, sd = _bf16(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda()
    yb = torch.full((M, N + 2), 5.0, dtype=torch.bfloat16, device="cuda")
    ops.qgemm(xd, cd, sd, out=yb[:, 1:N + 1], out_dtype=torch.bfloat16)
    y32 = ops.qgemm(xd, cd, sd)
    torch.cuda.synchronize()
    b = yb[:, 1:N + 1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(b, _bf16_bits_of(y32.cpu().numpy()))
    assert bool((yb[:, 0] == 5.0).all()) and bool((yb[:, N + 1] == 5.0).all())
