"""Pins of the oracle's fused-dequant GEMM: Y = X What^T, What = bf16(code * s) per row -- the
STE forward's dequantized weights (PR #69 card, section Other) consumed by the next matmul.

Checked against a hand-worked case, numpy float64 matmul over weights dequantized with torch's
own bf16 rounding, and the STE forward itself (its bf16 output is the GEMM's weight operand).
"""
import numpy as np
import pytest
import torch

import oracle


def test_hand_worked():
    x = oracle.f32_to_bf16(np.array([[1, 2, 3]], np.float32))
    c = np.array([[1, 1, 1], [2, 0, -1]], np.int8)
    s = np.array([0x3C00, 0x3800], np.uint16)            # fp16 1.0 and 0.5
    y, b = oracle.qgemm_bf16(x, c, s)
    assert y.tolist() == [[6.0, -0.5]] and b.tolist() == [[6.0, 2.5]]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 5, 3), (33, 40, 130), (64, 96, 528)])
def test_matches_numpy_with_torch_rounding(M, N, K):
    rng = np.random.default_rng(M * 1000 + N + K)
    x32 = (rng.standard_normal((M, K)) * 0.5).astype(np.float32)
    x = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes = rng.integers(-31, 32, (N, K)).astype(np.int8)
    scales = (rng.uniform(1e-4, 1e-2, N)).astype(np.float16).view(np.uint16)
    y, b = oracle.qgemm_bf16(x, codes, scales)
    wq = torch.from_numpy(codes.astype(np.float32) * scales.view(np.float16).astype(np.float32)[:, None])
    wq = wq.to(torch.bfloat16).to(torch.float64).numpy()
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ref = xd @ wq.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-300)
    assert np.allclose(b, np.abs(xd) @ np.abs(wq).T, rtol=1e-12, atol=1e-300)


def test_weight_operand_is_the_ste_forward_output():
    rng = np.random.default_rng(9)
    w = oracle.f32_to_bf16((rng.standard_normal((48, 200)) * 0.02).astype(np.float32))
    fq = oracle.fakequant_rows(w, 31)
    x = oracle.f32_to_bf16(rng.standard_normal((16, 200)).astype(np.float32))
    y, _ = oracle.qgemm_bf16(x, fq["codes"], fq["scales"])
    ref = oracle.bf16_to_f32(x).astype(np.float64) @ oracle.bf16_to_f32(fq["dq"]).astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-300)
