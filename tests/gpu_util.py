"""Helpers for the GPU parity tests: device transfer and bit-level comparison."""
import numpy as np
import torch


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    """fp16 bit patterns (uint16) as a device float16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.float16)


def u16(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def same_bits(got: np.ndarray, want: np.ndarray, what: str = ""):
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    g = got.view(np.uint8).reshape(-1)
    w = want.view(np.uint8).reshape(-1)
    if not np.array_equal(g, w):
        gi = got.reshape(-1)
        wi = want.reshape(-1)
        if got.dtype.itemsize in (2, 4):
            bad = np.nonzero(gi.view(f"u{got.dtype.itemsize}") != wi.view(f"u{got.dtype.itemsize}"))[0]
        else:
            bad = np.nonzero(gi != wi)[0]
        i = int(bad[0])
        idx = np.unravel_index(i, got.shape)
        raise AssertionError(f"{what}: {bad.size} of {gi.size} differ; first at {idx}: got {gi[i]!r} want {wi[i]!r}")


def f32_bits_equal(got: np.ndarray, want: np.ndarray, what: str = ""):
    """Bit equality of float32 arrays, sign of zero included."""
    same_bits(np.ascontiguousarray(got, dtype=np.float32), np.ascontiguousarray(want, dtype=np.float32), what)
