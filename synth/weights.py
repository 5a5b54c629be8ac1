"""Counter-based seeded generators and the synthetic weight sets.

Random bits come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) used as a counter-based generator:
draw i of stream `key` is mix(key + (i + 1) * 0x9E3779B97F4A7C15).  Uniforms take the
top 53 bits; normals use the Box-Muller transform in float64 and are then rounded
once to the storage type (float32 by numpy's round-to-nearest-even cast, bfloat16 by
torch's round-to-nearest-even cast).

The shapes follow the Parameter Golf submission cards:
  * PR #69 "SubSixteen v2" card, section Architecture: 9 layers, dim 512, MLP hidden
    1536, vocab 1024, 8 query / 4 KV heads, tied embeddings;
  * PR #1202 "Unified Attention + FA3 + Legal TTT" card, section Architecture:
    11 layers, dim 528, 4 heads, one unified Q/K/V projection, MLP 3x;
  * PR #1495 "12L 24min Vocab1792 ... Int6AWQ MixedBits", Submission summary and
    Mixed-bit quantization details: 12 layers, vocab 1792, untied tok_emb/lm_head.
Value distributions (N(0, 0.02^2) weights, N(0, 1e-4^2) gradients, LogNormal(0, 0.5^2)
activation scales, per-snapshot noise N(0, (0.002 k)^2)) are the stated synthetic
workloads that stand in for trained checkpoints, which the pages do not provide.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def key_of(*parts: int) -> int:
    """Derive a 64-bit stream key from a tuple of small non-negative integers."""
    k = 0x243F6A8885A308D3
    for p in parts:
        k = _mix64_int(k ^ ((int(p) * _GAMMA) & _MASK64))
    return k


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _bits(key: int, start: int, n: int) -> np.ndarray:
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        return _mix64(np.uint64(key) + i * np.uint64(_GAMMA))


def uniform01(key: int, n: int, start: int = 0) -> np.ndarray:
    """n uniforms in [0, 1) with 53 random bits each (float64)."""
    return (_bits(key, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(key: int, n: int) -> np.ndarray:
    """n standard normals (float64) by Box-Muller on consecutive uniform pairs."""
    m = (n + 1) // 2
    b = _bits(key, 0, 2 * m)
    u1 = ((b[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)  # (0, 1]
    u2 = (b[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)          # [0, 1)
    r = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * math.pi) * u2
    out = np.empty(2 * m, dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    return out[:n]


def gauss_f32(key: int, shape, sigma: float, mean: Optional[np.ndarray] = None) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    v = sigma * normal(key, n)
    if mean is not None:
        v = v + mean.reshape(-1).astype(np.float64)
    return v.astype(np.float32).reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even, by torch's cast); return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gauss_bf16(key: int, shape, sigma: float) -> np.ndarray:
    """bfloat16 N(0, sigma^2) as uint16 bit patterns (float64 -> float32 -> bfloat16)."""
    return f32_to_bf16_bits(gauss_f32(key, shape, sigma))


def student_t3_f32(key: int, shape, scale: float) -> np.ndarray:
    """scale * Student-t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3)."""
    n = int(np.prod(shape))
    z = normal(key_of(key, 0), n)
    c = normal(key_of(key, 1), 3 * n).reshape(n, 3)
    v = (c * c).sum(axis=1) / 3.0
    return (scale * z / np.sqrt(v)).astype(np.float32).reshape(shape)


def lognormal_f32(key: int, n: int, sigma: float) -> np.ndarray:
    return np.exp(sigma * normal(key, n)).astype(np.float32)


@dataclass
class SynthTensor:
    name: str
    data: np.ndarray                 # float32 array, or uint16 bfloat16 bit patterns
    dtype: str = "f32"               # "f32" or "bf16"
    awq_s: Optional[np.ndarray] = None   # per-input-column activation scale (float32)
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        return self.data.shape

    @property
    def numel(self) -> int:
        return int(self.data.size)


SIGMA_W = 0.02


def _map(fn, items, workers: int):
    """[fn(x) for x in items], on `workers` threads (numpy releases the GIL in the array work)."""
    if workers <= 1:
        return [fn(x) for x in items]
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(workers) as pool:
        return list(pool.map(fn, items))


def config1_batch(count: int, workers: int = 1) -> List[SynthTensor]:
    """`count` independent fp32 1536x512 matrices, N(0, 0.02^2), seeds 0..count-1."""
    return _map(lambda b: SynthTensor(f"mat{b}", gauss_f32(key_of(1, b), (1536, 512), SIGMA_W)), range(count), workers)


def config1() -> SynthTensor:
    return config1_batch(1)[0]


def _gpt_block_shapes(d: int, n_head: int, n_kv: int, hidden: int):
    hd = d // n_head
    return [
        ("attn.wq.weight", (n_head * hd, d)),
        ("attn.wk.weight", (n_kv * hd, d)),
        ("attn.wv.weight", (n_kv * hd, d)),
        ("attn.wo.weight", (d, n_head * hd)),
        ("mlp.up.weight", (hidden, d)),
        ("mlp.down.weight", (d, hidden)),
    ]


def _gpt_names_shapes(layers: int, d: int, n_head: int, n_kv: int, hidden: int, vocab: int,
                      tied: bool, vectors: bool):
    out = [("tok_emb.weight", (vocab, d))]
    if not tied:
        out.append(("lm_head.weight", (vocab, d)))
    for layer in range(layers):
        for nm, shp in _gpt_block_shapes(d, n_head, n_kv, hidden):
            out.append((f"blocks.{layer}.{nm}", shp))
        if vectors:
            out.append((f"blocks.{layer}.attn_scale", (d,)))
            out.append((f"blocks.{layer}.mlp_scale", (d,)))
    return out


def config2(cfg_id: int = 2, dist: str = "gauss") -> List[SynthTensor]:
    """9-layer GPT, d=512, 8/4 heads, MLP 1536, tied 1024x512 embedding, two 512-vectors per layer."""
    ts = []
    for i, (nm, shp) in enumerate(_gpt_names_shapes(9, 512, 8, 4, 1536, 1024, tied=True, vectors=True)):
        if dist == "gauss":
            a = gauss_f32(key_of(cfg_id, i), shp, SIGMA_W)
        elif dist == "t3":
            a = student_t3_f32(key_of(cfg_id, i), shp, SIGMA_W)
        else:
            raise ValueError(dist)
        ts.append(SynthTensor(nm, a))
    return ts


def config3_shapes(layers: int = 11):
    """11-layer d=528 model: unified QKV projection stored [out, in] = 1584x528, Wo 528x528,
    MLP 3x up 1584x528 and down 528x1584."""
    out = []
    for layer in range(layers):
        out.append((f"blocks.{layer}.attn.w_unified.weight", (1584, 528)))
        out.append((f"blocks.{layer}.attn.wo.weight", (528, 528)))
        out.append((f"blocks.{layer}.mlp.up.weight", (1584, 528)))
        out.append((f"blocks.{layer}.mlp.down.weight", (528, 1584)))
    return out


def config3_weights(layers: int = 11) -> List[SynthTensor]:
    return [SynthTensor(nm, gauss_bf16(key_of(3, i), shp, SIGMA_W), "bf16")
            for i, (nm, shp) in enumerate(config3_shapes(layers))]


def config3_grads(step: int, layers: int = 11) -> List[SynthTensor]:
    return [SynthTensor(nm + ".grad", gauss_bf16(key_of(3, i, 1000 + step), shp, 1e-4), "bf16")
            for i, (nm, shp) in enumerate(config3_shapes(layers))]


def config4() -> List[SynthTensor]:
    """12-layer GPT, d=512, GQA 8/4, MLP 3x, untied 1792x512 tok_emb and lm_head.
    Every block matrix carries a per-input-column activation scale s_j ~ LogNormal(0, 0.5^2)."""
    ts = []
    for i, (nm, shp) in enumerate(_gpt_names_shapes(12, 512, 8, 4, 1536, 1792, tied=False, vectors=False)):
        a = gauss_f32(key_of(4, i), shp, SIGMA_W)
        s = None
        if nm.startswith("blocks."):
            s = lognormal_f32(key_of(4, i, 77), shp[1], 0.5)
        ts.append(SynthTensor(nm, a, awq_s=s))
    return ts


def config5_base() -> List[SynthTensor]:
    return config2(cfg_id=2)


def config5_snapshot(k: int, base: Optional[List[SynthTensor]] = None) -> List[SynthTensor]:
    """Snapshot k (1-based) = base + N(0, (0.002 k)^2), rounded once to float32."""
    base = base if base is not None else config5_base()
    return [SynthTensor(t.name, gauss_f32(key_of(5, i, k), t.shape, 0.002 * k, mean=t.data))
            for i, t in enumerate(base)]


def config5_snapshots(ks, base: Optional[List[SynthTensor]] = None, workers: int = 1) -> List[List[SynthTensor]]:
    """config5_snapshot(k, base) for every k in ks."""
    base = base if base is not None else config5_base()
    return _map(lambda k: config5_snapshot(k, base), list(ks), workers)


def stress_s1() -> List[SynthTensor]:
    """Heavy-tailed weights of the 9-layer d=512 shapes: 0.02 * Student-t(3)."""
    return config2(cfg_id=101, dist="t3")


def stress_s2() -> List[SynthTensor]:
    """Long rows: 256x16384 and 64x65536 fp32 N(0, 0.02^2)."""
    return [SynthTensor("long.a", gauss_f32(key_of(102, 0), (256, 16384), SIGMA_W)),
            SynthTensor("long.b", gauss_f32(key_of(102, 1), (64, 65536), SIGMA_W))]


def stress_s4_weights(layers: int = 2) -> List[SynthTensor]:
    """bf16 weights of the d=528 shapes with heavy tails, for percentile-clipped fake quant."""
    out = []
    for i, (nm, shp) in enumerate(config3_shapes(layers)):
        out.append(SynthTensor(nm, f32_to_bf16_bits(student_t3_f32(key_of(104, i), shp, SIGMA_W)), "bf16"))
    return out
