"""Seeded synthetic inputs shared by the tests, the bench and the oracle legs.

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic (no quantisation, no dequantisation, no GEMM, no merge).
Both the CPU oracle and the GPU library receive exactly the bytes produced
here.

Each tensor has its own numpy ``Generator(PCG64)`` stream keyed by
``(seed, config, layer, projection, tensor_id)``; values are drawn as float64
standard normals, scaled, and cast to fp32.  bf16 tensors are then converted
with torch's own fp32 -> bf16 cast (a library routine) and handed out as
uint16 bit patterns.

Distributions follow the layer's workloads: W0 ~ N(0, 0.02^2) fp32;
A ~ N(0, 1/k); B ~ N(0, 0.01^2); activations x and dy ~ N(0, 1) in bf16.
"""

from __future__ import annotations

import numpy as np

TENSOR_W0, TENSOR_A, TENSOR_B, TENSOR_X, TENSOR_DY = 0, 1, 2, 3, 4


def _rng(key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def normal_f32(shape, std: float, key) -> np.ndarray:
    """fp32 array ~ N(0, std^2), drawn in float64 from the keyed stream."""
    x = _rng(key).standard_normal(size=shape, dtype=np.float64) * std
    return x.astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) via torch's built-in cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, std: float, key) -> np.ndarray:
    """bf16 bit patterns of N(0, std^2) draws."""
    return to_bf16_bits(normal_f32(shape, std, key))


def layer_inputs(d: int, k: int, r: int, M: int, *, seed: int = 0, cfg: int = 0,
                 layer: int = 0, proj: int = 0, b_zero: bool = False) -> dict:
    """All inputs of one adapted linear: W0 fp32, A/B/X/dY as bf16 bits."""
    base = (seed, cfg, layer, proj)
    out = {
        "W0": normal_f32((d, k), 0.02, base + (TENSOR_W0,)),
        "A": normal_bf16((r, k), float(k) ** -0.5, base + (TENSOR_A,)),
        "B": normal_bf16((d, r), 0.01, base + (TENSOR_B,)),
        "X": normal_bf16((M, k), 1.0, base + (TENSOR_X,)),
        "dY": normal_bf16((M, d), 1.0, base + (TENSOR_DY,)),
    }
    if b_zero:
        out["B"] = np.zeros((d, r), dtype=np.uint16)
    return out


# The workloads the layer is measured and checked on.  Each entry names the
# shapes (d x k), rank, alpha and token count of one configuration.
CONFIGS = {
    "small_256": dict(shapes=[(256, 256)], r=8, alpha=16.0, M=32),
    "attn_4096": dict(shapes=[(4096, 4096)], r=8, alpha=16.0, M=4096),
    "attn_4096_r16": dict(shapes=[(4096, 4096)], r=16, alpha=32.0, M=4096),
    "decode_m16": dict(shapes=[(4096, 4096), (11008, 4096), (4096, 11008)],
                       r=16, alpha=32.0, M=16),
    "stack_7b": dict(shapes=[(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)],
                     r=16, alpha=32.0, M=2048, layers=32),
    "stack_65b": dict(shapes=[(8192, 8192)] * 4 + [(22016, 8192)] * 2 + [(8192, 22016)],
                      r=64, alpha=16.0, M=4096, layers=80),
}
