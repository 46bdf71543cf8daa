"""Seeded generation of the workloads' inputs.

Recipe: numpy ``Generator(PCG64(seed))``; draws in the order ``Config.draws()``
lists them, each at its full unsharded shape, ``standard_normal(dtype=float32)``
multiplied by float32(1/sqrt(fan_in)) for weights.  bf16 workloads then round
each float32 value to bfloat16 with round-to-nearest-even.  Large tensors are
drawn in row chunks; a PCG64 stream consumed in chunks yields the same values as
one draw of the whole tensor.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

from .configs import Config

_CHUNK = 1 << 24  # elements per draw chunk


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.
    Inputs are finite normal draws, so NaN handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exact float32 values they encode."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class HostTensor:
    """One generated input.  ``dtype`` is "f32" or "bf16".  For bf16, ``bits`` holds the
    uint16 encoding (what the device receives) and ``values()`` decodes it exactly."""
    name: str
    dtype: str
    shape: tuple
    data: np.ndarray  # float32 values (f32) or uint16 bits (bf16)

    def values(self) -> np.ndarray:
        return self.data if self.dtype == "f32" else bf16_bits_to_f32(self.data)

    def device_array(self) -> np.ndarray:
        """What is copied to the device: float32 values, or the bf16 bits viewed as int16."""
        return self.data if self.dtype == "f32" else self.data.view(np.int16)


def _draw(rng: np.random.Generator, shape, fan_in: int, dtype: str) -> np.ndarray:
    rows, cols = shape
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    scale = np.float32(1.0 / np.sqrt(fan_in)) if fan_in else None
    step = max(1, _CHUNK // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = rng.standard_normal(size=(r1 - r0, cols), dtype=np.float32)
        if scale is not None:
            x *= scale
        out[r0:r1] = x if dtype == "f32" else f32_to_bf16_bits(x)
    return out


def generate(cfg: Config, only: Optional[set] = None) -> Dict[str, HostTensor]:
    """All inputs of ``cfg`` in draw order.  Tensors not in ``only`` are still drawn
    (to keep the stream aligned) but not kept."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    out: Dict[str, HostTensor] = {}
    for name, shape, fan_in in cfg.draws():
        arr = _draw(rng, shape, fan_in, cfg.dtype)
        if only is None or name in only:
            out[name] = HostTensor(name, cfg.dtype, tuple(shape), arr)
    if cfg.kind in ("mlp", "block", "attn"):
        ones = np.ones((cfg.hidden,), np.float32)
        zeros = np.zeros((cfg.hidden,), np.float32)
        enc = (lambda v: v) if cfg.dtype == "f32" else f32_to_bf16_bits
        out["gamma"] = HostTensor("gamma", cfg.dtype, (cfg.hidden,), enc(ones))
        out["beta"] = HostTensor("beta", cfg.dtype, (cfg.hidden,), enc(zeros))
    return out


def random_affine(cfg: Config, seed: int) -> Dict[str, HostTensor]:
    """Non-trivial LayerNorm gamma/beta for extra coverage (gamma ~ 1 + 0.5 N(0,1),
    beta ~ 0.5 N(0,1))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = (1.0 + 0.5 * rng.standard_normal(cfg.hidden)).astype(np.float32)
    b = (0.5 * rng.standard_normal(cfg.hidden)).astype(np.float32)
    enc = (lambda v: v) if cfg.dtype == "f32" else f32_to_bf16_bits
    return {"gamma": HostTensor("gamma", cfg.dtype, (cfg.hidden,), enc(g)),
            "beta": HostTensor("beta", cfg.dtype, (cfg.hidden,), enc(b))}


def integer_matrix(rng: np.random.Generator, shape, lo: int, hi: int, dtype: str,
                   nnz_per_row: Optional[int] = None) -> HostTensor:
    """Small-integer matrices for exactness pins: entries uniform in [lo, hi]; with
    ``nnz_per_row`` all but that many entries per row are zero."""
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    if nnz_per_row is not None:
        mask = np.zeros(shape, bool)
        for i in range(shape[0]):
            mask[i, rng.choice(shape[1], size=min(nnz_per_row, shape[1]), replace=False)] = True
        v = np.where(mask, v, np.float32(0))
    data = v if dtype == "f32" else f32_to_bf16_bits(v)
    return HostTensor("int", dtype, tuple(shape), data)


def from_values(name: str, v: np.ndarray, dtype: str) -> HostTensor:
    """Wrap caller-made float32 values (exactly representable in ``dtype``)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    data = v if dtype == "f32" else f32_to_bf16_bits(v)
    return HostTensor(name, dtype, tuple(v.shape), data)
