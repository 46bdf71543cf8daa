"""Seeded generation of the workloads' inputs.

Recipe: tensors are listed in the order ``Config.draws()`` gives (index i), each at
its full unsharded shape and cut into row chunks of ``rows_per_chunk = max(1, 2**22 //
cols)`` rows.  Chunk c of tensor i is ``Generator(PCG64(SeedSequence([seed, i, c])))
.standard_normal(dtype=float32)``, multiplied by float32(1/sqrt(fan_in)) for weights.
bf16 workloads then round each float32 value to bfloat16 (round to nearest, ties to
even).  Chunks are independent streams, so they are drawn on a thread pool and the
result does not depend on the number of threads.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

from .configs import Config

CHUNK_ELEMS = 1 << 22  # target elements per independently seeded chunk


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


def _draw(seed: int, index: int, shape, fan_in: int, dtype: str,
          threads: Optional[int] = None) -> np.ndarray:
    rows, cols = shape
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    scale = np.float32(1.0 / np.sqrt(fan_in)) if fan_in else None
    step = max(1, CHUNK_ELEMS // cols)

    def chunk(c: int) -> None:
        r0, r1 = c * step, min(rows, (c + 1) * step)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index, c])))
        x = g.standard_normal(size=(r1 - r0, cols), dtype=np.float32)
        if scale is not None:
            x *= scale
        out[r0:r1] = x if dtype == "f32" else f32_to_bf16_bits(x)

    n = (rows + step - 1) // step
    threads = threads or min(16, os.cpu_count() or 1)
    if n == 1 or threads == 1:
        for c in range(n):
            chunk(c)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(chunk, range(n)))
    return out


def generate(cfg: Config, only: Optional[set] = None,
             threads: Optional[int] = None) -> Dict[str, HostTensor]:
    """All inputs of ``cfg`` (or only the named ones), keyed by name."""
    out: Dict[str, HostTensor] = {}
    for index, (name, shape, fan_in) in enumerate(cfg.draws()):
        if only is not None and name not in only:
            continue
        arr = _draw(cfg.seed, index, shape, fan_in, cfg.dtype, threads)
        out[name] = HostTensor(name, cfg.dtype, tuple(shape), arr)
    if cfg.kind in ("mlp", "block", "attn"):
        ones = np.ones((cfg.hidden,), np.float32)
        zeros = np.zeros((cfg.hidden,), np.float32)
        enc = (lambda v: v) if cfg.dtype == "f32" else f32_to_bf16_bits
        out["gamma"] = HostTensor("gamma", cfg.dtype, (cfg.hidden,), enc(ones))
        out["beta"] = HostTensor("beta", cfg.dtype, (cfg.hidden,), enc(zeros))
    return out


def output_gradient(cfg: Config, threads: Optional[int] = None) -> HostTensor:
    """The gradient dZ [T, H] arriving at the layer's output in the backward pass: N(0, 1)
    in the io dtype, from its own stream (the draw index after the forward inputs)."""
    shape = (cfg.tokens, cfg.hidden)
    arr = _draw(cfg.seed, len(cfg.draws()), shape, 0, cfg.dtype, threads)
    return HostTensor("dZ", cfg.dtype, shape, arr)


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
