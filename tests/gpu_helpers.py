"""Helpers of the GPU parity tests: device upload, read-back, and the comparison rule.

The rule (the stated tolerance, per output tensor):
    max |gpu - ref| / max |ref|  <=  1e-4 (fp32 io)  or  2e-2 (bf16 io, fp32 accumulation)
A second, tighter guard on the root-mean-square error (a quarter of the same bound) catches
a wrong but small subset of elements that the max-relative rule could let through."""
from __future__ import annotations

import sys

import numpy as np
import torch

from workloads import HostTensor, f32_to_bf16_bits

TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(t: HostTensor, device="cuda:0") -> torch.Tensor:
    from megatron_tensor_transformer_linear_amd.pipeline import to_device
    return to_device(t.data, t.dtype, device)


def dev_values(v: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    from megatron_tensor_transformer_linear_amd.pipeline import to_device
    v = np.ascontiguousarray(v, dtype=np.float32)
    return to_device(v if dtype == "f32" else f32_to_bf16_bits(v), dtype, device)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 decoded exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a device tensor (uint16 for bf16, uint32 for fp32)."""
    if t.dtype == torch.bfloat16:
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def ref_bits(ref: np.ndarray, dtype: str) -> np.ndarray:
    r32 = np.ascontiguousarray(ref, dtype=np.float32)
    return f32_to_bf16_bits(r32) if dtype == "bf16" else r32.view(np.uint32)


def errors(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, f"shape {gpu.shape} vs {ref.shape}"
    d = gpu - ref
    mref = float(np.max(np.abs(ref)))
    rms_ref = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(d))) / mref, float(np.sqrt(np.mean(d * d))) / rms_ref


def check(name: str, gpu, ref: np.ndarray, dtype: str) -> None:
    g = host(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    mx, rms = errors(g, ref)
    tol = TOL[dtype]
    say(f"    {name:<28s} max_rel {mx:.3e}  rms_rel {rms:.3e}  (tol {tol:.0e})")
    assert mx <= tol, f"{name}: max rel err {mx:.3e} > {tol}"
    assert rms <= tol / 4, f"{name}: rms rel err {rms:.3e} > {tol / 4}"


def check_exact(name: str, gpu: torch.Tensor, ref: np.ndarray, dtype: str) -> None:
    g = bits(gpu)
    r = ref_bits(ref, dtype)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    bad = int(np.count_nonzero(g != r))
    say(f"    {name:<28s} bit-exact mismatches {bad} / {g.size}")
    assert bad == 0, f"{name}: {bad} elements differ bitwise"


def sample_rows(T: int, seq: int, seed: int, n_random: int = 6):
    rows = {0, 1, T - 1, min(T - 1, 255), min(T - 1, 256)}
    if seq:
        for b in range(T // seq):
            rows |= {b * seq, b * seq + seq - 1}
    rng = np.random.Generator(np.random.PCG64(seed))
    rows |= set(int(x) for x in rng.integers(0, T, n_random))
    return np.array(sorted(rows))

