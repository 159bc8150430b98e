"""Helpers shared by the GPU tests: move seeded numpy inputs to the device, compare to the oracle."""
from __future__ import annotations

import numpy as np

import synth

BF16_TOL = 2e-2  # max |gpu - oracle| for bf16 inputs, fp32 accumulation
F32_TOL = 1e-5   # max |gpu - oracle| for fp32 inputs


def torch_mod():
    import torch
    return torch


def to_dev(x: np.ndarray, dtype: str):
    """Seeded numpy array (fp32 values or bf16 bit patterns) -> contiguous CUDA tensor."""
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def to_host_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def values(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 values of a stored tensor (bf16 bit patterns are widened)."""
    return synth.as_f32(x, dtype)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0
