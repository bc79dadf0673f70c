"""Helpers for the GPU tests: host <-> device transfer of bf16 bit patterns and the error metrics
the parity bar is stated in."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W

# Output parity bar for bf16 outputs against the float64 oracle.
MAX_ABS_TOL = 2e-2
MEAN_ABS_TOL = 2e-3


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 tensor on cuda:0 (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> float64 numpy (exact)."""
    bits = t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def err(a, b, mask=None):
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    if mask is not None:
        d = d[mask]
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_output_parity(got, ref, what=""):
    mx, mean = err(got, ref)
    assert mx <= MAX_ABS_TOL and mean <= MEAN_ABS_TOL, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def announce(msg: str) -> None:
    """Print and flush the case about to run on the GPU."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()
