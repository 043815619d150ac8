"""Shared helpers for the GPU parity tests.

Tolerances (bf16 storage, fp32 accumulation): max-abs error <= 2e-2 and
relative L2 error ||gpu - oracle||_2 / ||oracle||_2 <= 5e-3 over the compared
outputs; fp32 path: max-abs <= 1e-5. The oracle's fp64 result is compared
unrounded.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
FP32_MAX_ABS = 1e-5


def have_gpu() -> bool:
    return torch.cuda.is_available()


def say(msg: str):
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def errors(gpu, ref):
    g = gpu.detach().float().cpu().double().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    diff = g - r
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(r))
    rel_l2 = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel_l2


def assert_parity(gpu, ref, dtype, what=""):
    max_abs, rel_l2 = errors(gpu, ref)
    if dtype == torch.float32:
        assert max_abs <= FP32_MAX_ABS, f"{what}: fp32 max-abs {max_abs:.3e} > {FP32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max-abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel_l2 <= BF16_REL_L2, f"{what}: rel-L2 {rel_l2:.3e} > {BF16_REL_L2}"
    return max_abs, rel_l2


def to_host(t: torch.Tensor) -> torch.Tensor:
    return t.detach().cpu().contiguous()
