"""Shared helpers for the parity tests: tolerances, comparisons, device moves.

Tolerances (written here once, used by every GPU parity test):
  bf16 inputs with fp32 accumulation: max |GPU - oracle| <= 2e-2 and
  mean |GPU - oracle| <= 2e-3 per output tensor;
  fp32: max |GPU - oracle| <= 1e-5.
Differences are taken in float64 after upcasting the GPU output exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
FP32_MAX_ABS = 1e-5


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault can be traced to it."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def errors(got, want):
    g, w = f64(got), f64(want)
    assert g.shape == w.shape, (g.shape, w.shape)
    finite = np.isfinite(w)
    assert np.array_equal(np.isfinite(g), finite), "non-finite values differ"
    d = np.abs(g[finite] - w[finite])
    if d.size == 0:
        return 0.0, 0.0
    return float(d.max()), float(d.mean())


def assert_bf16_close(got, want, what: str):
    mx, mean = errors(got, want)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def assert_fp32_close(got, want, what: str):
    mx, mean = errors(got, want)
    assert mx <= FP32_MAX_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def need_gpu():
    import pytest

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_19_amd as fa

    fa.load()  # raises when the HIP library is missing: no fallback
    return fa
