"""Shared helpers for the parity tests: tolerances, comparisons, device moves.

Tolerances (written here once, used by every GPU parity test):
  bf16 inputs with fp32 accumulation: |GPU - oracle| <= 2e-2 element-wise
  and mean |GPU - oracle| <= 2e-3 per output tensor;
  fp32: max |GPU - oracle| <= 1e-5.
Differences are taken in float64 after upcasting the GPU output exactly.

A bf16 output cannot resolve 2e-2 where the exact value has magnitude 4 or
more (one bf16 ulp is 2^-5 = 0.03125 on [4, 8)): there even the correctly
rounded exact answer can miss the bar. The element-wise bound is therefore
max(2e-2, one bf16 ulp of the exact value), which equals 2e-2 for every
|value| < 4 and is one ulp above that. fp32 outputs of the bf16 path (the
logsumexp) keep the plain 2e-2 bound.
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


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 0.0)


def assert_bf16_close(got, want, what: str):
    """Bound for a result of the bf16 path. Outputs stored as bf16 get the
    one-ulp allowance above; fp32 outputs of the bf16 path (LSE) do not."""
    mx, mean = errors(got, want)
    g, w = f64(got), f64(want)
    finite = np.isfinite(w)
    stored_bf16 = isinstance(got, torch.Tensor) and got.dtype == torch.bfloat16
    bound = np.maximum(BF16_MAX_ABS, bf16_ulp(w[finite])) if stored_bf16 else BF16_MAX_ABS
    over = np.abs(g[finite] - w[finite]) - bound
    worst = float(over.max()) if over.size else -1.0
    assert worst <= 0 and mean <= BF16_MEAN_ABS, f"{what}: max {mx:.3e} (over bound by {worst:.3e}) mean {mean:.3e}"
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
