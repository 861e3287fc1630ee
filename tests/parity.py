"""Shared helpers for the parity tests: tolerances, comparisons, device moves.

Tolerances (written here once, used by every GPU parity test):
  bf16 inputs with fp32 accumulation: |GPU - oracle| <= 2e-2 element-wise
  and mean |GPU - oracle| <= 2e-3 per output tensor;
  fp32: max |GPU - oracle| <= 1e-5.
Differences are taken in float64 after upcasting the GPU output exactly.

A bf16-stored output is a rounded value: storing even the exact answer
costs up to half a bf16 ulp of it (2^-9 relative, 0.0156 on [4, 8)). The
element-wise bound for a bf16-stored output is therefore 2e-2 + half a bf16
ulp of the exact value: the kernel's fp32 result within 2e-2, then the one
rounding no bf16 output can avoid. Below |x| = 1 the allowance is under 2e-3;
it reaches 2e-2 only from |x| = 8. fp32 outputs of the bf16 path (the
logsumexp) keep the plain 2e-2 bound. Every bf16 comparison reports how many
elements needed the allowance (error above 2e-2).
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


def bf16_bound(want: np.ndarray) -> np.ndarray:
    """Element-wise bound for a bf16-stored output with exact value ``want``:
    2e-2 plus half a bf16 ulp of that value."""
    return BF16_MAX_ABS + 0.5 * bf16_ulp(want)


def bf16_check(got, want, stored_bf16: bool):
    """(max |err|, mean |err|, worst excess over the bound, elements that
    needed the half-ulp allowance) over the finite entries of ``want``."""
    mx, mean = errors(got, want)
    g, w = f64(got), f64(want)
    finite = np.isfinite(w)
    err = np.abs(g[finite] - w[finite])
    bound = bf16_bound(w[finite]) if stored_bf16 else np.full(err.shape, BF16_MAX_ABS)
    over = err - bound
    worst = float(over.max()) if over.size else -1.0
    n_allow = int(np.count_nonzero((err > BF16_MAX_ABS) & (over <= 0)))
    return mx, mean, worst, n_allow


def assert_bf16_close(got, want, what: str):
    """Bound for a result of the bf16 path. Outputs stored as bf16 get the
    half-ulp output-rounding allowance; fp32 outputs of the bf16 path (LSE)
    do not."""
    stored_bf16 = isinstance(got, torch.Tensor) and got.dtype == torch.bfloat16
    mx, mean, worst, n_allow = bf16_check(got, want, stored_bf16)
    print(f"[parity] {what}: max {mx:.3e} mean {mean:.3e} elements over 2e-2 within the half-ulp allowance: "
          f"{n_allow}", flush=True)
    assert worst <= 0 and mean <= BF16_MEAN_ABS, f"{what}: max {mx:.3e} (over bound by {worst:.3e}) mean {mean:.3e}"
    return mx, mean


def assert_fp32_close(got, want, what: str):
    mx, mean = errors(got, want)
    print(f"[parity] {what}: max {mx:.3e} mean {mean:.3e} (fp32)", flush=True)
    assert mx <= FP32_MAX_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def need_gpu():
    import pytest

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_19_amd as fa

    fa.load()  # raises when the HIP library is missing: no fallback
    return fa
