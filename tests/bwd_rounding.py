"""CPU emulation of the bf16 rounding that the backward kernels cannot avoid.

Test infrastructure. The recompute backward (abeam summary, "学習時の backward
では再計算を使う") feeds two of its products with bf16 operands made from
fp32 intermediates: the probabilities P for dV = P^T dO, and the score
gradient dS = P (dP - D) for dK = scale dS^T Q and dQ = scale dS K. D is the
row sum of dO * O taken from the stored (bf16) O. This module repeats
exactly those roundings on top of exact fp64 arithmetic and rounds the
results to bf16, so a test can tell how far from the oracle rounding alone
puts a backward of a given shape and input scale, whatever the kernel does
beyond it.

The CPU tests use it to show that the suite's bf16 bound is attainable by
such a kernel for the backward shapes it checks at N(0,1) inputs, and that
a bound without the output-rounding allowance below |x| = 8 is not.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import workloads
from parity import bf16_check, f64


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 the way the kernels do: the fp32 value, then RNE."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def emulate_bwd(q, k, v, do, scale, causal, window=(-1, -1)):
    """dQ, dK, dV with P and dS rounded to bf16 (and D from bf16 O), every
    other step exact, the results rounded to bf16."""
    b_, n, hq, d = q.shape
    hkv = k.shape[2]
    g = hq // hkv
    o, _ = oracle.attn_fwd(q, k, v, scale, causal, window)
    o_b = to_bf16(o)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(b_):
        for h in range(hq):
            kh = h // g
            qh, kk, vv, doh = q[b, :, h], k[b, :, kh], v[b, :, kh], do[b, :, h]
            _, p, _ = oracle.head_probs(qh, kk, scale, causal, window=window)
            dp = doh @ vv.T
            dd = (doh * o_b[b, :, h]).sum(axis=1, keepdims=True)
            ds_b = to_bf16(p * (dp - dd))
            dv[b, :, kh] += to_bf16(p).T @ doh
            dk[b, :, kh] += scale * (ds_b.T @ qh)
            dq[b, :, h] = scale * (ds_b @ kk)
    return to_bf16(dq), to_bf16(dk), to_bf16(dv)


# Backward cases with 8 or 16 query heads summed into each dK, dV
# (B, N, Hq, Hkv, d); the GPU test draws them from seed many_heads_seed().
MANY_HEADS = [
    (1, 300, 16, 2, 128),
    (2, 200, 16, 1, 128),
    (1, 129, 8, 1, 64),
]


def many_heads_seed(shape) -> int:
    _, n, _, _, d = shape
    return 200 + n + d


# Backward sweep cases with query-head groups that are not powers of two
# (3, 6 and 5 query heads per kv head); the GPU sweep draws them from seed
# sweep_seed() at N(0,1).
ODD_GROUPS = [
    (2, 300, 6, 2, 128),
    (4, 260, 12, 2, 128),
    (1, 190, 5, 1, 64),
]


def sweep_seed(shape) -> int:
    _, n, _, _, d = shape
    return 100 + n + d


def emulation_report(shape, causal, mult=1.0, bound=None, seed=None):
    """Per output: (max err, mean err, worst excess over the bound, elements
    in the allowance) of the rounding emulation against the oracle. ``bound``
    maps exact values to element-wise bounds (default: the test suite's);
    ``seed`` defaults to many_heads_seed(shape)."""
    B, N, Hq, Hkv, d = shape
    seed = many_heads_seed(shape) if seed is None else seed
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=seed, mult=mult, do_mult=mult, with_do=True)
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    scale = 1 / math.sqrt(d)
    exact = oracle.attn_bwd(q, k, v, do, scale, causal)[:3]
    emul = emulate_bwd(q, k, v, do, scale, causal)
    out = {}
    for name, e, x in zip(("dQ", "dK", "dV"), emul, exact):
        if bound is None:
            out[name] = bf16_check(e, x, stored_bf16=True)
        else:
            err = np.abs(e - x)
            out[name] = (float(err.max()), float(err.mean()), float((err - bound(x)).max()), 0)
    return out
