"""GPU parity of fa_fwd against the fp64 oracle (through the C ABI)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (announce, assert_bf16_close, assert_fp32_close, errors, f64, need_gpu)

pytestmark = pytest.mark.gpu


def _run(fa, inp, causal, scale=None):
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


def test_c1_fp32_noncausal():
    fa = need_gpu()
    w = workloads.WORKLOADS["c1"]
    announce("fwd c1 fp32 B1 H1 N128 d64")
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "fp32", seed=0)
    o, lse = _run(fa, inp, False, w.scale)
    ro, rl = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), w.scale, False)
    assert_fp32_close(o, ro, "O")
    assert_fp32_close(lse, rl, "LSE")


@pytest.mark.parametrize("causal", [False, True])
def test_c2_bf16(causal):
    fa = need_gpu()
    w = workloads.WORKLOADS["c2"]
    announce(f"fwd c2 bf16 B2 H8 N1024 d64 causal={causal}")
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "bf16", seed=0)
    o, lse = _run(fa, inp, causal)
    ro, rl = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), w.scale, causal)
    assert_bf16_close(o, ro, "O")
    assert_bf16_close(lse, rl, "LSE")


SWEEP = [
    # B, N, Hq, Hkv, d
    (1, 1, 1, 1, 64),
    (1, 7, 2, 1, 128),
    (2, 63, 4, 2, 64),
    (1, 64, 2, 2, 128),
    (1, 65, 8, 1, 128),
    (1, 127, 4, 4, 64),
    (2, 129, 8, 2, 128),
    (1, 200, 8, 8, 128),
    (1, 1000, 4, 1, 128),
    (1, 333, 16, 2, 64),
    (1, 2113, 2, 1, 128),
    (1, 2113, 2, 1, 64),     # d = 64, key range split over the waves, 17 steps of 128 keys
    (4, 1100, 16, 4, 64),    # d = 64 with 576 workgroups of 128 rows: the DMA kernel with 128-byte rows
    (2, 1500, 16, 2, 64),    # d = 64 DMA kernel: ragged last tile, 8 query heads per kv head
    (3, 900, 12, 3, 64),     # d = 64 DMA kernel: 288 workgroups, B = 3, 4 query heads per kv head
    (2, 300, 6, 2, 128),     # 3 query heads per kv head (B*Hq = 12: plain block order)
    (4, 260, 6, 2, 128),     # 3 per kv head, B*Hq = 24: XCD order with a partial head group (3 of 4)
    (1, 190, 5, 1, 64),      # 5 query heads per kv head, d = 64 split-key kernel
    (4, 1100, 12, 2, 64),    # 6 per kv head, d = 64 DMA kernel (432 workgroups, XCD order)
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SWEEP, ids=[f"B{b}N{n}Hq{hq}Hkv{hk}d{d}" for b, n, hq, hk, d in SWEEP])
def test_bf16_sweep(shape, causal):
    fa = need_gpu()
    B, N, Hq, Hkv, d = shape
    announce(f"fwd bf16 sweep {shape} causal={causal}")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=N + 11 * Hq + d)
    o, lse = _run(fa, inp, causal)
    ro, rl = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 1 / math.sqrt(d), causal)
    assert_bf16_close(o, ro, "O")
    assert_bf16_close(lse, rl, "LSE")


FP32_SWEEP = [(1, 1, 1, 1, 64), (1, 65, 2, 1, 128), (2, 130, 4, 2, 64), (1, 257, 2, 2, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", FP32_SWEEP, ids=[f"B{b}N{n}Hq{hq}Hkv{hk}d{d}" for b, n, hq, hk, d in FP32_SWEEP])
def test_fp32_sweep(shape, causal):
    fa = need_gpu()
    B, N, Hq, Hkv, d = shape
    announce(f"fwd fp32 sweep {shape} causal={causal}")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "fp32", seed=3 * N + d)
    o, lse = _run(fa, inp, causal)
    ro, rl = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 1 / math.sqrt(d), causal)
    assert_fp32_close(o, ro, "O")
    assert_fp32_close(lse, rl, "LSE")


def test_first_causal_row_is_v0_exactly():
    """With one visible key, p = exp2(0) = 1 and l = 1, so O[0] equals V[0] bit for bit."""
    fa = need_gpu()
    announce("fwd first causal row")
    inp = workloads.prefill_inputs(2, 300, 8, 2, 128, "bf16", seed=5)
    o, _ = _run(fa, inp, True)
    v0 = inp["v"][:, 0].repeat_interleave(4, dim=1)
    assert torch.equal(o[:, 0].cpu(), v0)


def test_deterministic():
    fa = need_gpu()
    announce("fwd determinism")
    inp = workloads.prefill_inputs(1, 777, 8, 2, 128, "bf16", seed=9)
    o1, l1 = _run(fa, inp, True)
    o2, l2 = _run(fa, inp, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_identical_keys_and_shift():
    """Identical keys give the mean of the visible V rows; a large common
    shift of every key leaves O unchanged (exercises the running-max rescale)."""
    fa = need_gpu()
    announce("fwd identical keys / shift")
    B, N, H, d = 1, 190, 4, 128
    inp = workloads.prefill_inputs(B, N, H, H, d, "bf16", seed=21)
    kk = inp["k"].clone()
    kk[:] = kk[:, :1]
    o, lse = _run(fa, {"q": inp["q"], "k": kk, "v": inp["v"]}, True)
    vf = f64(inp["v"])
    mean = np.cumsum(vf, axis=1) / np.arange(1, N + 1)[None, :, None, None]
    assert_bf16_close(o, mean, "O identical keys")
    shifted = (inp["k"].float() + 8.0).to(torch.bfloat16)
    o1, _ = _run(fa, {"q": inp["q"], "k": shifted, "v": inp["v"]}, False)
    ro, _ = oracle.attn_fwd(f64(inp["q"]), f64(shifted), vf, 1 / math.sqrt(d), False)
    assert_bf16_close(o1, ro, "O shifted keys")


def test_error_no_larger_than_twice_bf16_baseline():
    """The upstream test rule: error against the exact result at most twice
    that of a plain attention computed in bf16 (torch on the CPU)."""
    fa = need_gpu()
    announce("fwd vs bf16 baseline error")
    B, N, H, d = 1, 512, 4, 128
    inp = workloads.prefill_inputs(B, N, H, H, d, "bf16", seed=33)
    o, _ = _run(fa, inp, True)
    ro, _ = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 1 / math.sqrt(d), True)
    q, k, v = (inp[n].transpose(1, 2) for n in ("q", "k", "v"))
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * (1 / math.sqrt(d))
    s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    base = torch.matmul(torch.softmax(s.float(), dim=-1).to(torch.bfloat16), v).transpose(1, 2)
    gpu_err, _ = errors(o, ro)
    base_err, _ = errors(base, ro)
    assert gpu_err <= 2 * base_err + 1e-6, (gpu_err, base_err)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_rising_scores_rescale_running_output(d, causal):
    """Key norms grow along the sequence (x0.1 at the start to x12 at the end),
    so a row's running maximum rises by far more than the kernel's rescale
    slack several times after O has accumulated real contributions: every
    rescale of a non-zero O is exercised and checked against the oracle."""
    fa = need_gpu()
    B, N, Hq, Hkv = 1, 1500, 4, 2
    announce(f"fwd rising scores N{N} d{d} causal={causal}")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=5)
    gain = torch.linspace(0.1, 12.0, N, dtype=torch.float32).view(1, N, 1, 1)
    inp["k"] = (inp["k"].float() * gain).to(torch.bfloat16)
    o, lse = _run(fa, inp, causal)
    ro, rl = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 1.0 / math.sqrt(d), causal)
    # the scores really do move: for the last row, the largest score among
    # the last 256 keys exceeds that among the first 256 by > 20 (natural log)
    qn, kn = f64(inp["q"])[0, N - 1, 0], f64(inp["k"])[0, :, 0]
    sc = kn @ qn / math.sqrt(d)
    assert sc[N - 256:].max() - sc[:256].max() > 20.0
    assert_bf16_close(o, ro, "O")
    assert_bf16_close(lse, rl, "LSE")
