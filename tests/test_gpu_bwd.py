"""GPU parity of fa_bwd against the fp64 oracle (through the C ABI)."""
from __future__ import annotations

import math

import pytest
import torch

import oracle
import workloads
import bwd_rounding
from parity import announce, assert_bf16_close, f64, need_gpu

pytestmark = pytest.mark.gpu

SWEEP = [
    # B, N, Hq, Hkv, d
    (1, 1, 1, 1, 64),
    (1, 64, 2, 2, 128),
    (1, 65, 2, 1, 64),
    (2, 130, 4, 2, 128),
    (1, 200, 4, 4, 64),
    (1, 257, 8, 2, 128),
    (1, 512, 2, 1, 128),
] + bwd_rounding.ODD_GROUPS  # 3, 6 (B*Hkv = 8: dK/dV in XCD order) and 5 query heads per kv head


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SWEEP, ids=[f"B{b}N{n}Hq{hq}Hkv{hk}d{d}" for b, n, hq, hk, d in SWEEP])
def test_bwd_sweep(shape, causal):
    fa = need_gpu()
    B, N, Hq, Hkv, d = shape
    announce(f"bwd sweep {shape} causal={causal}")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=bwd_rounding.sweep_seed(shape), with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    rdq, rdk, rdv, _ = oracle.attn_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]),
                                       1 / math.sqrt(d), causal)
    assert_bf16_close(dq, rdq, "dQ")
    assert_bf16_close(dk, rdk, "dK")
    assert_bf16_close(dv, rdv, "dV")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", bwd_rounding.MANY_HEADS,
                         ids=[f"B{b}N{n}Hq{hq}Hkv{hk}d{d}" for b, n, hq, hk, d in bwd_rounding.MANY_HEADS])
def test_bwd_many_query_heads_per_kv_head(shape, causal):
    """dK, dV summed over 8 or 16 query heads, inputs N(0,1)."""
    fa = need_gpu()
    B, N, Hq, Hkv, d = shape
    announce(f"bwd many heads {shape} causal={causal}")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=bwd_rounding.many_heads_seed(shape), with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    rdq, rdk, rdv, _ = oracle.attn_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]),
                                       1 / math.sqrt(d), causal)
    assert_bf16_close(dq, rdq, "dQ")
    assert_bf16_close(dk, rdk, "dK")
    assert_bf16_close(dv, rdv, "dV")


def test_bwd_deterministic():
    fa = need_gpu()
    announce("bwd determinism")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(1, 300, 8, 2, 128, "bf16", seed=3, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    a = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    b = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


ATOMIC = [
    # B, N, Hq, Hkv, d (d = 128 only)
    (1, 1, 1, 1, 128),
    (1, 64, 2, 2, 128),
    (2, 130, 4, 2, 128),
    (1, 257, 8, 2, 128),
    (1, 300, 16, 2, 128),
    (1, 512, 2, 1, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", ATOMIC, ids=[f"B{b}N{n}Hq{hq}Hkv{hk}d{d}" for b, n, hq, hk, d in ATOMIC])
def test_bwd_atomic(shape, causal):
    """fa_bwd_atomic: dQ, dK, dV against the oracle; dK and dV within one bf16
    ulp of the deterministic backward's (the same fp32 terms, summed in
    another order: the deterministic d = 128 kernel adds the two query halves
    of every tile in separate waves); every output written (NaN-filled)."""
    fa = need_gpu()
    B, N, Hq, Hkv, d = shape
    announce(f"bwd atomic {shape} causal={causal}")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=300 + N, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.fa_bwd(q, k, v, o, do, lse, causal=causal, dq=dq, dk=dk, dv=dv, deterministic=False)
    rq, rk, rv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    for name, x, y in (("dK", dk, rk), ("dV", dv, rv)):
        x64, y64 = x.double(), y.double()
        big = torch.maximum(x64.abs(), y64.abs())
        ulp = torch.ldexp(torch.ones_like(big), torch.frexp(big).exponent - 8)
        gap = (x64 - y64).abs()
        assert torch.isfinite(x64).all() and bool((gap <= ulp + 1e-6).all()), \
            f"{name}: atomic and deterministic differ by {float((gap - ulp).max()):.3e} beyond one ulp"
    rdq, rdk, rdv, _ = oracle.attn_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]),
                                       1 / math.sqrt(d), causal)
    assert_bf16_close(dq, rdq, "dQ")
    assert_bf16_close(dk, rdk, "dK")
    assert_bf16_close(dv, rdv, "dV")
