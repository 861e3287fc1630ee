"""Long sequences and tensors beyond 2 GiB: causal forward and backward at
N = 131072 with 64 heads of d = 128, so that each of Q, K, V, O, dO, dQ, dK
and dV holds 2 GiB (byte offsets past 2^31). Every output is written into a
NaN-filled buffer and must come back finite. Checks against the oracle, at
a cost linear in N per sampled row: forward rows, and dQ rows (row i of dQ
needs only row i of P and dP); and a property of dV that holds at any size:
rows of P sum to one, so the sum of dV over the keys equals the sum of dO
over the queries, up to the bf16 rounding of P and of dV."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import announce, assert_bf16_close, f64, need_gpu

pytestmark = pytest.mark.gpu

B, N, H, D = 1, 131072, 64, 128
HEADS = (0, 37, 63)


def _rows(rng):
    rows = {0, 1, 63, 64, 127, 128, 4095, 4096, N // 2, N - 129, N - 128, N - 2, N - 1}
    rows |= set(int(x) for x in rng.integers(0, N, 10))
    return np.array(sorted(rows))


def _head(t, h):
    """One head of a [B, N, H, d] device tensor as a float64 host array [1, N, 1, d]."""
    return f64(t[:, :, h:h + 1].cpu())


def test_causal_fwd_bwd_131072_tokens_64_heads():
    fa = need_gpu()
    dev = torch.device("cuda:0")
    announce(f"long causal fwd+bwd B={B} N={N} H={H} d={D} (2 GiB per tensor)")
    q = workloads.device_normal((B, N, H, D), seed=1301, mult=0.5)
    k = workloads.device_normal((B, N, H, D), seed=1302, mult=0.5)
    v = workloads.device_normal((B, N, H, D), seed=1303, mult=0.5)
    do = workloads.device_normal((B, N, H, D), seed=1304)
    assert q.numel() * q.element_size() == 1 << 31
    scale = 1 / math.sqrt(D)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_fwd(q, k, v, scale=scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert torch.equal(o[:, 0], v[:, 0])

    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    fa.fa_bwd(q, k, v, o, do, lse, scale=scale, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()

    rng = np.random.default_rng(1305)
    rows = _rows(rng)
    for h in HEADS:
        qh, kh, vh, doh = _head(q, h), _head(k, h), _head(v, h), _head(do, h)
        ro, rl = oracle.attn_fwd_rows(qh, kh, vh, scale, True, 0, 0, rows)
        assert_bf16_close(o[0, rows, h].cpu(), ro, f"O head {h}")
        assert_bf16_close(lse[0, h, rows].cpu(), rl, f"LSE head {h}")
        rdq, _ = oracle.attn_bwd_dq_rows(qh, kh, vh, doh, scale, True, 0, 0, rows)
        assert_bf16_close(dq[0, rows, h].cpu(), rdq, f"dQ head {h}")
        # sum_j dV_j = sum_i dO_i (P rows sum to one); P enters dV rounded to
        # bf16 (<= 2^-9 relative per term) and dV is stored in bf16 (<= 2^-9
        # relative per element): bound twice their sum, per column.
        dvh = f64(dv[0, :, h].cpu())
        lhs = dvh.sum(axis=0)
        rhs = doh[0, :, 0].sum(axis=0)
        bound = 2 * 2.0 ** -9 * (np.abs(doh[0, :, 0]).sum(axis=0) + np.abs(dvh).sum(axis=0))
        worst = float((np.abs(lhs - rhs) - bound).max())
        print(f"[parity] head {h}: sum dV vs sum dO, worst excess over bound {worst:.3e}")
        assert worst <= 0.0, f"head {h}: column sums of dV differ from those of dO beyond the rounding bound"
