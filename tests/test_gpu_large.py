"""Full-size parity: the workloads at their real sizes, launched exactly as the
benchmark launches them, checked against the fp64 oracle on sampled outputs
(rows, heads, sequences) plus properties that hold at every position."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import announce, assert_bf16_close, f64, need_gpu

pytestmark = pytest.mark.gpu


def _sample_rows(N, rng, extra=12):
    rows = {0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 65, N - 64, N - 2, N - 1}
    rows |= set(int(x) for x in rng.integers(0, N, extra))
    return np.array(sorted(r for r in rows if 0 <= r < N))


def _check_fwd_sampled(inp, o, lse, w, heads, rng):
    rows = _sample_rows(w.N, rng)
    g = w.Hq // w.Hkv
    for (b, h) in heads:
        kh = h // g
        q = f64(inp["q"][b:b + 1, :, h:h + 1])
        k = f64(inp["k"][b:b + 1, :, kh:kh + 1])
        v = f64(inp["v"][b:b + 1, :, kh:kh + 1])
        ro, rl = oracle.attn_fwd_rows(q, k, v, w.scale, w.causal, 0, 0, rows)
        assert_bf16_close(o[b, rows, h], ro, f"O b{b} h{h}")
        assert_bf16_close(lse[b, h, rows], rl, f"LSE b{b} h{h}")


@pytest.mark.parametrize("N", [512, 2048, 8192, 16384])
def test_causal_sweep_hidden2048(N):
    """Causal forward, 16 heads x 128 = hidden 2048, 16k tokens per batch, inputs N(0,1)*0.5."""
    fa = need_gpu()
    w = workloads.c3(N)
    announce(f"large fwd sweep N={N} B={w.B}")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "bf16", seed=0, mult=w.mult)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # first causal row of every (b, h) is V[0] exactly
    assert torch.equal(o[:, 0], v[:, 0])
    rng = np.random.default_rng(N)
    heads = [(0, 0), (w.B - 1, w.Hq - 1), (w.B // 2, 7)]
    _check_fwd_sampled(inp, o.cpu(), lse.cpu(), w, heads, rng)


def _c4_inputs(hkv):
    w = workloads.WORKLOADS["c4" if hkv == 96 else "c4g"]
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "bf16", seed=0, with_do=True)
    return w, inp


@pytest.mark.parametrize("hkv", [96, 12])
def test_b1_n8192_h96_forward(hkv):
    fa = need_gpu()
    announce(f"large fwd B1 N8192 Hq96 Hkv{hkv}")
    w, inp = _c4_inputs(hkv)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(hkv)
    _check_fwd_sampled(inp, o.cpu(), lse.cpu(), w, [(0, 0), (0, 47), (0, 95)], rng)


@pytest.mark.parametrize("hkv", [96, 12])
def test_b1_n8192_h96_backward(hkv):
    """dQ of sampled query heads and dK/dV of one kv head (summed over its
    query-head group) against the oracle's full backward of those heads."""
    fa = need_gpu()
    announce(f"large bwd B1 N8192 Hq96 Hkv{hkv}")
    w, inp = _c4_inputs(hkv)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    g = w.Hq // w.Hkv
    kh = w.Hkv - 1
    heads = list(range(kh * g, (kh + 1) * g))  # the whole group of the last kv head
    sl = slice(heads[0], heads[-1] + 1)
    rdq, rdk, rdv, _ = oracle.attn_bwd(f64(inp["q"][:, :, sl]), f64(inp["k"][:, :, kh:kh + 1]),
                                       f64(inp["v"][:, :, kh:kh + 1]), f64(inp["do"][:, :, sl]), w.scale, True)
    assert_bf16_close(dq[:, :, sl], rdq, "dQ")
    assert_bf16_close(dk[:, :, kh:kh + 1], rdk, "dK")
    assert_bf16_close(dv[:, :, kh:kh + 1], rdv, "dV")


def test_decode_64_sequences_32k_cache():
    """Decode at full size: 64 sequences, Hq=32, Hkv=8, d=128, lengths U[1024, 32768];
    six sequences (shortest, longest and four others) checked on every head."""
    fa = need_gpu()
    w = workloads.WORKLOADS["c5"]
    announce("large decode B64 Hq32 Hkv8 L32768")
    dev = torch.device("cuda:0")
    lens = workloads.decode_seqlens(w.B, w.seq_lo, w.seq_hi, seed=0)
    kc = torch.full((w.B, w.N, w.Hkv, w.d), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    for b in range(w.B):
        kr, vr = workloads.decode_kv_rows(b, int(lens[b]), w.Hkv, w.d, seed=0)
        kc[b, : int(lens[b])] = kr.to(dev)
        vc[b, : int(lens[b])] = vr.to(dev)
    qd = workloads.decode_query(w.B, w.Hq, w.d, seed=0)
    o, lse = fa.fa_decode_kvcache(qd.to(dev), kc, vc, lens.to(dev), scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    order = np.argsort(lens.numpy())
    picks = sorted({int(order[0]), int(order[-1]), 3, 17, 40, 63})
    for b in picks:
        L = int(lens[b])
        kr, vr = workloads.decode_kv_rows(b, L, w.Hkv, w.d, seed=0)
        ro, rl = oracle.attn_decode(f64(qd[b:b + 1]), f64(kr)[None], f64(vr)[None], np.array([L]), w.scale)
        assert_bf16_close(o[b:b + 1].cpu(), ro, f"O seq {b} (L={L})")
        assert_bf16_close(lse[b:b + 1].cpu(), rl, f"LSE seq {b} (L={L})")


def test_window_4095_forward_backward_full_size():
    """The sliding-window workload of the benchmark (B=1, N=8192, H=96, d=128,
    causal, window (4095, 0)): every output finite, and one head's O, LSE,
    dQ, dK, dV against the oracle's full forward and backward of that head."""
    fa = need_gpu()
    announce("large window fwd+bwd B1 N8192 H96 w4095")
    B, N, H, d, win = 1, 8192, 96, 128, (4095, 0)
    scale = 1 / math.sqrt(d)
    inp = workloads.prefill_inputs(B, N, H, H, d, "bf16", seed=7, with_do=True)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd_window(q, k, v, win, scale=scale, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, scale=scale, causal=True, window=win)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    h = H - 1
    sl = slice(h, h + 1)
    args = [f64(inp[n][:, :, sl]) for n in ("q", "k", "v")]
    ro, rl = oracle.attn_fwd(*args, scale, True, window=win)
    assert_bf16_close(o[:, :, sl].cpu(), ro, "O")
    assert_bf16_close(lse[:, sl].cpu(), rl, "LSE")
    rdq, rdk, rdv, _ = oracle.attn_bwd(*args, f64(inp["do"][:, :, sl]), scale, True, window=win)
    assert_bf16_close(dq[:, :, sl].cpu(), rdq, "dQ")
    assert_bf16_close(dk[:, :, sl].cpu(), rdk, "dK")
    assert_bf16_close(dv[:, :, sl].cpu(), rdv, "dV")


def test_varlen_benchmark_batch():
    """The varlen workload of the benchmark: sequences U[256, 4096] packed to
    at least 16k tokens, H=16, d=128, causal; all 16 heads against the oracle's
    varlen forward."""
    fa = need_gpu()
    announce("large varlen fwd U[256,4096] H16")
    rng = np.random.default_rng(2)
    lens = []
    while sum(lens) < 16384:
        lens.append(int(rng.integers(256, 4097)))
    vin = workloads.varlen_inputs(lens, lens, 16, 16, 128, seed=3)
    dev = torch.device("cuda:0")
    q, k, v = (vin[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd_varlen(q, k, v, vin["cu_q"].to(dev), vin["cu_k"].to(dev), max(lens), causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_varlen(f64(vin["q"]), f64(vin["k"]), f64(vin["v"]), vin["cu_q"].numpy(),
                                    vin["cu_k"].numpy(), 1 / math.sqrt(128), True)
    assert_bf16_close(o.cpu(), ro, "O")
    assert_bf16_close(lse.cpu(), rl, "LSE")
