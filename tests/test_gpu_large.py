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
    """Sampled rows of each listed (b, h) against the oracle's row forward
    (cost O(rows * N * d) per head)."""
    rows = _sample_rows(w.N, rng)
    g = w.Hq // w.Hkv
    worst = [0.0, 0.0]
    for (b, h) in heads:
        kh = h // g
        q = f64(inp["q"][b:b + 1, :, h:h + 1])
        k = f64(inp["k"][b:b + 1, :, kh:kh + 1])
        v = f64(inp["v"][b:b + 1, :, kh:kh + 1])
        ro, rl = oracle.attn_fwd_rows(q, k, v, w.scale, w.causal, 0, 0, rows)
        mo, _ = assert_bf16_close(o[b, rows, h], ro, f"O b{b} h{h}")
        ml, _ = assert_bf16_close(lse[b, h, rows], rl, f"LSE b{b} h{h}")
        worst = [max(worst[0], mo), max(worst[1], ml)]
    print(f"[parity] {len(heads)} heads x {len(rows)} rows: max O error {worst[0]:.3e}, max LSE error {worst[1]:.3e}")


def _nan_outputs(q, B, H, N):
    """Output buffers filled with NaN, so that a finite result everywhere
    proves every element was written."""
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    return o, lse


@pytest.mark.parametrize("N", [512, 2048, 8192, 16384])
def test_causal_sweep_hidden2048(N):
    """Causal forward, 16 heads x 128 = hidden 2048, 16k tokens per batch, inputs N(0,1)*0.5:
    every output written, sampled rows of every (b, h) against the oracle."""
    fa = need_gpu()
    w = workloads.c3(N)
    announce(f"large fwd sweep N={N} B={w.B}")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "bf16", seed=0, mult=w.mult)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = _nan_outputs(q, w.B, w.Hq, w.N)
    fa.fa_fwd(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # first causal row of every (b, h) is V[0] exactly
    assert torch.equal(o[:, 0], v[:, 0])
    rng = np.random.default_rng(N)
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    if len(heads) > 128:   # N = 512: 32 x 16 pairs; every head of 8 batches spread over the batch
        heads = [(b, h) for b in sorted({0, 5, 11, 16, 21, 26, 30, w.B - 1}) for h in range(w.Hq)]
    _check_fwd_sampled(inp, o.cpu(), lse.cpu(), w, heads, rng)


@pytest.mark.parametrize("N,causal", [(2048, True), (2048, False), (16384, True)])
def test_sweep_d64_hidden2048(N, causal):
    """Head dim 64 (32 heads x 64 = hidden 2048, 16k tokens per batch), inputs
    N(0,1)*0.5, through the DMA kernel with 128-byte rows: every output
    written, sampled rows of every head of two batches against the oracle."""
    fa = need_gpu()
    w = workloads.sweep_d64(N, causal)
    announce(f"large fwd d64 sweep N={N} B={w.B} causal={causal}")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "bf16", seed=1, mult=w.mult)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = _nan_outputs(q, w.B, w.Hq, w.N)
    fa.fa_fwd(q, k, v, scale=w.scale, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    if causal:
        assert torch.equal(o[:, 0], v[:, 0])
    rng = np.random.default_rng(N + int(causal))
    heads = [(b, h) for b in sorted({0, w.B - 1}) for h in range(w.Hq)]
    _check_fwd_sampled(inp, o.cpu(), lse.cpu(), w, heads, rng)


@pytest.mark.parametrize("N", [2048, 16384])
def test_backward_d64_hidden2048(N):
    """Causal backward at head dim 64 (32 heads x 64, 16k tokens per batch,
    inputs N(0,1)*0.5): every gradient written (NaN-filled buffers); the
    first head of the first batch in full against the oracle's backward;
    sampled dQ rows of every head of the first and last batch; and for every
    head, sum over keys of dV = sum over queries of dO within the bf16
    rounding of P and dV."""
    fa = need_gpu()
    w = workloads.sweep_d64(N, True)
    announce(f"large bwd d64 N={N} B={w.B}")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "bf16", seed=2, mult=w.mult, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.fa_bwd(q, k, v, o, do, lse, scale=w.scale, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    if N <= 2048:
        rdq, rdk, rdv, _ = oracle.attn_bwd(f64(inp["q"][:1, :, :1]), f64(inp["k"][:1, :, :1]), f64(inp["v"][:1, :, :1]),
                                           f64(inp["do"][:1, :, :1]), w.scale, True)
        assert_bf16_close(dq[:1, :, :1], rdq, "dQ b0 h0")
        assert_bf16_close(dk[:1, :, :1], rdk, "dK b0 h0")
        assert_bf16_close(dv[:1, :, :1], rdv, "dV b0 h0")
    rows = _sample_rows(w.N, np.random.default_rng(N + 64))
    for b in sorted({0, w.B - 1}):
        for h in range(w.Hq):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            rq, _ = oracle.attn_bwd_dq_rows(f64(inp["q"][sl]), f64(inp["k"][sl]), f64(inp["v"][sl]),
                                            f64(inp["do"][sl]), w.scale, True, 0, 0, rows)
            assert_bf16_close(dq[b, rows, h], rq, f"dQ rows b{b} h{h}")
    dvs, dos = f64(dv).sum(axis=1), f64(inp["do"]).sum(axis=1)
    bound = 2 * 2.0 ** -9 * (np.abs(f64(inp["do"])).sum(axis=1) + np.abs(f64(dv)).sum(axis=1))
    assert (np.abs(dvs - dos) <= bound).all(), "column sums of dV differ from those of dO beyond the rounding bound"


def _c4_inputs(hkv):
    w = workloads.WORKLOADS["c4" if hkv == 96 else "c4g"]
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "bf16", seed=0, with_do=True)
    return w, inp


@pytest.mark.parametrize("hkv", [96, 12])
def test_b1_n8192_h96_forward(hkv):
    """Every output written (NaN-filled buffers), sampled rows of all 96 heads."""
    fa = need_gpu()
    announce(f"large fwd B1 N8192 Hq96 Hkv{hkv}")
    w, inp = _c4_inputs(hkv)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = _nan_outputs(q, w.B, w.Hq, w.N)
    fa.fa_fwd(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(hkv)
    _check_fwd_sampled(inp, o.cpu(), lse.cpu(), w, [(0, h) for h in range(w.Hq)], rng)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("hkv", [96, 12])
def test_b1_n8192_h96_backward(hkv):
    """Every gradient written (NaN-filled buffers); dQ of the query heads and
    dK/dV of the first, middle and last kv head (each summed over its
    query-head group) against the oracle's full backward of those heads."""
    fa = need_gpu()
    announce(f"large bwd B1 N8192 Hq96 Hkv{hkv}")
    w, inp = _c4_inputs(hkv)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.fa_bwd(q, k, v, o, do, lse, scale=w.scale, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    g = w.Hq // w.Hkv
    for kh in (0, w.Hkv // 2, w.Hkv - 1):
        sl = slice(kh * g, (kh + 1) * g)
        rdq, rdk, rdv, _ = oracle.attn_bwd(f64(inp["q"][:, :, sl]), f64(inp["k"][:, :, kh:kh + 1]),
                                           f64(inp["v"][:, :, kh:kh + 1]), f64(inp["do"][:, :, sl]), w.scale, True)
        assert_bf16_close(dq[:, :, sl], rdq, f"dQ heads {sl.start}..{sl.stop - 1}")
        assert_bf16_close(dk[:, :, kh:kh + 1], rdk, f"dK kv head {kh}")
        assert_bf16_close(dv[:, :, kh:kh + 1], rdv, f"dV kv head {kh}")
    # Every query head: sampled dQ rows (row i of dQ needs only row i of P
    # and dP, so the oracle's cost is linear in N per row).
    rows = _sample_rows(w.N, np.random.default_rng(96 + hkv))
    worst = 0.0
    for h in range(w.Hq):
        kh = h // g
        rdq, _ = oracle.attn_bwd_dq_rows(f64(inp["q"][:, :, h:h + 1]), f64(inp["k"][:, :, kh:kh + 1]),
                                         f64(inp["v"][:, :, kh:kh + 1]), f64(inp["do"][:, :, h:h + 1]), w.scale,
                                         True, 0, 0, rows)
        m, _ = assert_bf16_close(dq[0, rows, h], rdq, f"dQ rows head {h}")
        worst = max(worst, m)
    print(f"[parity] dQ: {w.Hq} heads x {len(rows)} rows, max error {worst:.3e}")


@pytest.mark.timeout(600)
def test_decode_64_sequences_32k_cache():
    """Decode at full size: 64 sequences, Hq=32, Hkv=8, d=128, lengths U[1024, 32768];
    cache rows past each length and the outputs NaN-filled; every sequence
    checked on every head."""
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
    o = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_decode_kvcache(qd.to(dev), kc, vc, lens.to(dev), scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    o, lse = o.cpu(), lse.cpu()
    for b in range(w.B):
        L = int(lens[b])
        kr, vr = workloads.decode_kv_rows(b, L, w.Hkv, w.d, seed=0)
        ro, rl = oracle.attn_decode(f64(qd[b:b + 1]), f64(kr)[None], f64(vr)[None], np.array([L]), w.scale)
        assert_bf16_close(o[b:b + 1], ro, f"O seq {b} (L={L})")
        assert_bf16_close(lse[b:b + 1], rl, f"LSE seq {b} (L={L})")


def test_window_4095_forward_backward_full_size():
    """The sliding-window workload of the benchmark (B=1, N=8192, H=96, d=128,
    causal, window (4095, 0)): every output written (NaN-filled buffers), and
    one head's O, LSE, dQ, dK, dV against the oracle's full forward and
    backward of that head."""
    fa = need_gpu()
    announce("large window fwd+bwd B1 N8192 H96 w4095")
    B, N, H, d, win = 1, 8192, 96, 128, (4095, 0)
    scale = 1 / math.sqrt(d)
    inp = workloads.prefill_inputs(B, N, H, H, d, "bf16", seed=7, with_do=True)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = _nan_outputs(q, B, H, N)
    fa.fa_fwd_window(q, k, v, win, scale=scale, causal=True, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.fa_bwd(q, k, v, o, do, lse, scale=scale, causal=True, window=win, dq=dq, dk=dk, dv=dv)
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
