"""GPU parity of the sliding-window and variable-length forwards (fa_fwd_window,
fa_fwd_varlen, bf16, d = 128 and 64) and of the windowed backward against the
fp64 oracle, through the C ABI."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import announce, assert_bf16_close, f64, need_gpu

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _check_lse(got, want, what):
    """-inf exactly where the oracle has an empty row, bf16 bound elsewhere."""
    g, w = f64(got), f64(want)
    assert np.array_equal(np.isneginf(g), np.isneginf(w)), f"{what}: empty rows differ"
    fin = np.isfinite(w)
    assert_bf16_close(torch.from_numpy(g[fin]), w[fin], what)


WINDOWS = [(0, 0), (1, 0), (64, 0), (100, 37), (-1, 5), (7, -1), (300, 300)]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", WINDOWS, ids=[f"w{a}_{b}" for a, b in WINDOWS])
def test_window_dense(window, causal, d):
    fa = need_gpu()
    B, N, Hq, Hkv = 2, 333, 4, 2
    announce(f"fwd window {window} causal={causal} B{B} N{N} d{d}")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=31)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd_window(q, k, v, window, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 1 / math.sqrt(d), causal, window)
    assert_bf16_close(o.cpu(), ro, "O")
    _check_lse(lse.cpu(), rl, "LSE")


def test_window_unbounded_is_fa_fwd():
    fa = need_gpu()
    announce("fwd window (-1,-1) == fa_fwd")
    inp = workloads.prefill_inputs(1, 300, 2, 1, 128, "bf16", seed=32)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    a = fa.fa_fwd_window(q, k, v, (-1, -1), causal=True)
    b = fa.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


VARLEN_CASES = {
    # name: (lens_q, lens_k)
    "equal_lengths": ([200, 200, 200], [200, 200, 200]),
    "mixed": ([1, 130, 0, 64, 257, 5], [1, 130, 7, 64, 257, 5]),
    "chunked_prefill_nk_gt_nq": ([40, 130, 1], [300, 200, 513]),
    "nq_gt_nk_empty_rows": ([100, 64, 9], [30, 0, 9]),
}


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("name", sorted(VARLEN_CASES))
def test_varlen(name, causal, d):
    fa = need_gpu()
    lens_q, lens_k = VARLEN_CASES[name]
    announce(f"fwd varlen {name} causal={causal} d{d}")
    inp = workloads.varlen_inputs(lens_q, lens_k, 4, 2, d, seed=33)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd_varlen(q, k, v, inp["cu_q"].to(DEV), inp["cu_k"].to(DEV), max(lens_q), causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_q"].numpy(),
                                    inp["cu_k"].numpy(), 1 / math.sqrt(d), causal)
    assert_bf16_close(o.cpu(), ro, "O")
    _check_lse(lse.cpu(), rl, "LSE")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("window", [(16, 0), (50, 50), (0, -1)], ids=["w16_0", "w50_50", "w0_inf"])
def test_varlen_window(window, d):
    fa = need_gpu()
    lens_q, lens_k = [77, 300, 1, 129], [200, 300, 64, 129]
    announce(f"fwd varlen window {window} d{d}")
    inp = workloads.varlen_inputs(lens_q, lens_k, 8, 1, d, seed=34)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd_varlen(q, k, v, inp["cu_q"].to(DEV), inp["cu_k"].to(DEV), max(lens_q), causal=True,
                              window=window)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_q"].numpy(),
                                    inp["cu_k"].numpy(), 1 / math.sqrt(d), True, window)
    assert_bf16_close(o.cpu(), ro, "O")
    _check_lse(lse.cpu(), rl, "LSE")


# d = 64 dense batches of at most 256 workgroups of 128 rows run the split-key
# kernel, whose sums are ordered differently; 3 x 16 heads x 6 tiles = 288
# workgroups run the same 128-row kernel as the packed batch.
@pytest.mark.parametrize("shape", [(3, 320, 4, 2, 128), (3, 700, 16, 4, 64)], ids=["d128", "d64"])
def test_varlen_equal_lengths_matches_dense_bitwise(shape):
    """Packing equal-length sequences is the dense batch: same kernel arithmetic, same bits."""
    fa = need_gpu()
    B, N, Hq, Hkv, d = shape
    announce(f"fwd varlen == dense {shape}")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=35)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=DEV)
    for causal in (False, True):
        od, ld = fa.fa_fwd(q, k, v, causal=causal)
        ov, lv = fa.fa_fwd_varlen(q.view(B * N, Hq, d), k.view(B * N, Hkv, d), v.view(B * N, Hkv, d), cu, cu, N,
                                  causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(ov.view(B, N, Hq, d), od)
        assert torch.equal(lv.view(Hq, B, N).permute(1, 0, 2), ld)


def test_varlen_rows_past_max_seqlen_are_not_written():
    fa = need_gpu()
    announce("fwd varlen max_seqlen_q smaller than a sequence")
    lens = [100, 300]
    inp = workloads.varlen_inputs(lens, lens, 2, 2, 128, seed=36)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    # max_seqlen_q = 200 < 300: rows 256.. of sequence 1 lie past the last launched tile
    o, lse = fa.fa_fwd_varlen(q, k, v, inp["cu_q"].to(DEV), inp["cu_k"].to(DEV), 200)
    torch.cuda.synchronize()
    ro, _ = oracle.attn_fwd_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_q"].numpy(),
                                   inp["cu_k"].numpy(), 1 / math.sqrt(128), False)
    assert_bf16_close(o[:100 + 256].cpu(), ro[:100 + 256], "O of launched rows")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [(0, 0), (64, 0), (100, 37), (-1, 5), (7, -1), (200, 200)],
                         ids=["w0_0", "w64_0", "w100_37", "winf_5", "w7_inf", "w200_200"])
def test_window_backward(window, causal, d):
    fa = need_gpu()
    B, N, Hq, Hkv = 1, 333, 4, 2
    announce(f"bwd window {window} causal={causal} N{N} d{d}")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=37, with_do=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd_window(q, k, v, window, causal=causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, window=window)
    torch.cuda.synchronize()
    rdq, rdk, rdv, _ = oracle.attn_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]),
                                       1 / math.sqrt(d), causal, window)
    assert_bf16_close(dq.cpu(), rdq, "dQ")
    assert_bf16_close(dk.cpu(), rdk, "dK")
    assert_bf16_close(dv.cpu(), rdv, "dV")


def test_window_backward_deterministic():
    fa = need_gpu()
    announce("bwd window determinism")
    inp = workloads.prefill_inputs(1, 700, 8, 2, 128, "bf16", seed=38, with_do=True)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd_window(q, k, v, (128, 0), causal=True)
    r1 = fa.fa_bwd(q, k, v, o, do, lse, causal=True, window=(128, 0))
    r2 = fa.fa_bwd(q, k, v, o, do, lse, causal=True, window=(128, 0))
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
