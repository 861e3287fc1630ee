"""GPU parity of fa_fwd_blocksparse (128 x 128 block mask, bf16, d = 128 and
64) against the fp64 oracle, through the C ABI."""
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


def _check(o, lse, ro, rl):
    assert_bf16_close(o.cpu(), ro, "O")
    g, w = f64(lse.cpu()), rl
    assert np.array_equal(np.isneginf(g), np.isneginf(w)), "empty rows differ"
    fin = np.isfinite(w)
    assert_bf16_close(torch.from_numpy(g[fin]), w[fin], "LSE")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("per_head", [False, True])
def test_random_mask(per_head, causal, d):
    fa = need_gpu()
    B, N, Hq, Hkv = 2, 700, 4, 2
    nb = (N + 127) // 128
    announce(f"fwd blocksparse per_head={per_head} causal={causal} d{d}")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=60)
    rng = np.random.default_rng(61)
    mask = (rng.random((B, Hq, nb, nb) if per_head else (nb, nb)) < 0.45).astype(np.uint8)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd_blocksparse(q, k, v, torch.from_numpy(mask).to(DEV), causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_blocksparse(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), mask, 128,
                                         1 / math.sqrt(d), causal)
    _check(o, lse, ro, rl)


# At d = 64 the dense batch must launch more than 256 workgroups of 128 rows
# (2 x 16 heads x 8 tiles = 256 + 16 here) to run the same kernel as the
# block-sparse path rather than the split-key one.
@pytest.mark.parametrize("shape", [(1, 1000, 4, 1, 128), (2, 1000, 17, 1, 64)], ids=["d128", "d64"])
def test_all_ones_is_dense_bitwise_and_all_zeros_is_empty(shape):
    fa = need_gpu()
    B, N, Hq, Hkv, d = shape
    announce(f"fwd blocksparse all-ones / all-zeros {shape}")
    nb = (N + 127) // 128
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=62)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    for causal in (False, True):
        ob, lb = fa.fa_fwd_blocksparse(q, k, v, torch.ones((nb, nb), dtype=torch.uint8, device=DEV), causal=causal)
        od, ld = fa.fa_fwd(q, k, v, causal=causal)
        oz, lz = fa.fa_fwd_blocksparse(q, k, v, torch.zeros((nb, nb), dtype=torch.uint8, device=DEV), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(ob, od) and torch.equal(lb, ld)
        assert (oz == 0).all() and torch.isneginf(lz).all()


def test_local_plus_global_pattern_n8192():
    """A sliding band of blocks plus the first block column (a common sparse
    layout), N = 8192, checked on sampled rows of every head."""
    fa = need_gpu()
    announce("fwd blocksparse local+global N8192")
    B, N, Hq, Hkv, d = 1, 8192, 8, 8, 128
    nb = N // 128
    i = np.arange(nb)
    mask = ((np.abs(i[:, None] - i[None, :]) <= 2) | (i[None, :] == 0)).astype(np.uint8)
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=63)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd_blocksparse(q, k, v, torch.from_numpy(mask).to(DEV), causal=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 500, 4095, 4096, 6000, 8190, 8191])
    keep = oracle.block_keep(mask, 128, N, N)
    for h in range(Hq):
        qh = f64(inp["q"][0, rows, h])[None, :, None, :]
        kh, vh = f64(inp["k"][0, :, h])[None, :, None, :], f64(inp["v"][0, :, h])[None, :, None, :]
        _, p, rl = oracle.head_probs(qh[0, :, 0], kh[0, :, 0], 1 / math.sqrt(d), True, rows=rows, nq=N,
                                     keep_extra=keep[rows])
        ro = p @ vh[0, :, 0]
        assert_bf16_close(o[0, rows, h].cpu(), ro, f"O h{h}")
        assert_bf16_close(lse[0, h, rows].cpu(), rl, f"LSE h{h}")
