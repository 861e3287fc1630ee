"""GPU parity of fa_decode_kvcache against the fp64 oracle (through the C ABI)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import announce, assert_bf16_close, f64, need_gpu

pytestmark = pytest.mark.gpu


def _make_cache(B, Lmax, Hkv, d, lens, seed, dev, fill=float("nan")):
    """Cache tensors on the GPU: valid rows from the seeded generator, the
    rest NaN so that a read past cache_seqlens[b] shows up in the output."""
    kc = torch.full((B, Lmax, Hkv, d), fill, dtype=torch.bfloat16, device=dev)
    vc = torch.full((B, Lmax, Hkv, d), fill, dtype=torch.bfloat16, device=dev)
    for b in range(B):
        kr, vr = workloads.decode_kv_rows(b, int(lens[b]), Hkv, d, seed=seed)
        kc[b, : int(lens[b])] = kr.to(dev)
        vc[b, : int(lens[b])] = vr.to(dev)
    return kc, vc


def _oracle_seq(q, b, L, Hkv, d, seed, scale):
    kr, vr = workloads.decode_kv_rows(b, L, Hkv, d, seed=seed)
    return oracle.attn_decode(f64(q[b:b + 1]), f64(kr)[None], f64(vr)[None], np.array([L]), scale)


SMALL = [
    # B, Hq, Hkv, d, Lmax, lens
    (3, 8, 2, 128, 300, [300, 1, 77]),
    (2, 4, 4, 64, 1000, [999, 513]),
    (4, 32, 8, 128, 1500, [1500, 1024, 7, 640]),
    (2, 16, 1, 128, 700, [700, 65]),
    (3, 24, 8, 128, 900, [900, 1, 333]),    # 3 query heads per kv head: one head per workgroup
    (2, 10, 2, 64, 500, [500, 77]),         # 5 per kv head, d = 64
    (2, 24, 2, 128, 700, [700, 300]),       # 12 per kv head: groups of 4
]


@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}d{c[3]}L{c[4]}" for c in SMALL])
def test_small(case, num_splits):
    fa = need_gpu()
    B, Hq, Hkv, d, Lmax, lens = case
    announce(f"decode small {case} splits={num_splits}")
    dev = torch.device("cuda:0")
    seed = 4 + Lmax
    kc, vc = _make_cache(B, Lmax, Hkv, d, lens, seed, dev)
    q = workloads.decode_query(B, Hq, d, seed=seed)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    o, lse = fa.fa_decode_kvcache(q.to(dev), kc, vc, sl, num_splits=num_splits)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    for b in range(B):
        ro, rl = _oracle_seq(q, b, lens[b], Hkv, d, seed, scale)
        assert_bf16_close(o[b:b + 1], ro, f"O seq {b}")
        assert_bf16_close(lse[b:b + 1], rl, f"LSE seq {b}")


def test_split_count_invariance_and_determinism():
    """One split against the automatic split count: the partials merge with
    exact LSE weights, so only rounding differs."""
    fa = need_gpu()
    announce("decode split invariance")
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, Lmax = 4, 16, 4, 128, 4096
    lens = [4096, 3000, 1025, 17]
    kc, vc = _make_cache(B, Lmax, Hkv, d, lens, 77, dev)
    q = workloads.decode_query(B, Hq, d, seed=77).to(dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    o1, l1 = fa.fa_decode_kvcache(q, kc, vc, sl, num_splits=1)
    oa, la = fa.fa_decode_kvcache(q, kc, vc, sl, num_splits=0)
    ob, lb = fa.fa_decode_kvcache(q, kc, vc, sl, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    ulp = (o1.float().abs() * 2.0 ** -7).clamp_min(1e-30)  # one bf16 ulp at each value
    assert ((o1.float() - oa.float()).abs() <= ulp + 1e-6).all()
    assert (l1 - la).abs().max().item() < 1e-4


def test_decode_matches_last_causal_row_of_fwd():
    fa = need_gpu()
    announce("decode vs fwd last causal row")
    dev = torch.device("cuda:0")
    N, Hq, Hkv, d = 777, 8, 2, 128
    inp = workloads.prefill_inputs(1, N, Hq, Hkv, d, "bf16", seed=12)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    of, lf = fa.fa_fwd(q, k, v, causal=True)
    od, ld = fa.fa_decode_kvcache(q[:, N - 1].contiguous(), k, v, torch.tensor([N], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert_bf16_close(od, of[:, N - 1], "O")
    assert_bf16_close(ld, lf[:, :, N - 1], "LSE")


def test_out_of_range_lengths_give_zero_output():
    fa = need_gpu()
    announce("decode out-of-range lengths")
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, Lmax = 3, 4, 2, 64, 128
    kc = torch.randn(B, Lmax, Hkv, d, device=dev).to(torch.bfloat16)
    vc = torch.randn(B, Lmax, Hkv, d, device=dev).to(torch.bfloat16)
    q = torch.randn(B, Hq, d, device=dev).to(torch.bfloat16)
    sl = torch.tensor([0, 129, 5], dtype=torch.int32, device=dev)
    o, lse = fa.fa_decode_kvcache(q, kc, vc, sl)
    torch.cuda.synchronize()
    assert (o[:2] == 0).all() and torch.isneginf(lse[:2]).all()
    assert torch.isfinite(lse[2]).all()


# Cases for the balanced split (automatic split count, Hkv a multiple of
# 512 / d, B <= 1024): all sequences' rows are cut into equal ranges, so a
# range can span many short sequences, and with few rows most ranges are
# empty. Lengths 0 and > Lmax are invalid (output 0, LSE -inf).
BALANCED = [
    # B, Hq, Hkv, d, Lmax, lens
    (5, 32, 8, 128, 16, [1, 1, 2, 1, 3]),                   # fewer rows than ranges
    (6, 16, 8, 128, 2000, [2000, 0, 1, 5000, 1999, 37]),     # invalid lengths between valid ones
    (3, 64, 8, 64, 900, [900, 450, 3]),                      # d = 64: 8 kv heads per wave instruction
    (2, 8, 4, 128, 40000, [40000, 33]),                      # ranges far longer than a chunk
    (4, 8, 8, 128, 3000, [3000, 1, 2500, 17]),               # one query head per kv head
    (3, 64, 4, 128, 5000, [5000, 4096, 1]),                  # 16 query heads per kv head
    (4, 24, 8, 128, 1200, [1200, 5, 640, 1199]),             # 3 query heads per kv head
    (3, 20, 4, 64, 800, [800, 2, 513]),                      # 5 per kv head, d = 64
]


@pytest.mark.parametrize("case", BALANCED, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}d{c[3]}L{c[4]}" for c in BALANCED])
def test_balanced_split(case):
    fa = need_gpu()
    B, Hq, Hkv, d, Lmax, lens = case
    announce(f"decode balanced {case}")
    dev = torch.device("cuda:0")
    seed = 9 + Lmax
    valid = [1 <= L <= Lmax for L in lens]
    kc, vc = _make_cache(B, Lmax, Hkv, d, [L if ok else 0 for L, ok in zip(lens, valid)], seed, dev)
    q = workloads.decode_query(B, Hq, d, seed=seed)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    o, lse = fa.fa_decode_kvcache(q.to(dev), kc, vc, sl, num_splits=0)
    o2, lse2 = fa.fa_decode_kvcache(q.to(dev), kc, vc, sl, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    scale = 1 / math.sqrt(d)
    for b in range(B):
        if not valid[b]:
            assert (o[b] == 0).all() and torch.isneginf(lse[b]).all(), f"seq {b}"
            continue
        ro, rl = _oracle_seq(q, b, lens[b], Hkv, d, seed, scale)
        assert_bf16_close(o[b:b + 1], ro, f"O seq {b}")
        assert_bf16_close(lse[b:b + 1], rl, f"LSE seq {b}")


def test_many_sequences_fall_back_to_chunks():
    """More sequences than the balanced split keeps prefix sums for: the
    chunked split runs instead; sampled sequences against the oracle."""
    fa = need_gpu()
    announce("decode B=1100 chunked fallback")
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, Lmax = 1100, 8, 8, 128, 48
    rng = np.random.default_rng(5)
    lens = rng.integers(1, Lmax + 1, size=B).tolist()
    kc, vc = _make_cache(B, Lmax, Hkv, d, lens, 21, dev)
    q = workloads.decode_query(B, Hq, d, seed=21)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    o, lse = fa.fa_decode_kvcache(q.to(dev), kc, vc, sl)
    torch.cuda.synchronize()
    for b in (0, 1, 517, 1023, 1024, 1099):
        ro, rl = _oracle_seq(q, b, lens[b], Hkv, d, 21, 1 / math.sqrt(d))
        assert_bf16_close(o[b:b + 1], ro, f"O seq {b}")
        assert_bf16_close(lse[b:b + 1], rl, f"LSE seq {b}")
