"""GPU parity of fa_decode_kvcache_ext (paged KV cache, in-place append)
against the fp64 oracle, through the C ABI."""
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


def _paged_setup(lens, Hkv, d, page_size, max_pages, seed, spare=3):
    """Random pages in a shuffled pool: returns host pages, the block table,
    and the contiguous [B, max_pages*page_size, Hkv, d] view of the same rows."""
    B = len(lens)
    gen = torch.Generator().manual_seed(seed)
    num_pages = B * max_pages + spare
    kp = torch.randn((num_pages, page_size, Hkv, d), generator=gen).to(torch.bfloat16)
    vp = torch.randn((num_pages, page_size, Hkv, d), generator=gen).to(torch.bfloat16)
    perm = torch.randperm(num_pages, generator=gen)[: B * max_pages]
    table = perm.view(B, max_pages).to(torch.int32)
    kc = kp[table.long()].reshape(B, max_pages * page_size, Hkv, d)
    vc = vp[table.long()].reshape(B, max_pages * page_size, Hkv, d)
    return kp, vp, table, kc, vc


CASES = [
    # lens, Hq, Hkv, page_size, max_pages
    ([1, 17, 64, 200], 4, 2, 16, 13),
    ([700, 1, 1500], 8, 2, 64, 24),
    ([2047, 333], 32, 8, 256, 8),
]


@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_decode(case, append):
    fa = need_gpu()
    lens, Hq, Hkv, ps, mp = CASES[case]
    B, d = len(lens), 128
    announce(f"decode paged case {case} append={append}")
    kp, vp, table, _, _ = _paged_setup(lens, Hkv, d, ps, mp, seed=40 + case)
    q = workloads.decode_query(B, Hq, d, seed=case)
    gen = torch.Generator().manual_seed(50 + case)
    kn = torch.randn((B, Hkv, d), generator=gen).to(torch.bfloat16) if append else None
    vn = torch.randn((B, Hkv, d), generator=gen).to(torch.bfloat16) if append else None
    seq = torch.tensor(lens, dtype=torch.int32)
    kpd, vpd = kp.to(DEV), vp.to(DEV)
    o, lse = fa.fa_decode_kvcache_ext(q.to(DEV), kpd, vpd, seq.to(DEV), block_table=table.to(DEV),
                                      k_new=None if kn is None else kn.to(DEV),
                                      v_new=None if vn is None else vn.to(DEV))
    torch.cuda.synchronize()
    ro, rl, rkp, rvp = oracle.attn_decode_paged(f64(q), f64(kp), f64(vp), table.numpy(), seq.numpy(),
                                                1 / math.sqrt(d), None if kn is None else f64(kn),
                                                None if vn is None else f64(vn))
    assert_bf16_close(o.cpu(), ro, "O")
    assert_bf16_close(lse.cpu(), rl, "LSE")
    # the cache after the call: exactly the oracle's (the new rows copied bit for bit)
    assert np.array_equal(f64(kpd.cpu()), rkp) and np.array_equal(f64(vpd.cpu()), rvp)


def test_paged_equals_contiguous_bitwise():
    """Same logical rows, same chunking: the paged kernel is the contiguous one
    with another address per row, so outputs agree bit for bit."""
    fa = need_gpu()
    announce("decode paged == contiguous")
    lens, Hq, Hkv, ps, mp = [3000, 1, 4096, 777], 32, 8, 128, 32
    B, d = len(lens), 128
    kp, vp, table, kc, vc = _paged_setup(lens, Hkv, d, ps, mp, seed=44)
    q = workloads.decode_query(B, Hq, d, seed=5).to(DEV)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    op, lp = fa.fa_decode_kvcache_ext(q, kp.to(DEV), vp.to(DEV), seq, block_table=table.to(DEV))
    oc, lc = fa.fa_decode_kvcache(q, kc.to(DEV), vc.to(DEV), seq)
    torch.cuda.synchronize()
    assert torch.equal(op, oc) and torch.equal(lp, lc)


def test_contiguous_append():
    fa = need_gpu()
    announce("decode contiguous append")
    B, Hq, Hkv, d, N = 5, 8, 2, 128, 600
    lens = torch.tensor([0, 1, 299, 598, 599], dtype=torch.int32)
    gen = torch.Generator().manual_seed(46)
    kc = torch.randn((B, N, Hkv, d), generator=gen).to(torch.bfloat16)
    vc = torch.randn((B, N, Hkv, d), generator=gen).to(torch.bfloat16)
    kn = torch.randn((B, Hkv, d), generator=gen).to(torch.bfloat16)
    vn = torch.randn((B, Hkv, d), generator=gen).to(torch.bfloat16)
    q = workloads.decode_query(B, Hq, d, seed=6)
    kcd, vcd = kc.to(DEV), vc.to(DEV)
    o, lse = fa.fa_decode_kvcache_ext(q.to(DEV), kcd, vcd, lens.to(DEV), k_new=kn.to(DEV), v_new=vn.to(DEV))
    torch.cuda.synchronize()
    want_k, want_v = kc.clone(), vc.clone()
    for b in range(B):
        want_k[b, lens[b]], want_v[b, lens[b]] = kn[b], vn[b]
    assert torch.equal(kcd.cpu(), want_k) and torch.equal(vcd.cpu(), want_v)
    ro, rl = oracle.attn_decode(f64(q), f64(want_k), f64(want_v), (lens + 1).numpy(), 1 / math.sqrt(d))
    assert_bf16_close(o.cpu(), ro, "O")
    assert_bf16_close(lse.cpu(), rl, "LSE")


def test_append_past_capacity_is_not_written():
    fa = need_gpu()
    announce("decode append past capacity")
    B, Hq, Hkv, d, N = 2, 4, 1, 128, 64
    lens = torch.tensor([64, 10], dtype=torch.int32)   # sequence 0 is full
    kc = torch.zeros((B, N, Hkv, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kn = torch.ones((B, Hkv, d), dtype=torch.bfloat16, device=DEV)
    q = torch.ones((B, Hq, d), dtype=torch.bfloat16, device=DEV)
    o, lse = fa.fa_decode_kvcache_ext(q, kc, vc, lens.to(DEV), k_new=kn, v_new=kn)
    torch.cuda.synchronize()
    assert torch.isneginf(lse[0]).all() and (o[0] == 0).all()
    assert (kc[0] == 0).all() and (kc[1, 10] == 1).all() and torch.isfinite(lse[1]).all()


def test_paged_full_size_decode_64_sequences():
    """Decode workload at full size (64 sequences, Hq=32, Hkv=8, d=128, lengths
    U[1024, 32768]) in 256-row pages: bitwise equal to the contiguous cache."""
    fa = need_gpu()
    w = workloads.WORKLOADS["c5"]
    announce("decode paged full size")
    lens = workloads.decode_seqlens(w.B, w.seq_lo, w.seq_hi, seed=0)
    ps, mp = 256, w.N // 256
    kc = torch.zeros((w.B, w.N, w.Hkv, w.d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    for b in range(w.B):
        kr, vr = workloads.decode_kv_rows(b, int(lens[b]), w.Hkv, w.d, seed=0)
        kc[b, : int(lens[b])] = kr.to(DEV)
        vc[b, : int(lens[b])] = vr.to(DEV)
    gen = torch.Generator().manual_seed(7)
    perm = torch.randperm(w.B * mp, generator=gen)
    table = torch.argsort(perm).view(w.B, mp).to(torch.int32).to(DEV)  # logical (b, p) -> physical page
    kp = torch.empty((w.B * mp, ps, w.Hkv, w.d), dtype=torch.bfloat16, device=DEV)
    vp = torch.empty_like(kp)
    kp[table.view(-1).long()] = kc.view(w.B * mp, ps, w.Hkv, w.d)
    vp[table.view(-1).long()] = vc.view(w.B * mp, ps, w.Hkv, w.d)
    q = workloads.decode_query(w.B, w.Hq, w.d, seed=0).to(DEV)
    sl = lens.to(DEV)
    op, lp = fa.fa_decode_kvcache_ext(q, kp, vp, sl, block_table=table)
    oc, lc = fa.fa_decode_kvcache(q, kc, vc, sl)
    torch.cuda.synchronize()
    assert torch.equal(op, oc) and torch.equal(lp, lc)


def test_paged_long_ranges_small_pages():
    """Balanced split with ranges longer than one page-list load (16-row
    pages, over a thousand rows per range): paged equals contiguous bitwise,
    and both agree with the chunked split (explicit split count) to one bf16
    ulp."""
    fa = need_gpu()
    announce("decode paged long ranges, 16-row pages")
    B, Hq, Hkv, d, ps = 2, 16, 4, 128, 16
    lens = [600000, 100000]
    N = 600016
    mp = N // ps
    gen = torch.Generator(device=DEV).manual_seed(3)
    kc = torch.randn((B, N, Hkv, d), generator=gen, device=DEV).to(torch.bfloat16)
    vc = torch.randn((B, N, Hkv, d), generator=gen, device=DEV).to(torch.bfloat16)
    perm = torch.randperm(B * mp, generator=torch.Generator().manual_seed(4))
    table = torch.argsort(perm).view(B, mp).to(torch.int32).to(DEV)
    kp = torch.empty((B * mp, ps, Hkv, d), dtype=torch.bfloat16, device=DEV)
    vp = torch.empty_like(kp)
    kp[table.view(-1).long()] = kc.view(B * mp, ps, Hkv, d)
    vp[table.view(-1).long()] = vc.view(B * mp, ps, Hkv, d)
    q = torch.randn((B, Hq, d), generator=gen, device=DEV).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    op, lp = fa.fa_decode_kvcache_ext(q, kp, vp, sl, block_table=table)
    oc, lc = fa.fa_decode_kvcache(q, kc, vc, sl)
    os_, ls_ = fa.fa_decode_kvcache(q, kc, vc, sl, num_splits=600)
    torch.cuda.synchronize()
    assert torch.equal(op, oc) and torch.equal(lp, lc)
    ulp = (os_.float().abs() * 2.0 ** -7).clamp_min(1e-30)
    assert ((os_.float() - oc.float()).abs() <= ulp + 1e-6).all()
    assert ((ls_ - lc).abs() <= 1e-4).all()
