"""fa_decode_kvcache_noalloc recorded into a HIP graph (the use it exists
for: code under graph capture cannot allocate a workspace), through the C
ABI. The graph is replayed several times, with eager work and host
synchronisation between replays and new query and cache-length values
written into the captured input buffers before some of them; every replay
must equal an eager call on the same inputs bit for bit, and the oracle
within the bf16 bound."""
from __future__ import annotations

import math

import pytest
import torch

import oracle
import workloads
from exact_attention_19_amd import _lib
from parity import announce, assert_bf16_close, f64, need_gpu

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
B, HQ, HKV, N, D = 8, 32, 8, 2048, 128


def _cache(lens, seed):
    kc = torch.full((B, N, HKV, D), float("nan"), dtype=torch.bfloat16)
    vc = torch.full_like(kc, float("nan"))
    for b in range(B):
        kr, vr = workloads.decode_kv_rows(b, int(lens[b]), HKV, D, seed=seed)
        kc[b, :int(lens[b])] = kr
        vc[b, :int(lens[b])] = vr
    return kc, vc


def _decode(lib, q, kc, vc, lens, o, lse):
    st = lib.fa_decode_kvcache_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), lens.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), B, HQ, HKV, N, D, 1 / math.sqrt(D), 0, 0, _lib.FA_BF16,
                                       torch.cuda.current_stream(DEV).cuda_stream)
    _lib.check(st)


def test_noalloc_decode_replayed_from_a_graph():
    fa = need_gpu()
    lib = fa.load()
    announce(f"no-alloc decode under graph capture B={B} Hq={HQ} Hkv={HKV} N={N} d={D}")
    # Every cache row up to N holds real values; the lengths pick how many count.
    full = torch.full((B,), N, dtype=torch.int32)
    kc, vc = (t.to(DEV) for t in _cache(full, seed=81))
    lens = workloads.decode_seqlens(B, 1, N, seed=81).to(DEV)
    q = workloads.decode_query(B, HQ, D, seed=81).to(DEV)
    o_g = torch.full((B, HQ, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    l_g = torch.full((B, HQ), float("nan"), dtype=torch.float32, device=DEV)
    o_e, l_e = torch.empty_like(o_g), torch.empty_like(l_g)

    # One eager call first: it looks up the scratch array's address and the
    # split plan's device figures, which capture must not have to do.
    _decode(lib, q, kc, vc, lens, o_e, l_e)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        _decode(lib, q, kc, vc, lens, o_g, l_g)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _decode(lib, q, kc, vc, lens, o_g, l_g)
    torch.cuda.synchronize()

    for rep in range(4):
        if rep >= 2:
            # New inputs in the captured buffers.
            q.copy_(workloads.decode_query(B, HQ, D, seed=90 + rep).to(DEV))
            lens.copy_(workloads.decode_seqlens(B, 1, N, seed=90 + rep).to(DEV))
        o_g.fill_(float("nan"))
        l_g.fill_(float("nan"))
        _decode(lib, q, kc, vc, lens, o_e, l_e)  # eager reference, same scratch array, before the replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {rep}: output differs from the eager call"
        assert torch.equal(l_g, l_e), f"replay {rep}: lse differs from the eager call"
        if rep in (0, 3):
            qh, kh, vh, lh = q.cpu(), kc.cpu(), vc.cpu(), lens.cpu()
            ro, rl = oracle.attn_decode(f64(qh), f64(kh), f64(vh), lh.numpy(), 1 / math.sqrt(D))
            assert_bf16_close(o_g.cpu(), ro, f"replay {rep} O")
            assert_bf16_close(l_g.cpu(), rl, f"replay {rep} LSE")
