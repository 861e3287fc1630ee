"""Every tile is computed exactly once under the XCD-aware workgroup order.

When the number of heads (B*Hq for the forward and dQ kernels, B*Hkv for the
dK/dV kernel) is a multiple of 8, workgroups are remapped so that each XCD
takes whole heads, visited in groups of a few heads with the heaviest tile of
each head first. These shapes give 1, 2, 3, 5 and 9 heads per XCD (a last
group shorter than the others, or a single one) with ragged tiles; the
outputs start as NaN, so a tile that no workgroup writes shows up, and every
value is compared with the fp64 oracle.
"""
from __future__ import annotations

import math

import pytest
import torch

import oracle
import workloads
from parity import announce, assert_bf16_close, f64, need_gpu

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, N, Hq, Hkv  (d = 128)
    (1, 320, 8, 8),
    (2, 320, 8, 8),
    (1, 320, 24, 24),
    (1, 320, 40, 8),
    (3, 200, 24, 24),
    (1, 448, 72, 24),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{b}N{n}Hq{hq}Hkv{hk}" for b, n, hq, hk in SHAPES])
def test_every_tile_written_once(shape, causal):
    fa = need_gpu()
    from exact_attention_19_amd import _lib

    B, N, Hq, Hkv = shape
    d = 128
    announce(f"workgroup order {shape} causal={causal}")
    dev = torch.device("cuda:0")
    inp = workloads.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=7 + Hq + N, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full((B, Hq, N), nan, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(v, nan)
    lib = _lib.load()
    ws_bytes = lib.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d)
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    scale = 1 / math.sqrt(d)
    P = lambda t: t.data_ptr()  # noqa: E731
    _lib.check(lib.fa_fwd(P(q), P(k), P(v), P(o), P(lse), B, Hq, Hkv, N, d, scale, int(causal), _lib.FA_BF16,
                          stream))
    _lib.check(lib.fa_bwd(P(q), P(k), P(v), P(o), P(do), P(lse), P(dq), P(dk), P(dv), P(ws), ws_bytes, B, Hq,
                          Hkv, N, d, scale, int(causal), _lib.FA_BF16, stream))
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale, causal)
    rdq, rdk, rdv, _ = oracle.attn_bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]), scale, causal)
    assert_bf16_close(o, ro, "O")
    assert_bf16_close(lse, rlse, "LSE")
    assert_bf16_close(dq, rdq, "dQ")
    assert_bf16_close(dk, rdk, "dK")
    assert_bf16_close(dv, rdv, "dV")
