"""Seeded synthetic inputs for the attention workloads.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic, so both the fp64 oracle and the HIP path can be fed
from it without sharing any computation.

Every tensor is drawn on the CPU from a ``torch.Generator`` as float32
standard normals, multiplied by an optional factor, then rounded to the
storage dtype (round-to-nearest-even for bfloat16). The same seed always
gives the same bits, on any machine.

Workload shapes follow the pages' benchmark settings: the README sweep
(head dim 64 or 128, hidden 2048, sequence 512 to 16k, batch = 16k / seqlen;
hysenlabs digest of the flash-attention README, "FlashAttentionで見る対応範囲の
読み方") and the B=1, T=8192, H=96, d=128 shape timed on GB200 in the zocula
guide to flash-linear-attention (benchmark section).
"""
from __future__ import annotations

import itertools
import math
from dataclasses import dataclass, field

import torch

DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _randn(shape, gen, mult, dtype):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if mult != 1.0:
        x = x * mult
    return x.to(dtype)


def device_normal(shape, seed, mult=1.0, dtype="bf16", device="cuda:0"):
    """Standard normals drawn directly on a GPU from torch's seeded generator
    (for inputs of several GiB, which drawing on the host and copying would
    make slow), times ``mult``, rounded to the storage dtype. The same seed
    gives the same bits on the same torch build and device type; a check
    copies to the host only the slices it needs."""
    gen = torch.Generator(device=device).manual_seed(seed)
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(DTYPES[dtype])


def prefill_inputs(B, N, Hq, Hkv, d, dtype="bf16", seed=0, mult=1.0, with_do=False, Nk=None, do_mult=1.0):
    """Q [B, N, Hq, d], K and V [B, Nk, Hkv, d] (and dO like Q), drawn in that order.
    ``mult`` scales Q, K and V; ``do_mult`` scales dO."""
    nk = N if Nk is None else Nk
    dt = DTYPES[dtype]
    gen = torch.Generator().manual_seed(seed)
    q = _randn((B, N, Hq, d), gen, mult, dt)
    k = _randn((B, nk, Hkv, d), gen, mult, dt)
    v = _randn((B, nk, Hkv, d), gen, mult, dt)
    out = {"q": q, "k": k, "v": v}
    if with_do:
        out["do"] = _randn((B, N, Hq, d), gen, do_mult, dt)
    return out


def varlen_inputs(lens_q, lens_k, Hq, Hkv, d, dtype="bf16", seed=0, mult=1.0):
    """Packed variable-length sequences: q [sum(lens_q), Hq, d], k/v
    [sum(lens_k), Hkv, d] drawn in that order, and int32 prefix sums
    cu_q, cu_k of shape [B + 1]."""
    dt = DTYPES[dtype]
    gen = torch.Generator().manual_seed(seed)
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    q = _randn((tq, Hq, d), gen, mult, dt)
    k = _randn((tk, Hkv, d), gen, mult, dt)
    v = _randn((tk, Hkv, d), gen, mult, dt)
    cu_q = torch.tensor([0] + list(itertools.accumulate(int(x) for x in lens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(itertools.accumulate(int(x) for x in lens_k)), dtype=torch.int32)
    return {"q": q, "k": k, "v": v, "cu_q": cu_q, "cu_k": cu_k}


def decode_seqlens(B, lo, hi, seed=0):
    """Per-sequence cache lengths, integers uniform on [lo, hi] inclusive."""
    gen = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int32)


def decode_query(B, Hq, d, dtype="bf16", seed=0):
    """The single query token per sequence, [B, Hq, d]."""
    gen = torch.Generator().manual_seed(seed * 7919 + 1)
    return _randn((B, Hq, d), gen, 1.0, DTYPES[dtype])


def decode_kv_rows(b, L, Hkv, d, dtype="bf16", seed=0):
    """K and V rows 0 .. L-1 of sequence b, each [L, Hkv, d].

    Each sequence has its own generator, so one sequence can be rebuilt
    without drawing the others (the full cache is gigabytes).
    """
    gen = torch.Generator().manual_seed(seed * 1_000_003 + 17 + b)
    dt = DTYPES[dtype]
    k = _randn((L, Hkv, d), gen, 1.0, dt)
    v = _randn((L, Hkv, d), gen, 1.0, dt)
    return k, v


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "fwd", "fwd_bwd" or "decode"
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str
    causal: bool
    mult: float = 1.0
    seq_lo: int = 0
    seq_hi: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def fwd_flops(self) -> float:
        """4 * B * Hq * N^2 * d, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """2.5 times the forward count (five N x N x d products against two)."""
        return 2.5 * self.fwd_flops()


def c3(N: int) -> Workload:
    return Workload(f"c3_causal_fwd_N{N}", "fwd", 16384 // N, 16, 16, N, 128, "bf16", True, 0.5,
                    note="hidden 2048 = 16 heads x 128, 16k tokens per batch")


def sweep_d64(N: int, causal: bool = True) -> Workload:
    """The head-dim-64 member of the same benchmark sweep: hidden 2048 = 32
    heads x 64, 16k tokens per batch."""
    return Workload(f"sweep_d64_{'causal_' if causal else ''}fwd_N{N}", "fwd", 16384 // N, 32, 32, N, 64, "bf16",
                    causal, 0.5, note="hidden 2048 = 32 heads x 64, 16k tokens per batch")


WORKLOADS = {
    "c1": Workload("c1_fp32_fwd", "fwd", 1, 1, 1, 128, 64, "fp32", False),
    "c2": Workload("c2_bf16_fwd", "fwd", 2, 8, 8, 1024, 64, "bf16", False),
    "c2c": Workload("c2_bf16_fwd_causal", "fwd", 2, 8, 8, 1024, 64, "bf16", True),
    "c3_512": c3(512),
    "c3_2048": c3(2048),
    "c3_8192": c3(8192),
    "c3_16384": c3(16384),
    "c4": Workload("c4_causal_fwd_bwd_mha", "fwd_bwd", 1, 96, 96, 8192, 128, "bf16", True),
    "c4g": Workload("c4_causal_fwd_bwd_gqa", "fwd_bwd", 1, 96, 12, 8192, 128, "bf16", True),
    "c5": Workload("c5_decode_gqa", "decode", 64, 32, 8, 32768, 128, "bf16", False,
                   seq_lo=1024, seq_hi=32768),
}
