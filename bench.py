#!/usr/bin/env python
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass over every stage of the path, on seeded synthetic inputs
already resident in device memory:
  * forward  (fa_fwd) and backward (fa_bwd, timed stage by stage) of causal
    bf16 attention at B=1, N=8192, Hq=Hkv=96, d=128 -- the shape of the
    flash_attn fwd+bwd timing on GB200 in the zocula guide to
    flash-linear-attention (benchmark section);
  * one KV-cache decode (fa_decode_kvcache: split kernel + merge kernel) of
    64 sequences x 1 query, Hq=32, Hkv=8, d=128, cache lengths uniform in
    [1024, 32768].

`value` is attention TFLOP/s of the forward+backward part, with the FLOP
convention forward = 4*B*Hq*N^2*d (halved when causal), backward = 2.5 x
forward. The decode line reports HBM GB/s over the algorithmic bytes
4096*sum(L_b) + q/o/lse bytes. Every kernel is timed with HIP events on the
stream it runs on. `roofline` describes the kernel with the largest share of
the step time; `cpu_baseline` times the fp64 oracle on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s at 1 MI355X (% bf16 MFMA peak); decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 4096 dense bf16 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_causal_fwd_bwd_N8192_H96_d128_and_decode_B64_L32k.txt")
KERNEL_SOURCES = {
    "fwd_bf16_kernel": "fa_fwd.hip",
    "bwd_dkdv_kernel": "fa_bwd.hip",
    "bwd_dq_kernel": "fa_bwd.hip",
    "bwd_preprocess_kernel": "fa_bwd.hip",
    "decode_split_kernel": "fa_decode.hip",
    "decode_merge_kernel": "fa_decode.hip",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads of the oracle sample")
    ap.add_argument("--no-decode", action="store_true", help="leave the decode stage out (profiling only)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the reference "
                         "kernel for scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    """A copy kernel of known size: an elementwise kernel (y = x * 1 in fp32)
    that reads and writes exactly `mib` MiB per launch."""
    import torch

    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": 4 * n, "launches": 3}))


def source_sha(name: str) -> str:
    path = os.path.join(ROOT, "exact_attention_19_amd", "csrc", name)
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "exact_attention_19_amd", "csrc", "fa_common.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, if the kernel
    source is unchanged since the counters were taken; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = source_sha(KERNEL_SOURCES[kernel])
    for line in open(TRAFFIC_FILE):
        if not line.startswith("kernel="):
            continue
        kv = dict(tok.split("=", 1) for tok in line.split())
        if kv.get("kernel") == kernel and kv.get("source_sha") == want:
            return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:  # noqa: BLE001
        pass
    return os.cpu_count() or 1


def cpu_baseline(inp, w, heads: int):
    """fp64 oracle forward+backward on `heads` full heads of the workload."""
    import torch

    import oracle

    def f64(t):
        return t.to(dtype=torch.float64).numpy()

    t0 = time.perf_counter()
    for h in range(heads):
        q = f64(inp["q"][:, :, h:h + 1])
        k = f64(inp["k"][:, :, h:h + 1])
        v = f64(inp["v"][:, :, h:h + 1])
        do = f64(inp["do"][:, :, h:h + 1])
        oracle.attn_fwd(q, k, v, w.scale, w.causal)
        oracle.attn_bwd(q, k, v, do, w.scale, w.causal)
        del q, k, v, do
    dt = time.perf_counter() - t0
    per_head = 3.5 * 4.0 * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    return {
        "value": round(per_head * heads / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.Hq} heads (b=0, h<{heads}) at full N={w.N}: fp64 forward + backward "
                  f"with S materialised; {dt:.1f} s wall",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(pass --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import exact_attention_19_amd as fa
    import workloads
    from exact_attention_19_amd import _lib

    lib = fa.load()
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS["c4"]
    wd = workloads.WORKLOADS["c5"]

    # ---- inputs (seeded, generated on the host, copied once) -------------
    inp = workloads.prefill_inputs(w.B, w.N, w.Hq, w.Hkv, w.d, "bf16", seed=0, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = lib.fa_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    run_decode = not args.no_decode
    if run_decode:
        lens = workloads.decode_seqlens(wd.B, wd.seq_lo, wd.seq_hi, seed=0)
        kc = torch.zeros((wd.B, wd.N, wd.Hkv, wd.d), dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)
        for b in range(wd.B):
            kr, vr = workloads.decode_kv_rows(b, int(lens[b]), wd.Hkv, wd.d, seed=0)
            kc[b, : int(lens[b])] = kr.to(dev)
            vc[b, : int(lens[b])] = vr.to(dev)
            del kr, vr
        qd = workloads.decode_query(wd.B, wd.Hq, wd.d, seed=0).to(dev)
        sl = lens.to(dev)
        od = torch.empty_like(qd)
        ld = torch.empty((wd.B, wd.Hq), dtype=torch.float32, device=dev)
        dws_bytes = lib.fa_decode_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.N, wd.d, 0)
        dws = torch.empty(dws_bytes, dtype=torch.uint8, device=dev)
        decode_bytes = 2 * 2 * wd.d * wd.Hkv * int(lens.sum()) + 2 * wd.B * wd.Hq * wd.d * 2 + 4 * wd.B * wd.Hq
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731

    def fwd():
        _lib.check(lib.fa_fwd(P(q), P(k), P(v), P(o), P(lse), w.B, w.Hq, w.Hkv, w.N, w.d, w.scale, 1,
                              _lib.FA_BF16, sp))

    def bwd(stage):
        _lib.check(lib.fa_bwd_stage(stage, P(q), P(k), P(v), P(o), P(do), P(lse), P(dq), P(dk), P(dv), P(ws),
                                    ws_bytes, w.B, w.Hq, w.Hkv, w.N, w.d, w.scale, 1, _lib.FA_BF16, sp))

    def decode():
        _lib.check(lib.fa_decode_kvcache(P(qd), P(kc), P(vc), P(sl), P(od), P(ld), P(dws), dws_bytes, wd.B, wd.Hq,
                                         wd.Hkv, wd.N, wd.d, wd.scale, 0, 0, _lib.FA_BF16, sp))

    stages = [("fwd_bf16_kernel", fwd), ("bwd_preprocess_kernel", lambda: bwd(0)),
              ("bwd_dkdv_kernel", lambda: bwd(1)), ("bwd_dq_kernel", lambda: bwd(2))]
    if run_decode:
        stages.append(("decode", decode))

    for _ in range(args.warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev = events[s]
        ev[0].record(stream)
        for i, (_, fn) in enumerate(stages):
            fn()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {name: float(np.mean([events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]))
           for i, (name, _) in enumerate(stages)}
    step_ms = float(np.mean([events[s][0].elapsed_time(events[s][-1]) for s in range(args.steps)]))

    fwd_flops = w.fwd_flops()
    bwd_flops = w.bwd_flops()
    t_fb = (per["fwd_bf16_kernel"] + per["bwd_preprocess_kernel"] + per["bwd_dkdv_kernel"] + per["bwd_dq_kernel"])
    value = (fwd_flops + bwd_flops) / (t_fb * 1e-3) / 1e12

    # Algorithmic work per launch. The backward's five N x N x d products
    # are attributed to the kernel that needs them: S, dP, dV, dK to the dK/dV
    # kernel (8 of the 10 N^2 d units), dQ to the dQ kernel (2 of 10); the dQ
    # kernel's recomputation of S and dP is overhead and is not counted.
    causal_f = 0.5 if w.causal else 1.0
    unit = w.B * w.Hq * w.N * w.N * w.d * causal_f
    algo = {
        "fwd_bf16_kernel": ("mfma", 4.0 * unit),
        "bwd_dkdv_kernel": ("mfma", 8.0 * unit),
        "bwd_dq_kernel": ("mfma", 2.0 * unit),
        "bwd_preprocess_kernel": ("hbm", 2 * 2 * w.B * w.N * w.Hq * w.d + 4 * w.B * w.Hq * w.N),
    }
    kernels = {}
    for name, (bound, work) in algo.items():
        ms = per[name]
        if bound == "mfma":
            ach = work / (ms * 1e-3) / 1e12
            kernels[name] = {"ms": round(ms, 4), "TFLOP/s": round(ach, 1), "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = work / (ms * 1e-3) / 1e9
            kernels[name] = {"ms": round(ms, 4), "GB/s": round(ach, 1), "frac": round(ach / PEAK_HBM_GBS, 4)}
    if run_decode:
        gbs = decode_bytes / (per["decode"] * 1e-3) / 1e9
        kernels["decode"] = {"ms": round(per["decode"], 4), "GB/s": round(gbs, 1),
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": decode_bytes}

    dom = max((n for n in algo), key=lambda n: per[n])
    bound, work = algo[dom]
    ms = per[dom]
    if bound == "mfma":
        ach, peak, unit_s = work / (ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        ach, peak, unit_s = work / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"kernel": dom, "bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit_s,
                "frac": round(ach / peak, 4), "traffic": measured_traffic(dom),
                "algorithmic_per_launch": work, "avg_launch_ms": round(ms, 4)}
    if run_decode and per["decode"] > ms:
        roofline["note"] = "decode (split+merge) takes longer than this kernel; see decode"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, w, args.cpu_heads)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal attention fwd+bwd B=1 N=8192 Hq=Hkv=96 d=128 bf16"
                        + (" + KV-cache decode 64 seqs x 1 query Hq=32 Hkv=8 d=128 L~U[1024,32768]"
                           if run_decode else ""),
            "global_batch": w.B, "seq_len": w.N, "heads_q": w.Hq, "heads_kv": w.Hkv, "head_dim": w.d,
            "causal": w.causal, "parallelism": "single GPU",
        },
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
        "decode": ({"GB/s": kernels["decode"]["GB/s"], "frac_of_hbm_peak": kernels["decode"]["frac"],
                    "ms": kernels["decode"]["ms"], "sum_cache_len": int(lens.sum())} if run_decode else None),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 3),
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
