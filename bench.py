#!/usr/bin/env python
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass over every stage of the path, on seeded synthetic inputs
already resident in device memory:
  * forward  (fa_fwd) and backward (fa_bwd, timed stage by stage) of causal
    bf16 attention at B=1, N=8192, Hq=Hkv=96, d=128 -- the shape of the
    flash_attn fwd+bwd timing on GB200 in the zocula guide to
    flash-linear-attention (benchmark section);
  * one KV-cache decode (fa_decode_kvcache: balanced split kernel + merge kernel) of
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
import statistics
import subprocess
import sys
import threading
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
    "decode_split_bal_kernel": "fa_decode.hip",
    "decode_merge_bal_kernel": "fa_decode.hip",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads of the oracle sample")
    ap.add_argument("--no-decode", action="store_true", help="leave the decode stage out (profiling only)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the amd-smi clock/power reading (profiling runs: it starts a child process and "
                         "adds steps outside the timed region)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the secondary measurements (window, varlen, paged decode, block-sparse)")
    ap.add_argument("--sweep-only", type=int, default=0, metavar="LAUNCHES",
                    help="only run the causal forward sweep (H=16, d=128, 16k tokens at N = 512, 2048, 8192, "
                         "16384), LAUNCHES launches per point after two warm-up launches, and exit (profiling)")
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


def sweep_only(launches: int) -> None:
    """The causal forward sweep of the extras (same inputs), `launches`
    back-to-back launches per point after two warm-up launches, for a
    profiler to take apart point by point (the launches run in the order
    N = 512, 2048, 8192, 16384)."""
    import torch

    import exact_attention_19_amd as fa
    import workloads

    fa.load()
    dev = torch.device("cuda:0")
    done = {}
    for N in (512, 2048, 8192, 16384):
        B = 16384 // N
        inp = workloads.prefill_inputs(B, N, 16, 16, 128, "bf16", seed=5, mult=0.5)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        del inp
        o_, l_ = torch.empty_like(q), torch.empty((B, 16, N), dtype=torch.float32, device=dev)
        for _ in range(2 + launches):
            fa.fa_fwd(q, k, v, causal=True, out=o_, lse=l_)
        torch.cuda.synchronize()
        done[f"N={N} B={B}"] = 2 + launches
        del q, k, v, o_, l_
    print(json.dumps({"sweep_only_launches": done}))


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


def blas_info() -> dict:
    """BLAS library behind numpy and its thread count (threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_info

        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            b = max(blas, key=lambda i: i.get("num_threads", 0))
            return {"vendor": b.get("internal_api"), "threads": b.get("num_threads"),
                    "version": b.get("version"), "threading_layer": b.get("threading_layer")}
    except Exception:  # noqa: BLE001
        pass
    return {"vendor": None, "threads": os.cpu_count() or 1}


def host_cpus() -> dict:
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = None
    return {"os_cpu_count": os.cpu_count(), "sched_affinity": aff}


def _num(x):
    """A number out of amd-smi's JSON ({"value": v, "unit": u}, "123 MHz" or 123)."""
    if isinstance(x, dict):
        x = x.get("value")
    if isinstance(x, str):
        x = x.split()[0] if x.strip() else "N/A"
        try:
            return float(x)
        except ValueError:
            return None
    return float(x) if isinstance(x, (int, float)) else None


def smi_sample():
    """One amd-smi reading of GPU 0: shader (gfx) clocks in MHz, socket power
    in W and throttle status; None where amd-smi is unavailable."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True, text=True,
                           timeout=30)
        d = json.loads(r.stdout)
    except Exception:  # noqa: BLE001
        return None
    if isinstance(d, dict) and "gpu_data" in d:
        d = d["gpu_data"]
    if isinstance(d, list):
        d = d[0] if d else {}
    clk = d.get("clock", {}) if isinstance(d, dict) else {}
    pw = d.get("power", {}) if isinstance(d, dict) else {}
    gfx = [v for k, c in clk.items() if k.startswith("gfx_") and isinstance(c, dict)
           for v in [_num(c.get("clk"))] if v]
    return {"t": time.perf_counter(), "gfx_mhz": gfx, "mem_mhz": _num(clk.get("mem_0", {}).get("clk"))
            if isinstance(clk.get("mem_0"), dict) else None,
            "socket_w": _num(pw.get("socket_power")), "throttle": pw.get("throttle_status")}


def sustained_clock(step, seconds: float):
    """Run `step` back to back for `seconds` while amd-smi is read on a side
    thread; returns the median gfx clock and socket power seen under that load."""
    import torch

    samples, stop = [], threading.Event()

    def sampler():
        time.sleep(0.3)
        while not stop.is_set():
            smp = smi_sample()
            if smp is None:
                return
            samples.append(smp)

    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        step()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=60)
    if not samples:
        return {"note": "amd-smi unavailable"}
    gfx = [v for smp in samples for v in smp["gfx_mhz"]]
    pw = [smp["socket_w"] for smp in samples if smp["socket_w"]]
    return {"samples": len(samples), "steps": n, "seconds": round(time.perf_counter() - t0, 2),
            "gfx_clock_mhz_median": statistics.median(gfx) if gfx else None,
            "gfx_clock_mhz_min": min(gfx) if gfx else None, "gfx_clock_mhz_max": max(gfx) if gfx else None,
            "socket_power_w_median": statistics.median(pw) if pw else None,
            "mem_clock_mhz": samples[-1]["mem_mhz"], "throttle_status": sorted({str(smp["throttle"]) for smp in samples}),
            "source": "amd-smi metric -g 0 -c -p, read while the step runs back to back"}


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
        "cores": blas_info()["threads"],
        "kind": "oracle",
        "blas": blas_info(),
        "host": host_cpus(),
        "sample": f"{heads} of {w.B * w.Hq} heads (b=0, h<{heads}) at full N={w.N}: fp64 forward + backward "
                  f"with S materialised; {dt:.1f} s wall",
    }


def _time_ms(fn, reps=None, warm=5):
    """Per-launch times of fn() from HIP events on the current stream:
    {"ms": median, "mean_ms", "min_ms", "reps"}. With reps=None the count
    follows one timed launch: 100 below 0.1 ms, else 20."""
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    if reps is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        reps = 100 if e0.elapsed_time(e1) < 0.1 else 20
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    # A spin kernel ahead of the timed launches lets the host queue them all
    # while the GPU is busy, so short launches run back to back and the events
    # do not count time spent waiting for the host.
    try:
        torch.cuda._sleep(50_000_000)
    except Exception:  # noqa: BLE001
        pass
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return {"ms": round(statistics.median(t), 4), "mean_ms": round(sum(t) / reps, 4), "min_ms": round(min(t), 4),
            "reps": reps}


def _fwd_roofline(flops, B, N, Hq, Hkv, d, ms):
    """Where a forward point sits on the roofline: its minimum HBM bytes (Q, K,
    V read once, O and the fp32 LSE written once), the rate that makes, and
    which of the two bounds (bf16 MFMA peak, HBM peak) is the larger time; the
    fraction is that bound's time over the measured time."""
    nbytes = 2 * B * N * d * (2 * Hq + 2 * Hkv) + 4 * B * Hq * N
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if t_hbm > t_mfma else "mfma"
    return {"min_bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bound": bound,
            "roofline_frac": round(max(t_mfma, t_hbm) / (ms * 1e-3), 4)}


def _pairs_band(nq, nk, causal, wl=-1, wr=-1):
    """Visible (query, key) pairs of one head: keys j with i + off - wl <= j <=
    i + off + wr (and j <= i + off when causal), off = nk - nq."""
    import numpy as np

    i = np.arange(nq, dtype=np.int64)
    diag = i + (nk - nq)
    hi = np.full(nq, nk - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, diag)
    if wr >= 0:
        hi = np.minimum(hi, diag + wr)
    lo = np.zeros(nq, dtype=np.int64) if wl < 0 else np.maximum(diag - wl, 0)
    return int(np.maximum(hi - lo + 1, 0).sum())


def extras(fa_mod, lib, dev):
    """Secondary lines: the causal forward sweep, the two small forward
    configs and GQA fwd+bwd of the workload configs, and the sliding-window, varlen, paged-decode and
    block-sparse paths on workloads of the pages' shapes. Each rate uses the
    algorithmic work (4*d FLOP per visible query-key pair in a forward,
    2.5x that in a backward; bytes read once for decode)."""
    import numpy as np
    import torch

    import workloads
    from exact_attention_19_amd import _lib

    out = {}
    # Causal forward sweep: hidden 2048 (16 heads x 128), 16k tokens per batch.
    sweep = {}
    for N in (512, 2048, 8192, 16384):
        B = 16384 // N
        inp = workloads.prefill_inputs(B, N, 16, 16, 128, "bf16", seed=5, mult=0.5)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        del inp
        o_, l_ = torch.empty_like(q), torch.empty((B, 16, N), dtype=torch.float32, device=dev)
        t = _time_ms(lambda: fa_mod.fa_fwd(q, k, v, causal=True, out=o_, lse=l_))
        pairs = _pairs_band(N, N, True) * B * 16
        tf = 4 * 128 * pairs / (t["ms"] * 1e9)
        sweep[f"N={N} B={B}"] = {**t, "TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                 **_fwd_roofline(4 * 128 * pairs, B, N, 16, 16, 128, t["ms"])}
        del o_, l_
        del q, k, v
    out["fwd_sweep_h2048"] = {"workload": "causal forward, H=16 d=128, B*N = 16384 tokens", "points": sweep}
    # The same sweep at head dim 64 (hidden 2048 = 32 heads x 64), causal and not.
    sweep = {}
    for N in (512, 2048, 8192, 16384):
        for causal in (True, False):
            B = 16384 // N
            inp = workloads.prefill_inputs(B, N, 32, 32, 64, "bf16", seed=6, mult=0.5)
            q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
            del inp
            o_, l_ = torch.empty_like(q), torch.empty((B, 32, N), dtype=torch.float32, device=dev)
            t = _time_ms(lambda: fa_mod.fa_fwd(q, k, v, causal=causal, out=o_, lse=l_))
            pairs = _pairs_band(N, N, causal) * B * 32
            tf = 4 * 64 * pairs / (t["ms"] * 1e9)
            sweep[f"N={N} B={B}{' causal' if causal else ''}"] = {
                **t, "TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                **_fwd_roofline(4 * 64 * pairs, B, N, 32, 32, 64, t["ms"])}
            del o_, l_
            del q, k, v
    out["fwd_sweep_h2048_d64"] = {"workload": "forward, H=32 d=64, B*N = 16384 tokens", "points": sweep}
    # The two small configs: an fp32 forward (B=1, H=1, N=128, d=64, non-causal)
    # and a bf16 d=64 forward (B=2, H=8, N=1024, non-causal and causal). Both
    # are a few workgroups and launch-bound; they are timed through the C ABI
    # directly (the torch binding's per-call checks would dominate).
    small = {}
    for name, (B, N, H, d, dt, causal) in {"fp32 B=1 H=1 N=128 d=64": (1, 128, 1, 64, "fp32", False),
                                           "bf16 B=2 H=8 N=1024 d=64": (2, 1024, 8, 64, "bf16", False),
                                           "bf16 B=2 H=8 N=1024 d=64 causal": (2, 1024, 8, 64, "bf16", True)}.items():
        inp = workloads.prefill_inputs(B, N, H, H, d, dt, seed=0)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        sp = torch.cuda.current_stream(dev).cuda_stream
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H, N, d,
                1.0 / d ** 0.5, int(causal), _lib.FA_FP32 if dt == "fp32" else _lib.FA_BF16, sp)
        t = _time_ms(lambda: _lib.check(lib.fa_fwd(*args)), reps=200, warm=20)
        pairs = _pairs_band(N, N, causal) * B * H
        small[name] = {**t, "TFLOP/s": round(4 * d * pairs / (t["ms"] * 1e9), 2)}
        del inp, q, k, v, o, lse
    out["small_configs_fwd"] = small
    # Forward + backward with GQA (Hkv = 12) at the GB200 timing shape.
    B, N, H, Hkv, d = 1, 8192, 96, 12, 128
    inp = workloads.prefill_inputs(B, N, H, Hkv, d, "bf16", seed=6, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    del inp
    o, lse = fa_mod.fa_fwd(q, k, v, causal=True)
    pairs = _pairs_band(N, N, True) * B * H
    tf_ = _time_ms(lambda: fa_mod.fa_fwd(q, k, v, causal=True, out=o, lse=lse))
    tb_ = _time_ms(lambda: fa_mod.fa_bwd(q, k, v, o, do, lse, causal=True))
    ms_f, ms_b = tf_["ms"], tb_["ms"]
    ta_ = _time_ms(lambda: fa_mod.fa_bwd(q, k, v, o, do, lse, causal=True, deterministic=False))
    out["gqa_bwd_atomic"] = {"workload": f"B={B} N={N} Hq={H} Hkv={Hkv} d={d} causal", **ta_,
                             "TFLOP/s": round(2.5 * 4 * d * pairs / (ta_["ms"] * 1e9), 1),
                             "note": "fa_bwd_atomic: preprocess + fused dK/dV/dQ (fp32 atomic dQ) + dQ convert"}
    out["gqa_fwd_bwd"] = {"workload": f"B={B} N={N} Hq={H} Hkv={Hkv} d={d} causal", "fwd": tf_, "bwd": tb_,
                          "fwd_TFLOP/s": round(4 * d * pairs / (ms_f * 1e9), 1),
                          "fwd+bwd TFLOP/s": round(3.5 * 4 * d * pairs / ((ms_f + ms_b) * 1e9), 1),
                          "note": "fa_bwd: preprocess + dK/dV + dQ kernels"}
    del q, k, v, do, o, lse
    # Causal fwd + bwd at head dim 64 (hidden 2048 = 32 heads x 64, 16k tokens).
    pts = {}
    for N in (2048, 16384):
        B, H, d = 16384 // N, 32, 64
        inp = workloads.prefill_inputs(B, N, H, H, d, "bf16", seed=7, mult=0.5, with_do=True)
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        del inp
        o, lse = fa_mod.fa_fwd(q, k, v, causal=True)
        pairs = _pairs_band(N, N, True) * B * H
        tf_ = _time_ms(lambda: fa_mod.fa_fwd(q, k, v, causal=True, out=o, lse=lse))
        tb_ = _time_ms(lambda: fa_mod.fa_bwd(q, k, v, o, do, lse, causal=True))
        pts[f"N={N} B={B}"] = {"fwd": tf_, "bwd": tb_, "bwd_TFLOP/s": round(2.5 * 4 * d * pairs / (tb_["ms"] * 1e9), 1),
                               "fwd+bwd TFLOP/s": round(3.5 * 4 * d * pairs / ((tf_["ms"] + tb_["ms"]) * 1e9), 1)}
        del q, k, v, do, o, lse
    out["fwd_bwd_d64_h2048"] = {"workload": "causal fwd + bwd, H=32 d=64, B*N = 16384 tokens", "points": pts,
                                "note": "fa_bwd: preprocess + dK/dV + dQ kernels (d = 64 on the DMA kernels, 128-byte rows)"}
    # Sliding window at the GB200 timing shape, window of 4096 keys (causal).
    B, N, H, d = 1, 8192, 96, 128
    wl = 4095
    inp = workloads.prefill_inputs(B, N, H, H, d, "bf16", seed=1, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    del inp
    o, lse = fa_mod.fa_fwd_window(q, k, v, (wl, 0), causal=True)
    pairs = _pairs_band(N, N, True, wl, 0) * B * H
    tf_ = _time_ms(lambda: fa_mod.fa_fwd_window(q, k, v, (wl, 0), causal=True, out=o, lse=lse))
    tb_ = _time_ms(lambda: fa_mod.fa_bwd(q, k, v, o, do, lse, causal=True, window=(wl, 0)))
    ms_f, ms_b = tf_["ms"], tb_["ms"]
    o_full, lse_full = fa_mod.fa_fwd(q, k, v, causal=True)
    ta_ = _time_ms(lambda: fa_mod.fa_bwd(q, k, v, o_full, do, lse_full, causal=True, deterministic=False))
    pairs_full = _pairs_band(N, N, True) * B * H
    out["bwd_atomic"] = {"workload": f"B={B} N={N} H={H} d={d} causal", **ta_,
                         "TFLOP/s": round(2.5 * 4 * d * pairs_full / (ta_["ms"] * 1e9), 1),
                         "note": "fa_bwd_atomic: preprocess + fused dK/dV/dQ (fp32 atomic dQ) + dQ convert; "
                                 "compare kernels.bwd_* (deterministic)"}
    del o_full, lse_full
    out["window_fwd"] = {"workload": f"B={B} N={N} H={H} d={d} causal window (4095, 0)", **tf_,
                         "TFLOP/s": round(4 * d * pairs / (ms_f * 1e9), 1)}
    out["window_bwd"] = {"workload": out["window_fwd"]["workload"], **tb_,
                         "TFLOP/s": round(2.5 * 4 * d * pairs / (ms_b * 1e9), 1),
                         "note": "fa_bwd_window: preprocess + dK/dV + dQ kernels"}
    # Block-sparse at the same shape: a band of 5 blocks plus the first block column.
    nb = N // 128
    ib = np.arange(nb)
    bm = ((np.abs(ib[:, None] - ib[None, :]) <= 2) | (ib[None, :] == 0)).astype(np.uint8)
    keep = np.kron(bm, np.ones((128, 128), dtype=np.uint8)).astype(bool) & np.tri(N, dtype=bool)
    pairs = int(keep.sum()) * B * H
    del keep
    bmd = torch.from_numpy(bm).to(dev)
    t = _time_ms(lambda: fa_mod.fa_fwd_blocksparse(q, k, v, bmd, causal=True))
    out["blocksparse_fwd"] = {"workload": f"B={B} N={N} H={H} d={d} causal, 128x128 blocks: band |i-j|<=2 "
                                          f"plus block column 0 ({bm.mean() * 100:.1f}% of blocks)",
                              **t, "TFLOP/s": round(4 * d * pairs / (t["ms"] * 1e9), 1)}
    del q, k, v, do, o, lse
    # Varlen prefill: hidden 2048 (16 heads x 128), sequences U[256, 4096] packed to >= 16k tokens.
    rng = np.random.default_rng(2)
    lens = []
    while sum(lens) < 16384:
        lens.append(int(rng.integers(256, 4097)))
    vin = workloads.varlen_inputs(lens, lens, 16, 16, d, seed=3)
    vq, vk, vv = (vin[n].to(dev) for n in ("q", "k", "v"))
    cq, ck = vin["cu_q"].to(dev), vin["cu_k"].to(dev)
    pairs = sum(_pairs_band(n, n, True) for n in lens) * 16
    t = _time_ms(lambda: fa_mod.fa_fwd_varlen(vq, vk, vv, cq, ck, max(lens), causal=True))
    out["varlen_fwd"] = {"workload": f"{len(lens)} sequences (U[256,4096], {sum(lens)} tokens) H=16 d=128 causal",
                         **t, "TFLOP/s": round(4 * d * pairs / (t["ms"] * 1e9), 1)}
    del vq, vk, vv
    # Paged decode with append: the decode workload in 256-row pages.
    wd = workloads.WORKLOADS["c5"]
    seq = workloads.decode_seqlens(wd.B, wd.seq_lo, wd.seq_hi, seed=0)
    seq = torch.clamp(seq, max=wd.N - 1)                # room for the appended token
    ps, mp = 256, wd.N // 256
    kp = torch.randn((wd.B * mp, ps, wd.Hkv, wd.d), device=dev, dtype=torch.bfloat16)
    vp = torch.randn_like(kp)
    perm = torch.randperm(wd.B * mp, generator=torch.Generator().manual_seed(4))
    table = perm.view(wd.B, mp).to(torch.int32).to(dev)
    qd = workloads.decode_query(wd.B, wd.Hq, wd.d, seed=0).to(dev)
    kn = torch.randn((wd.B, wd.Hkv, wd.d), device=dev, dtype=torch.bfloat16)
    sl = seq.to(dev)
    t = _time_ms(lambda: fa_mod.fa_decode_kvcache_ext(qd, kp, vp, sl, block_table=table, k_new=kn, v_new=kn))
    ms = t["ms"]
    nbytes = 2 * 2 * wd.d * wd.Hkv * int((seq + 1).sum()) + 2 * wd.B * wd.Hq * wd.d * 2 + 4 * wd.B * wd.Hq
    out["paged_decode_append"] = {"workload": "64 seqs x 1 query, Hq=32 Hkv=8 d=128, L~U[1024,32768]+1, "
                                              "256-row pages in a shuffled pool, in-place append",
                                  **t, "GB/s": round(nbytes / (ms * 1e6), 1),
                                  "note": "append + split + merge kernels; bytes = cache rows read once + q/o/lse"}
    del kp, vp
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(pass --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.sweep_only:
        sweep_only(args.sweep_only)
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
    times = {name: [events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]
             for i, (name, _) in enumerate(stages)}
    per = {name: float(np.mean(t)) for name, t in times.items()}
    step_t = [events[s][0].elapsed_time(events[s][-1]) for s in range(args.steps)]
    step_ms = float(np.mean(step_t))

    # Clock and power under this load: the step back to back for a few
    # seconds while amd-smi is read (outside the timed region).
    clock = None if args.no_clock else sustained_clock(lambda: [fn() for _, fn in stages], 4.0)

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
        spread = {"median_ms": round(float(np.median(times[name])), 4), "min_ms": round(float(min(times[name])), 4)}
        if bound == "mfma":
            ach = work / (ms * 1e-3) / 1e12
            kernels[name] = {"ms": round(ms, 4), **spread, "TFLOP/s": round(ach, 1),
                             "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = work / (ms * 1e-3) / 1e9
            kernels[name] = {"ms": round(ms, 4), **spread, "GB/s": round(ach, 1), "frac": round(ach / PEAK_HBM_GBS, 4)}
    if run_decode:
        gbs = decode_bytes / (per["decode"] * 1e-3) / 1e9
        kernels["decode"] = {"ms": round(per["decode"], 4), "median_ms": round(float(np.median(times["decode"])), 4),
                             "min_ms": round(float(min(times["decode"])), 4), "GB/s": round(gbs, 1),
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
                "algorithmic_per_launch": work, "avg_launch_ms": round(ms, 4),
                "median_launch_ms": round(float(np.median(times[dom])), 4)}
    if run_decode and per["decode"] > ms:
        roofline["note"] = "decode (split+merge) takes longer than this kernel; see decode"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, w, args.cpu_heads)

    extra = None
    if not args.no_extras:
        if run_decode:
            del kc, vc
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
        extra = extras(fa, lib, dev)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_median": round(float(np.median(step_t)), 4),
        "ms_per_step_min": round(float(min(step_t)), 4),
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
        "extras": extra,
        "wall_s_timed_region": round(wall, 3),
        "gpu": torch.cuda.get_device_name(0),
        "gpu_clock_power": clock,
        "timing": "HIP events on the library's stream around every launch; per kernel mean (ms), median and "
                  "min over the timed steps; extras: median of >= 20 launches (>= 100 below 0.1 ms)",
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
