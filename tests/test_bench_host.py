"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the visible
(query, key) pair counts behind every rate, the FLOP convention of the
workload configs, and the rule that a counter summary only counts while the
kernel source it was measured on is unchanged."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _pairs_brute(nq, nk, causal, wl=-1, wr=-1):
    off = nk - nq
    n = 0
    for i in range(nq):
        for j in range(nk):
            if causal and j > i + off:
                continue
            if wl >= 0 and j < i + off - wl:
                continue
            if wr >= 0 and j > i + off + wr:
                continue
            n += 1
    return n


@pytest.mark.parametrize("nq,nk,causal,wl,wr", [
    (1, 1, True, -1, -1), (7, 7, False, -1, -1), (7, 7, True, -1, -1), (5, 9, True, -1, -1),
    (9, 5, True, -1, -1), (16, 16, True, 3, 0), (16, 16, False, 2, 5), (12, 20, True, 4, -1),
    (20, 12, False, -1, 3), (30, 30, True, 0, 0),
])
def test_visible_pairs_match_brute_force(nq, nk, causal, wl, wr):
    assert bench._pairs_band(nq, nk, causal, wl, wr) == _pairs_brute(nq, nk, causal, wl, wr)


def test_causal_pairs_closed_form():
    # N (N + 1) / 2 visible pairs per head with a square causal mask.
    for n in (1, 2, 64, 8192):
        assert bench._pairs_band(n, n, True) == n * (n + 1) // 2


def test_flop_convention_of_the_configs():
    w = workloads.WORKLOADS["c4"]
    # 4 * B * Hq * N^2 * d, halved for causal; backward counted as 2.5x.
    assert w.fwd_flops() == 4 * 1 * 96 * 8192 * 8192 * 128 / 2
    assert w.bwd_flops() == 2.5 * w.fwd_flops()
    assert abs(w.fwd_flops() - 1.649e12) / 1.649e12 < 1e-3
    for n, b in ((512, 32), (2048, 8), (8192, 2), (16384, 1)):
        c = workloads.c3(n)
        assert (c.B, c.Hq, c.Hkv, c.N, c.d, c.causal) == (b, 16, 16, n, 128, True)


def test_traffic_only_counts_for_the_measured_source(tmp_path, monkeypatch):
    sha = bench.source_sha(bench.KERNEL_SOURCES["bwd_dkdv_kernel"])
    f = tmp_path / "traffic.txt"
    f.write_text("# header\n"
                 f"kernel=bwd_dkdv_kernel source_sha={sha} fetch_bytes=100 write_bytes=20 fetch_kib_raw=1 write_kib_raw=1\n"
                 "kernel=bwd_dq_kernel source_sha=0000000000000000 fetch_bytes=5 write_bytes=5 fetch_kib_raw=1 write_kib_raw=1\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("bwd_dkdv_kernel") == 120
    assert bench.measured_traffic("bwd_dq_kernel") is None  # measured on another source
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("bwd_dkdv_kernel") is None

