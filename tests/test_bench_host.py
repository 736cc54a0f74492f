"""Host logic of bench.py (no GPU): algorithmic byte counts against the per-token figures worked out from the
problem statement, the counter-traffic guard, and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

T, H, K, E = 65536, 2048, 3, 2


def test_training_step_bytes():
    # forward: B, C, xv read (3 x 4 KiB) and y written (4 KiB) per token, plus the 12 KiB weight
    assert bench.algo_bytes_fwd(T, H, K, E) == T * 16384 + 12288 == 1_073_754_112
    # backward: dy, B, C, xv read and dB, dC, dxv written (7 x 4 KiB) per token, the weight, fp32 dW (24 KiB)
    assert bench.algo_bytes_bwd(T, H, K, E) == T * 28672 + 12288 + 24576 == 1_879_085_056
    assert bench.algo_bytes_fwd(T, H, K, E) + bench.algo_bytes_bwd(T, H, K, E) == 2_952_839_168


def test_small_call_bytes():
    # decode: per sequence 12 KiB in_proj + 4 KiB y + 2 x 12 KiB state (read and written), weight, slot ids
    assert bench.algo_bytes_decode(256, H, K, E) == 256 * (12288 + 4096 + 2 * 12288) + 12288 + 4 * 256
    # verify: per draft token in_proj, y and a 12 KiB tape entry; per sequence the state read
    assert bench.algo_bytes_verify(64, 8, H, K, E) == 512 * (12288 + 4096 + 12288) + 64 * 12288 + 12288 + 256
    # ragged prefill: per token in_proj + y, per sequence the state read and written, offsets and slot ids
    assert bench.algo_bytes_prefill(1000, 8, H, K, E) == 1000 * 16384 + 8 * 2 * 12288 + 12288 + 4 * 17


def test_traffic_only_for_the_measured_sources(monkeypatch):
    path = os.path.join(ROOT, "profiles", "backward_T65536_counters.txt")
    vals = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: vals["kernel_source_sha256_16"].strip())
    assert bench.read_traffic(None) == float(vals["hbm_bytes_per_backward_call"])
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_traffic(None) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
