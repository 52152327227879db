"""Host-side checks of bench.py's measurement contract (no GPU): the one-GPU
refusal, the traffic figure's tie to the kernel source it was measured on, and
the algorithmic FLOP and byte counts against their closed forms."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_is_read_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    t = bench.read_traffic()
    assert t is not None and t > 3.0e8          # the committed summary matches the source
    other = tmp_path / "gemm_q4.hip"
    other.write_bytes(open(bench.KERNEL_SRC, "rb").read() + b"\n// changed\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(other))
    assert bench.read_traffic() is None         # any edit of the kernel voids the figure


def test_algorithmic_counts():
    # 2 (T k + T) 3 H I flops: gate, up and down for every routed row and shared row
    assert bench.layer_flops(512, 2048, 512, 8, 512) == pytest.approx(28.99e9, rel=1e-3)
    assert bench.layer_flops(2048, 2048, 512, 8, 512) == pytest.approx(115.96e9, rel=1e-4)
    # packed bytes per weight: half a byte of code plus a bf16 scale and bias per 64
    assert bench.BYTES_PER_WEIGHT * 64 == 36
    assert int(2 * 512 * 2048 * bench.BYTES_PER_WEIGHT) == 1_179_648   # gate + up per expert
    assert int(3 * 512 * 2048 * bench.BYTES_PER_WEIGHT) == 1_769_472   # one expert
