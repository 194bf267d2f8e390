"""bench.py on the host: the byte accounting and the one-GPU contract (no GPU needed)."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_touched_bytes_formula():
    # T = 2rd + 2 ffn r + 4 ffn + (m + 1) count 2d + 4 count + 2d + 4d + 8 count
    d, r, ffn, c = 7168, 1024, 28672, 2867
    want = 2 * r * d + 2 * ffn * r + 4 * ffn + 2 * c * 2 * d + 4 * c + 2 * d + 4 * d + 8 * c
    assert bench.touched_bytes("relu", d, r, ffn, c) == want
    assert bench.touched_bytes("reglu", d, r, ffn, c) == want + c * 2 * d
    assert bench.touched_bytes("swiglu", d, r, ffn, c) == bench.touched_bytes("reglu", d, r, ffn, c)
    assert bench.dense_bytes("relu", d, ffn) == 2 * ffn * 2 * d + 4 * ffn + 6 * d
