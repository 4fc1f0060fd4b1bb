"""bench.py pieces that need no GPU: the one-GPU guard and the algorithmic work it divides by."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_decode_bytes_of_the_default_workload():
    # 64 x 4096 tokens of 1152-byte rows, 147,456 B of q_lat and 131,072 B of latent output
    # per query, 4 bytes of block table per page
    assert bench.decode_bytes([4096] * 64) == 64 * (1152 * 4096 + 147456 + 131072 + 4 * 64) == 319832064


def test_per_head_decode_bytes():
    # 1536-byte rows (256 + 16 x 32 bf16), 9,216 B of q_lat, 8,192 B of output per query
    assert bench.per_head_decode_bytes([4096] * 64) == 64 * (1536 * 4096 + 9216 + 8192 + 256) == 403783680


def test_prefill_flops_count_visible_pairs():
    class _Shape:
        n_heads, row, d_latent = 128, 576, 512

    class _Case:
        shape = _Shape()
        batch = 1
        cu_q = np.array([0, 2048])
        q_start = np.array([16384])

    pairs = 2048 * 16384 + 2048 * 2049 // 2
    assert bench.prefill_flops(_Case()) == 2.0 * 128 * (576 + 512) * pairs
