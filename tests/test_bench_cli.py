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
    # 64 x 4096 tokens of 1152-byte rows, 147,456 B of bf16 q_lat and 262,144 B of float32
    # latent output per query, 4 bytes of block table per page
    assert bench.decode_bytes([4096] * 64) == 64 * (1152 * 4096 + 147456 + 262144 + 4 * 64) == 328220672


def test_per_head_decode_bytes():
    # 1536-byte rows (256 + 16 x 32 bf16), 18,432 B of float32 q_lat, 16,384 B of float32 output per query
    assert bench.per_head_decode_bytes([4096] * 64, q_elt=4) == 64 * (1536 * 4096 + 18432 + 16384 + 256) == 404897792


def test_every_workload_has_its_own_metric():
    import argparse

    import synth

    seen = set()
    for cfg, maker in (("c1", synth.config1), ("c2", synth.config2)):
        args = argparse.Namespace(config=cfg, front="none", score="one", prefill_form="absorbed")
        seen.add(bench.metric_name(args, maker(), False))
    args = argparse.Namespace(config="c3", front="none", score="one", prefill_form="absorbed")
    case3 = synth.direct_decode(synth.DSV2, "bf16", [64], seed=0)
    assert bench.metric_name(args, case3, False) == bench.METRIC
    for cfg in ("c4", "c5a"):
        seen.add(bench.metric_name(argparse.Namespace(config=cfg, front="none", score="one",
                                                      prefill_form="absorbed"), case3, False))
    pre = synth.direct_prefill(synth.DSV2, "bf16", [4], [4], seed=0)
    for form in ("absorbed", "materialised"):
        seen.add(bench.metric_name(argparse.Namespace(config="c5b", front="none", score="one", prefill_form=form),
                                   pre, False))
    assert len(seen) == 6 and bench.METRIC not in seen


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
