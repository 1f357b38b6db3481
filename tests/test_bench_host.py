"""bench.py host logic (CPU only): the one-GPU contract and the flop count of a call."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr and not r.stdout.strip()


def test_attention_flops_of_the_540p_call():
    # 6120 queries x (5 x 6120) keys x 128 dims x 24 heads, a multiply and an add for each of the
    # two products Q.K^T and P.V
    assert bench.attn_flops(6120, 24, 128, 5 * 6120) == 2 * 2 * 6120 * 30600 * 128 * 24
    assert abs(bench.attn_flops(6120, 24, 128, 5 * 6120) / 1e12 - 2.301) < 1e-3


def test_traffic_is_reported_only_for_the_profiled_source():
    rec = bench.load_traffic("c2")
    assert rec is None or rec > 0
    assert bench.load_traffic("no_such_workload") is None
