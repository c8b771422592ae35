"""bench.py's accounting and its one-GPU contract, without a GPU."""
import os
import subprocess
import sys

import numpy as np

import bench
from paged_kv_cache_v2_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kv_bytes_and_work_count():
    inp = W.make_inputs(W.CONFIGS["tiny_f32_d64"], seed=1)
    # lengths {37, 100}: 137 tokens, 4 kv heads, K and V rows of 64 fp32 each
    assert bench.kv_bytes(inp) == 137 * 4 * 2 * 64 * 4 == 280_576
    assert bench.qhead_tokens(inp) == 137 * 4


def test_work_count_with_several_query_tokens():
    """Token m of M (the sequence's last positions) sees L - M + m + 1 keys."""
    cfg = W.CONFIGS["gqa_bf16_g4_m4"].replace(num_seqs=3)
    inp = W.make_inputs(cfg, seed=1, lens=[0, 2, 10])
    keys = (0 + 0 + 0 + 0) + (0 + 0 + 1 + 2) + (7 + 8 + 9 + 10)
    assert bench.qhead_tokens(inp) == keys * cfg.num_heads


def test_quantiles():
    v = list(range(100))
    assert bench.quantile(v, 0.5) == 50 and bench.quantile(v, 0.1) == 10
    assert np.isclose(bench.pct(4000.0), 50.0)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
