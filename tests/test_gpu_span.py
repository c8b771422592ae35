"""Workgroups that span several partitions, and the multi-wavefront reduce.

A partition workgroup may own two, four or eight consecutive partitions of
one (sequence, kv head); each partition is still computed and stored on its
own, so every intermediate must match the oracle exactly as for one partition
per workgroup. The shapes below are chosen so that the launch plan takes
spans of two, four and eight (asserted through paged_attn_partition_span) on
every kernel family, with partition counts that leave a shorter last span,
partitions that are not a multiple of four pages (wavefronts cross a
partition edge between two of their pages), and sequence lengths at every
span edge. The reduce cases cover one, two and four wavefronts per row and
more than 64 partitions (a second chunk of statistics).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built():
    pa.ensure_built()
    import oracle
    oracle.build(force=False)


def span_lens(S, BS, PS, P, seed):
    edges = [0, 1, BS - 1, BS, PS - 1, PS, PS + 1, 2 * PS - 1, 2 * PS, 2 * PS + 1, 3 * PS,
             4 * PS - 1, 4 * PS, 4 * PS + 1, 8 * PS - 1, 8 * PS, 8 * PS + 1, P * PS - 1, P * PS]
    edges = [e for e in edges if 0 <= e <= P * PS]
    rng = np.random.default_rng(seed)
    rest = rng.integers(0, P * PS + 1, size=max(0, S - len(edges))).tolist()
    return (edges + rest)[:S]


# dtype, H, KH, D, BS, PS, P, S, span the plan takes on MI355X
SPAN_CASES = [
    ("bf16", 32, 8, 128, 16, 64, 5, 104, 4),   # MFMA G=4, spans of 4 + 1 partitions
    ("bf16", 32, 8, 128, 16, 48, 6, 96, 4),    # MFMA G=4, 3 pages per partition, 4 + 2
    ("bf16", 64, 8, 128, 16, 64, 8, 64, 4),    # MFMA G=8
    ("bf16", 32, 2, 128, 16, 64, 8, 256, 2),   # MFMA G=16: 66 KiB of parked state per span
    ("bf16", 32, 8, 128, 16, 64, 5, 128, 8),   # MFMA G=4, one span over all 5 partitions
    ("bf16", 32, 8, 128, 16, 48, 9, 128, 8),   # MFMA, 3 pages per partition, spans of 8 + 1
    ("f16", 32, 32, 128, 16, 64, 8, 32, 4),    # vector G=1
    ("bf16", 16, 8, 64, 32, 64, 8, 256, 8),    # vector G=2, D=64, BS=32
    ("f32", 8, 8, 64, 16, 64, 4, 128, 2),      # vector fp32
    ("f32", 8, 8, 64, 16, 64, 6, 256, 8),      # vector fp32, one span over all 6 partitions
    ("f16", 16, 16, 256, 32, 64, 4, 64, 4),    # vector D=256, BS=32
    ("fp8", 32, 8, 128, 16, 64, 5, 104, 2),    # MFMA, 8-bit cache, odd P (largest-first order)
    ("fp8", 32, 8, 128, 16, 64, 6, 128, 4),    # MFMA, 8-bit cache, spans of 4 + 2
    ("fp8", 16, 16, 128, 16, 64, 5, 104, 4),   # vector, 8-bit cache, spans of 4 + 1
    ("fp8", 16, 16, 128, 16, 64, 8, 160, 8),   # vector, 8-bit cache, spans of 8
]


def case_config(name, dtype, H, KH, D, BS, PS, P, S):
    fp8 = dict(q_dtype="bf16", k_scale=0.015, v_scale=0.02) if dtype == "fp8" else {}
    return W.DecodeConfig(name, num_seqs=S, num_heads=H, num_kv_heads=KH, head_size=D,
                          block_size=BS, partition_size=PS, dtype=dtype, len_lo=0,
                          len_hi=P * PS, **fp8)


@pytest.mark.parametrize("c", SPAN_CASES, ids=lambda c: "_".join(map(str, c)))
@pytest.mark.parametrize("split", [False, True], ids=["decode", "split"])
def test_multi_partition_span(c, split):
    dtype, H, KH, D, BS, PS, P, S, C = c
    span = pa.partition_span(S, H, KH, D, BS, P, PS, W.DTYPES[dtype])
    assert span == C, f"plan chose span {span}; the case no longer exercises spans of {C}"
    cfg = case_config(f"span_{dtype}", dtype, H, KH, D, BS, PS, P, S)
    lens = span_lens(S, BS, PS, P, seed=S + P)
    inp = W.make_inputs(cfg, seed=41, lens=lens, extra_blocks=3)
    W.poison_unused(inp)
    U.note(f"span case {c} split={split}")
    res = U.run_decode(U.to_device(inp), split=split)
    assert res["P"] == P
    U.check_against_oracle(inp, res, label=f"span {c}")


# dtype, H, KH, D, BS, PS, P, lens: reduce rows over 1, 2 and 4 wavefronts, > 64 partitions
REDUCE_CASES = [
    ("bf16", 16, 4, 128, 16, 16, 130, [2080, 1030, 5]),  # 4 wavefronts per row, 3 chunks
    ("f16", 8, 8, 256, 16, 16, 70, [1120, 1000]),        # D=256: 4 wavefronts, 2 chunks
    ("f32", 4, 4, 64, 16, 16, 20, [320, 17]),            # D=64: 2 wavefronts per row
    ("f32", 4, 4, 64, 16, 16, 12, [192, 17]),            # D=64: one wavefront per row
    ("bf16", 32, 8, 128, 16, 16, 24, [384, 200, 0]),     # 4 wavefronts per row
    ("bf16", 32, 8, 128, 16, 16, 12, [192, 100, 0]),     # 2 wavefronts per row
    ("bf16", 32, 8, 128, 16, 16, 8, [128, 100, 0]),      # one wavefront per row
]


@pytest.mark.parametrize("c", REDUCE_CASES, ids=lambda c: "_".join(map(str, c[:7])))
def test_reduce_row_spread(c):
    dtype, H, KH, D, BS, PS, P, lens = c
    cfg = W.DecodeConfig(f"red_{dtype}", num_seqs=len(lens), num_heads=H, num_kv_heads=KH,
                         head_size=D, block_size=BS, partition_size=PS, dtype=dtype, len_lo=0,
                         len_hi=P * PS)
    inp = W.make_inputs(cfg, seed=43, lens=lens, extra_blocks=2)
    W.poison_unused(inp)
    U.note(f"reduce case {c[:7]}")
    res = U.run_decode(U.to_device(inp), split=True)
    assert res["P"] == P
    U.check_against_oracle(inp, res, label=f"reduce {c[:7]}")


def test_span_plan_keeps_occupancy():
    """A two-partition span's parked state may take the LDS that the kernel's
    register-limited occupancy leaves: 66 KiB for 16 columns at head size 128
    fits the 16-bit MFMA kernel (two workgroups per CU) but not the 8-bit one
    (four per CU), which keeps one partition per workgroup there."""
    args = (256, 32, 2, 128, 16, 8, 512)  # G = 16: one full column tile
    assert pa.partition_span(*args, torch.bfloat16) == 2
    assert pa.partition_span(*args, torch.float8_e4m3fn) == 1
    assert pa.partition_span(256, 32, 8, 128, 16, 8, 512, torch.float8_e4m3fn) == 4  # G = 4


def test_span_results_match_single_partition_workgroups():
    """Same inputs, one and two partitions per workgroup: tmp/statistics identical.

    The two plans differ only in how units are grouped; each partition's
    arithmetic is the same, so the intermediates agree bit for bit. The
    single-partition plan is reached by a small batch of the same sequences."""
    dtype, H, KH, D, BS, PS, P = "bf16", 32, 8, 128, 16, 64, 5
    S_big = 104
    cfg = W.DecodeConfig("span_eq", num_seqs=S_big, num_heads=H, num_kv_heads=KH, head_size=D,
                         block_size=BS, partition_size=PS, dtype=dtype, len_lo=0, len_hi=P * PS)
    lens = span_lens(S_big, BS, PS, P, seed=5)
    inp = W.make_inputs(cfg, seed=47, lens=lens)
    assert pa.partition_span(S_big, H, KH, D, BS, P, PS, torch.bfloat16) >= 2
    assert pa.partition_span(4, H, KH, D, BS, P, PS, torch.bfloat16) == 1
    U.note("span vs single-partition plan")
    big = U.run_decode(U.to_device(inp), split=True)
    small_inp = dict(inp)
    small_inp["query"] = inp["query"][:4]
    small_inp["block_tables"] = inp["block_tables"][:4]
    small_inp["seq_lens"] = inp["seq_lens"][:4]
    small = U.run_decode(U.to_device(small_inp), split=True)
    for k in ("es", "ml"):
        assert torch.equal(small[k], big[k][:4]), k
    n = [-(-int(L) // PS) for L in lens[:4]]
    for s in range(4):
        assert torch.equal(small["tmp"][s, :, :n[s]], big["tmp"][s, :, :n[s]]), s
    assert torch.equal(small["out"], big["out"][:4])


# More (sequence, span) pairs than the largest-first ranking takes (4096): the
# vector and 8-bit kernels fall back to index order. Short ragged sequences
# keep the oracle quick.
@pytest.mark.parametrize("dtype,H,KH", [("f16", 8, 8), ("fp8", 16, 4)], ids=["vec_f16", "mfma_fp8"])
def test_many_pairs_index_order(dtype, H, KH):
    S, D, BS, PS, P = 4200, 64, 16, 32, 2
    assert S * P > 4096
    cfg = case_config(f"pairs_{dtype}", dtype, H, KH, D, BS, PS, P, S)
    lens = np.random.default_rng(9).integers(0, P * PS + 1, size=S).tolist()
    inp = W.make_inputs(cfg, seed=49, lens=lens)
    W.poison_unused(inp)
    U.note(f"many pairs {dtype} S={S}")
    res = U.run_decode(U.to_device(inp), split=True)
    U.check_against_oracle(inp, res, seqs=list(range(0, S, 7)), label=f"pairs {dtype}")
    # every sequence: sentinels exactly past its partitions, finite statistics before
    for s_, L in enumerate(lens):
        n = -(-L // PS)
        assert torch.all(res["ml"][s_, :, n:] == -np.inf) and torch.all(res["es"][s_, :, n:] == 0)
        assert torch.isfinite(res["ml"][s_, :, :n]).all() and torch.all(res["es"][s_, :, :n] >= 1)
