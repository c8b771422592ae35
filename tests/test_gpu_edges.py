"""Edge cases of the HIP path against the oracle.

Lengths at every block / partition boundary (0, 1, BS-1, BS, BS+1, PS-1, PS,
PS+1, 2PS-1, P*PS), a partition-size sweep (BS, 2BS, 64, 512, >= longest),
every group size the library builds (vector and MFMA paths, every dtype, head
size and block size), guard bytes after every output, NaN in unread memory,
garbage block-table padding, and the empty batch.
"""
import math

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


def geom(dtype, H, KH, D, BS, PS, S, hi):
    return W.DecodeConfig(f"edge_{dtype}_{H}_{KH}_{D}_{BS}", num_seqs=S, num_heads=H,
                          num_kv_heads=KH, head_size=D, block_size=BS, partition_size=PS,
                          dtype=dtype, len_lo=0, len_hi=hi)


EDGE_GEOMS = [
    ("bf16", 32, 8, 128, 16, 512),   # MFMA, G=4
    ("bf16", 64, 8, 128, 16, 512),   # MFMA, G=8
    ("f16", 32, 32, 128, 16, 512),   # vector, G=1
    ("f16", 16, 16, 256, 32, 512),   # vector, G=1, D=256, BS=32
    ("f32", 4, 4, 64, 16, 64),       # vector fp32
    ("bf16", 8, 4, 64, 32, 64),      # vector, G=2, D=64, BS=32
    ("f16", 16, 1, 256, 16, 128),    # MFMA, G=16, D=256
]


@pytest.mark.parametrize("g", EDGE_GEOMS, ids=lambda g: "_".join(map(str, g)))
def test_length_edges(g):
    dtype, H, KH, D, BS, PS = g
    P = 3
    lens = [0, 1, BS - 1, BS, BS + 1, PS - 1, PS, PS + 1, 2 * PS - 1, P * PS]
    cfg = geom(dtype, H, KH, D, BS, PS, len(lens), P * PS)
    inp = W.make_inputs(cfg, seed=31, lens=lens, extra_blocks=4)
    W.poison_unused(inp)
    U.note(f"length edges {g}")
    res = U.run_decode(U.to_device(inp))
    U.check_against_oracle(inp, res, label=f"edges {g}")
    assert torch.all(res["out"][0] == 0)  # empty sequence -> 0, no NaN


@pytest.mark.parametrize("g", [("bf16", 32, 8, 128, 16), ("f16", 32, 32, 128, 16),
                               ("f16", 16, 16, 256, 32), ("f32", 4, 4, 64, 16)],
                         ids=lambda g: "_".join(map(str, g)))
@pytest.mark.parametrize("PS_rule", ["BS", "2BS", "64", "512", "max"])
def test_partition_size_sweep(g, PS_rule):
    dtype, H, KH, D, BS = g
    hi = 1100
    PS = {"BS": BS, "2BS": 2 * BS, "64": 64, "512": 512, "max": 1120}[PS_rule]
    PS = max(PS, BS)
    cfg = geom(dtype, H, KH, D, BS, PS, 4, hi)
    inp = W.make_inputs(cfg, seed=41, lens=[1, 300, 777, 1100])
    W.poison_unused(inp)
    U.note(f"PS sweep {g} PS={PS}")
    res = U.run_decode(U.to_device(inp), PS=PS)
    U.check_against_oracle(inp, res, label=f"PS={PS} {g}")


@pytest.mark.parametrize("dtype,G", [("bf16", 2), ("bf16", 3), ("f16", 5), ("bf16", 6),
                                     ("f16", 7), ("bf16", 12), ("bf16", 16), ("f32", 3),
                                     ("f32", 4), ("f16", 4)])
@pytest.mark.parametrize("D,BS", [(64, 16), (128, 32), (256, 16)])
def test_group_sizes(dtype, G, D, BS):
    KH = 2
    cfg = geom(dtype, G * KH, KH, D, BS, 256, 3, 700)
    inp = W.make_inputs(cfg, seed=G * 100 + D + BS, lens=[5, 256, 700], extra_blocks=2)
    W.poison_unused(inp)
    U.note(f"group {dtype} G={G} D={D} BS={BS}")
    res = U.run_decode(U.to_device(inp))
    U.check_against_oracle(inp, res, label=f"G={G} {dtype} D={D} BS={BS}")


def test_guard_bytes_untouched():
    cfg = geom("bf16", 32, 8, 128, 16, 512, 3, 1500)
    inp = W.make_inputs(cfg, seed=51, lens=[3, 700, 1500])
    d = U.to_device(inp)
    S, H, D, P = 3, 32, 128, cfg.max_num_partitions
    G = 4096
    pat = 12345.5
    tmp_b = torch.full((S * H * P * D + G,), pat, device=U.DEV)
    es_b = torch.full((S * H * P + G,), pat, device=U.DEV)
    ml_b = torch.full((S * H * P + G,), pat, device=U.DEV)
    out_b = torch.full((S * H * D + G,), pat, device=U.DEV)
    tmp = tmp_b[:S * H * P * D].view(S, H, P, D)
    es = es_b[:S * H * P].view(S, H, P)
    ml = ml_b[:S * H * P].view(S, H, P)
    out = out_b[:S * H * D].view(S, H, D)
    U.note("guard bytes")
    pa.paged_attn_decode(out, tmp, es, ml, d["query"], d["key_cache"], d["value_cache"],
                         d["block_tables"], d["seq_lens"], d["scale"], 512)
    torch.cuda.synchronize()
    for b in (tmp_b, es_b, ml_b, out_b):
        assert torch.all(b[-G:] == pat)


def test_block_table_padding_never_read():
    cfg = geom("f16", 16, 8, 128, 16, 256, 3, 900)
    inp = W.make_inputs(cfg, seed=61, lens=[17, 400, 900])
    base = U.run_decode(U.to_device(inp))
    bt = inp["block_tables"].clone()
    bt[bt < 0] = 2_000_000_000  # documented: entries past ceil(L/BS) are never read
    inp["block_tables"] = bt
    U.note("padding garbage")
    res = U.run_decode(U.to_device(inp))
    for k in ("out", "es", "ml"):
        assert torch.equal(base[k], res[k]), k


def test_empty_batch_is_noop():
    q = torch.empty(0, 8, 128, dtype=torch.bfloat16, device=U.DEV)
    kc = torch.zeros(4, 2, 16, 16, 8, dtype=torch.bfloat16, device=U.DEV)
    vc = torch.zeros(4, 2, 128, 16, dtype=torch.bfloat16, device=U.DEV)
    bt = torch.empty(0, 4, dtype=torch.int32, device=U.DEV)
    sl = torch.empty(0, dtype=torch.int32, device=U.DEV)
    tmp = torch.empty(0, 8, 1, 128, device=U.DEV)
    es = torch.empty(0, 8, 1, device=U.DEV)
    ml = torch.empty(0, 8, 1, device=U.DEV)
    out = torch.empty(0, 8, 128, device=U.DEV)
    U.note("empty batch")
    pa.paged_attn_decode(out, tmp, es, ml, q, kc, vc, bt, sl, 0.1, 512)
    torch.cuda.synchronize()


def test_many_empty_partitions():
    """P far above what any sequence uses: every extra unit only writes sentinels."""
    cfg = geom("bf16", 16, 4, 128, 16, 64, 4, 200)
    inp = W.make_inputs(cfg, seed=71, lens=[1, 64, 65, 200])
    U.note("many empty partitions")
    res = U.run_decode(U.to_device(inp), PS=64, P=40)
    U.check_against_oracle(inp, res, label="P=40")


# The largest partition the launchers accept: PS / BS = 256 pages, one page per
# thread of the block-table hoist (and one partition per workgroup), on each
# kernel family; lengths around one and two full partitions.
@pytest.mark.parametrize("dtype,H,KH,D,BS,extra", [
    ("bf16", 32, 8, 128, 16, {}),                                          # MFMA
    ("f16", 16, 16, 128, 32, {}),                                          # vector, BS=32
    ("fp8", 32, 8, 128, 16, dict(q_dtype="bf16", k_scale=0.02, v_scale=0.03)),  # 8-bit MFMA
    ("fp8", 8, 8, 64, 16, dict(q_dtype="f16", k_scale=0.02, v_scale=0.03)),     # 8-bit vector
], ids=["mfma_bf16", "vec_f16_bs32", "mfma_fp8", "vec_fp8"])
def test_max_pages_per_partition(dtype, H, KH, D, BS, extra):
    PS = 256 * BS
    lens = [0, 1, PS - 1, PS, PS + 1, 2 * PS]
    cfg = W.DecodeConfig(f"maxps_{dtype}", num_seqs=len(lens), num_heads=H, num_kv_heads=KH,
                         head_size=D, block_size=BS, partition_size=PS, dtype=dtype, len_lo=0,
                         len_hi=2 * PS, **extra)
    inp = W.make_inputs(cfg, seed=37, lens=lens, extra_blocks=2)
    W.poison_unused(inp)
    assert pa.partition_span(len(lens), H, KH, D, BS, 2, PS, W.DTYPES[dtype]) == 1
    U.note(f"max pages per partition {dtype} PS={PS}")
    res = U.run_decode(U.to_device(inp))
    U.check_against_oracle(inp, res, label=f"max PS {dtype}")
