"""Several query tokens per sequence (the last M positions, causal) through the C ABI.

Every output row and every partition intermediate is compared with the
oracle's multi-token mode (which is pinned to the single-query oracle on each
row's causal prefix): several (group, M) mixes that fill one MFMA column tile
(G * M <= 16), two column tiles (17 to 32 columns, head sizes up to 128) and
wider windows that run in several launches over the pages (one of them ending
part-way through a token's heads), 8-bit caches, lengths shorter than M, equal
to M and at block / partition edges, the two-call and one-call forms, and
M = 1 against the single-query entry points bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import workloads as W
from tests import rows as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built():
    pa.ensure_built()
    oracle.build(force=False)


def run_mq(d, PS, P, split=False, out_dtype=torch.float32):
    """The two calls (paged_attn_v2_partition_mq + paged_attn_v2_reduce_mq: `tmp`,
    `es`, `ml` and their output); with split=False also paged_attn_decode_mq on
    its own workspace, whose output is `out` (the two calls' is `out_split`)."""
    q = d["query"]
    S, M, H, D = q.shape

    def ws():
        return (torch.full((S, M, H, P, D), float("nan"), device=U.DEV),
                torch.full((S, M, H, P), float("nan"), device=U.DEV),
                torch.full((S, M, H, P), float("nan"), device=U.DEV))

    args = (q, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"], PS)
    sc = dict(k_scale=d.get("k_scale", 1.0), v_scale=d.get("v_scale", 1.0))
    tmp, es, ml = ws()
    out_s = torch.full((S, M, H, D), float("nan"), device=U.DEV).to(out_dtype)
    pa.paged_attn_v2_partition_mq(tmp, es, ml, *args, **sc)
    pa.paged_attn_v2_reduce_mq(out_s, tmp, es, ml, d["seq_lens"], PS)
    res = dict(tmp=tmp, es=es, ml=ml, out=out_s)
    if not split:
        out = torch.full((S, M, H, D), float("nan"), device=U.DEV).to(out_dtype)
        pa.paged_attn_decode_mq(out, *ws(), *args, **sc)
        res.update(out=out, out_split=out_s)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in res.items()}


def check(inp, res, PS, P, label):
    a = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
         inp["seq_lens"], inp["scale"])
    sc = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    ref = oracle.attention(*a, **sc)
    U.assert_close(f"{label} out", res["out"].float(), ref)
    if "out_split" in res:
        U.assert_close(f"{label} out (two calls)", res["out_split"].float(), ref)
    tmp, es, ml = oracle.partition_stats(*a, P, PS, **sc)
    M = inp["query"].shape[1]
    for s, L in enumerate(inp["seq_lens"].tolist()):
        for m in range(M):
            n = -(-R.causal_len(L, M, m) // PS)
            if n:
                U.assert_close(f"{label} ml s={s} m={m}", res["ml"][s, m, :, :n], ml[s, m, :, :n])
                U.assert_close(f"{label} es s={s} m={m}", res["es"][s, m, :, :n], es[s, m, :, :n])
                U.assert_close(f"{label} tmp s={s} m={m}", res["tmp"][s, m, :, :n],
                               tmp[s, m, :, :n])
            assert torch.all(res["ml"][s, m, :, n:] == -math.inf), (label, s, m)
            assert torch.all(res["es"][s, m, :, n:] == 0), (label, s, m)


def mq_geom(dtype, H, KH, D, BS, PS, M, lens, q_dtype=None, **kw):
    return W.DecodeConfig(f"mq_{dtype}", num_seqs=len(lens), num_heads=H, num_kv_heads=KH,
                          head_size=D, block_size=BS, partition_size=PS, dtype=dtype,
                          q_dtype=q_dtype, len_lo=0, len_hi=max(max(lens), 1), num_queries=M,
                          **kw)


# dtype, H, KH, D, BS, PS, M
CASES = [
    ("bf16", 32, 8, 128, 16, 64, 4),    # G=4 x M=4: a full column tile
    ("bf16", 64, 8, 128, 16, 64, 2),    # G=8 x M=2
    ("f16", 8, 8, 128, 16, 64, 8),      # G=1 x M=8
    ("bf16", 16, 8, 64, 32, 64, 3),     # G=2 x M=3 (6 columns), D=64, BS=32
    ("f16", 16, 2, 256, 16, 128, 2),    # G=8 x M=2, D=256
    ("fp8", 32, 8, 128, 16, 64, 4),     # 8-bit cache, G=4 x M=4
    ("fp8", 8, 4, 256, 32, 64, 5),      # 8-bit cache, G=2 x M=5, D=256, BS=32
    # 17 to 32 columns, head size <= 128: one launch with two column tiles
    ("bf16", 64, 8, 128, 16, 64, 4),    # G=8 x M=4: 32 columns
    ("f16", 32, 8, 128, 16, 64, 7),     # G=4 x M=7: 28 columns
    ("bf16", 40, 8, 64, 16, 64, 5),     # G=5 x M=5: 25 columns, D=64
    ("fp8", 32, 8, 128, 16, 64, 6),     # 8-bit cache, G=4 x M=6: 24 columns
    # wider: several launches over the pages
    ("bf16", 16, 1, 64, 32, 64, 3),     # G=16 x M=3: launches of 32 and 16 columns
    ("bf16", 48, 8, 128, 16, 64, 6),    # G=6 x M=6: 32 + 4, token 5's heads split
    ("f16", 32, 2, 256, 16, 128, 3),    # G=16 x M=3, D=256: three 16-column launches
    ("fp8", 64, 2, 128, 32, 64, 2),     # 8-bit cache, G=32 x M=2: two 32-column launches
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: "_".join(map(str, c)))
@pytest.mark.parametrize("split", [False, True], ids=["decode", "split"])
def test_multi_token_parity(c, split):
    dtype, H, KH, D, BS, PS, M = c
    lens = [0, 1, M - 1, M, M + 1, BS, PS - 1, PS, PS + M - 1, 2 * PS + 3, 3 * PS]
    kw = dict(q_dtype="bf16" if H // KH != 1 else "f16", k_scale=0.03, v_scale=0.045) \
        if dtype == "fp8" else {}
    cfg = mq_geom(dtype, H, KH, D, BS, PS, M, lens, **kw)
    inp = W.make_inputs(cfg, seed=51, lens=lens, extra_blocks=3)
    W.poison_unused(inp)
    P = cfg.max_num_partitions
    U.note(f"multi-token {c} split={split}")
    res = run_mq(U.to_device(inp), PS, P, split=split)
    check(inp, res, PS, P, f"mq {c}")
    assert torch.all(res["out"][0] == 0)  # a sequence with no keys


@pytest.mark.parametrize("name", ["gqa_bf16_g4", "longctx_bf16_g8"])
def test_multi_token_reduced_workload(name):
    """The GQA / long-context shapes with 4 (resp. 2) draft tokens per sequence."""
    M = 4 if name == "gqa_bf16_g4" else 2
    cfg = U.small_config(name).replace(num_queries=M)
    inp = W.make_inputs(cfg, seed=13)
    W.poison_unused(inp)
    U.note(f"multi-token reduced {name} M={M}")
    P = cfg.max_num_partitions
    res = run_mq(U.to_device(inp), cfg.partition_size, P)
    check(inp, res, cfg.partition_size, P, f"mq {name}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_multi_token_two_partition_spans(dtype):
    """4 heads x 4 tokens (16 columns) over enough units that the host takes
    two-partition spans (66 KiB of parked state per workgroup at head size 128)."""
    S, PS, P, M = 64, 64, 8, 4
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(0, P * PS + 1, size=S)]
    lens[:4] = [0, 3, PS + 1, P * PS]
    kw = dict(q_dtype="bf16", k_scale=0.03, v_scale=0.045) if dtype == "fp8" else {}
    cfg = mq_geom(dtype, 32, 8, 128, 16, PS, M, lens, **kw)
    inp = W.make_inputs(cfg, seed=52, lens=lens, extra_blocks=3)
    W.poison_unused(inp)
    U.note(f"multi-token spans {dtype}")
    res = run_mq(U.to_device(inp), PS, P)
    check(inp, res, PS, P, f"mq spans {dtype}")


@pytest.mark.parametrize("name", ["gqa_bf16_g4", "mha_f16_d128", "gqa_fp8_g4"])
def test_one_query_token_matches_single_query_calls(name):
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=17)
    d = U.to_device(inp)
    U.note(f"mq M=1 vs single {name}")
    single = U.run_decode(d)
    d4 = dict(d, query=d["query"][:, None].contiguous())
    if cfg.group > 16 or cfg.query_dtype == "f32":
        pytest.skip("not an MFMA-path shape")
    res = run_mq(d4, cfg.partition_size, single["P"])
    # the single-query calls use the vector path for G < 4; the MFMA path then
    # differs in rounding only, so compare at tolerance, bitwise where both are MFMA
    if cfg.group >= 4:
        assert torch.equal(res["out"][:, 0], single["out"])
        assert torch.equal(res["es"][:, 0], single["es"])
    else:
        U.assert_close("M=1 vs vector path", res["out"][:, 0], single["out"].double().numpy())


def test_multi_token_rejects_fp32_query():
    cfg = mq_geom("f32", 8, 2, 64, 16, 64, 2, [10, 20])   # the MFMA path needs a 16-bit query
    d = U.to_device(W.make_inputs(cfg, seed=1, lens=[10, 20]))
    with pytest.raises(RuntimeError):
        run_mq(d, 64, 1)


_FULL = {}


@pytest.mark.parametrize("name", W.MQ_ORDER)
@pytest.mark.parametrize("ps", ["config", "planned"])
def test_multi_token_full_size(name, ps):
    """The multi-token workloads at full size, at the configured and at the
    planned partition size, through the one call and the two calls: every
    output row and every used partition's row and statistics against the
    oracle, sentinels exact past each row's causal prefix."""
    cfg = W.CONFIGS[name]
    if name not in _FULL:
        _FULL.clear()
        inp = W.make_inputs(cfg, seed=W.workload_seed(name))
        _FULL[name] = (inp, U.to_device(inp))
    inp, d = _FULL[name]
    if ps == "config":
        PS, P = cfg.partition_size, cfg.max_num_partitions
    else:
        PS = pa.plan_partition_size(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads,
                                    cfg.head_size, cfg.block_size, cfg.max_len,
                                    W.DTYPES[cfg.dtype])
        P = max(1, -(-cfg.max_len // PS))
    U.note(f"multi-token full {name} ps={PS}")
    res = run_mq(d, PS, P)
    assert torch.isfinite(res["out"]).all()
    check(inp, res, PS, P, f"mq full {name} PS={PS}")
