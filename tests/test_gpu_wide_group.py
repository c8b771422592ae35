"""Query groups wider than one MFMA column tile (G > 16 query heads per kv
head, e.g. multi-query attention with one kv head) through the single-query
entry points.

A (sequence, kv head) unit has G columns; the MFMA kernel takes up to 32 of
them in one launch with two column tiles (head sizes up to 128) and runs wider
groups, and head size 256, as several launches over the same pages, each
writing its own heads' rows. Every output row, row log-sum-exp and partition
intermediate is compared with the oracle: two-tile launches (G = 20, 24, 32),
several launches (G = 64; G = 32 at head size 256; G = 48 in launches of 32
and 16), 8-bit caches, ALiBi, the one-call and two-call forms, and the
single-query call against the multi-token call with M = 1 bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built():
    pa.ensure_built()
    oracle.build(force=False)


def geom(dtype, H, KH, D, BS, PS, lens, **kw):
    return W.DecodeConfig(f"wide_group_{dtype}", num_seqs=len(lens), num_heads=H,
                          num_kv_heads=KH, head_size=D, block_size=BS, partition_size=PS,
                          dtype=dtype, len_lo=0, len_hi=max(max(lens), 1), **kw)


FP8 = dict(q_dtype="bf16", k_scale=0.02, v_scale=0.03)
# label, (dtype, H, KH, D, BS, PS), extra config
CASES = [
    ("g32_bf16_d128", ("bf16", 32, 1, 128, 16, 256), {}),     # one two-tile launch
    ("g24_f16_d64_bs32", ("f16", 48, 2, 64, 32, 128), {}),    # 24 columns
    ("g20_fp8_d128", ("fp8", 40, 2, 128, 16, 256), FP8),      # 8-bit cache, 20 columns
    ("g64_bf16_d128", ("bf16", 64, 1, 128, 16, 256), {}),     # two 32-column launches
    ("g48_bf16_d64", ("bf16", 96, 2, 64, 16, 128), {}),       # launches of 32 and 16
    ("g32_f16_d256", ("f16", 64, 2, 256, 16, 256), {}),       # two 16-column launches
    ("g32_fp8_d256_bs32", ("fp8", 32, 1, 256, 32, 256), FP8),  # 8-bit, 16-column launches
]
BY_LABEL = {c[0]: c for c in CASES}


def case(label, seed):
    _, g, extra = BY_LABEL[label]
    PS, BS = g[5], g[4]
    lens = [0, 1, BS - 1, PS, PS + 1, 3 * PS - 5]
    cfg = geom(*g, lens, **extra)
    inp = W.make_inputs(cfg, seed=seed, lens=lens, extra_blocks=3)
    W.poison_unused(inp)
    return cfg, inp, PS, cfg.max_num_partitions


def run(d, PS, P, split, slopes=None):
    """The two calls (paged_attn_v2_partition_ex + paged_attn_v2_reduce_lse: `tmp`,
    `es`, `ml`, their output and lse); unless split, also paged_attn_decode_ex on
    its own workspace, whose output and lse are `out` and `lse`."""
    q = d["query"]
    S, H, D = q.shape

    def ws():
        return (torch.full((S, H, P, D), float("nan"), device=U.DEV),
                torch.full((S, H, P), float("nan"), device=U.DEV),
                torch.full((S, H, P), float("nan"), device=U.DEV))

    args = (q, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"], PS)
    sc = dict(k_scale=d.get("k_scale", 1.0), v_scale=d.get("v_scale", 1.0),
              alibi_slopes=slopes.to(U.DEV) if slopes is not None else None)
    tmp, es, ml = ws()
    out_s = torch.full((S, H, D), float("nan"), device=U.DEV)
    lse_s = torch.full((S, H), float("nan"), device=U.DEV)
    pa.paged_attn_v2_partition_ex(tmp, es, ml, *args, **sc)
    pa.paged_attn_v2_reduce_lse(out_s, lse_s, tmp, es, ml, d["seq_lens"], PS)
    res = dict(tmp=tmp, es=es, ml=ml, out=out_s, lse=lse_s)
    if not split:
        out = torch.full((S, H, D), float("nan"), device=U.DEV)
        lse = torch.full((S, H), float("nan"), device=U.DEV)
        pa.paged_attn_decode_ex(out, *ws(), *args, lse=lse, **sc)
        res.update(out=out, lse=lse, out_split=out_s, lse_split=lse_s)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in res.items()}


def check(inp, res, PS, P, label, slopes=None):
    a = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
         inp["seq_lens"], inp["scale"])
    sc = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"], alibi_slopes=slopes)
    ref, ref_lse = oracle.attention_lse(*a, **sc)
    empty = np.isneginf(ref_lse)
    for o, l in (("out", "lse"), ("out_split", "lse_split")):
        if o not in res:
            continue
        U.assert_close(f"{label} {o}", res[o], ref)
        got_lse = res[l].double().numpy()
        assert np.array_equal(np.isneginf(got_lse), empty), f"{label} {l} -inf rows"
        U.assert_close(f"{label} {l}", got_lse[~empty], ref_lse[~empty])
    tmp, es, ml = oracle.partition_stats(*a, P, PS, **sc)
    for s, L in enumerate(inp["seq_lens"].tolist()):
        n = -(-L // PS)
        if n:
            U.assert_close(f"{label} ml s={s}", res["ml"][s][:, :n], ml[s][:, :n])
            U.assert_close(f"{label} es s={s}", res["es"][s][:, :n], es[s][:, :n])
            U.assert_close(f"{label} tmp s={s}", res["tmp"][s][:, :n], tmp[s][:, :n])
        assert torch.all(res["ml"][s][:, n:] == -math.inf), (label, s)
        assert torch.all(res["es"][s][:, n:] == 0), (label, s)


@pytest.mark.parametrize("label", [c[0] for c in CASES])
@pytest.mark.parametrize("split", [False, True], ids=["decode", "split"])
def test_wide_group_matches_oracle(label, split):
    cfg, inp, PS, P = case(label, seed=71)
    U.note(f"wide group {label} split={split}")
    res = run(U.to_device(inp), PS, P, split)
    check(inp, res, PS, P, f"wide group {label}")
    assert torch.all(res["out"][0] == 0)  # a sequence with no keys


@pytest.mark.parametrize("label", ["g32_bf16_d128", "g48_bf16_d64", "g20_fp8_d128"])
def test_wide_group_alibi(label):
    cfg, inp, PS, P = case(label, seed=72)
    slopes = W.alibi_slopes(cfg.num_heads)
    U.note(f"wide group alibi {label}")
    res = run(U.to_device(inp), PS, P, False, slopes)
    check(inp, res, PS, P, f"wide group alibi {label}", slopes)


@pytest.mark.parametrize("label", ["g32_bf16_d128", "g64_bf16_d128", "g32_f16_d256"])
def test_single_query_equals_one_token_window(label):
    """The single-query call and the multi-token call with M = 1 launch the same
    kernels over the same columns: identical bits."""
    cfg, inp, PS, P = case(label, seed=73)
    d = U.to_device(inp)
    U.note(f"wide group M=1 {label}")
    single = run(d, PS, P, False)
    q4 = d["query"][:, None].contiguous()
    S, _, H, D = q4.shape
    def ws():
        return (torch.full((S, 1, H, P, D), float("nan"), device=U.DEV),
                torch.full((S, 1, H, P), float("nan"), device=U.DEV),
                torch.full((S, 1, H, P), float("nan"), device=U.DEV))

    a = (q4, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"], PS)
    out = torch.full((S, 1, H, D), float("nan"), device=U.DEV)
    pa.paged_attn_decode_mq(out, *ws(), *a)           # the one-call form
    tmp, es, ml = ws()
    pa.paged_attn_v2_partition_mq(tmp, es, ml, *a)    # phase 1 alone
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0].cpu(), single["out"])
    assert torch.equal(es[:, 0].cpu(), single["es"])
    assert torch.equal(ml[:, 0].cpu(), single["ml"])
