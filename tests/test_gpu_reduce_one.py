"""Calls whose rows each have a single partition (max_num_partitions = 1),
which the reduce serves with its one-partition form.

With one partition the combine's weight is e^(m - m) l / l = 1, so every row
with keys must come out as its partition row bit for bit (f32 output; the
16-bit output as that row rounded to nearest even), a row with no keys as 0
with lse -inf, and out and lse must agree with the oracle: single-query and
multi-token rows (some shorter than the query window), head sizes 64, 128 and
256, the two-call and one-call forms.
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


# dtype, H, KH, D, BS, PS, M
CASES = [
    ("bf16", 32, 8, 128, 16, 512, 1),   # MFMA partition kernel
    ("f16", 8, 8, 64, 16, 256, 1),      # vector kernel, 8 rows per wavefront in the reduce
    ("f16", 4, 4, 256, 32, 512, 1),     # one row per wavefront
    ("bf16", 16, 4, 128, 16, 256, 3),   # three query tokens
    ("bf16", 16, 2, 256, 32, 256, 2),
]


def inputs(c, seed):
    dtype, H, KH, D, BS, PS, M = c
    lens = [0, 1, M - 1, BS - 1, BS, PS // 2 + 3, PS - 1, PS]
    lens = [max(0, x) for x in lens]
    cfg = W.DecodeConfig(f"one_partition_{dtype}", num_seqs=len(lens), num_heads=H,
                         num_kv_heads=KH, head_size=D, block_size=BS, partition_size=PS,
                         dtype=dtype, len_lo=0, len_hi=PS, num_queries=M)
    inp = W.make_inputs(cfg, seed=seed, lens=lens, extra_blocks=2)
    W.poison_unused(inp)
    if M == 1:
        inp["query"] = inp["query"][:, 0] if inp["query"].dim() == 4 else inp["query"]
    return cfg, inp


def keys_seen(lens, M):
    """[S, M] keys each query token sees (its causal prefix)."""
    return np.array([[R.causal_len(L, M, m) for m in range(M)] for L in lens])


@pytest.mark.parametrize("c", CASES, ids=lambda c: "_".join(map(str, c)))
def test_single_partition_rows_are_the_partition_rows(c):
    dtype, H, KH, D, BS, PS, M = c
    cfg, inp = inputs(c, seed=81)
    d = U.to_device(inp)
    q = d["query"]
    S = q.shape[0]
    shp = (S, M, H) if M > 1 else (S, H)
    tmp = torch.full((*shp, 1, D), float("nan"), device=U.DEV)
    es = torch.full((*shp, 1), float("nan"), device=U.DEV)
    ml = torch.full((*shp, 1), float("nan"), device=U.DEV)
    out = torch.full((*shp, D), float("nan"), device=U.DEV)
    lse = torch.full(shp, float("nan"), device=U.DEV)
    U.note(f"one partition {c}")
    args = (q, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"], PS)
    pa.paged_attn_v2_partition_ex(tmp, es, ml, *args)
    pa.paged_attn_v2_reduce_lse(out, lse, tmp, es, ml, d["seq_lens"], PS)
    # the one-call form with a 16-bit output
    out16 = torch.full((*shp, D), float("nan"), device=U.DEV).to(q.dtype)
    tmp2, es2, ml2 = (torch.full_like(t, float("nan")) for t in (tmp, es, ml))
    lse2 = torch.full(shp, float("nan"), device=U.DEV)
    pa.paged_attn_decode_ex(out16, tmp2, es2, ml2, *args, lse=lse2)
    torch.cuda.synchronize()
    out, lse, tmp, es, ml = (t.cpu() for t in (out, lse, tmp, es, ml))
    out16, lse2 = out16.cpu(), lse2.cpu()

    seen = keys_seen(inp["seq_lens"].tolist(), M).reshape((S, M) if M > 1 else (S,))
    has = torch.from_numpy(seen > 0)
    rows = has[..., None].expand(*shp)          # rows with keys
    assert torch.equal(out[rows], tmp[rows][:, 0]), c
    assert torch.all(out[~rows] == 0), c
    assert torch.equal(out16[rows], tmp[rows][:, 0].to(q.dtype)), c
    assert torch.all(out16[~rows] == 0), c
    assert torch.all(lse[~rows] == -math.inf) and torch.all(lse2[~rows] == -math.inf), c
    assert torch.equal(lse, lse2), c
    # the oracle
    ref, ref_lse = oracle.attention_lse(inp["query"], inp["key_cache"], inp["value_cache"],
                                        inp["block_tables"], inp["seq_lens"], inp["scale"])
    U.assert_close(f"one partition {c} out", out, ref)
    r = rows.numpy()
    U.assert_close(f"one partition {c} lse", lse.double().numpy()[r], ref_lse[r])
    U.assert_close(f"one partition {c} lse vs stats", lse[rows],
                   (ml[rows][:, 0].double() + torch.log(es[rows][:, 0].double())).numpy())
