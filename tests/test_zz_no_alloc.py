"""The allocation-free one-call decode (paged_attn_decode_noalloc): the span
entries live in the library's static per-GPU scratch instead of a caller
workspace. It runs the kernels of paged_attn_decode_ex, so on the same inputs
its output and row log-sum-exp must equal that call's bit for bit (and the
oracle's within the tolerance). Two calls in a row, the second smaller, show
that nothing left in the scratch by a call changes the next one; a call whose
workspace would not fit is rejected on the host."""
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


def batch(name, dtype, S, H, KH, D, BS, PS, M, lo, hi, seed, **kw):
    cfg = W.DecodeConfig(name, num_seqs=S, num_heads=H, num_kv_heads=KH, head_size=D,
                         block_size=BS, partition_size=PS, dtype=dtype, len_lo=lo, len_hi=hi,
                         num_queries=M, **kw)
    inp = W.make_inputs(cfg, seed=seed, extra_blocks=2)
    W.poison_unused(inp)
    if M == 1 and inp["query"].dim() == 4:
        inp["query"] = inp["query"][:, 0]
    return cfg, inp


def both(cfg, inp, slopes=None):
    """(out, lse) of paged_attn_decode_noalloc, then of paged_attn_decode_ex on a
    NaN-filled caller workspace; host copies."""
    d = U.to_device(inp)
    q = d["query"]
    P = cfg.max_num_partitions
    lead = tuple(q.shape[:-1])
    args = (q, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"],
            cfg.partition_size)
    sc = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"],
              alibi_slopes=slopes.to(U.DEV) if slopes is not None else None)
    out_n = torch.full(q.shape, float("nan"), device=U.DEV)
    lse_n = torch.full(lead, float("nan"), device=U.DEV)
    pa.paged_attn_decode_noalloc(out_n, *args, P, lse=lse_n, **sc)
    ws = (torch.full(lead + (P, q.shape[-1]), float("nan"), device=U.DEV),
          torch.full(lead + (P,), float("nan"), device=U.DEV),
          torch.full(lead + (P,), float("nan"), device=U.DEV))
    out_e = torch.full(q.shape, float("nan"), device=U.DEV)
    lse_e = torch.full(lead, float("nan"), device=U.DEV)
    pa.paged_attn_decode_ex(out_e, *ws, *args, lse=lse_e, **sc)
    torch.cuda.synchronize()
    return out_n.cpu(), lse_n.cpu(), out_e.cpu(), lse_e.cpu()


def check(cfg, inp, slopes=None, label=""):
    S, H, D = cfg.num_seqs, cfg.num_heads, cfg.head_size
    plan = pa.decode_plan(S, cfg.num_queries, H, cfg.num_kv_heads, D, cfg.block_size,
                          cfg.max_num_partitions, cfg.partition_size,
                          W.DTYPES[cfg.query_dtype], W.DTYPES[cfg.dtype])
    U.note(f"no-alloc {label} S={S} plan={plan}")
    out_n, lse_n, out_e, lse_e = both(cfg, inp, slopes)
    assert torch.equal(out_n.view(torch.int32), out_e.view(torch.int32)), label
    assert torch.equal(lse_n.view(torch.int32), lse_e.view(torch.int32)), label
    a = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
         inp["seq_lens"], inp["scale"])
    ref, ref_lse = oracle.attention_lse(*a, k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                                        alibi_slopes=slopes)
    U.assert_close(f"no-alloc {label} out", out_n, ref)
    got = lse_n.double().numpy()
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got), empty)
    U.assert_close(f"no-alloc {label} lse", got[~empty], ref_lse[~empty])
    return plan


def test_two_calls_in_a_row_second_smaller():
    # span entries per row > 1: the scratch holds them between the two kernels
    big_cfg, big = batch("noalloc_big", "bf16", 64, 32, 8, 128, 16, 512, 1, 1, 8192, seed=301)
    small_cfg, small = batch("noalloc_small", "bf16", 6, 32, 8, 128, 16, 512, 1, 1, 3000,
                             seed=302)
    p1 = check(big_cfg, big, label="first (larger)")
    p2 = check(small_cfg, small, label="second (smaller)")
    assert p1["entries"] > 1 and p2["entries"] > 1, (p1, p2)


def test_multi_token_alibi_fp8_calls():
    cfg, inp = batch("noalloc_mq", "bf16", 16, 32, 8, 128, 16, 256, 4, 0, 3000, seed=303)
    plan = check(cfg, inp, W.alibi_slopes(32), label="4 query tokens, ALiBi")
    cfg, inp = batch("noalloc_fp8", "fp8", 12, 16, 4, 128, 16, 512, 1, 1, 5000, seed=304,
                     q_dtype="f16", k_scale=0.02, v_scale=0.03)
    check(cfg, inp, label="8-bit cache")
    # one span per row: the scratch is not touched, results still equal
    cfg, inp = batch("noalloc_one", "f16", 40, 16, 16, 256, 32, 4096, 1, 1, 4000, seed=305)
    check(cfg, inp, label="one span per row")


def test_workspace_beyond_the_scratch_is_rejected():
    """4096 sequences x 64 heads x 64 partitions of 512 tokens would need far
    more than 32 MiB of span entries: PA_ERR_UNSUPPORTED, nothing enqueued."""
    S, H, KH, D, BS, P = 4096, 64, 64, 128, 16, 64
    q = torch.zeros(S, H, D, dtype=torch.bfloat16, device=U.DEV)
    kc = torch.zeros(2, KH, D // 8, BS, 8, dtype=torch.bfloat16, device=U.DEV)
    vc = torch.zeros(2, KH, D, BS, dtype=torch.bfloat16, device=U.DEV)
    bt = torch.zeros(S, P * 512 // BS, dtype=torch.int32, device=U.DEV)
    sl = torch.ones(S, dtype=torch.int32, device=U.DEV)
    out = torch.zeros(S, H, D, device=U.DEV)
    plan = pa.decode_plan(S, 1, H, KH, D, BS, P, 512, torch.bfloat16, torch.bfloat16)
    assert S * H * plan["entries"] * (D + 2) * 4 > 32 << 20, plan
    with pytest.raises(RuntimeError, match="scratch"):
        pa.paged_attn_decode_noalloc(out, q, kc, vc, bt, sl, 0.1, 512, P)
    torch.cuda.synchronize()
