"""Seeded random configurations through the general entry point.

Each case draws a geometry (dtype pair, head counts, head size, block and
partition size, batch, lengths with empty and partial partitions, query
tokens, ALiBi on or off, output dtype) within what the launchers accept and
runs paged_attn_decode_ex; the output, the row log-sum-exp and every
partition intermediate are compared with the oracle. Sizes stay small so the
oracle finishes in well under a second per case. The cases from N_NARROW to
N_FIRST, and the odd ones after it, draw 16-bit queries with more than 16
(query token, head) columns per kv head: two MFMA column tiles, or several
launches over the pages. The
large-batch cases draw 150-320 short sequences, enough work units that the
launch plan takes spans of several partitions and the largest-first order.
The planned cases run at the partition size the library plans for the batch.
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

N_NARROW = 40
N_FIRST = 56   # cases before this one: narrow below N_NARROW, wide from it
N_CASES = 120  # cases from N_FIRST on alternate: even narrow, odd wide


@pytest.fixture(scope="module", autouse=True)
def built():
    pa.ensure_built()
    oracle.build(force=False)


def draw(i):
    rng = np.random.default_rng(1000 + i)
    wide = i >= N_NARROW if i < N_FIRST else i % 2 == 1
    kv = rng.choice(["f32", "f16", "bf16", "fp8"], p=[0, 0.35, 0.35, 0.3] if wide else
                    [0.15, 0.3, 0.3, 0.25])
    q = kv if kv != "fp8" else str(rng.choice(["f16", "bf16"]))
    D = int(rng.choice([64, 128, 256]))
    BS = int(rng.choice([16, 32]))
    PS = BS * int(rng.choice([1, 2, 3, 4, 8]))
    KH = int(rng.choice([1, 2, 4]))
    if q == "f32":
        G = int(rng.choice([1, 2, 3, 4]))
        M = 1
    elif wide:  # 17 .. ~50 columns per kv head
        G = int(rng.choice([2, 3, 5, 6, 8, 12, 17, 24, 32]))
        M = int(rng.integers(max(1, 17 // G + (17 % G > 0)), max(2, 48 // G) + 1))
    else:
        G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        # up to 16 columns per pass; wider windows run in several passes
        M = 1 if rng.random() < 0.6 else int(rng.integers(2, max(3, 16 // G + 1) + 3))
    S = int(rng.integers(1, 7))
    P = int(rng.integers(1, 6))
    lens = rng.integers(0, P * PS + 1, size=S)
    lens[rng.integers(0, S)] = P * PS  # one full sequence
    extra = dict(q_dtype=q, k_scale=float(rng.uniform(0.01, 0.05)),
                 v_scale=float(rng.uniform(0.01, 0.05))) if kv == "fp8" else {}
    cfg = W.DecodeConfig(f"rand{i}", num_seqs=S, num_heads=G * KH, num_kv_heads=KH, head_size=D,
                         block_size=BS, partition_size=PS, dtype=kv, len_lo=0, len_hi=P * PS,
                         num_queries=M, **extra)
    alibi = rng.random() < 0.4
    out16 = q != "f32" and rng.random() < 0.3
    return cfg, [int(x) for x in lens], alibi, out16


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config(i):
    cfg, lens, alibi, out16 = draw(i)
    inp = W.make_inputs(cfg, seed=2000 + i, lens=lens, extra_blocks=2)
    W.poison_unused(inp)
    d = U.to_device(inp)
    q = d["query"]
    lead = tuple(q.shape[:-1])
    P, PS, D = cfg.max_num_partitions, cfg.partition_size, cfg.head_size
    slopes = W.alibi_slopes(cfg.num_heads) if alibi else None
    tmp = torch.full(lead + (P, D), float("nan"), device=U.DEV)
    es = torch.full(lead + (P,), float("nan"), device=U.DEV)
    ml = torch.full(lead + (P,), float("nan"), device=U.DEV)
    out = torch.full(q.shape, float("nan"), device=U.DEV)
    lse = torch.full(lead, float("nan"), device=U.DEV)
    U.note(f"random case {i}: {cfg} lens={lens} alibi={alibi}")
    call = (q, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"], PS)
    sc = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"],
              alibi_slopes=slopes.to(U.DEV) if alibi else None)
    # the one call (its workspace: a copy of the NaN-filled buffers), then phase
    # 1 alone for the per-partition rows and statistics
    pa.paged_attn_decode_ex(out, tmp.clone(), es.clone(), ml.clone(), *call, lse=lse, **sc)
    if out16:  # the same call with a 16-bit output is the RNE cast of the fp32 one
        o16 = torch.empty(q.shape, dtype=q.dtype, device=U.DEV)
        pa.paged_attn_decode_ex(o16, tmp.clone(), es.clone(), ml.clone(), *call, **sc)
    pa.paged_attn_v2_partition_ex(tmp, es, ml, *call, **sc)
    torch.cuda.synchronize()
    a = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
         inp["seq_lens"], inp["scale"])
    sc = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"], alibi_slopes=slopes)
    ref, ref_lse = oracle.attention_lse(*a, **sc)
    U.assert_close(f"case {i} out", out.cpu(), ref)
    got_lse = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse)), f"case {i} lse -inf"
    fin = ~np.isneginf(ref_lse)
    U.assert_close(f"case {i} lse", got_lse[fin], ref_lse[fin])
    rtmp, res_, rml = oracle.partition_stats(*a, P, PS, **sc)
    M = cfg.num_queries
    gt, ge, gm = tmp.cpu(), es.cpu(), ml.cpu()
    for s, L in enumerate(lens):
        for m in range(M):
            n = -(-R.causal_len(L, M, m) // PS)
            idx = (s, m) if M > 1 else (s,)
            if n:
                U.assert_close(f"case {i} ml {s},{m}", gm[idx][:, :n], rml[idx][:, :n])
                U.assert_close(f"case {i} es {s},{m}", ge[idx][:, :n], res_[idx][:, :n])
                U.assert_close(f"case {i} tmp {s},{m}", gt[idx][:, :n], rtmp[idx][:, :n])
            assert torch.all(gm[idx][:, n:] == -math.inf) and torch.all(ge[idx][:, n:] == 0)
    if out16:
        assert torch.equal(out.to(q.dtype).cpu().view(torch.int16), o16.cpu().view(torch.int16))


N_BATCH_CASES = 24


def draw_batch(i):
    """Larger batches of short sequences: enough units that the launch plan
    takes spans of 2, 4 or 8 partitions (and the largest-first order)."""
    rng = np.random.default_rng(5000 + i)
    kv = str(rng.choice(["f32", "f16", "bf16", "fp8"], p=[0.1, 0.3, 0.35, 0.25]))
    q = kv if kv != "fp8" else str(rng.choice(["f16", "bf16"]))
    D = int(rng.choice([64, 128, 256], p=[0.4, 0.45, 0.15]))
    BS = int(rng.choice([16, 32]))
    PS = BS * int(rng.choice([1, 2, 4]))
    P = int(rng.integers(3, 10))
    KH = int(rng.choice([2, 4, 8]))
    if q == "f32":
        G, M = int(rng.choice([1, 2, 4])), 1
    else:
        G = int(rng.choice([1, 2, 4, 8, 16]))
        M = 1 if rng.random() < 0.5 else int(rng.integers(2, 4))
    while G * KH > 64:
        KH //= 2
    S = int(rng.integers(150, 321))
    lens = [int(x) for x in rng.integers(0, P * PS + 1, size=S)]
    extra = dict(q_dtype=q, k_scale=float(rng.uniform(0.01, 0.05)),
                 v_scale=float(rng.uniform(0.01, 0.05))) if kv == "fp8" else {}
    cfg = W.DecodeConfig(f"batch{i}", num_seqs=S, num_heads=G * KH, num_kv_heads=KH,
                         head_size=D, block_size=BS, partition_size=PS, dtype=kv, len_lo=0,
                         len_hi=P * PS, num_queries=M, **extra)
    return cfg, lens, rng.random() < 0.3


@pytest.mark.parametrize("i", range(N_BATCH_CASES))
def test_random_large_batch(i):
    cfg, lens, alibi = draw_batch(i)
    inp = W.make_inputs(cfg, seed=6000 + i, lens=lens, extra_blocks=2)
    W.poison_unused(inp)
    d = U.to_device(inp)
    q = d["query"]
    lead = tuple(q.shape[:-1])
    P, PS, D, M = cfg.max_num_partitions, cfg.partition_size, cfg.head_size, cfg.num_queries
    slopes = W.alibi_slopes(cfg.num_heads) if alibi else None
    span = (pa.partition_span(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, D, cfg.block_size,
                              P, PS, W.DTYPES[cfg.dtype]) if M == 1 else None)
    tmp = torch.full(lead + (P, D), float("nan"), device=U.DEV)
    es = torch.full(lead + (P,), float("nan"), device=U.DEV)
    ml = torch.full(lead + (P,), float("nan"), device=U.DEV)
    out = torch.full(q.shape, float("nan"), device=U.DEV)
    lse = torch.full(lead, float("nan"), device=U.DEV)
    U.note(f"random batch {i}: {cfg} alibi={alibi} span={span}")
    call = (q, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"], PS)
    sc = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"],
              alibi_slopes=slopes.to(U.DEV) if alibi else None)
    pa.paged_attn_decode_ex(out, tmp.clone(), es.clone(), ml.clone(), *call, lse=lse, **sc)
    pa.paged_attn_v2_partition_ex(tmp, es, ml, *call, **sc)   # phase 1 alone
    torch.cuda.synchronize()
    a = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
         inp["seq_lens"], inp["scale"])
    sc = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"], alibi_slopes=slopes)
    ref, ref_lse = oracle.attention_lse(*a, **sc)
    U.assert_close(f"batch {i} out", out.cpu(), ref)
    got_lse = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse)), f"batch {i} lse -inf"
    fin = ~np.isneginf(ref_lse)
    U.assert_close(f"batch {i} lse", got_lse[fin], ref_lse[fin])
    # statistics of every used partition at once; sentinels past each row's prefix
    rtmp, res_, rml = oracle.partition_stats(*a, P, PS, **sc)
    n = np.array([[-(-R.causal_len(L, M, m) // PS) for m in range(M)] for L in lens])
    used = np.arange(P)[None, None, :] < n[:, :, None]          # [S, M, P]
    used = used.reshape((len(lens),) + ((M,) if M > 1 else ()) + (1, P))
    used = np.broadcast_to(used, tuple(es.shape))
    ge, gm, gt = es.cpu().numpy(), ml.cpu().numpy(), tmp.cpu().numpy()
    U.assert_close(f"batch {i} es", ge[used], np.asarray(res_)[used])
    U.assert_close(f"batch {i} ml", gm[used], np.asarray(rml)[used])
    U.assert_close(f"batch {i} tmp", gt[used], np.asarray(rtmp)[used])
    assert np.all(gm[~used] == -np.inf) and np.all(ge[~used] == 0), f"batch {i} sentinels"


N_PLANNED = 8


@pytest.mark.parametrize("i", range(N_PLANNED))
def test_random_planned_partition_size(i):
    """The partition size paged_attn_plan_partition_size picks for the batch
    (one partition per row for the large batches of short sequences, several
    for the small batches of long ones), through the one-call form: out and lse
    against the oracle."""
    if i < N_PLANNED // 2:
        cfg, lens, alibi = draw_batch(i)
    else:
        rng = np.random.default_rng(7000 + i)
        kv = str(rng.choice(["f16", "bf16", "fp8"]))
        q = kv if kv != "fp8" else "bf16"
        if i < N_PLANNED - 2:   # a few long sequences: many short partitions
            KH, G = int(rng.choice([1, 2])), int(rng.choice([1, 4, 8]))
            S, hi = int(rng.integers(1, 4)), 6000
        else:                   # a dozen: a few partitions of 2048 or 4096 tokens
            KH, G, S, hi = 8, 4, 12, 12000
        lens = [int(x) for x in rng.integers(1, hi + 1, size=S)]
        extra = dict(q_dtype=q, k_scale=0.03, v_scale=0.04) if kv == "fp8" else {}
        cfg = W.DecodeConfig(f"planned{i}", num_seqs=S, num_heads=G * KH, num_kv_heads=KH,
                             head_size=128, block_size=16, partition_size=128, dtype=kv,
                             len_lo=0, len_hi=max(lens), **extra)
        alibi = False
    L = max(lens)
    PS = pa.plan_partition_size(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size,
                                cfg.block_size, L, W.DTYPES[cfg.dtype])
    P = max(1, -(-L // PS))
    inp = W.make_inputs(cfg, seed=8000 + i, lens=lens, extra_blocks=2)
    W.poison_unused(inp)
    d = U.to_device(inp)
    q = d["query"]
    lead = tuple(q.shape[:-1])
    D = cfg.head_size
    slopes = W.alibi_slopes(cfg.num_heads) if alibi else None
    tmp = torch.full(lead + (P, D), float("nan"), device=U.DEV)
    es = torch.full(lead + (P,), float("nan"), device=U.DEV)
    ml = torch.full(lead + (P,), float("nan"), device=U.DEV)
    out = torch.full(q.shape, float("nan"), device=U.DEV)
    lse = torch.full(lead, float("nan"), device=U.DEV)
    U.note(f"planned {i}: {cfg} PS={PS} P={P} alibi={alibi}")
    pa.paged_attn_decode_ex(out, tmp, es, ml, q, d["key_cache"], d["value_cache"],
                            d["block_tables"], d["seq_lens"], d["scale"], PS,
                            k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                            alibi_slopes=slopes.to(U.DEV) if alibi else None, lse=lse)
    torch.cuda.synchronize()
    a = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
         inp["seq_lens"], inp["scale"])
    ref, ref_lse = oracle.attention_lse(*a, k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                                        alibi_slopes=slopes)
    U.assert_close(f"planned {i} out", out.cpu(), ref)
    got_lse = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse)), f"planned {i} lse -inf"
    fin = ~np.isneginf(ref_lse)
    U.assert_close(f"planned {i} lse", got_lse[fin], ref_lse[fin])
