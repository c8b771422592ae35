"""Pins of the oracle's multi-token mode (M query tokens per sequence; CPU only).

Reading taken: the M query tokens are a sequence's last M positions; token m
sits at L - M + m and attends to keys t <= L - M + m (the causal rule of the
Flash Attention Metal forward kernel, aligned to the end of the cached
sequence); every later step is per (sequence, query token, head) row.

* each query row equals the single-query oracle run on that row's causal
  prefix (lengths computed here from the definition);
* a library routine: torch fp64 softmax/matmul with an explicit causal mask
  over K/V gathered by a permute/reshape route;
* a pure-Python brute force on tiny inputs, including lengths shorter than M;
* partition + combine equals dense; M = 1 equals the single-query mode.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_v2_amd import workloads as W
from tests import rows as R
from tests import dense_views as DV


def mq_cfg(M, dtype="bf16", H=8, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=90, **kw):
    return W.DecodeConfig("mq_tiny", num_seqs=S, num_heads=H, num_kv_heads=KH, head_size=D,
                          block_size=BS, partition_size=PS, dtype=dtype, len_lo=lo, len_hi=hi,
                          num_queries=M, **kw)


def run(inp, fn=oracle.attention, *extra):
    return fn(inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
              inp["seq_lens"], inp["scale"], *extra, k_scale=inp["k_scale"],
              v_scale=inp["v_scale"])


def rel_close(a, b, rtol=1e-10, atol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= atol + rtol * np.abs(b))


@pytest.mark.parametrize("M,dtype", [(2, "bf16"), (5, "f16"), (4, "fp8")])
def test_rows_equal_single_query_on_causal_prefix(M, dtype):
    kw = dict(q_dtype="bf16", k_scale=0.03, v_scale=0.05) if dtype == "fp8" else {}
    cfg = mq_cfg(M, dtype, S=4, **kw)
    inp = W.make_inputs(cfg, seed=2, lens=[1, M, 33, 90])
    got = run(inp)
    for s in range(4):
        L = int(inp["seq_lens"][s])
        for m in range(M):
            e = max(0, min(L, L - M + m + 1))
            one = oracle.attention(inp["query"][s:s + 1, m], inp["key_cache"], inp["value_cache"],
                                   inp["block_tables"][s:s + 1],
                                   torch.tensor([e], dtype=torch.int32), inp["scale"],
                                   k_scale=inp["k_scale"], v_scale=inp["v_scale"])
            assert np.array_equal(got[s, m], one[0]), (s, m)


def library_causal(inp):
    q = inp["query"].to(torch.float64)
    S, M, H, D = q.shape
    KH = inp["key_cache"].shape[1]
    G = H // KH
    out = torch.zeros(S, M, H, D, dtype=torch.float64)
    for s in range(S):
        K, V = DV.gathered(inp, s)
        L = K.shape[0]
        if L == 0:
            continue
        Kh = K.repeat_interleave(G, dim=1).permute(1, 0, 2)  # [H, L, D]
        Vh = V.repeat_interleave(G, dim=1).permute(1, 0, 2)
        scores = torch.matmul(q[s].permute(1, 0, 2), Kh.transpose(1, 2)) * float(inp["scale"])
        pos = torch.arange(L)[None, :]
        qpos = (L - M + torch.arange(M))[:, None]
        scores = scores.masked_fill((pos > qpos)[None], -math.inf)  # [H, M, L]
        w = torch.softmax(scores, dim=-1).nan_to_num(0.0)           # rows with no keys -> 0
        out[s] = torch.matmul(w, Vh).permute(1, 0, 2)
    return out


@pytest.mark.parametrize("M,G", [(3, 4), (8, 1), (2, 8)])
def test_library_routine_causal(M, G):
    cfg = mq_cfg(M, "bf16", H=2 * G, KH=2, D=64, BS=16, S=4)
    inp = W.make_inputs(cfg, seed=5, lens=[M - 1, M, 47, 90])
    got = run(inp)
    ref = library_causal(inp).numpy()
    assert rel_close(got, ref)


def test_brute_force_tiny():
    cfg = mq_cfg(3, "f32", H=2, KH=1, D=8, BS=4, S=3, lo=0, hi=9)
    inp = W.make_inputs(cfg, seed=7, lens=[2, 3, 9])
    got = run(inp)
    q = inp["query"].to(torch.float64).tolist()
    kc = inp["key_cache"].to(torch.float64).tolist()
    vc = inp["value_cache"].to(torch.float64).tolist()
    bt = inp["block_tables"].tolist()
    BS, x = 4, 4
    for s, L in enumerate(inp["seq_lens"].tolist()):
        for m in range(3):
            for h in range(2):
                toks = [(bt[s][t // BS], t % BS) for t in range(L) if t <= L - 3 + m]
                if not toks:
                    assert np.all(got[s, m, h] == 0)
                    continue
                sc = [inp["scale"] * math.fsum(q[s][m][h][d] * kc[b][0][d // x][o][d % x]
                                               for d in range(8)) for b, o in toks]
                mx = max(sc)
                w = [math.exp(a - mx) for a in sc]
                z = math.fsum(w)
                want = [math.fsum(wi * vc[b][0][d][o] for wi, (b, o) in zip(w, toks)) / z
                        for d in range(8)]
                assert rel_close(got[s, m, h], want, rtol=1e-12, atol=1e-13), (s, m, h)


@pytest.mark.parametrize("PS", [16, 32, 64])
def test_partition_combine_equals_dense(PS):
    M = 4
    cfg = mq_cfg(M, "bf16", PS=PS, S=3)
    inp = W.make_inputs(cfg, seed=4, lens=[3, 40, 90])
    P = -(-90 // PS)
    tmp, es, ml = run(inp, oracle.partition_stats, P, PS)
    assert tmp.shape == (3, M, 8, P, 64)
    cmb = oracle.combine(tmp, es, ml, inp["seq_lens"], PS)
    assert rel_close(cmb, run(inp), rtol=1e-12, atol=1e-14)
    # sentinels exactly where a query row's causal prefix ends
    for s, L in enumerate(inp["seq_lens"].tolist()):
        for m in range(M):
            n = -(-R.causal_len(L, M, m) // PS)
            assert np.all(ml[s, m, :, n:] == -np.inf) and np.all(es[s, m, :, n:] == 0)
            assert np.all(np.isfinite(ml[s, m, :, :n]))


def test_single_query_mode_is_m_equal_1():
    cfg = mq_cfg(1, "bf16", S=3)
    inp = W.make_inputs(cfg, seed=9, lens=[1, 50, 90])
    a = run(inp)
    q4 = inp["query"][:, None]  # [S, 1, H, D]
    b = oracle.attention(q4, inp["key_cache"], inp["value_cache"], inp["block_tables"],
                         inp["seq_lens"], inp["scale"])
    assert np.array_equal(a, b[:, 0])
