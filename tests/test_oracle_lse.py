"""Pins of the oracle's log-sum-exp output and its merge of two attention states
(CPU only).

Reading taken: a row's log-sum-exp is lse = m + log(l) = log(sum_t exp(s_t))
over the same scaled scores the softmax uses (the Flash Attention Metal forward
kernel stores this per row); a row with no keys has lse = -inf. Two results of
the same query rows over disjoint key sets merge by the V2 reduce's
log-sum-exp combine with each side's (max, exp-sum) folded into its lse.

* lse against torch.logsumexp over scores from the library route (dense,
  causal multi-token, 8-bit caches with scales);
* lse against the partition statistics: M' + log(sum_p e^{m_p - M'} l_p);
* merging the states of two disjoint page ranges equals attention over the
  whole sequence (the cascade / context-parallel split);
* closed forms: two single-key states, the -inf identities, symmetry,
  associativity, a pure-Python brute force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_v2_amd import workloads as W
from tests import dense_views as DV


def cfg(dtype="bf16", M=1, H=8, KH=2, D=64, BS=16, PS=32, S=4, lo=1, hi=90, **kw):
    return W.DecodeConfig("lse_tiny", num_seqs=S, num_heads=H, num_kv_heads=KH, head_size=D,
                          block_size=BS, partition_size=PS, dtype=dtype, len_lo=lo, len_hi=hi,
                          num_queries=M, **kw)


def run_lse(inp, **kw):
    return oracle.attention_lse(inp["query"], inp["key_cache"], inp["value_cache"],
                                inp["block_tables"], inp["seq_lens"], inp["scale"],
                                k_scale=inp["k_scale"], v_scale=inp["v_scale"], **kw)


def library_lse(inp):
    """lse[S, (M,) H] from torch.logsumexp over library-route scores (causal rule
    for several query tokens: token m of M sees keys t <= L - M + m)."""
    q = inp["query"].to(torch.float64)
    q4 = q if q.dim() == 4 else q[:, None]
    S, M, H, D = q4.shape
    G = H // inp["key_cache"].shape[1]
    lse = torch.full((S, M, H), -math.inf, dtype=torch.float64)
    for s in range(S):
        K, _ = DV.gathered(inp, s)
        L = K.shape[0]
        if L == 0:
            continue
        Kh = K.repeat_interleave(G, dim=1).permute(1, 0, 2)  # [H, L, D]
        scores = torch.matmul(q4[s].permute(1, 0, 2), Kh.transpose(1, 2)) * float(inp["scale"])
        pos = torch.arange(L)[None, :]
        qpos = (L - M + torch.arange(M))[:, None]
        scores = scores.masked_fill((pos > qpos)[None], -math.inf)  # [H, M, L]
        lse[s] = torch.logsumexp(scores, dim=-1).permute(1, 0)
    return (lse if q.dim() == 4 else lse[:, 0]).numpy()


def close(a, b, rtol=1e-12, atol=1e-13):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    same_inf = (a == b) & np.isinf(b)
    with np.errstate(invalid="ignore"):
        return np.all(same_inf | (np.abs(a - b) <= atol + rtol * np.abs(b)))


@pytest.mark.parametrize("dtype,M", [("bf16", 1), ("f16", 3), ("f32", 1), ("fp8", 2)])
def test_lse_matches_library_logsumexp(dtype, M):
    kw = dict(q_dtype="bf16", k_scale=0.03, v_scale=0.05) if dtype == "fp8" else {}
    inp = W.make_inputs(cfg(dtype, M, **kw), seed=3, lens=[0, 1, 37, 90])
    out, lse = run_lse(inp)
    want = library_lse(inp)
    assert lse.shape == want.shape
    assert close(lse, want)
    # the output is the plain attention oracle's, unchanged
    base = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                            inp["block_tables"], inp["seq_lens"], inp["scale"],
                            k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    assert np.array_equal(out, base)
    assert np.all(lse[0] == -np.inf) and np.all(out[0] == 0)


@pytest.mark.parametrize("PS", [16, 32, 64])
def test_lse_matches_partition_statistics(PS):
    inp = W.make_inputs(cfg("bf16", 2, PS=PS), seed=6, lens=[2, 17, 64, 90])
    _, lse = run_lse(inp)
    P = -(-90 // PS)
    _, es, ml = oracle.partition_stats(inp["query"], inp["key_cache"], inp["value_cache"],
                                       inp["block_tables"], inp["seq_lens"], inp["scale"], P, PS)
    with np.errstate(divide="ignore", invalid="ignore"):
        Mx = ml.max(axis=-1)
        want = Mx + np.log(np.sum(np.exp(ml - Mx[..., None]) * es, axis=-1))
    assert close(lse, want, rtol=1e-12, atol=1e-12)


def split_pages(inp, cut_pages):
    """Two inputs over disjoint page ranges of every sequence: pages
    [0, cut) and [cut, nb) (cut_pages[s] in pages, clamped to the sequence)."""
    bt, sl = inp["block_tables"], inp["seq_lens"]
    BS = inp["key_cache"].shape[3]
    a, b = dict(inp), dict(inp)
    bt_b = torch.zeros_like(bt)
    la, lb = [], []
    for s, L in enumerate(sl.tolist()):
        c = min(cut_pages[s] * BS, L)
        la.append(c)
        lb.append(L - c)
        rest = bt[s, c // BS:]
        bt_b[s, :rest.numel()] = rest
    a["seq_lens"] = torch.tensor(la, dtype=torch.int32)
    b["seq_lens"] = torch.tensor(lb, dtype=torch.int32)
    b["block_tables"] = bt_b
    return a, b


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 1), ("fp8", 8)])
def test_merge_of_disjoint_splits_is_full_attention(dtype, G):
    kw = dict(q_dtype="f16", k_scale=0.02, v_scale=0.04) if dtype == "fp8" else {}
    inp = W.make_inputs(cfg(dtype, 1, H=2 * G, KH=2, **kw), seed=8, lens=[0, 10, 48, 90])
    full, full_lse = run_lse(inp)
    # cut points: everything on one side, nothing on one side, and mid-sequence
    a, b = split_pages(inp, [1, 0, 1, 3])
    oa, la = run_lse(a)
    ob, lb = run_lse(b)
    out, lse = oracle.merge_states(oa, la, ob, lb)
    assert close(out, full, rtol=1e-12, atol=1e-14)
    assert close(lse, full_lse)


def test_merge_two_single_keys_closed_form():
    rng = np.random.default_rng(1)
    R, D = 32, 8
    v1, v2 = rng.normal(size=(R, D)), rng.normal(size=(R, D))
    s1, s2 = rng.normal(scale=4, size=R), rng.normal(scale=4, size=R)
    s2[:4] = s1[:4]          # equal weights: the plain average
    s2[4:8] = s1[4:8] + 700  # one side dominates beyond exp's range
    out, lse = oracle.merge_states(v1, s1, v2, s2)
    p1 = 1.0 / (1.0 + np.exp(s2 - s1))
    assert close(out, p1[:, None] * v1 + (1 - p1)[:, None] * v2, rtol=1e-13, atol=1e-14)
    assert close(lse, np.logaddexp(s1, s2), rtol=1e-14)
    assert np.allclose(out[:4], (v1[:4] + v2[:4]) / 2, rtol=1e-15, atol=0)
    assert np.array_equal(out[4:8], v2[4:8])


def test_merge_infinite_identities_and_symmetry():
    rng = np.random.default_rng(2)
    R, D = 12, 16
    a, b = rng.normal(size=(R, D)), rng.normal(size=(R, D))
    la, lb = rng.normal(size=R), rng.normal(size=R)
    lb_empty = np.full(R, -np.inf)
    out, lse = oracle.merge_states(a, la, b, lb_empty)
    assert np.array_equal(out, a) and np.array_equal(lse, la)
    out, lse = oracle.merge_states(b, lb_empty, a, la)
    assert np.array_equal(out, a) and np.array_equal(lse, la)
    out, lse = oracle.merge_states(a, lb_empty, b, lb_empty)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    o1, l1 = oracle.merge_states(a, la, b, lb)
    o2, l2 = oracle.merge_states(b, lb, a, la)
    assert close(o1, o2, rtol=1e-15, atol=1e-15) and np.array_equal(l1, l2)


def test_merge_is_associative():
    rng = np.random.default_rng(3)
    R, D = 10, 8
    xs = [rng.normal(size=(R, D)) for _ in range(3)]
    ls = [rng.normal(scale=3, size=R) for _ in range(3)]
    left = oracle.merge_states(*oracle.merge_states(xs[0], ls[0], xs[1], ls[1]), xs[2], ls[2])
    right = oracle.merge_states(xs[0], ls[0], *oracle.merge_states(xs[1], ls[1], xs[2], ls[2]))
    assert close(left[0], right[0], rtol=1e-13, atol=1e-14)
    assert close(left[1], right[1], rtol=1e-14)


def test_lse_brute_force_tiny():
    inp = W.make_inputs(cfg("f32", 1, H=2, KH=1, D=8, BS=4, S=3, lo=0, hi=9), seed=11,
                        lens=[0, 3, 9])
    _, lse = run_lse(inp)
    q = inp["query"].to(torch.float64).tolist()
    kc = inp["key_cache"].to(torch.float64).tolist()
    bt = inp["block_tables"].tolist()
    for s, L in enumerate(inp["seq_lens"].tolist()):
        for h in range(2):
            sc = [inp["scale"] * math.fsum(q[s][h][d] * kc[bt[s][t // 4]][0][d // 4][t % 4][d % 4]
                                           for d in range(8)) for t in range(L)]
            want = math.log(math.fsum(math.exp(x) for x in sc)) if sc else -math.inf
            assert close(lse[s, h], want, rtol=1e-13, atol=1e-14), (s, h)
