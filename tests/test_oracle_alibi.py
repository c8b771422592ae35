"""Pins of the oracle's ALiBi mode (per-head linear position bias; CPU only).

Reading taken (the pages name the slopes argument but give no formula): the
published ALiBi definition (Press, Smith and Lewis, ICLR 2022). A query at
position i adds slope_h * (j - i) to its scaled score for the key at
position j; i = L - 1 for single-query decode, L - M + m for query token m
of M.

* a library route: torch fp64 matmul / softmax / logsumexp with the bias
  built by broadcasting position vectors (single and multi-token, GQA, MHA,
  8-bit caches);
* closed forms: with a zero query the weights are geometric in the distance,
  so out and lse have closed forms (sum of a truncated geometric series and
  its mean);
* a steep slope puts all the weight on the query's own position; zero slopes
  give exactly the plain oracle;
* partition statistics + combine equal dense; a brute force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_v2_amd import workloads as W
from tests import dense_views as DV


def cfg(dtype="bf16", M=1, H=8, KH=2, D=64, BS=16, PS=32, S=4, lo=1, hi=90, **kw):
    return W.DecodeConfig("alibi_tiny", num_seqs=S, num_heads=H, num_kv_heads=KH, head_size=D,
                          block_size=BS, partition_size=PS, dtype=dtype, len_lo=lo, len_hi=hi,
                          num_queries=M, **kw)


def slopes_for(H):
    """The ALiBi paper's slopes for H heads: 2^(-8 (h + 1) / H)."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def run(inp, slopes, fn=oracle.attention_lse, *extra):
    return fn(inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
              inp["seq_lens"], inp["scale"], *extra, k_scale=inp["k_scale"],
              v_scale=inp["v_scale"], alibi_slopes=slopes)


def library(inp, slopes):
    """(out, lse) from torch ops with the ALiBi bias as a broadcast difference of
    key and query position vectors."""
    q = inp["query"].to(torch.float64)
    q4 = q if q.dim() == 4 else q[:, None]
    S, M, H, D = q4.shape
    G = H // inp["key_cache"].shape[1]
    sl = slopes.to(torch.float64)
    out = torch.zeros(S, M, H, D, dtype=torch.float64)
    lse = torch.full((S, M, H), -math.inf, dtype=torch.float64)
    for s in range(S):
        K, V = DV.gathered(inp, s)
        L = K.shape[0]
        if L == 0:
            continue
        Kh = K.repeat_interleave(G, dim=1).permute(1, 0, 2)  # [H, L, D]
        Vh = V.repeat_interleave(G, dim=1).permute(1, 0, 2)
        scores = torch.matmul(q4[s].permute(1, 0, 2), Kh.transpose(1, 2)) * float(inp["scale"])
        kpos = torch.arange(L, dtype=torch.float64)[None, :]
        qpos = (L - M + torch.arange(M, dtype=torch.float64))[:, None]
        scores = scores + sl[:, None, None] * (kpos - qpos)[None]      # [H, M, L]
        scores = scores.masked_fill((kpos > qpos)[None], -math.inf)
        w = torch.softmax(scores, dim=-1).nan_to_num(0.0)
        out[s] = torch.matmul(w, Vh).permute(1, 0, 2)
        lse[s] = torch.logsumexp(scores, dim=-1).permute(1, 0)
    if q.dim() == 3:
        return out[:, 0].numpy(), lse[:, 0].numpy()
    return out.numpy(), lse.numpy()


def close(a, b, rtol=1e-10, atol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    same_inf = (a == b) & np.isinf(b)
    with np.errstate(invalid="ignore"):
        return np.all(same_inf | (np.abs(a - b) <= atol + rtol * np.abs(b)))


@pytest.mark.parametrize("dtype,M,G", [("bf16", 1, 4), ("f16", 1, 1), ("f32", 1, 2),
                                       ("bf16", 3, 4), ("fp8", 2, 8)])
def test_library_route(dtype, M, G):
    kw = dict(q_dtype="bf16", k_scale=0.03, v_scale=0.05) if dtype == "fp8" else {}
    inp = W.make_inputs(cfg(dtype, M, H=2 * G, KH=2, **kw), seed=12, lens=[0, 1, 45, 90])
    sl = slopes_for(2 * G)
    out, lse = run(inp, sl)
    ref_out, ref_lse = library(inp, sl)
    assert close(out, ref_out) and close(lse, ref_lse)


def test_zero_slopes_are_the_plain_oracle():
    inp = W.make_inputs(cfg("bf16", 2), seed=13, lens=[1, 17, 64, 90])
    a = run(inp, torch.zeros(8))
    b = run(inp, None)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_steep_slope_selects_the_query_position():
    inp = W.make_inputs(cfg("f32", 1, H=4, KH=4, D=64), seed=14, lens=[1, 16, 33, 90])
    out = run(inp, torch.full((4,), 1e4))[0]
    for s, L in enumerate(inp["seq_lens"].tolist()):
        _, V = DV.gathered(inp, s)
        assert close(out[s], V[L - 1].numpy(), rtol=1e-12, atol=1e-15), s


@pytest.mark.parametrize("slope", [0.5, 2.0 ** -8, 0.0625])
def test_zero_query_closed_form(slope):
    """q = 0: w_t = r^(L-1-t) with r = e^-slope. With V_t = t in every element,
    out = (L-1) - E[j] for j = L-1-t truncated geometric, and
    lse = ln((1 - r^L) / (1 - r))."""
    H, KH = 4, 2
    inp = W.make_inputs(cfg("f32", 1, H=H, KH=KH, D=64, BS=16), seed=15, lens=[1, 2, 40, 90])
    inp["query"].zero_()
    vc, bt, BS = inp["value_cache"], inp["block_tables"], 16
    for s, L in enumerate(inp["seq_lens"].tolist()):
        for t in range(L):
            vc[int(bt[s, t // BS]), :, :, t % BS] = float(t)
    out, lse = run(inp, torch.full((H,), slope))
    r = math.exp(-slope)
    for s, L in enumerate(inp["seq_lens"].tolist()):
        mean_j = r * (1 - L * r ** (L - 1) + (L - 1) * r ** L) / ((1 - r) * (1 - r ** L))
        assert close(out[s], np.full((H, 64), (L - 1) - mean_j), rtol=1e-11, atol=1e-11), s
        assert close(lse[s], np.full(H, math.log((1 - r ** L) / (1 - r))), rtol=1e-12), s


@pytest.mark.parametrize("PS,M", [(16, 1), (32, 3)])
def test_partition_combine_equals_dense(PS, M):
    inp = W.make_inputs(cfg("bf16", M, PS=PS), seed=16, lens=[3, 31, 64, 90])
    sl = slopes_for(8)
    P = -(-90 // PS)
    tmp, es, ml = oracle.partition_stats(inp["query"], inp["key_cache"], inp["value_cache"],
                                         inp["block_tables"], inp["seq_lens"], inp["scale"], P,
                                         PS, alibi_slopes=sl)
    dense, _ = run(inp, sl)
    assert close(oracle.combine(tmp, es, ml, inp["seq_lens"], PS), dense, rtol=1e-12,
                 atol=1e-14)


def test_brute_force_tiny():
    inp = W.make_inputs(cfg("f32", 2, H=2, KH=1, D=8, BS=4, S=3, lo=0, hi=9), seed=17,
                        lens=[1, 4, 9])
    sl = [0.75, 0.125]
    out, lse = run(inp, torch.tensor(sl))
    q = inp["query"].to(torch.float64).tolist()
    kc = inp["key_cache"].to(torch.float64).tolist()
    vc = inp["value_cache"].to(torch.float64).tolist()
    bt = inp["block_tables"].tolist()
    for s, L in enumerate(inp["seq_lens"].tolist()):
        for m in range(2):
            i = L - 2 + m  # query position
            for h in range(2):
                toks = [t for t in range(L) if t <= i]
                if not toks:
                    assert np.all(out[s, m, h] == 0) and lse[s, m, h] == -np.inf
                    continue
                sc = [inp["scale"] * math.fsum(q[s][m][h][d] *
                                               kc[bt[s][t // 4]][0][d // 4][t % 4][d % 4]
                                               for d in range(8)) + sl[h] * (t - i)
                      for t in toks]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                z = math.fsum(w)
                want = [math.fsum(wi * vc[bt[s][t // 4]][0][d][t % 4] for wi, t in zip(w, toks)) / z
                        for d in range(8)]
                assert close(out[s, m, h], want, rtol=1e-12, atol=1e-13), (s, m, h)
                assert close(lse[s, m, h], mx + math.log(z), rtol=1e-13), (s, m, h)
