"""Pins of the fp64 oracle against things other than itself (CPU only).

* the binary16 / bfloat16 decoders, exhaustively, against numpy / torch casts;
* hand-derived closed-form fixtures under tests/golden/;
* a pure-Python brute force on tiny inputs;
* a library routine: torch fp64 softmax/matmul on K/V gathered by a
  permute/reshape route with repeat_interleave'd kv heads (GQA);
* invariants: partition + combine == dense, P = 1 equals the unpartitioned
  result bit for bit, physical-block relabelling, GQA == repeated-KV MHA,
  seq_len = 1 returns V, q = 0 or scale = 0 gives the mean of V, L = 0 gives 0,
  unread memory (NaN) never matters, empty-partition sentinels.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_v2_amd import workloads as W
from tests import dense_views as DV

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_cfg(dtype="bf16", H=4, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=70, **kw):
    return W.DecodeConfig(f"tiny_{dtype}", num_seqs=S, num_heads=H, num_kv_heads=KH,
                          head_size=D, block_size=BS, partition_size=PS, dtype=dtype,
                          len_lo=lo, len_hi=hi, **kw)


def rel_close(a, b, rtol=1e-10, atol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= atol + rtol * np.abs(b))


# --------------------------------------------------------------------- decoders
def test_binary16_decoder_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_bfloat16_decoder_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# --------------------------------------------------------------------- golden fixtures
def _fixture_inputs(fx, key_cache, value_cache, query):
    return dict(query=query, key_cache=key_cache, value_cache=value_cache,
                block_tables=torch.tensor(fx["block_tables"], dtype=torch.int32),
                seq_lens=torch.tensor(fx["seq_lens"], dtype=torch.int32))


def _nanify(a):
    if isinstance(a, list):
        return [_nanify(b) for b in a]
    return float("nan") if a == "NaN" else float(a)


def test_golden_uniform_scores():
    fx = json.load(open(os.path.join(GOLDEN, "uniform_scores.json")))
    q = torch.tensor(_nanify(fx["query"]), dtype=torch.float32)
    kc = torch.tensor(_nanify(fx["key_cache"]), dtype=torch.float32)
    vc = torch.tensor(_nanify(fx["value_cache"]), dtype=torch.float32)
    inp = _fixture_inputs(fx, kc, vc, q)
    args = (inp["query"], kc, vc, inp["block_tables"], inp["seq_lens"], fx["scale"])
    out = oracle.attention(*args)
    assert np.array_equal(out, np.array(fx["expected_out"], np.float64))
    tmp, es, ml = oracle.partition_stats(*args, fx["max_num_partitions"], fx["partition_size"])
    assert np.array_equal(ml, np.array(fx["expected_max_logits"], np.float64))
    assert np.array_equal(es, np.array(fx["expected_exp_sums"], np.float64))
    assert np.array_equal(tmp, np.array(fx["expected_tmp_output"], np.float64))
    comb = oracle.combine(tmp, es, ml, inp["seq_lens"], fx["partition_size"])
    assert np.allclose(comb, np.array(fx["expected_out"], np.float64), rtol=0, atol=1e-14)
    blk, slot = oracle.gather_indices(inp["block_tables"], inp["seq_lens"], fx["block_size"])
    assert [list(p) for p in zip(blk.tolist(), slot.tolist())] == fx["expected_gather"]


def _argmax_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "argmax_selection.json")))
    S, H, KH, D, BS, NB = (len(fx["seq_lens"]), fx["num_heads"], fx["num_kv_heads"],
                           fx["head_size"], fx["block_size"], fx["num_blocks"])
    x = 4
    q = torch.zeros(S, H, D)
    for s in range(S):
        for h in range(H):
            q[s, h, 1 if h % 2 == 0 else 6] = 30.0
    kc = torch.zeros(NB, KH, D // x, BS, x)
    for b, kh, c, o, e in fx["key_nonzero"]:
        kc[b, kh, c, o, e] = 120.0
    vc = torch.zeros(NB, KH, D, BS)
    for b in range(NB):
        for kh in range(KH):
            for d in range(D):
                for o in range(BS):
                    vc[b, kh, d, o] = 1000 * kh + 100 * b + 10 * o + d
    for t in (kc, vc):
        t[2] = float("nan")
    kc[0, :, :, 1, :] = float("nan")
    vc[0, :, :, 1] = float("nan")
    return fx, _fixture_inputs(fx, kc, vc, q)


def test_golden_argmax_selection():
    fx, inp = _argmax_fixture()
    args = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
            inp["seq_lens"], fx["scale"])
    out = oracle.attention(*args)
    D = fx["head_size"]
    base = np.array(fx["expected_out_base"], np.float64)
    expect = base[:, :, None] + np.arange(D)[None, None, :]
    assert np.array_equal(out, expect)
    tmp, es, ml = oracle.partition_stats(*args, fx["max_num_partitions"], fx["partition_size"])
    assert np.array_equal(ml, np.array(fx["expected_max_logits"], np.float64))
    assert np.array_equal(es, np.array(fx["expected_exp_sums"], np.float64))
    blk, slot = oracle.gather_indices(inp["block_tables"], inp["seq_lens"], fx["block_size"])
    assert [list(p) for p in zip(blk.tolist(), slot.tolist())] == fx["expected_gather"]


# --------------------------------------------------------------------- brute force / library
@pytest.mark.parametrize("dtype,H,KH,D,BS", [("f32", 2, 2, 8, 4), ("bf16", 4, 2, 16, 2),
                                             ("f16", 3, 1, 8, 3)])
def test_brute_force_tiny(dtype, H, KH, D, BS):
    cfg = tiny_cfg(dtype, H=H, KH=KH, D=D, BS=BS, PS=4, S=3, lo=0, hi=9)
    inp = W.make_inputs(cfg, seed=7, lens=[0, 1, 9])
    got = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                           inp["block_tables"], inp["seq_lens"], cfg.scale_f32)
    ref = np.array(DV.brute_force_attention(inp, cfg.scale_f32))
    assert rel_close(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dtype,H,KH,D,BS", [("f32", 4, 4, 64, 16), ("f16", 8, 2, 128, 16),
                                             ("bf16", 8, 1, 64, 32), ("bf16", 16, 2, 256, 32)])
@pytest.mark.parametrize("seed", [0, 1])
def test_library_routine_dense(dtype, H, KH, D, BS, seed):
    cfg = tiny_cfg(dtype, H=H, KH=KH, D=D, BS=BS, PS=64, S=4, lo=1, hi=150)
    inp = W.make_inputs(cfg, seed=seed)
    got = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                           inp["block_tables"], inp["seq_lens"], cfg.scale_f32)
    ref = DV.library_attention(inp, cfg.scale_f32).numpy()
    assert rel_close(got, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f16", 1), ("f32", 2)])
def test_library_routine_partitions(dtype, G):
    cfg = tiny_cfg(dtype, H=2 * G, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=100)
    inp = W.make_inputs(cfg, seed=3, lens=[1, 64, 100])
    P = cfg.max_num_partitions
    tmp, es, ml = oracle.partition_stats(inp["query"], inp["key_cache"], inp["value_cache"],
                                         inp["block_tables"], inp["seq_lens"], cfg.scale_f32,
                                         P, cfg.partition_size)
    rtmp, res, rml = (t.numpy() for t in DV.library_partitions(inp, cfg.scale_f32, P,
                                                                 cfg.partition_size))
    valid = np.isfinite(rml)
    assert np.array_equal(valid, np.isfinite(ml))
    assert rel_close(ml[valid], rml[valid]) and rel_close(es[valid], res[valid])
    assert rel_close(tmp[valid], rtmp[valid])
    # empty partitions: sentinels exactly
    assert np.all(ml[~valid] == -np.inf) and np.all(es[~valid] == 0.0)


# --------------------------------------------------------------------- invariants
@pytest.mark.parametrize("PS", [16, 32, 64, 512])
def test_partition_combine_equals_dense(PS):
    cfg = tiny_cfg("bf16", H=8, KH=2, D=128, BS=16, PS=PS, S=4, lo=1, hi=300)
    inp = W.make_inputs(cfg, seed=11, lens=[1, 16, 17, 300])
    args = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
            inp["seq_lens"], cfg.scale_f32)
    dense = oracle.attention(*args)
    tmp, es, ml = oracle.partition_stats(*args, cfg.max_num_partitions, PS)
    comb = oracle.combine(tmp, es, ml, inp["seq_lens"], PS)
    assert np.all(np.abs(comb - dense) <= 1e-12 * (1 + np.abs(dense)))


def test_single_partition_is_bitwise_dense():
    cfg = tiny_cfg("f16", H=4, KH=4, D=64, BS=16, PS=512, S=3, lo=1, hi=500)
    inp = W.make_inputs(cfg, seed=5)
    args = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
            inp["seq_lens"], cfg.scale_f32)
    dense = oracle.attention(*args)
    tmp, es, ml = oracle.partition_stats(*args, 1, 512)
    assert np.array_equal(tmp[:, :, 0, :], dense)
    comb = oracle.combine(tmp, es, ml, inp["seq_lens"], 512)
    assert np.array_equal(comb, dense)


def test_block_relabelling_invariance():
    cfg = tiny_cfg("bf16", H=4, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=90)
    inp = W.make_inputs(cfg, seed=2)
    NB = inp["key_cache"].shape[0]
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(9))
    kc2 = torch.empty_like(inp["key_cache"])
    vc2 = torch.empty_like(inp["value_cache"])
    kc2[perm] = inp["key_cache"]
    vc2[perm] = inp["value_cache"]
    bt = inp["block_tables"].clone()
    m = bt >= 0
    bt[m] = perm[bt[m].long()].to(torch.int32)
    a = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
                         inp["seq_lens"], cfg.scale_f32)
    b = oracle.attention(inp["query"], kc2, vc2, bt, inp["seq_lens"], cfg.scale_f32)
    assert np.array_equal(a, b)


def test_gqa_equals_repeated_kv_mha():
    G = 4
    cfg = tiny_cfg("bf16", H=8, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=90)
    inp = W.make_inputs(cfg, seed=4)
    kc_rep = inp["key_cache"].repeat_interleave(G, dim=1).contiguous()
    vc_rep = inp["value_cache"].repeat_interleave(G, dim=1).contiguous()
    a = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                         inp["block_tables"], inp["seq_lens"], cfg.scale_f32)
    b = oracle.attention(inp["query"], kc_rep, vc_rep, inp["block_tables"], inp["seq_lens"],
                         cfg.scale_f32)
    assert np.array_equal(a, b)


def test_seq_len_one_returns_v():
    cfg = tiny_cfg("f16", H=4, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=1)
    inp = W.make_inputs(cfg, seed=6, lens=[1, 1, 1])
    out = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                           inp["block_tables"], inp["seq_lens"], cfg.scale_f32)
    v = inp["value_cache"].to(torch.float64)
    for s in range(3):
        b = int(inp["block_tables"][s, 0])
        for h in range(4):
            assert np.array_equal(out[s, h], v[b, h // 2, :, 0].numpy())


@pytest.mark.parametrize("mode", ["zero_q", "zero_scale"])
def test_equal_scores_give_mean(mode):
    cfg = tiny_cfg("bf16", H=4, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=80)
    inp = W.make_inputs(cfg, seed=8)
    scale = cfg.scale_f32
    if mode == "zero_q":
        inp["query"] = torch.zeros_like(inp["query"])
    else:
        scale = 0.0
    out = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                           inp["block_tables"], inp["seq_lens"], scale)
    for s in range(3):
        _, V = DV.gathered(inp, s)
        mean = V.mean(dim=0).numpy()  # [KH, D]
        for h in range(4):
            assert rel_close(out[s, h], mean[h // 2], rtol=1e-13, atol=1e-14)


def test_scale_multiplies_the_dot():
    # Doubling q and halving the scale changes nothing, bit for bit (both exact).
    cfg = tiny_cfg("f32", H=4, KH=2, D=64, BS=16, PS=32, S=2, lo=5, hi=60)
    inp = W.make_inputs(cfg, seed=12)
    a = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                         inp["block_tables"], inp["seq_lens"], 0.25)
    b = oracle.attention(inp["query"] * 2, inp["key_cache"], inp["value_cache"],
                         inp["block_tables"], inp["seq_lens"], 0.125)
    assert np.array_equal(a, b)
    c = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                         inp["block_tables"], inp["seq_lens"], 0.5)
    assert not np.allclose(a, c)


def test_zero_length_gives_zero_and_sentinels():
    cfg = tiny_cfg("bf16", H=4, KH=2, D=64, BS=16, PS=32, S=2, lo=0, hi=40)
    inp = W.make_inputs(cfg, seed=1, lens=[0, 40])
    args = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
            inp["seq_lens"], cfg.scale_f32)
    out = oracle.attention(*args)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert not np.any(np.isnan(out))
    tmp, es, ml = oracle.partition_stats(*args, cfg.max_num_partitions, 32)
    assert np.all(ml[0] == -np.inf) and np.all(es[0] == 0)
    assert np.all(np.isfinite(ml[1, :, :2])) and np.all(ml[1, :, 2:] == -np.inf)
    comb = oracle.combine(tmp, es, ml, inp["seq_lens"], 32)
    assert np.array_equal(comb[0], np.zeros_like(comb[0]))


def test_unread_memory_never_matters():
    cfg = tiny_cfg("bf16", H=4, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=77,
                   num_blocks=40)
    inp = W.make_inputs(cfg, seed=13)
    args = lambda i: (i["query"], i["key_cache"], i["value_cache"], i["block_tables"],  # noqa
                      i["seq_lens"], cfg.scale_f32)
    clean = oracle.attention(*args(inp))
    tclean = oracle.partition_stats(*args(inp), cfg.max_num_partitions, 32)
    poisoned = dict(inp)
    poisoned["key_cache"] = inp["key_cache"].clone()
    poisoned["value_cache"] = inp["value_cache"].clone()
    W.poison_unused(poisoned)
    bt = inp["block_tables"].clone()
    bt[bt < 0] = 123456  # padding past a sequence's blocks is never dereferenced
    poisoned["block_tables"] = bt
    assert np.array_equal(clean, oracle.attention(*args(poisoned)))
    tpois = oracle.partition_stats(*args(poisoned), cfg.max_num_partitions, 32)
    for a, b in zip(tclean, tpois):
        assert np.array_equal(a, b, equal_nan=True)


def test_gather_indices_brute_force():
    cfg = tiny_cfg("f16", H=2, KH=1, D=64, BS=16, PS=32, S=5, lo=0, hi=70)
    inp = W.make_inputs(cfg, seed=21)
    blk, slot = oracle.gather_indices(inp["block_tables"], inp["seq_lens"], 16)
    expect = []
    bt = inp["block_tables"].tolist()
    for s, L in enumerate(inp["seq_lens"].tolist()):
        for t in range(L):
            expect.append((bt[s][t // 16], t % 16))
    assert list(zip(blk.tolist(), slot.tolist())) == expect


def test_subset_rows_match_full():
    cfg = tiny_cfg("bf16", H=4, KH=2, D=64, BS=16, PS=32, S=5, lo=1, hi=70)
    inp = W.make_inputs(cfg, seed=22)
    args = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
            inp["seq_lens"], cfg.scale_f32)
    full = oracle.attention(*args)
    part = oracle.attention(*args, seqs=[3, 1])
    assert np.array_equal(part[[1, 3]], full[[1, 3]])
    assert np.all(np.isnan(part[[0, 2, 4]]))
