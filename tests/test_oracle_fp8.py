"""Pins of the oracle's 8-bit (OCP FP8 E4M3) cache mode (CPU only).

Reading taken (the pages give the launcher's cache dtype and per-tensor
k_scale / v_scale arguments, and an e4m3fn element type, but no formula): a
stored key byte stands for decode(byte) * k_scale, a value byte for
decode(byte) * v_scale; the query keeps its 16-bit dtype; the key cache packs
x = 16 one-byte elements.

* the decoder, exhaustively against torch's float8_e4m3fn cast, and at the
  closed-form points of the format definition;
* a pure-Python brute force and a library routine (torch fp64 softmax/matmul
  over a permute/reshape gather, torch's own fp8 decode) with scales that are
  not powers of two;
* the fp8 mode equals the fp32-cache mode on the same values repacked to the
  fp32 layout (x = 4), bit for bit, when the scale is a power of two;
* closed forms: v_scale scales the output, k_scale = 0 gives the mean of V.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_v2_amd import workloads as W
from tests import dense_views as DV


def fp8_cfg(q_dtype="bf16", H=8, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=90, k_scale=0.03,
            v_scale=0.045, **kw):
    return W.DecodeConfig("fp8_tiny", num_seqs=S, num_heads=H, num_kv_heads=KH, head_size=D,
                          block_size=BS, partition_size=PS, dtype="fp8", q_dtype=q_dtype,
                          len_lo=lo, len_hi=hi, k_scale=k_scale, v_scale=v_scale, **kw)


def run(inp, fn=oracle.attention, *extra, **kw):
    return fn(inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
              inp["seq_lens"], inp["scale"], *extra, k_scale=inp["k_scale"],
              v_scale=inp["v_scale"], **kw)


def rel_close(a, b, rtol=1e-10, atol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= atol + rtol * np.abs(b))


def test_e4m3_decoder_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode(codes, "fp8")
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decoder_closed_forms():
    """Points fixed by the format (1 sign, 4 exponent bits with bias 7, 3 fraction
    bits, subnormals at exponent 0, no infinities, only S.1111.111 is NaN)."""
    d = lambda c: float(oracle.decode(np.array([c], np.uint8), "fp8")[0])
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x38) == 1.0 and d(0x3C) == 1.5 and d(0xB8) == -1.0
    assert d(0x77) == 240.0              # exponent 14, fraction 7
    assert d(0x78) == 256.0              # exponent 15 is still finite ...
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0   # ... up to the largest value
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))


@pytest.mark.parametrize("q_dtype,H,KH,D,BS", [("bf16", 4, 2, 16, 2), ("f16", 3, 1, 32, 3)])
def test_fp8_brute_force_tiny(q_dtype, H, KH, D, BS):
    cfg = fp8_cfg(q_dtype, H=H, KH=KH, D=D, BS=BS, PS=4, S=3, lo=0, hi=9)
    inp = W.make_inputs(cfg, seed=7, lens=[0, 1, 9])
    got = run(inp)
    ref = np.array(DV.brute_force_attention(inp, inp["scale"]))
    assert rel_close(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("q_dtype,H,KH,D,BS", [("bf16", 8, 2, 128, 16), ("f16", 4, 4, 64, 32),
                                               ("bf16", 16, 2, 256, 16)])
@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_library_routine_dense(q_dtype, H, KH, D, BS, seed):
    cfg = fp8_cfg(q_dtype, H=H, KH=KH, D=D, BS=BS, PS=64, S=4, lo=1, hi=150)
    inp = W.make_inputs(cfg, seed=seed)
    got = run(inp)
    ref = DV.library_attention(inp, inp["scale"]).numpy()
    assert rel_close(got, ref, rtol=1e-10, atol=1e-12)


def test_fp8_library_routine_partitions():
    cfg = fp8_cfg("bf16", H=8, KH=2, D=64, BS=16, PS=32, S=3, lo=1, hi=100)
    inp = W.make_inputs(cfg, seed=3, lens=[1, 64, 100])
    P = 4
    tmp, es, ml = run(inp, oracle.partition_stats, P, 32)
    rt, re_, rm = DV.library_partitions(inp, inp["scale"], P, 32)
    assert np.array_equal(np.isnan(tmp), np.isnan(rt.numpy()))
    assert rel_close(tmp[~np.isnan(tmp)], rt.numpy()[~np.isnan(tmp)])
    assert rel_close(es, re_.numpy()) and np.array_equal(ml == -np.inf, rm.numpy() == -np.inf)
    fin = np.isfinite(ml)
    assert rel_close(ml[fin], rm.numpy()[fin])


def test_fp8_equals_repacked_fp32_cache():
    """Same values through the fp32 path: bytes decoded by torch, times a
    power-of-two scale (exact in fp32), repacked from x = 16 to x = 4."""
    ks, vs = 2.0 ** -5, 2.0 ** -6
    cfg = fp8_cfg("bf16", H=8, KH=2, D=64, BS=16, PS=32, S=3, lo=0, hi=120, k_scale=ks,
                  v_scale=vs)
    inp = W.make_inputs(cfg, seed=9, lens=[0, 17, 120])
    got = run(inp)
    B, KH, Dx, BS, x = inp["key_cache"].shape
    D = Dx * x
    k32 = (inp["key_cache"].to(torch.float32) * ks).permute(0, 1, 3, 2, 4).reshape(B, KH, BS, D)
    k32 = k32.reshape(B, KH, BS, D // 4, 4).permute(0, 1, 3, 2, 4).contiguous()
    v32 = (inp["value_cache"].to(torch.float32) * vs).contiguous()
    q32 = inp["query"].to(torch.float32)
    ref = oracle.attention(q32, k32, v32, inp["block_tables"], inp["seq_lens"], inp["scale"])
    assert np.array_equal(got, ref)


def test_fp8_scales_closed_forms():
    cfg = fp8_cfg("bf16", H=4, KH=2, D=64, BS=16, PS=32, S=2, lo=1, hi=60)
    inp = W.make_inputs(cfg, seed=11, lens=[1, 60])
    base = run(inp)
    doubled = dict(inp, v_scale=inp["v_scale"] * 2)
    assert np.array_equal(run(doubled), 2 * base)        # out is linear in v_scale
    flat = dict(inp, k_scale=0.0)                         # all scores 0: mean of V
    got = run(flat)
    for s in range(2):
        K, V = DV.gathered(inp, s)
        mean = V.mean(dim=0).numpy()                      # [KH, D]
        G = 2
        assert rel_close(got[s], np.repeat(mean, G, axis=0), rtol=1e-12, atol=1e-15)


def test_fp8_rejects_fp8_query_and_mixed_16_bit():
    cfg = fp8_cfg("bf16", H=4, KH=2, D=64, BS=16, PS=32, S=1, lo=5, hi=5)
    inp = W.make_inputs(cfg, seed=1)
    with pytest.raises(ValueError):
        oracle.attention(inp["key_cache"].reshape(-1)[:256].reshape(1, 4, 64),
                         inp["key_cache"], inp["value_cache"], inp["block_tables"],
                         inp["seq_lens"], 0.1)
    with pytest.raises(ValueError):
        oracle.attention(inp["query"].to(torch.float16), inp["query"].reshape(1, 2, 8, 1, 16),
                         inp["value_cache"], inp["block_tables"], inp["seq_lens"], 0.1)
