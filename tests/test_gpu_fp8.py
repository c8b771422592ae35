"""8-bit (OCP E4M3) key/value caches through the C ABI, against the oracle.

* every finite E4M3 code, decoded by the kernels' gfx950 conversions: one
  token per sequence makes the output the value row times v_scale exactly
  (probability 1, a power-of-two scale), on the MFMA path (bf16 and f16
  queries) and the vector path (group sizes 1 and 2), block sizes 16 and 32;
* lengths at every block / partition edge and a partition-size sweep for
  each kernel family, with NaN bytes in every unread slot;
* seq_len = 1 returns that token's V (times v_scale) bit for bit;
* k_scale = 0 gives the mean of the values; scales enter linearly.
"""
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


def geom(q_dtype, H, KH, D, BS, PS, S, hi, k_scale=0.03, v_scale=0.045):
    return W.DecodeConfig(f"fp8_{q_dtype}_{H}_{KH}_{D}_{BS}", num_seqs=S, num_heads=H,
                          num_kv_heads=KH, head_size=D, block_size=BS, partition_size=PS,
                          dtype="fp8", q_dtype=q_dtype, len_lo=0, len_hi=hi, k_scale=k_scale,
                          v_scale=v_scale)


@pytest.mark.parametrize("q_dtype,H,KH,BS", [("bf16", 16, 4, 16), ("f16", 16, 4, 32),
                                             ("bf16", 4, 4, 32), ("f16", 4, 4, 16),
                                             ("bf16", 8, 4, 16)])
def test_every_e4m3_code_decodes_exactly(q_dtype, H, KH, BS):
    """D = 256 value dims hold the codes 0..255 (the two NaN codes replaced by 0)."""
    D, S = 256, 3
    cfg = geom(q_dtype, H, KH, D, BS, 64, S, 1, v_scale=0.125)
    inp = W.make_inputs(cfg, seed=5, lens=[1] * S)
    codes = torch.arange(256, dtype=torch.uint8)
    codes[0x7F] = 0
    codes[0xFF] = 0
    vb = inp["value_cache"].view(torch.uint8)
    vb[:, :, :, 0] = codes
    U.note(f"fp8 codes {q_dtype} H={H} KH={KH} BS={BS}")
    res = U.run_decode(U.to_device(inp))
    want = codes.view(torch.float8_e4m3fn).to(torch.float32) * 0.125
    assert torch.equal(res["out"], want.expand(S, H, D))


EDGE_GEOMS = [
    ("bf16", 32, 8, 128, 16, 512),   # MFMA, G=4
    ("bf16", 64, 8, 128, 16, 512),   # MFMA, G=8
    ("f16", 16, 1, 256, 32, 128),    # MFMA, G=16, D=256, BS=32
    ("f16", 32, 32, 128, 16, 512),   # vector, G=1
    ("bf16", 8, 4, 64, 32, 64),      # vector, G=2, D=64, BS=32
    ("f16", 12, 4, 256, 16, 128),    # vector, G=3, D=256
]


@pytest.mark.parametrize("g", EDGE_GEOMS, ids=lambda g: "_".join(map(str, g)))
@pytest.mark.parametrize("split", [False, True], ids=["decode", "split"])
def test_fp8_length_edges(g, split):
    q_dtype, H, KH, D, BS, PS = g
    P = 3
    lens = [0, 1, BS - 1, BS, BS + 1, PS - 1, PS, PS + 1, 2 * PS - 1, P * PS]
    cfg = geom(q_dtype, H, KH, D, BS, PS, len(lens), P * PS)
    inp = W.make_inputs(cfg, seed=31, lens=lens, extra_blocks=4)
    W.poison_unused(inp)
    U.note(f"fp8 length edges {g} split={split}")
    res = U.run_decode(U.to_device(inp), split=split)
    U.check_against_oracle(inp, res, label=f"fp8 edges {g}")
    assert torch.all(res["out"][0] == 0)


@pytest.mark.parametrize("g", [("bf16", 32, 8, 128, 16), ("f16", 32, 32, 128, 16),
                               ("bf16", 16, 16, 256, 32)], ids=lambda g: "_".join(map(str, g)))
@pytest.mark.parametrize("PS_rule", ["BS", "2BS", "64", "512", "1024", "max"])
def test_fp8_partition_size_sweep(g, PS_rule):
    q_dtype, H, KH, D, BS = g
    hi = 1300
    PS = {"BS": BS, "2BS": 2 * BS, "64": 64, "512": 512, "1024": 1024,
          "max": -(-hi // BS) * BS}[PS_rule]
    cfg = geom(q_dtype, H, KH, D, BS, PS, 4, hi)
    inp = W.make_inputs(cfg, seed=37, lens=[hi, 700, 33, 1])
    W.poison_unused(inp)
    U.note(f"fp8 PS sweep {g} PS={PS}")
    res = U.run_decode(U.to_device(inp))
    U.check_against_oracle(inp, res, label=f"fp8 PS={PS} {g}")


@pytest.mark.parametrize("name", W.FP8_ORDER)
def test_fp8_seq_len_one_returns_scaled_v(name):
    """Power-of-two scales: out = V * v_scale exactly, and equals the oracle bit for bit."""
    cfg = U.small_config(name).replace(k_scale=1 / 64, v_scale=1 / 32)
    inp = W.make_inputs(cfg, seed=3, lens=[1] * cfg.num_seqs)
    W.poison_unused(inp)
    U.note(f"fp8 T2 {name}")
    res = U.run_decode(U.to_device(inp))
    ref = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                           inp["block_tables"], inp["seq_lens"], inp["scale"],
                           k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    assert np.array_equal(res["out"].double().numpy(), ref)
    assert np.array_equal(res["out_split"].double().numpy(), ref)
    v = inp["value_cache"].to(torch.float32) / 32
    G = cfg.group
    for s in range(cfg.num_seqs):
        b = int(inp["block_tables"][s, 0])
        for h in range(cfg.num_heads):
            assert torch.equal(res["out"][s, h], v[b, h // G, :, 0])


@pytest.mark.parametrize("name", ["gqa_fp8_g4", "mha_fp8_d128"])
def test_fp8_scale_closed_forms(name):
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=8)
    W.poison_unused(inp)
    d = U.to_device(inp)
    U.note(f"fp8 scales {name}")
    flat = U.run_decode(dict(d, k_scale=0.0))          # all scores equal: mean of V * v_scale
    ref = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                           inp["block_tables"], inp["seq_lens"], inp["scale"], k_scale=0.0,
                           v_scale=inp["v_scale"])
    U.assert_close("k_scale=0", flat["out"], ref)
    a = U.run_decode(d)
    b = U.run_decode(dict(d, v_scale=2 * inp["v_scale"]))  # a power-of-two factor: exact
    assert torch.equal(b["out"], 2 * a["out"])


def test_fp8_calls_reject_wrong_dtypes():
    cfg = U.small_config("gqa_fp8_g4")
    inp = U.to_device(W.make_inputs(cfg, seed=2))
    S, H, D = inp["query"].shape
    tmp, es, ml = pa.workspace(S, H, D, cfg.max_num_partitions, U.DEV)
    out = torch.empty(S, H, D, device=U.DEV)
    args = (inp["key_cache"], inp["value_cache"], inp["block_tables"], inp["seq_lens"])
    with pytest.raises(ValueError):   # the plain call does not take 8-bit caches
        pa.paged_attn_decode(out, tmp, es, ml, inp["query"], *args, 0.1, 512)
    with pytest.raises(ValueError):   # fp32 query with an 8-bit cache
        pa.paged_attn_decode_fp8(out, tmp, es, ml, inp["query"].float(), *args, 0.1, 1.0, 1.0,
                                 512)
    with pytest.raises(RuntimeError):  # non-finite scale (checked by the library)
        pa.paged_attn_decode_fp8(out, tmp, es, ml, inp["query"], *args, 0.1, float("inf"), 1.0,
                                 512)
