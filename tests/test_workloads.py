"""The seeded input generator: determinism, shapes, block-table structure (CPU)."""
import numpy as np
import pytest
import torch

from paged_kv_cache_v2_amd import workloads as W


def small(name, **kw):
    cfg = W.CONFIGS[name]
    base = dict(num_seqs=min(cfg.num_seqs, 4))
    if cfg.fixed_lens is None:
        base.update(len_hi=min(cfg.len_hi, 700), len_lo=min(cfg.len_lo, 300))
    else:
        base.update(fixed_lens=tuple(min(n, 700) for n in cfg.fixed_lens[:base["num_seqs"]]))
    base.update(kw)
    return cfg.replace(**base)


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_shapes_and_determinism(name):
    cfg = small(name)
    a = W.make_inputs(cfg, seed=3)
    b = W.make_inputs(cfg, seed=3)
    c = W.make_inputs(cfg, seed=4)
    S, H, KH, D, BS, x = (cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size,
                          cfg.block_size, cfg.x)
    NB = a["num_blocks"]
    assert a["query"].shape == (S, H, D)
    assert a["key_cache"].shape == (NB, KH, D // x, BS, x)
    assert a["value_cache"].shape == (NB, KH, D, BS)
    assert a["block_tables"].shape == (S, cfg.max_blocks_per_seq)
    assert a["query"].dtype == W.DTYPES[cfg.dtype]
    for k in ("query", "key_cache", "value_cache", "block_tables", "seq_lens"):
        assert torch.equal(a[k].view(torch.uint8) if a[k].is_floating_point() else a[k],
                           b[k].view(torch.uint8) if b[k].is_floating_point() else b[k])
    assert not torch.equal(a["key_cache"], c["key_cache"])


def test_block_tables_are_a_permutation_slice_padded():
    cfg = small("gqa_bf16_g4", num_seqs=6)
    inp = W.make_inputs(cfg, seed=1)
    bt, sl = inp["block_tables"], inp["seq_lens"]
    used = []
    for s in range(cfg.num_seqs):
        nb = -(-int(sl[s]) // cfg.block_size)
        assert torch.all(bt[s, nb:] == -1)
        used += bt[s, :nb].tolist()
    assert sorted(used) == list(range(inp["num_blocks"]))  # each block used once, none missing


def test_lengths_in_range_and_fixed():
    cfg = W.CONFIGS["gqa_bf16_g4"]
    lens = W.draw_lengths(cfg, seed=3)
    assert lens.min() >= 1 and lens.max() <= 4096 and lens.shape == (128,)
    assert list(W.draw_lengths(W.CONFIGS["tiny_f32_d64"], 1)) == [37, 100]


def test_tiny_config_geometry():
    inp = W.make_inputs(W.CONFIGS["tiny_f32_d64"], seed=1)
    assert inp["num_blocks"] == 32 and inp["used_blocks"] == 10
    assert inp["max_blocks_per_seq"] == 7 and inp["max_num_partitions"] == 2
    assert inp["scale"] == 0.125


def test_distribution_sigma():
    cfg = small("longctx_bf16_g8")
    inp = W.make_inputs(cfg, seed=2)
    v = inp["value_cache"].float()
    assert abs(float(v.std()) - 0.5) < 0.01 and abs(float(v.mean())) < 0.01


def test_poison_unused_leaves_read_slots():
    cfg = small("mha_f16_d128", num_seqs=3, num_blocks=None)
    inp = W.make_inputs(cfg, seed=5)
    before = inp["value_cache"].clone()
    W.poison_unused(inp)
    bt, sl = inp["block_tables"], inp["seq_lens"]
    for s in range(3):
        L = int(sl[s])
        for t in range(L):
            b, o = int(bt[s, t // 16]), t % 16
            assert torch.equal(inp["value_cache"][b, :, :, o], before[b, :, :, o])
        if L % 16:
            b = int(bt[s, (L - 1) // 16])
            assert torch.isnan(inp["value_cache"][b, :, :, L % 16:].float()).all()
