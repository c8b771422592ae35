"""Bit-exact checks of the integer gather through the production kernels.

A single wrong token moves a long-context output by about 1/L, far below the
floating-point tolerance, so the gather is proven exactly instead:

* index-encoding selector: V stores (block mod 256, block div 256, slot,
  kv head) in its first four dims (for an 8-bit E4M3 cache, which holds
  integers exactly only up to 16: the hexadecimal digits of block, slot and
  kv head in its first eight dims), K is zero except a 1 at (target token,
  head-specific dim d_h), q = c * e_{d_h} with c * scale >= 128. Every other
  token's weight underflows to exactly 0 in fp32, so out[s, h, 0:4] must equal
  the encoding of the target's (block, slot) as the oracle's gather gives it,
  exactly. The random d_h also proves the x-packed key layout. Exhaustive over
  target tokens on the tiny workload, 64 seeded rounds at full shape on the others;
* seq_len = 1 returns that token's V exactly;
* relabelling physical blocks leaves every output bit-identical;
* two runs give bit-identical results.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_v2_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
C_Q = 4096.0  # exact in every dtype; C_Q * scale >= 256 * (1/16) * 16 = 256 for all workloads


@pytest.fixture(scope="module", autouse=True)
def built():
    import paged_kv_cache_v2_amd as pa
    pa.ensure_built()
    oracle.build(force=False)


class Selector:
    """Device-side K/V/q of the index-encoding construction for one geometry."""

    def __init__(self, cfg: W.DecodeConfig, seed: int, lens=None):
        base = W.make_metadata(cfg, seed, lens)
        self.cfg = cfg
        self.bt = base["block_tables"]
        self.sl = base["seq_lens"]
        self.NB = base["num_blocks"]
        S, H, KH, D, BS, x = (cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size,
                              cfg.block_size, cfg.x)
        dt = W.DTYPES[cfg.dtype]
        self.fp8 = cfg.dtype == "fp8"
        self.kc = torch.zeros(self.NB, KH, D // x, BS, x, dtype=dt, device=U.DEV)
        # writable view of K (8-bit caches are edited byte-wise: 1.0 is 0x38)
        self.kw = self.kc.view(torch.uint8) if self.fp8 else self.kc
        self.one = (torch.tensor([1.0]).to(dt).view(torch.uint8)[0].item() if self.fp8 else 1.0)
        vc = torch.zeros(self.NB, KH, D, BS, dtype=torch.float32, device=U.DEV)
        b = torch.arange(self.NB, device=U.DEV, dtype=torch.float32)[:, None, None]
        o = torch.arange(BS, device=U.DEV, dtype=torch.float32)[None, None, :]
        k = torch.arange(KH, device=U.DEV, dtype=torch.float32)[None, :, None]
        for d, val in enumerate(self.encode(b, o, k)):
            vc[:, :, d, :] = val.expand(self.NB, KH, BS)
        self.vc = vc.to(dt)
        self.q = torch.zeros(S, H, D, dtype=W.DTYPES[cfg.query_dtype], device=U.DEV)
        self.blk, self.slot = oracle.gather_indices(self.bt, self.sl, BS)
        self.start = np.concatenate([[0], np.cumsum(self.sl.numpy())])
        self.d = dict(query=self.q, key_cache=self.kc, value_cache=self.vc,
                      block_tables=self.bt.to(U.DEV), seq_lens=self.sl.to(U.DEV),
                      scale=cfg.scale_f32, partition_size=cfg.partition_size,
                      max_num_partitions=cfg.max_num_partitions, k_scale=1.0, v_scale=1.0)

    def encode(self, b, o, k):
        """Values of V's first dims for block b, slot o, kv head k (exact in the cache dtype)."""
        if not self.fp8:
            return [torch.remainder(b, 256), torch.floor(b / 256), o, k]
        hexd = lambda v, i: torch.remainder(torch.floor(v / 16 ** i), 16)
        return [hexd(b, 0), hexd(b, 1), hexd(b, 2), hexd(b, 3), hexd(o, 0), hexd(o, 1),
                hexd(k, 0), hexd(k, 1)]

    def round(self, targets: np.ndarray, dims: np.ndarray):
        """targets[s, h] = token index, dims[s, h] = d_h; runs the decode, returns results."""
        cfg = self.cfg
        S, H, KH, D, x = (cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size, cfg.x)
        G = H // KH
        flat = self.start[:-1, None] + targets  # index into the oracle's gather list
        b = torch.from_numpy(self.blk[flat].astype(np.int64))
        o = torch.from_numpy(self.slot[flat].astype(np.int64))
        kh = torch.arange(H)[None, :].expand(S, H) // G
        dd = torch.from_numpy(dims.astype(np.int64))
        idx = (b.flatten(), kh.flatten(), (dd // x).flatten(), o.flatten(), (dd % x).flatten())
        idx = tuple(t.to(U.DEV) for t in idx)
        self.kw.index_put_(idx, torch.full((S * H,), self.one, dtype=self.kw.dtype, device=U.DEV))
        self.q.zero_()
        si = torch.arange(S)[:, None].expand(S, H).flatten().to(U.DEV)
        hi = torch.arange(H)[None, :].expand(S, H).flatten().to(U.DEV)
        self.q.index_put_((si, hi, dd.flatten().to(U.DEV)),
                          torch.full((S * H,), C_Q, dtype=self.q.dtype, device=U.DEV))
        res = U.run_decode(self.d)
        self.kw.index_put_(idx, torch.zeros(S * H, dtype=self.kw.dtype, device=U.DEV))
        expect = torch.stack(self.encode(b.double(), o.double(), kh.double()), dim=-1)
        return res, expect.to(torch.float32)

    def random_round(self, rng):
        cfg = self.cfg
        S, H, KH, D = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size
        G = H // KH
        sl = self.sl.numpy()
        targets = (rng.random((S, H)) * np.maximum(sl, 1)[:, None]).astype(np.int64)
        dims = np.empty((S, H), np.int64)
        for s in range(S):
            for k in range(KH):
                dims[s, k * G:(k + 1) * G] = rng.permutation(D)[:G]
        return targets, dims


def check(res, expect, label):
    for k in ("out", "out_split"):  # the one call, and the two calls
        got = res[k][:, :, :expect.shape[-1]]
        if not torch.equal(got, expect):
            bad = (got != expect).any(-1).nonzero()[:5].tolist()
            raise AssertionError(f"{label} ({k}): gathered indices differ at (s, h) {bad}")


def test_selector_exhaustive_tiny():
    cfg = W.CONFIGS["tiny_f32_d64"]
    sel = Selector(cfg, seed=1)
    sl = sel.sl.numpy()
    rng = np.random.default_rng(0)
    U.note("T1 tiny exhaustive")
    for t in range(int(sl.max())):
        targets = np.stack([(t + 7 * np.arange(cfg.num_heads)) % sl[s] for s in range(len(sl))])
        _, dims = sel.random_round(rng)
        res, expect = sel.round(targets, dims)
        check(res, expect, f"tiny t={t}")


@pytest.mark.parametrize("name", ["mha_f16_d128", "gqa_bf16_g4", "longctx_bf16_g8",
                                  "wide_f16_d256", "gqa_fp8_g4", "longctx_fp8_g8", "mha_fp8_d128"])
def test_selector_full_shape(name):
    cfg = W.CONFIGS[name]
    sel = Selector(cfg, seed=W.workload_seed(name))
    rng = np.random.default_rng(W.workload_seed(name) - 1)
    U.note(f"T1 full {name}")
    for r in range(64):
        targets, dims = sel.random_round(rng)
        res, expect = sel.round(targets, dims)
        check(res, expect, f"{name} round {r}")
        if r == 0:  # max_logits closed form: c*scale in the target's partition, 0 elsewhere
            PS = cfg.partition_size
            m = res["ml"].double()
            tp = torch.from_numpy(targets // PS)
            tgt = m.gather(2, tp[..., None]).squeeze(-1)
            assert torch.allclose(tgt, torch.full_like(tgt, C_Q * cfg.scale_f32), rtol=1e-5)
            n = (sel.sl + PS - 1) // PS
            for s in range(cfg.num_seqs):
                mask = torch.ones(cfg.num_heads, int(n[s]), dtype=torch.bool)
                mask[torch.arange(cfg.num_heads), tp[s]] = False
                assert torch.all(m[s, :, :int(n[s])][mask] == 0)


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_seq_len_one_returns_v(name):
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=3, lens=[1] * cfg.num_seqs)
    W.poison_unused(inp)
    U.note(f"T2 {name}")
    res = U.run_decode(U.to_device(inp))
    ref = oracle.attention(inp["query"], inp["key_cache"], inp["value_cache"],
                           inp["block_tables"], inp["seq_lens"], inp["scale"])
    assert np.array_equal(res["out"].double().numpy(), ref)
    assert np.array_equal(res["out_split"].double().numpy(), ref)
    v = inp["value_cache"].float()
    G = cfg.group
    for s in range(cfg.num_seqs):
        b = int(inp["block_tables"][s, 0])
        for h in range(cfg.num_heads):
            assert torch.equal(res["out"][s, h], v[b, h // G, :, 0])


@pytest.mark.parametrize("name", W.CONFIG_ORDER + W.FP8_ORDER)
def test_block_relabelling_bit_identical(name):
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=4, extra_blocks=3)
    NB = inp["key_cache"].shape[0]
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(17))
    inp2 = dict(inp)
    inp2["key_cache"] = torch.empty_like(inp["key_cache"])
    inp2["value_cache"] = torch.empty_like(inp["value_cache"])
    inp2["key_cache"][perm] = inp["key_cache"]
    inp2["value_cache"][perm] = inp["value_cache"]
    bt = inp["block_tables"].clone()
    m = bt >= 0
    bt[m] = perm[bt[m].long()].to(torch.int32)
    inp2["block_tables"] = bt
    U.note(f"T3 {name}")
    a = U.run_decode(U.to_device(inp))
    b = U.run_decode(U.to_device(inp2))
    for k in ("out", "out_split", "es", "ml"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["tmp"].nan_to_num(nan=3.0), b["tmp"].nan_to_num(nan=3.0))


@pytest.mark.parametrize("name", W.CONFIG_ORDER + W.FP8_ORDER)
def test_run_to_run_bit_identical(name):
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=6)
    d = U.to_device(inp)
    U.note(f"determinism {name}")
    a = U.run_decode(d)
    b = U.run_decode(d)
    for k in ("out", "out_split", "es", "ml"):
        assert torch.equal(a[k], b[k]), k
