"""Seeded synthetic inputs for paged single-query decode attention.

This module only *constructs inputs*: shapes, sequence lengths, a shuffled
physical-block assignment and normally distributed query/key/value values.
It holds none of the attention arithmetic, so both the HIP path and the fp64
oracle can consume the same tensors without sharing any code of the method.

Layouts follow the problem statement of the Triton PagedAttention V2 page
(argument comments of the phase-1 partition kernel):

* query        ``[S, H, D]``
* key_cache    ``[B, KH, D/x, BS, x]`` with ``x = 16 / sizeof(dtype)``
* value_cache  ``[B, KH, D, BS]``
* block_tables ``[S, MB]`` int32, padded with -1 past a sequence's blocks
* seq_lens     ``[S]`` int32

Random numbers come from numpy's PCG64, one independent stream per
(tensor, 4 Mi-element chunk), keyed by ``SeedSequence(seed, spawn_key=...)``.
The values therefore do not depend on how many threads generate them.
Normals are drawn in float32 and rounded to the storage dtype with
round-to-nearest-even (torch's ``.to``), so every consumer reads the same bits.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "fp8": torch.float8_e4m3fn}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
FP8_MAX = 448.0  # largest finite OCP E4M3 value

# Stream keys (first element of spawn_key) for each random quantity.
_KEY_LENS, _KEY_PERM, _KEY_Q, _KEY_K, _KEY_V = 0, 1, 2, 3, 4
_CHUNK = 1 << 22


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One decode workload: head structure, cache geometry and length mix."""

    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    partition_size: int
    dtype: str
    len_lo: int = 0  # inclusive lower bound of uniform integer lengths
    len_hi: int = 0  # inclusive upper bound; also sizes max_blocks and P
    fixed_lens: Optional[Sequence[int]] = None
    sigma: float = 1.0
    scale: Optional[float] = None  # None means 1/sqrt(head_size)
    num_blocks: Optional[int] = None  # None means exactly the blocks used
    q_dtype: Optional[str] = None  # None means the cache dtype
    k_scale: float = 1.0  # 8-bit caches: a stored key byte stands for decode(byte) * k_scale
    v_scale: float = 1.0
    num_queries: int = 1  # query tokens per sequence (the last positions; query [S, M, H, D])
    alibi: bool = False  # per-head ALiBi slopes (alibi_slopes) come with the inputs

    @property
    def query_dtype(self) -> str:
        return self.q_dtype or self.dtype

    @property
    def x(self) -> int:
        return 16 // torch.tensor([], dtype=DTYPES[self.dtype]).element_size()

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def max_len(self) -> int:
        if self.fixed_lens is not None:
            return max(self.fixed_lens)
        return self.len_hi

    @property
    def max_blocks_per_seq(self) -> int:
        return max(1, -(-self.max_len // self.block_size))

    @property
    def max_num_partitions(self) -> int:
        return max(1, -(-self.max_len // self.partition_size))

    @property
    def scale_f32(self) -> float:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_size)
        return float(np.float32(s))

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


# The five workloads the measurements are quoted on, named by what they are.
CONFIGS: Dict[str, DecodeConfig] = {
    "tiny_f32_d64": DecodeConfig(
        "tiny_f32_d64", num_seqs=2, num_heads=4, num_kv_heads=4, head_size=64,
        block_size=16, partition_size=64, dtype="f32", fixed_lens=(37, 100),
        scale=1.0 / 8.0, num_blocks=32),
    "mha_f16_d128": DecodeConfig(
        "mha_f16_d128", num_seqs=64, num_heads=32, num_kv_heads=32, head_size=128,
        block_size=16, partition_size=512, dtype="f16", len_lo=512, len_hi=2048),
    "gqa_bf16_g4": DecodeConfig(
        "gqa_bf16_g4", num_seqs=128, num_heads=32, num_kv_heads=8, head_size=128,
        block_size=16, partition_size=512, dtype="bf16", len_lo=1, len_hi=4096),
    "longctx_bf16_g8": DecodeConfig(
        "longctx_bf16_g8", num_seqs=8, num_heads=64, num_kv_heads=8, head_size=128,
        block_size=16, partition_size=512, dtype="bf16", fixed_lens=(32768,) * 8,
        sigma=0.5),
    "wide_f16_d256": DecodeConfig(
        "wide_f16_d256", num_seqs=32, num_heads=16, num_kv_heads=16, head_size=256,
        block_size=32, partition_size=512, dtype="f16", len_lo=4096, len_hi=8192,
        scale=1.0 / 16.0),
}
CONFIG_ORDER = ["tiny_f32_d64", "mha_f16_d128", "gqa_bf16_g4", "longctx_bf16_g8",
                "wide_f16_d256"]

# 8-bit (OCP E4M3) key/value caches with per-tensor scales: the GQA, long-context
# and MHA shapes above with the caches stored in one byte per element and the
# query kept in its 16-bit dtype. The scales are deliberately not powers of two.
FP8_CONFIGS: Dict[str, DecodeConfig] = {
    "gqa_fp8_g4": CONFIGS["gqa_bf16_g4"].replace(
        name="gqa_fp8_g4", dtype="fp8", q_dtype="bf16", k_scale=0.015, v_scale=0.02),
    "longctx_fp8_g8": CONFIGS["longctx_bf16_g8"].replace(
        name="longctx_fp8_g8", dtype="fp8", q_dtype="bf16", k_scale=0.0075, v_scale=0.01),
    "mha_fp8_d128": CONFIGS["mha_f16_d128"].replace(
        name="mha_fp8_d128", dtype="fp8", q_dtype="f16", k_scale=0.015, v_scale=0.02),
}
FP8_ORDER = ["gqa_fp8_g4", "longctx_fp8_g8", "mha_fp8_d128"]
CONFIGS.update(FP8_CONFIGS)

# Several query tokens per sequence (speculative decoding: the last M positions
# of each sequence query the cache causally): the GQA workload with 4 tokens
# (4 heads x 4 tokens fill one 16-column tile) and the long-context one with 2
# (16 columns) and 4 (8 heads x 4 tokens: 32 columns, two tiles).
MQ_CONFIGS: Dict[str, DecodeConfig] = {
    "gqa_bf16_g4_m4": CONFIGS["gqa_bf16_g4"].replace(name="gqa_bf16_g4_m4", num_queries=4),
    "longctx_bf16_g8_m2": CONFIGS["longctx_bf16_g8"].replace(name="longctx_bf16_g8_m2",
                                                            num_queries=2),
    "longctx_bf16_g8_m4": CONFIGS["longctx_bf16_g8"].replace(name="longctx_bf16_g8_m4",
                                                            num_queries=4),
}
MQ_ORDER = ["gqa_bf16_g4_m4", "longctx_bf16_g8_m2", "longctx_bf16_g8_m4"]
CONFIGS.update(MQ_CONFIGS)

# ALiBi position bias: the MHA workload (the head structure of the published
# ALiBi models) and the GQA one, with the ALiBi paper's slopes.
ALIBI_CONFIGS: Dict[str, DecodeConfig] = {
    "mha_f16_d128_alibi": CONFIGS["mha_f16_d128"].replace(name="mha_f16_d128_alibi", alibi=True),
    "gqa_bf16_g4_alibi": CONFIGS["gqa_bf16_g4"].replace(name="gqa_bf16_g4_alibi", alibi=True),
}
ALIBI_ORDER = ["mha_f16_d128_alibi", "gqa_bf16_g4_alibi"]
CONFIGS.update(ALIBI_CONFIGS)


def alibi_slopes(num_heads: int) -> torch.Tensor:
    """The ALiBi paper's head slopes (Press, Smith and Lewis, ICLR 2022): for a
    power-of-two head count H, the geometric sequence 2^(-8 (h + 1) / H);
    otherwise the slopes of the next lower power of two followed by every
    other slope of the next higher one."""
    def pow2(n):
        return [2.0 ** (-8.0 * (h + 1) / n) for h in range(n)]
    p = 1 << (num_heads.bit_length() - 1)
    sl = pow2(p) if p == num_heads else pow2(p) + pow2(2 * p)[0::2][:num_heads - p]
    return torch.tensor(sl, dtype=torch.float32)


def workload_seed(name: str) -> int:
    """Seed of a named workload's reported runs: its index in its list, plus 1
    (the 8-bit workloads from 101, the multi-token ones from 201); an ALiBi
    workload reuses its base workload's seed (the same inputs plus slopes)."""
    if name in CONFIG_ORDER:
        return CONFIG_ORDER.index(name) + 1
    if name in FP8_ORDER:
        return FP8_ORDER.index(name) + 101
    if name in ALIBI_ORDER:
        return workload_seed(name[:-len("_alibi")])
    return MQ_ORDER.index(name) + 201


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normals(seed: int, key: int, n: int, sigma: float) -> np.ndarray:
    """n float32 normals N(0, sigma^2), chunked PCG64 streams, thread-count independent."""
    out = np.empty(n, dtype=np.float32)
    nchunks = -(-n // _CHUNK) if n else 0

    def work(i: int) -> None:
        ss = np.random.SeedSequence(seed, spawn_key=(key, i))
        rng = np.random.Generator(np.random.PCG64(ss))
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, range(nchunks)))
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


def _rng(seed: int, key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(key,))))


def draw_lengths(cfg: DecodeConfig, seed: int) -> np.ndarray:
    if cfg.fixed_lens is not None:
        lens = np.asarray(cfg.fixed_lens, dtype=np.int64)
        assert lens.shape == (cfg.num_seqs,)
        return lens
    return _rng(seed, _KEY_LENS).integers(cfg.len_lo, cfg.len_hi + 1, size=cfg.num_seqs)


def make_metadata(cfg: DecodeConfig, seed: int, lens: Optional[Sequence[int]] = None,
                  extra_blocks: int = 0) -> Dict[str, object]:
    """Lengths, shuffled block tables and sizes of one input set (no K/V values).

    ``lens`` overrides the drawn lengths; ``extra_blocks`` adds physical blocks
    that no sequence references (decoys).
    """
    S, BS = cfg.num_seqs, cfg.block_size
    seq_lens = np.asarray(lens if lens is not None else draw_lengths(cfg, seed), dtype=np.int64)
    assert seq_lens.shape == (S,)
    MB = cfg.max_blocks_per_seq
    P = cfg.max_num_partitions
    assert int(seq_lens.max(initial=0)) <= min(MB * BS, P * cfg.partition_size)
    blocks_per_seq = [-(-int(n) // BS) for n in seq_lens]
    used = sum(blocks_per_seq)
    NB = (cfg.num_blocks if cfg.num_blocks is not None else max(1, used)) + extra_blocks
    assert NB >= used, "num_blocks too small for the drawn lengths"
    perm = _rng(seed, _KEY_PERM).permutation(NB).astype(np.int32)
    bt = np.full((S, MB), -1, dtype=np.int32)
    pos = 0
    for s, nb in enumerate(blocks_per_seq):
        bt[s, :nb] = perm[pos:pos + nb]
        pos += nb
    return dict(block_tables=torch.from_numpy(bt),
                seq_lens=torch.from_numpy(seq_lens.astype(np.int32)),
                num_seqs=S, num_heads=cfg.num_heads, num_kv_heads=cfg.num_kv_heads,
                head_size=cfg.head_size, block_size=BS, num_blocks=NB, max_blocks_per_seq=MB,
                max_num_partitions=P, partition_size=cfg.partition_size, scale=cfg.scale_f32,
                dtype=cfg.dtype, q_dtype=cfg.query_dtype, x=cfg.x, used_blocks=used,
                k_scale=float(np.float32(cfg.k_scale)), v_scale=float(np.float32(cfg.v_scale)))


def make_inputs(cfg: DecodeConfig, seed: int, lens: Optional[Sequence[int]] = None,
                device: str = "cpu", extra_blocks: int = 0) -> Dict[str, object]:
    """Build one seeded input set for ``cfg``.

    Returns the metadata of ``make_metadata`` plus torch tensors ``query``,
    ``key_cache`` and ``value_cache`` drawn N(0, sigma^2) and rounded to the
    workload's dtypes. For an 8-bit cache the drawn values are divided by the
    cache scale, clamped to the format's finite range and rounded to E4M3
    (the stored bytes then stand for roughly N(0, sigma^2) values).
    """
    S, H, KH, D, BS = (cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_size,
                       cfg.block_size)
    x = cfg.x
    assert H % KH == 0 and D % x == 0
    out = make_metadata(cfg, seed, lens, extra_blocks)
    NB = out["num_blocks"]

    def tensor(key: int, shape, dtype: str, cache_scale: float = 1.0) -> torch.Tensor:
        n = int(np.prod(shape))
        vals = torch.from_numpy(_normals(seed, key, n, cfg.sigma)).reshape(shape)
        if dtype == "fp8":
            vals = (vals / np.float32(cache_scale)).clamp_(-FP8_MAX, FP8_MAX)
        return vals.to(DTYPES[dtype])

    M = cfg.num_queries
    out["query"] = tensor(_KEY_Q, (S, H, D) if M == 1 else (S, M, H, D), cfg.query_dtype)
    out["num_queries"] = M
    out["key_cache"] = tensor(_KEY_K, (NB, KH, D // x, BS, x), cfg.dtype, cfg.k_scale)
    out["value_cache"] = tensor(_KEY_V, (NB, KH, D, BS), cfg.dtype, cfg.v_scale)
    out["alibi_slopes"] = alibi_slopes(H) if cfg.alibi else None
    if device != "cpu":
        for k in ("query", "key_cache", "value_cache", "block_tables", "seq_lens"):
            out[k] = out[k].to(device)
    return out


def poison_unused(inp: Dict[str, object], value: float = float("nan")) -> None:
    """Fill every cache slot no sequence may read with ``value`` (in place, CPU tensors).

    That is: physical blocks no block table references, and the slots of each
    sequence's last block at or past its length.
    """
    kc, vc = inp["key_cache"], inp["value_cache"]
    if kc.dtype == torch.float8_e4m3fn:  # fill through the byte view (same storage)
        value = int(torch.tensor([value]).to(kc.dtype).view(torch.uint8)[0])
        kc, vc = kc.view(torch.uint8), vc.view(torch.uint8)
    bt, sl = inp["block_tables"], inp["seq_lens"]
    BS = inp["block_size"]
    NB = kc.shape[0]
    referenced = torch.zeros(NB, dtype=torch.bool)
    for s in range(bt.shape[0]):
        n = int(sl[s])
        nb = -(-n // BS)
        for i in range(nb):
            referenced[int(bt[s, i])] = True
        if n % BS:
            last = int(bt[s, nb - 1])
            kc[last, :, :, n % BS:, :] = value
            vc[last, :, :, n % BS:] = value
    kc[~referenced] = value
    vc[~referenced] = value
