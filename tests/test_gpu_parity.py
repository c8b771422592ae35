"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

* reduced-size versions of all five workloads (every output compared), with
  NaN in every cache slot no sequence reads and NaN-prefilled workspace;
* the five workloads and their 8-bit-cache variants at full size, at the
  configured and at the planned partition size, through the one-call decode
  (partitions combined inside the kernel) and the two calls (per-partition
  rows, then the reduce): every output row and every used partition's row and
  statistics against the oracle, sentinels exact;
* the output cast: bf16 / fp16 `out` equals round-to-nearest-even of the
  kernel's own fp32 result, bit for bit.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
ALL = W.CONFIG_ORDER + W.FP8_ORDER  # the five configurations, then their 8-bit-cache variants


@pytest.fixture(scope="module", autouse=True)
def built():
    import paged_kv_cache_v2_amd as pa
    pa.ensure_built()
    import oracle
    oracle.build(force=False)


@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("seed", [11, 12])
def test_parity_reduced(name, seed):
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=seed, extra_blocks=5 if cfg.num_blocks is None else 0)
    W.poison_unused(inp)
    U.note(f"parity reduced {name} seed={seed} lens={inp['seq_lens'].tolist()}")
    res = U.run_decode(U.to_device(inp))
    U.check_against_oracle(inp, res, label=name)


@pytest.mark.parametrize("name", ALL)
def test_one_call_matches_two_calls(name):
    """paged_attn_decode (partitions combined inside the partition kernel) and
    paged_attn_v2_partition + paged_attn_v2_reduce agree within the tolerance;
    both are compared with the oracle by the other tests. The one-call form
    leaves its workspace unwritten when one span holds every partition of a
    row, and otherwise writes only its first ceil(P / span) entries per row."""
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=21)
    d = U.to_device(inp)
    U.note(f"one call vs two calls {name}")
    r = U.run_decode(d)
    U.assert_close(f"{name} one call vs two", r["out"], r["out_split"].double().numpy())
    S, H, D = inp["query"].shape
    plan = pa.decode_plan(S, 1, H, inp["num_kv_heads"], D, cfg.block_size, r["P"], r["PS"],
                          W.DTYPES[cfg.query_dtype], W.DTYPES[cfg.dtype])
    Pq = plan["entries"]
    assert Pq == -(-r["P"] // plan["span"])
    if Pq == 1:
        for k in ("ws_tmp", "ws_es", "ws_ml"):
            assert torch.isnan(r[k]).all(), k
    else:
        flat_es = r["ws_es"].reshape(-1)
        assert torch.isnan(flat_es[S * H * Pq:]).all()
        assert not torch.isnan(flat_es[:S * H * Pq]).any()


_FULL = {}


def full_inputs(name):
    if name not in _FULL:
        _FULL.clear()
        cfg = W.CONFIGS[name]
        inp = W.make_inputs(cfg, seed=W.workload_seed(name))
        _FULL[name] = (inp, U.to_device(inp))
    return _FULL[name]


@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("ps", ["config", "planned"])
def test_parity_full_size(name, ps):
    """Full-size inputs at the configured partition size and at the size the
    library plans for the batch, in both launch forms bench.py times (the one
    call and the two calls): every output row, and every used partition's
    statistics and row, against the oracle; sentinels exact everywhere."""
    inp, d = full_inputs(name)
    cfg = W.CONFIGS[name]
    PS = None
    if ps == "planned":
        PS = pa.plan_partition_size(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads,
                                    cfg.head_size, cfg.block_size, cfg.max_len,
                                    W.DTYPES[cfg.dtype])
    U.note(f"parity full {name} ps={ps} S={inp['num_seqs']} blocks={inp['num_blocks']}")
    res = U.run_decode(d, PS=PS, P=max(1, -(-cfg.max_len // PS)) if PS else None)
    assert torch.isfinite(res["out"]).all()
    U.check_against_oracle(inp, res, label=f"{name} full PS={res['PS']}")


@pytest.mark.parametrize("name", ["mha_f16_d128", "gqa_bf16_g4", "wide_f16_d256", "gqa_fp8_g4",
                                  "mha_fp8_d128"])
def test_out_cast_is_rne_of_fp32(name):
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=5)
    d = U.to_device(inp)
    U.note(f"cast {name}")
    f32 = U.run_decode(d)
    low = U.run_decode(d, out_dtype=W.DTYPES[cfg.query_dtype])
    for k in ("out", "out_split"):  # the one-call kernel's cast, and the reduce's
        assert low[k].dtype == W.DTYPES[cfg.query_dtype]
        assert torch.equal(low[k].view(torch.int16), f32[k].to(low[k].dtype).view(torch.int16)), k
