"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

* reduced-size versions of all five workloads (every output compared), with
  NaN in every cache slot no sequence reads and NaN-prefilled workspace;
* the five workloads at full size in the launch configuration the benchmark
  times (paged_attn_decode, the workload's partition size), compared on
  sampled sequences the oracle computes one by one, plus properties that hold
  at any size (finite outputs, exact sentinels);
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
def test_parity_reduced_split_calls(name):
    """paged_attn_v2_partition + paged_attn_v2_reduce give what paged_attn_decode gives."""
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=21)
    d = U.to_device(inp)
    U.note(f"split vs fused {name}")
    a = U.run_decode(d)
    b = U.run_decode(d, split=True)
    for k in ("out", "es", "ml"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(torch.nan_to_num(a["tmp"], nan=7.0), torch.nan_to_num(b["tmp"], nan=7.0))


_FULL = {}


def full_inputs(name):
    if name not in _FULL:
        _FULL.clear()
        cfg = W.CONFIGS[name]
        inp = W.make_inputs(cfg, seed=W.workload_seed(name))
        _FULL[name] = (inp, U.to_device(inp))
    return _FULL[name]


def sample_seqs(inp, k=3, seed=0):
    sl = inp["seq_lens"].numpy()
    S = len(sl)
    picks = {int(np.argmax(sl)), int(np.argmin(sl))}
    rng = np.random.default_rng(seed)
    while len(picks) < min(S, k + 2):
        picks.add(int(rng.integers(S)))
    return sorted(picks)


@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("ps", ["config", "planned"])
def test_parity_full_size_sampled(name, ps):
    """Full-size inputs, in the launch configurations bench.py times: the
    configured partition size through the two calls, and the library's
    partition size the library plans for the batch through paged_attn_decode."""
    inp, d = full_inputs(name)
    cfg = W.CONFIGS[name]
    seqs = sample_seqs(inp, k=1 if name == "longctx_bf16_g8" else 3)
    PS = None
    if ps == "planned":
        PS = pa.plan_partition_size(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads,
                                    cfg.head_size, cfg.block_size, cfg.max_len,
                                    W.DTYPES[cfg.dtype])
    U.note(f"parity full {name} ps={ps} S={inp['num_seqs']} blocks={inp['num_blocks']} "
           f"seqs={seqs}")
    res = U.run_decode(d, PS=PS, P=max(1, -(-cfg.max_len // PS)) if PS else None,
                       split=(ps == "config"))
    assert torch.isfinite(res["out"]).all()
    U.check_against_oracle(inp, res, seqs=seqs, label=f"{name} full")
    # properties at every row: sentinels exact, valid partitions finite and l >= 1
    sl = inp["seq_lens"].tolist()
    for s in range(inp["num_seqs"]):
        n = -(-sl[s] // res["PS"])
        assert torch.all(res["ml"][s, :, n:] == -np.inf) and torch.all(res["es"][s, :, n:] == 0)
        assert torch.isfinite(res["ml"][s, :, :n]).all() and torch.all(res["es"][s, :, :n] >= 1)
        assert torch.isfinite(res["tmp"][s, :, :n]).all()


@pytest.mark.parametrize("name", ["mha_f16_d128", "gqa_bf16_g4", "wide_f16_d256", "gqa_fp8_g4",
                                  "mha_fp8_d128"])
def test_out_cast_is_rne_of_fp32(name):
    cfg = U.small_config(name)
    inp = W.make_inputs(cfg, seed=5)
    d = U.to_device(inp)
    U.note(f"cast {name}")
    f32 = U.run_decode(d)["out"]
    low = U.run_decode(d, out_dtype=W.DTYPES[cfg.query_dtype])["out"]
    assert low.dtype == W.DTYPES[cfg.query_dtype]
    assert torch.equal(low.view(torch.int16), f32.to(low.dtype).view(torch.int16))
