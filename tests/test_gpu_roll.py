"""The one-call decode's rolling merge: spans whose parked per-partition
states would not fit on chip (several query tokens, wide groups, head size
256) merge each partition over the wavefronts as the span streams and fold it
into a running log-sum-exp combination.

Each case is planned (paged_attn_decode_plan, asserted) to take the rolling
merge with one or two ring slots, head sizes 64, 128 and 256 (one, two and
four owned d-blocks per wavefront), one and two column tiles, spans that hold
a whole row (the output written by the partition kernel) and spans that do
not (span entries, then the reduce), lengths at partition and span edges,
rows shorter than the query window and empty sequences, ALiBi, the row
log-sum-exp and a 16-bit output; with 16-bit and 8-bit (E4M3, scaled) caches
(an 8-bit cache takes the rolling merge for every span of two or more
partitions). Every output row and lse is compared with
the oracle, and with the two calls (paged_attn_v2_partition_ex +
paged_attn_v2_reduce_lse), whose per-partition rows the other tests compare.
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


# label, (cache dtype, H, KH, D, BS, PS, M, S, P); 8-bit caches with a bf16
# or f16 query (the q_dtype column of FP8_QUERY)
CASES = [
    ("g4m4_d128", ("bf16", 32, 8, 128, 16, 64, 4, 128, 8)),
    ("g4m4_d128_entries", ("bf16", 32, 8, 128, 16, 64, 4, 128, 16)),
    ("g8m4_two_tiles", ("bf16", 64, 8, 128, 16, 64, 4, 128, 8)),
    ("g8m2_d64_bs32", ("f16", 32, 4, 64, 32, 64, 2, 256, 8)),
    ("g8_d256", ("bf16", 16, 2, 256, 16, 32, 1, 512, 8)),
    ("g16_d128_single", ("f16", 64, 4, 128, 16, 64, 1, 256, 8)),
    ("fp8_g8_d128", ("fp8", 64, 8, 128, 16, 64, 1, 64, 8)),
    ("fp8_g4_d128_entries", ("fp8", 32, 8, 128, 16, 64, 1, 128, 16)),
    ("fp8_g8m4_two_tiles", ("fp8", 64, 8, 128, 16, 64, 4, 64, 8)),
    ("fp8_g4_d64_bs32", ("fp8", 16, 4, 64, 32, 64, 1, 256, 8)),
    ("fp8_g8_d256", ("fp8", 16, 2, 256, 16, 32, 1, 256, 8)),
    ("fp8_g8_d256_bs32", ("fp8", 16, 2, 256, 32, 64, 1, 256, 8)),
]
# Head size 256 with an 8-bit cache and 16-token blocks: the rolling kernel's
# ring slot (~66 KiB) exceeds the LDS its register occupancy leaves a
# workgroup, so the host may plan one-partition spans there instead; the case
# checks whichever plan it takes.
MAY_NOT_ROLL = {"fp8_g8_d256"}
FP8_QUERY = {"fp8_g4_d64_bs32": "f16"}  # the others: bf16
FP8_SCALES = (0.015, 0.02)  # k_scale, v_scale
BY = {c[0]: c for c in CASES}


def lens_for(S, BS, PS, P, M, seed):
    edges = [0, 1, 2, M - 1, M, BS - 1, BS, PS - 1, PS, PS + 1, 2 * PS, 4 * PS - 1, 4 * PS,
             4 * PS + 1, 8 * PS - 1, 8 * PS, P * PS - 1, P * PS]
    edges = [e for e in edges if 0 <= e <= P * PS]
    rng = np.random.default_rng(seed)
    return (edges + rng.integers(0, P * PS + 1, size=S).tolist())[:S]


def cfg_of(label):
    _, (dtype, H, KH, D, BS, PS, M, S, P) = BY[label]
    extra = {}
    if dtype == "fp8":
        extra = dict(q_dtype=FP8_QUERY.get(label, "bf16"), k_scale=FP8_SCALES[0],
                     v_scale=FP8_SCALES[1])
    cfg = W.DecodeConfig(f"roll_{label}", num_seqs=S, num_heads=H, num_kv_heads=KH,
                         head_size=D, block_size=BS, partition_size=PS, dtype=dtype, len_lo=0,
                         len_hi=P * PS, num_queries=M, **extra)
    return cfg, PS, P


def case(label, seed):
    cfg, PS, P = cfg_of(label)
    S, BS, M = cfg.num_seqs, cfg.block_size, cfg.num_queries
    inp = W.make_inputs(cfg, seed=seed, lens=lens_for(S, BS, PS, P, M, seed), extra_blocks=2)
    W.poison_unused(inp)
    if M == 1 and inp["query"].dim() == 4:
        inp["query"] = inp["query"][:, 0]
    return cfg, inp, PS, P


def plan_of(cfg, P, PS):
    return pa.decode_plan(cfg.num_seqs, cfg.num_queries, cfg.num_heads, cfg.num_kv_heads,
                          cfg.head_size, cfg.block_size, P, PS, W.DTYPES[cfg.query_dtype],
                          W.DTYPES[cfg.dtype])


def test_cases_cover_the_plans():
    """The cases take the rolling merge with one and with two ring slots, with
    spans that hold whole rows and spans whose entries the reduce combines."""
    plans = [plan_of(cfg, P, PS) for cfg, PS, P in (cfg_of(c[0]) for c in CASES)]
    assert all(p["roll"] in (1, 2) and p["span"] >= 2
               for c, p in zip(CASES, plans) if c[0] not in MAY_NOT_ROLL), plans
    rolling = [p for c, p in zip(CASES, plans) if c[0] not in MAY_NOT_ROLL]
    assert {p["roll"] for p in rolling} == {1, 2}, plans
    assert any(p["entries"] == 1 for p in rolling) and any(p["entries"] > 1 for p in rolling), plans
    fp8 = [p for c, p in zip(CASES, plans) if c[1][0] == "fp8" and c[0] not in MAY_NOT_ROLL]
    assert any(p["entries"] == 1 for p in fp8) and any(p["entries"] > 1 for p in fp8), fp8
    assert any(p["launches"] == 1 and c[1][6] * c[1][1] // c[1][2] > 16
               for c, p in zip(CASES, plans) if c[1][0] == "fp8"), fp8  # two column tiles


def run(d, PS, P, slopes, out_dtype):
    """The one call (with lse), then the two calls; host copies."""
    q = d["query"]
    scales = dict(k_scale=d["k_scale"], v_scale=d["v_scale"]) if "k_scale" in d else {}
    lead = tuple(q.shape[:-1])
    D = q.shape[-1]

    def ws():
        return (torch.full(lead + (P, D), float("nan"), device=U.DEV),
                torch.full(lead + (P,), float("nan"), device=U.DEV),
                torch.full(lead + (P,), float("nan"), device=U.DEV))

    args = (q, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"], PS)
    al = slopes.to(U.DEV) if slopes is not None else None
    out = torch.full(q.shape, float("nan"), device=U.DEV).to(out_dtype)
    lse = torch.full(lead, float("nan"), device=U.DEV)
    pa.paged_attn_decode_ex(out, *ws(), *args, alibi_slopes=al, lse=lse, **scales)
    tmp, es, ml = ws()
    out_s = torch.full(q.shape, float("nan"), device=U.DEV).to(out_dtype)
    lse_s = torch.full(lead, float("nan"), device=U.DEV)
    pa.paged_attn_v2_partition_ex(tmp, es, ml, *args, alibi_slopes=al, **scales)
    pa.paged_attn_v2_reduce_lse(out_s, lse_s, tmp, es, ml, d["seq_lens"], PS)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), out_s.cpu(), lse_s.cpu()


def check_lse(name, got, ref):
    got = got.double().numpy()
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), f"{name}: -inf rows differ"
    return U.assert_close(name, got[~empty], ref[~empty])


@pytest.mark.parametrize("label", [c[0] for c in CASES])
@pytest.mark.parametrize("variant", ["plain", "alibi", "bf16_out"])
def test_rolling_merge_matches_oracle(label, variant):
    cfg, inp, PS, P = case(label, seed=91)
    S, H, D = cfg.num_seqs, cfg.num_heads, cfg.head_size
    qdt = W.DTYPES[cfg.query_dtype]
    plan = plan_of(cfg, P, PS)
    if label not in MAY_NOT_ROLL:
        assert plan["span"] >= 2 and plan["roll"] in (1, 2), plan
    slopes = W.alibi_slopes(H) if variant == "alibi" else None
    out_dtype = qdt if variant == "bf16_out" else torch.float32
    U.note(f"rolling merge {label} {variant} plan={plan}")
    d = U.to_device(inp)
    out, lse, out_s, lse_s = run(d, PS, P, slopes, out_dtype)
    a = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
         inp["seq_lens"], inp["scale"])
    scales = {k: inp[k] for k in ("k_scale", "v_scale") if k in inp}
    ref, ref_lse = oracle.attention_lse(*a, alibi_slopes=slopes, **scales)
    if out_dtype == torch.float32:
        w = U.assert_close(f"{label} {variant} out", out, ref)
        U.assert_close(f"{label} {variant} out (two calls)", out_s, ref)
    else:  # a 16-bit output: within its rounding of the reference
        ref16 = torch.from_numpy(ref).to(out_dtype).double().numpy()
        w = U.assert_close(f"{label} {variant} out", out, ref16, atol=1e-3, rtol=2 ** -7)
    wl = check_lse(f"{label} {variant} lse", lse, ref_lse)
    check_lse(f"{label} {variant} lse (two calls)", lse_s, ref_lse)
    U.note(f"{label} {variant}: worst err/limit out={w:.3g} lse={wl:.3g}")
    # rows with no keys: exactly 0 and -inf
    empty = np.isneginf(ref_lse)
    assert np.all(out.float().numpy()[empty] == 0)


@pytest.mark.parametrize("label", ["g4m4_d128", "g8m4_two_tiles", "fp8_g8_d128"])
def test_rolling_merge_run_to_run_identical(label):
    cfg, inp, PS, P = case(label, seed=92)
    d = U.to_device(inp)
    U.note(f"rolling merge determinism {label}")
    a = run(d, PS, P, None, torch.float32)
    b = run(d, PS, P, None, torch.float32)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
