"""ALiBi position bias through the C ABI (paged_attn_v2_partition_ex /
paged_attn_decode_ex with alibi_slopes).

Every output row, every partition intermediate and every row log-sum-exp is
compared with the oracle's ALiBi mode (pinned to a torch route, closed forms
and a brute force) on both partition kernels: the MFMA path (group 4 and 8,
several query tokens, 8-bit caches, 256-wide heads) and the vector path (MHA,
group 2, fp32, 8-bit caches); zero slopes give the plain kernels' bits, and
the two-call form equals the one-call form. Slopes follow the ALiBi paper's
geometric sequence 2^(-8 (h + 1) / H), plus a steep set that concentrates
each row on its last keys.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import workloads as W
from tests import rows as R
from tests import gpu_util as U
from tests.test_oracle_alibi import slopes_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built():
    pa.ensure_built()
    oracle.build(force=False)


def workspace(q, P):
    lead = tuple(q.shape[:-1])
    D = q.shape[-1]
    return (torch.full(lead + (P, D), float("nan"), device=U.DEV),
            torch.full(lead + (P,), float("nan"), device=U.DEV),
            torch.full(lead + (P,), float("nan"), device=U.DEV))


def run_ex(d, PS, P, slopes, split=False, out_dtype=torch.float32):
    """The two calls (paged_attn_v2_partition_ex + paged_attn_v2_reduce_lse: `tmp`,
    `es`, `ml`, their output and lse); with split=False also paged_attn_decode_ex
    on its own workspace, whose output and lse are `out` and `lse` (the two
    calls' are then `out_split` and `lse_split`)."""
    q = d["query"]
    args = (q, d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"], PS)
    sc = dict(k_scale=d.get("k_scale", 1.0), v_scale=d.get("v_scale", 1.0))
    al = slopes.to(U.DEV) if slopes is not None else None
    tmp, es, ml = workspace(q, P)
    out_s = torch.full(q.shape, float("nan"), device=U.DEV).to(out_dtype)
    lse_s = torch.full(q.shape[:-1], float("nan"), device=U.DEV)
    pa.paged_attn_v2_partition_ex(tmp, es, ml, *args, alibi_slopes=al, **sc)
    pa.paged_attn_v2_reduce_lse(out_s, lse_s, tmp, es, ml, d["seq_lens"], PS)
    res = dict(tmp=tmp, es=es, ml=ml, out=out_s, lse=lse_s)
    if not split:
        out = torch.full(q.shape, float("nan"), device=U.DEV).to(out_dtype)
        lse = torch.full(q.shape[:-1], float("nan"), device=U.DEV)
        pa.paged_attn_decode_ex(out, *workspace(q, P), *args, alibi_slopes=al, lse=lse, **sc)
        res.update(out=out, lse=lse, out_split=out_s, lse_split=lse_s)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in res.items()}


def check(inp, res, PS, P, slopes, label, seqs=None):
    a = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
         inp["seq_lens"], inp["scale"])
    sc = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"], alibi_slopes=slopes)
    rows = list(range(inp["query"].shape[0])) if seqs is None else seqs
    ref, ref_lse = oracle.attention_lse(*a, seqs=rows, **sc)
    empty = np.isneginf(ref_lse[rows])
    for o, l in (("out", "lse"), ("out_split", "lse_split")):
        if o not in res:
            continue
        U.assert_close(f"{label} {o}", res[o][rows].float(), ref[rows])
        got_lse = res[l][rows].double().numpy()
        assert np.array_equal(np.isneginf(got_lse), empty), f"{label} {l} -inf rows"
        U.assert_close(f"{label} {l}", got_lse[~empty], ref_lse[rows][~empty])
    tmp, es, ml = oracle.partition_stats(*a, P, PS, seqs=rows, **sc)
    q = inp["query"]
    M = q.shape[1] if q.dim() == 4 else 1
    for s in rows:
        L = int(inp["seq_lens"][s])
        for m in range(M):
            n = -(-R.causal_len(L, M, m) // PS)
            idx = (s, m) if M > 1 else (s,)
            if n:
                U.assert_close(f"{label} ml s={s} m={m}", res["ml"][idx][:, :n], ml[idx][:, :n])
                U.assert_close(f"{label} es s={s} m={m}", res["es"][idx][:, :n], es[idx][:, :n])
                U.assert_close(f"{label} tmp s={s} m={m}", res["tmp"][idx][:, :n],
                               tmp[idx][:, :n])
            assert torch.all(res["ml"][idx][:, n:] == -math.inf), (label, s, m)
            assert torch.all(res["es"][idx][:, n:] == 0), (label, s, m)


def geom(dtype, H, KH, D, BS, PS, lens, M=1, **kw):
    return W.DecodeConfig(f"alibi_{dtype}", num_seqs=len(lens), num_heads=H, num_kv_heads=KH,
                          head_size=D, block_size=BS, partition_size=PS, dtype=dtype,
                          len_lo=0, len_hi=max(max(lens), 1), num_queries=M, **kw)


FP8 = dict(k_scale=0.015, v_scale=0.02)
# label, (dtype, H, KH, D, BS, PS), lens, extra config, slope set
CASES = [
    ("mfma_g4_bf16", ("bf16", 32, 8, 128, 16, 512), [0, 1, 17, 512, 700, 1600], {}, "paper"),
    ("mfma_g8_bf16_steep", ("bf16", 64, 8, 128, 16, 512), [3, 1300, 2500], {}, "steep"),
    ("mfma_g4_m4", ("bf16", 32, 8, 128, 16, 256), [0, 2, 4, 5, 300, 900], dict(M=4), "paper"),
    ("mfma_g4_fp8", ("fp8", 32, 8, 128, 16, 512), [0, 40, 777, 1600],
     dict(q_dtype="bf16", **FP8), "paper"),
    ("mfma_g4_d256_bs32", ("f16", 16, 4, 256, 32, 512), [31, 33, 1000], {}, "paper"),
    ("vec_mha_f16", ("f16", 32, 32, 128, 16, 512), [1, 15, 513, 1100], {}, "paper"),
    ("vec_g2_bf16", ("bf16", 16, 8, 64, 32, 256), [0, 64, 65, 700], {}, "steep"),
    ("vec_f32", ("f32", 4, 4, 64, 16, 64), [37, 100], {}, "paper"),
    ("vec_mha_fp8", ("fp8", 16, 16, 128, 16, 512), [5, 600, 1100], dict(q_dtype="f16", **FP8),
     "paper"),
]
BY_LABEL = {c[0]: c for c in CASES}


def slope_set(kind, H):
    if kind == "paper":
        return slopes_for(H)
    # steep: 0.5 .. 4 per token (the last few keys dominate every row)
    return torch.tensor([0.5 * (1 + (h % 8)) for h in range(H)], dtype=torch.float32)


def case_inputs(label, seed):
    _, g, lens, extra, kind = BY_LABEL[label]
    cfg = geom(*g, lens, **extra)
    inp = W.make_inputs(cfg, seed=seed, lens=lens)
    PS = cfg.partition_size
    return cfg, inp, PS, max(1, -(-max(lens) // PS)), kind


@pytest.mark.parametrize("label", [c[0] for c in CASES])
def test_alibi_matches_oracle(label):
    cfg, inp, PS, P, kind = case_inputs(label, seed=41)
    d = U.to_device(inp)
    slopes = slope_set(kind, cfg.num_heads)
    U.note(f"alibi {label} lens={inp['seq_lens'].tolist()} PS={PS}")
    res = run_ex(d, PS, P, slopes)
    check(inp, res, PS, P, slopes, label)


@pytest.mark.parametrize("label", ["mfma_g4_bf16", "vec_mha_f16", "mfma_g4_fp8", "mfma_g4_m4"])
def test_zero_slopes_give_the_plain_bits(label):
    cfg, inp, PS, P, _ = case_inputs(label, seed=42)
    d = U.to_device(inp)
    U.note(f"alibi zero slopes {label}")
    a = run_ex(d, PS, P, torch.zeros(cfg.num_heads))
    b = run_ex(d, PS, P, None)
    for k in ("out", "lse", "out_split", "lse_split", "es", "ml"):
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), (label, k)
    valid = ~torch.isnan(b["tmp"])
    assert torch.equal(a["tmp"][valid].view(torch.int32), b["tmp"][valid].view(torch.int32))


@pytest.mark.parametrize("name", ["mha_f16_d128", "gqa_bf16_g4"])
def test_alibi_full_size(name):
    """The full-size MHA f16 batch (64 sequences, 32 heads, head size 128,
    lengths 512..2048; the vector kernel) and GQA bf16 batch (128 sequences,
    32 / 8 heads, lengths 1..4096; the MFMA kernel) with the paper's slopes,
    at their configured partition size, one call and two calls: every row
    against the oracle."""
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg, seed=W.workload_seed(name))
    d = U.to_device(inp)
    slopes = slopes_for(cfg.num_heads)
    U.note(f"alibi full {name}")
    res = run_ex(d, cfg.partition_size, cfg.max_num_partitions, slopes)
    assert torch.isfinite(res["out"]).all() and torch.isfinite(res["lse"]).all()
    check(inp, res, cfg.partition_size, cfg.max_num_partitions, slopes, "alibi full")
