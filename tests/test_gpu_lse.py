"""Row log-sum-exp export and the merge of two attention states, through the C ABI.

* paged_attn_v2_reduce_lse / paged_attn_decode_lse: lse against the oracle's
  (pinned to torch.logsumexp and to the partition statistics), exact -inf for
  rows with no keys, and out bit-identical to the plain calls;
* paged_attn_merge_states: against the oracle's merge on random states with
  the special rows (one side or both -inf, equal lse, far-apart lse), every
  dtype and head size, in place and without out_lse;
* the cascade / context-parallel use: each sequence's pages split in two,
  each half decoded with its lse, the halves merged, equal to the oracle's
  attention over the whole sequence (reduced sizes, and sampled rows of the
  full-size GQA batch).

Bar: |gpu - oracle| <= 1e-3 + 1e-3 |oracle| on fp32 results (lse included);
16-bit merge outputs may also differ by their final rounding (half an ulp of
the output format, relative).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import workloads as W
from tests import gpu_util as U
from tests.test_oracle_lse import split_pages

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built():
    pa.ensure_built()
    oracle.build(force=False)


def oracle_lse(inp, seqs=None):
    return oracle.attention_lse(inp["query"], inp["key_cache"], inp["value_cache"],
                                inp["block_tables"], inp["seq_lens"], inp["scale"], seqs=seqs,
                                k_scale=inp["k_scale"], v_scale=inp["v_scale"])


def assert_lse(name, got, ref):
    got = got.double().numpy()
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), f"{name}: -inf rows differ"
    U.assert_close(name, got[~empty], ref[~empty])


def decode_lse(d, PS, P, out_dtype=torch.float32):
    q = d["query"]
    lead = tuple(q.shape[:-1])
    D = q.shape[-1]
    tmp = torch.full(lead[:-1] + (lead[-1], P, D), float("nan"), device=U.DEV)
    es = torch.full(lead + (P,), float("nan"), device=U.DEV)
    ml = torch.full(lead + (P,), float("nan"), device=U.DEV)
    out = torch.full(q.shape, float("nan"), device=U.DEV).to(out_dtype)
    lse = torch.full(lead, float("nan"), device=U.DEV)
    pa.paged_attn_decode_lse(out, lse, tmp, es, ml, q, d["key_cache"], d["value_cache"],
                             d["block_tables"], d["seq_lens"], d["scale"], PS,
                             k_scale=d.get("k_scale", 1.0), v_scale=d.get("v_scale", 1.0))
    return out, lse, (tmp, es, ml)


# name, M, lens
CASES = [
    ("gqa_bf16_g4", 1, [0, 1, 16, 511, 512, 513, 1600]),
    ("tiny_f32_d64", 1, [0, 37, 100]),
    ("mha_f16_d128", 1, [3, 1024, 1100]),
    ("gqa_fp8_g4", 1, [0, 700, 1600]),
    ("gqa_bf16_g4", 4, [0, 2, 4, 5, 600, 1600]),
]


@pytest.mark.parametrize("name,M,lens", CASES, ids=[f"{c[0]}-m{c[1]}" for c in CASES])
def test_reduce_and_decode_lse_match_oracle(name, M, lens):
    cfg = U.small_config(name).replace(num_seqs=len(lens), num_queries=M)
    if M > 1:
        cfg = cfg.replace(name=f"{name}_m{M}")
    inp = W.make_inputs(cfg, seed=31, lens=lens)
    d = U.to_device(inp)
    PS = cfg.partition_size
    P = max(1, -(-max(lens) // PS))
    U.note(f"lse {name} M={M} lens={lens} PS={PS}")
    out_l, lse_l, _ = decode_lse(d, PS, P)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_lse(inp)
    U.assert_close(f"{name} decode_lse out", out_l.cpu().float(), ref_out)
    assert_lse(f"{name} decode_lse lse", lse_l.cpu(), ref_lse)
    # the two calls: phase 1 alone, then the plain reduce and the reduce_lse
    # entry point over the same statistics give the same bits, and match the
    # oracle too
    q = d["query"]
    lead = tuple(q.shape[:-1])
    D = q.shape[-1]
    tmp = torch.full(lead + (P, D), float("nan"), device=U.DEV)
    es = torch.full(lead + (P,), float("nan"), device=U.DEV)
    ml = torch.full(lead + (P,), float("nan"), device=U.DEV)
    pa.paged_attn_v2_partition_ex(tmp, es, ml, q, d["key_cache"], d["value_cache"],
                                  d["block_tables"], d["seq_lens"], d["scale"], PS,
                                  k_scale=d.get("k_scale", 1.0), v_scale=d.get("v_scale", 1.0))
    out_p = torch.full_like(out_l, float("nan"))
    out_r = torch.full_like(out_l, float("nan"))
    lse_r = torch.full_like(lse_l, float("nan"))
    if M == 1:
        pa.paged_attn_v2_reduce(out_p, tmp, es, ml, d["seq_lens"], PS)
    else:
        pa.paged_attn_v2_reduce_mq(out_p, tmp, es, ml, d["seq_lens"], PS)
    pa.paged_attn_v2_reduce_lse(out_r, lse_r, tmp, es, ml, d["seq_lens"], PS)
    torch.cuda.synchronize()
    assert torch.equal(out_r.cpu().view(torch.int32), out_p.cpu().view(torch.int32))
    U.assert_close(f"{name} reduce_lse out", out_r.cpu().float(), ref_out)
    assert_lse(f"{name} reduce_lse lse", lse_r.cpu(), ref_lse)


def test_decode_lse_16bit_out_is_cast_of_fp32():
    cfg = U.small_config("gqa_bf16_g4").replace(num_seqs=4)
    inp = W.make_inputs(cfg, seed=32, lens=[0, 77, 512, 1500])
    d = U.to_device(inp)
    P = -(-1500 // cfg.partition_size)
    U.note("lse bf16 out")
    o32, l32, _ = decode_lse(d, cfg.partition_size, P)
    o16, l16, _ = decode_lse(d, cfg.partition_size, P, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16).cpu().view(torch.int16), o16.cpu().view(torch.int16))
    assert torch.equal(l32.cpu().view(torch.int32), l16.cpu().view(torch.int32))


def random_states(R, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(R, D, generator=g).to(dtype)
    b = torch.randn(R, D, generator=g).to(dtype)
    la = torch.randn(R, generator=g) * 5
    lb = torch.randn(R, generator=g) * 5
    k = R // 8
    la[:k] = -math.inf                      # only b has keys
    lb[k:2 * k] = -math.inf                 # only a has keys
    la[2 * k:3 * k] = -math.inf             # neither
    lb[2 * k:3 * k] = -math.inf
    lb[3 * k:4 * k] = la[3 * k:4 * k]       # equal weights
    lb[4 * k:5 * k] = la[4 * k:5 * k] + 90  # b dominates past fp32 exp's range
    la[5 * k:6 * k] += 300                  # large magnitudes
    lb[5 * k:6 * k] = la[5 * k:6 * k] - 2
    return a, la, b, lb, k


ROUND = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_merge_states_ignores_the_rows_of_empty_sides(dtype):
    """A side whose lse is -inf has no keys; its row is unspecified (a decode
    leaves it 0, a caller's buffer may hold anything) and must not reach the
    output: NaN-filled rows there give the other side's row, or 0 when both
    sides are empty."""
    R, D = 96, 128
    a, la, b, lb, k = random_states(R, D, dtype, seed=7)
    a[:k] = float("nan")              # la = -inf on these rows
    b[k:2 * k] = float("inf")         # lb = -inf on these rows
    a[2 * k:3 * k] = float("nan")     # both -inf
    b[2 * k:3 * k] = float("nan")
    U.note(f"merge empty sides {dtype}")
    ga, gb, gla, glb = (t.to(U.DEV) for t in (a, b, la, lb))
    out = torch.full_like(ga, float("nan"))
    out_lse = torch.full_like(gla, float("nan"))
    pa.paged_attn_merge_states(out, out_lse, ga, gla, gb, glb)
    torch.cuda.synchronize()
    got, got_lse = out.cpu(), out_lse.cpu()
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(got[:k].view(bits), b[:k].view(bits))
    assert torch.equal(got[k:2 * k].view(bits), a[k:2 * k].view(bits))
    assert torch.all(got[2 * k:3 * k] == 0) and torch.all(got_lse[2 * k:3 * k] == -math.inf)
    assert torch.isfinite(got[:3 * k]).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_merge_states_matches_oracle(dtype, D):
    R = 200  # rows; several workgroups for every head size, plus a ragged last one
    a, la, b, lb, k = random_states(R, D, dtype, seed=D)
    ref, ref_lse = oracle.merge_states(a.double().numpy(), la.double().numpy(),
                                       b.double().numpy(), lb.double().numpy())
    U.note(f"merge {dtype} D={D} R={R}")
    ga, gb, gla, glb = (t.to(U.DEV) for t in (a, b, la, lb))
    out = torch.full_like(ga, float("nan"))
    out_lse = torch.full_like(gla, float("nan"))
    pa.paged_attn_merge_states(out, out_lse, ga, gla, gb, glb)
    torch.cuda.synchronize()
    got, got_lse = out.cpu(), out_lse.cpu()
    U.assert_close(f"merge {dtype} D={D} out", got.float(), ref,
                   rtol=U.RTOL + ROUND[dtype])
    assert_lse(f"merge {dtype} D={D} lse", got_lse, ref_lse)
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    # one side empty: the other side's row and lse, exactly; both empty: 0, -inf
    assert torch.equal(got[:k].view(bits), b[:k].view(bits))
    assert torch.equal(got[k:2 * k].view(bits), a[k:2 * k].view(bits))
    assert torch.equal(got_lse[:k], lb[:k]) and torch.equal(got_lse[k:2 * k], la[k:2 * k])
    assert torch.all(got[2 * k:3 * k] == 0) and torch.all(got_lse[2 * k:3 * k] == -math.inf)
    # in place into a (and a's lse), and without out_lse: the same bits
    pa.paged_attn_merge_states(ga, gla, ga, gla, gb, glb)
    out2 = torch.full_like(gb, float("nan"))
    pa.paged_attn_merge_states(out2, None, gb.clone(), glb, gb, glb)  # b with itself
    torch.cuda.synchronize()
    assert torch.equal(ga.cpu().view(bits), got.view(bits))
    assert torch.equal(gla.cpu().view(torch.int32), got_lse.view(torch.int32))
    # merging a state with itself keeps its rows (equal weights, up to
    # rounding); its rows with no keys stay 0
    keys = torch.isfinite(lb)
    U.assert_close("merge self", out2.cpu()[keys].float(), b[keys].double().numpy(),
                   rtol=U.RTOL + ROUND[dtype])
    assert torch.all(out2.cpu()[~keys] == 0)


def cascade(inp, PS, cut_pages, seqs=None):
    """Decode each half of a page split with its lse, merge; compare with the
    oracle's whole-sequence attention (rows `seqs`, all if None)."""
    a, b = split_pages(inp, cut_pages)
    P = max(1, -(-int(inp["seq_lens"].max()) // PS))
    oa, la, _ = decode_lse(U.to_device(a), PS, P)
    ob, lb, _ = decode_lse(U.to_device(b), PS, P)
    out = torch.full_like(oa, float("nan"))
    lse = torch.full_like(la, float("nan"))
    pa.paged_attn_merge_states(out, lse, oa, la, ob, lb)
    torch.cuda.synchronize()
    rows = list(range(inp["query"].shape[0])) if seqs is None else seqs
    ref, ref_lse = oracle_lse(inp, seqs=rows)
    return out.cpu()[rows], lse.cpu()[rows], ref[rows], ref_lse[rows]


@pytest.mark.parametrize("name", ["gqa_bf16_g4", "mha_f16_d128", "gqa_fp8_g4"])
def test_cascade_split_and_merge_equals_full_attention(name):
    cfg = U.small_config(name).replace(num_seqs=5)
    lens = [0, 20, 512, 1000, cfg.len_hi]
    inp = W.make_inputs(cfg, seed=33, lens=lens)
    # cut at: page 1 of an empty sequence, mid-page-run, a partition edge, the
    # whole sequence on one side
    cuts = [1, 1, 32, 20, 200]
    U.note(f"cascade {name} lens={lens} cuts={cuts}")
    out, lse, ref, ref_lse = cascade(inp, cfg.partition_size, cuts)
    U.assert_close(f"cascade {name} out", out.float(), ref)
    assert_lse(f"cascade {name} lse", lse, ref_lse)


def test_cascade_full_size_gqa_sampled():
    """The full-size GQA bf16 batch (128 sequences, 32 query / 8 kv heads,
    lengths 1..4096), each sequence split at its middle page; sampled rows
    against the oracle."""
    name = "gqa_bf16_g4"
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg, seed=W.workload_seed(name))
    sl = inp["seq_lens"].numpy()
    cuts = [int(-(-L // cfg.block_size)) // 2 for L in sl]
    seqs = sorted({int(np.argmax(sl)), int(np.argmin(sl)), 5, 64, 100})
    U.note(f"cascade full {name} seqs={seqs}")
    out, lse, ref, ref_lse = cascade(inp, cfg.partition_size, cuts, seqs=seqs)
    U.assert_close(f"cascade full {name} out", out.float(), ref)
    assert_lse(f"cascade full {name} lse", lse, ref_lse)
