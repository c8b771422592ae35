"""Streams and graph capture through the C ABI.

The library keeps no device state between calls and never allocates, copies
to the host or synchronises, so
* two decodes enqueued on two streams at once give the same bits as each
  alone;
* a cascade (two decode_lse calls over a page split, then merge_states) can
  be captured in a HIP graph: every replay, with eager work and
  synchronisation between replays and new query values written in place,
  gives the bits of the same calls run eagerly;
* so can a call that the host splits into several column launches.
"""
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


def decode_into(d, bufs, stream=None):
    out, tmp, es, ml = bufs
    args = (d["query"], d["key_cache"], d["value_cache"], d["block_tables"], d["seq_lens"],
            d["scale"], d["partition_size"])
    if d["key_cache"].dtype == torch.float8_e4m3fn:
        pa.paged_attn_decode_fp8(out, tmp, es, ml, *args[:6], d["k_scale"], d["v_scale"],
                                 args[6], stream=stream)
    else:
        pa.paged_attn_decode(out, tmp, es, ml, *args, stream=stream)


def buffers(d):
    S, H, D = d["query"].shape
    P = d["max_num_partitions"]
    return (torch.zeros(S, H, D, device=U.DEV),) + pa.workspace(S, H, D, P, U.DEV)


def test_two_streams_at_once_match_each_alone():
    a = U.to_device(W.make_inputs(U.small_config("gqa_bf16_g4"), seed=61))
    b = U.to_device(W.make_inputs(U.small_config("mha_fp8_d128"), seed=62))
    ref_a, ref_b = buffers(a), buffers(b)
    decode_into(a, ref_a)
    decode_into(b, ref_b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got_a, got_b = buffers(a), buffers(b)
    U.note("two streams")
    for _ in range(3):  # several rounds in flight on both streams
        decode_into(a, got_a, stream=s1)
        decode_into(b, got_b, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(got_a[0], ref_a[0]) and torch.equal(got_b[0], ref_b[0])


def test_cascade_in_a_graph_matches_eager():
    cfg = U.small_config("gqa_bf16_g4").replace(num_seqs=4)
    lens = [0, 300, 777, 1600]
    inp = W.make_inputs(cfg, seed=63, lens=lens)
    ha, hb = split_pages(inp, [0, 5, 20, 40])
    da, db = U.to_device(ha), U.to_device(hb)
    db["query"] = da["query"]  # one query tensor: rewritten in place between replays
    S, H, D = da["query"].shape
    PS, P = cfg.partition_size, cfg.max_num_partitions

    def alloc():
        return dict(oa=torch.zeros(S, H, D, device=U.DEV), la=torch.zeros(S, H, device=U.DEV),
                    ob=torch.zeros(S, H, D, device=U.DEV), lb=torch.zeros(S, H, device=U.DEV),
                    out=torch.zeros(S, H, D, device=U.DEV), lse=torch.zeros(S, H, device=U.DEV),
                    wa=pa.workspace(S, H, D, P, U.DEV), wb=pa.workspace(S, H, D, P, U.DEV))

    def cascade(b):
        for d, o, l, w in ((da, b["oa"], b["la"], b["wa"]), (db, b["ob"], b["lb"], b["wb"])):
            pa.paged_attn_decode_lse(o, l, *w, d["query"], d["key_cache"], d["value_cache"],
                                     d["block_tables"], d["seq_lens"], d["scale"], PS)
        pa.paged_attn_merge_states(b["out"], b["lse"], b["oa"], b["la"], b["ob"], b["lb"])

    g_bufs, e_bufs = alloc(), alloc()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the path outside capture
        cascade(g_bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    U.note("capture cascade")
    with torch.cuda.graph(graph):
        cascade(g_bufs)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(64)
    for rep in range(4):
        newq = torch.randn(S, H, D, generator=gen).to(torch.bfloat16).to(U.DEV)
        da["query"].copy_(newq)  # eager work between replays
        torch.cuda.synchronize()
        U.note(f"replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        cascade(e_bufs)
        torch.cuda.synchronize()
        for k in ("out", "lse", "oa", "la", "ob", "lb"):
            assert torch.equal(g_bufs[k].view(torch.int32), e_bufs[k].view(torch.int32)), (rep, k)
    # the eager cascade itself equals the oracle's whole-sequence attention
    full = dict(inp)
    full["query"] = da["query"].cpu()
    ref, ref_lse = oracle.attention_lse(full["query"], full["key_cache"], full["value_cache"],
                                        full["block_tables"], full["seq_lens"], full["scale"])
    U.assert_close("graph cascade out", e_bufs["out"].cpu(), ref)


@pytest.mark.parametrize("ps", [256, 1024], ids=["four_partitions", "one_partition"])
def test_multi_launch_call_in_a_graph_matches_eager(ps):
    """A call that the host splits into several column launches (8 query heads
    x 6 query tokens = 48 columns per kv head: launches of 32 and 16) captured
    in a graph: every replay, with the query rewritten in place between
    replays, gives the bits of the same call run eagerly. With 1024-token
    partitions every row has one partition (the reduce's one-partition form)."""
    lens = [0, 5, 300, 777]
    cfg = W.DecodeConfig("graph_mq", num_seqs=len(lens), num_heads=32, num_kv_heads=4,
                         head_size=128, block_size=16, partition_size=ps, dtype="bf16",
                         len_lo=0, len_hi=max(lens), num_queries=6)
    inp = W.make_inputs(cfg, seed=65, lens=lens)
    d = U.to_device(inp)
    q = d["query"]
    S, M, H, D = q.shape
    P = cfg.max_num_partitions

    def alloc():
        return dict(out=torch.zeros(S, M, H, D, device=U.DEV),
                    lse=torch.zeros(S, M, H, device=U.DEV),
                    tmp=torch.zeros(S, M, H, P, D, device=U.DEV),
                    es=torch.zeros(S, M, H, P, device=U.DEV),
                    ml=torch.zeros(S, M, H, P, device=U.DEV))

    def call(b):
        pa.paged_attn_decode_ex(b["out"], b["tmp"], b["es"], b["ml"], q, d["key_cache"],
                                d["value_cache"], d["block_tables"], d["seq_lens"], d["scale"],
                                cfg.partition_size, lse=b["lse"])

    g_bufs, e_bufs = alloc(), alloc()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the path outside capture
        call(g_bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    U.note(f"capture multi-launch call ps={ps}")
    with torch.cuda.graph(graph):
        call(g_bufs)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(66)
    for rep in range(3):
        q.copy_(torch.randn(S, M, H, D, generator=gen).to(torch.bfloat16).to(U.DEV))
        torch.cuda.synchronize()
        U.note(f"replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        call(e_bufs)
        torch.cuda.synchronize()
        for k in ("out", "lse", "es", "ml"):
            assert torch.equal(g_bufs[k].view(torch.int32), e_bufs[k].view(torch.int32)), (rep, k)
    host = dict(inp)
    host["query"] = q.cpu()
    ref = oracle.attention(host["query"], host["key_cache"], host["value_cache"],
                           host["block_tables"], host["seq_lens"], host["scale"])
    U.assert_close("graph multi-launch out", e_bufs["out"].cpu(), ref)
