"""The Python binding's argument checks (CPU only, no device work).

The binding only marshals arguments: it checks dtypes, ranks, shapes and
that every tensor is a contiguous device tensor, and raises ValueError with a
message naming the problem before the library is called. These checks run in
a fixed order (ranks and dtypes first), so CPU tensors exercise the ones
before the device check, and the device check itself.
"""
import pytest
import torch

import paged_kv_cache_v2_amd as pa


def tensors(S=2, H=8, KH=2, D=64, BS=16, B=8, MB=4, P=2, dt=torch.float16):
    x = 16 // torch.empty(0, dtype=dt).element_size()
    return dict(
        out=torch.zeros(S, H, D),
        tmp=torch.zeros(S, H, P, D), es=torch.zeros(S, H, P), ml=torch.zeros(S, H, P),
        q=torch.zeros(S, H, D, dtype=dt),
        kc=torch.zeros(B, KH, D // x, BS, x, dtype=dt), vc=torch.zeros(B, KH, D, BS, dtype=dt),
        bt=torch.zeros(S, MB, dtype=torch.int32), sl=torch.zeros(S, dtype=torch.int32))


def decode(t, **over):
    a = dict(t, **over)
    pa.paged_attn_decode(a["out"], a["tmp"], a["es"], a["ml"], a["q"], a["kc"], a["vc"], a["bt"],
                         a["sl"], 0.125, 64)


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="device tensors"):
        decode(tensors())


def test_index_tensors_must_be_int32():
    t = tensors()
    with pytest.raises(ValueError, match="int32"):
        decode(t, bt=t["bt"].long())
    with pytest.raises(ValueError, match="int32"):
        decode(t, sl=t["sl"].long())


def test_query_and_caches_share_a_dtype():
    t = tensors()
    with pytest.raises(ValueError, match="one dtype"):
        decode(t, q=t["q"].to(torch.bfloat16))


def test_8bit_caches_need_the_fp8_calls():
    t = tensors()
    kc8 = torch.zeros(t["kc"].shape[0], 2, 4, 16, 16).to(torch.float8_e4m3fn)
    vc8 = t["vc"].to(torch.float8_e4m3fn)
    with pytest.raises(ValueError, match="_fp8"):
        decode(t, kc=kc8, vc=vc8)
    with pytest.raises(ValueError, match="float8_e4m3fn"):
        pa.paged_attn_decode_fp8(t["out"], t["tmp"], t["es"], t["ml"], t["q"], t["kc"], t["vc"],
                                 t["bt"], t["sl"], 0.125, 1.0, 1.0, 64)


def test_ranks_are_checked():
    t = tensors()
    with pytest.raises(ValueError, match=r"query \[S,H,D\]"):
        decode(t, q=t["q"][None])
    with pytest.raises(ValueError, match=r"\[S, H, D\]"):
        pa.paged_attn_v2_reduce(t["out"][None], t["tmp"], t["es"], t["ml"], t["sl"], 64)


def test_multi_token_calls_check_their_ranks():
    t = tensors()
    with pytest.raises(ValueError):
        pa.paged_attn_decode_mq(t["out"], t["tmp"], t["es"], t["ml"], t["q"], t["kc"], t["vc"],
                                t["bt"], t["sl"], 0.125, 64)


def test_host_helpers_reject_unknown_dtypes():
    with pytest.raises(ValueError, match="cache dtype"):
        pa.plan_partition_size(4, 8, 2, 128, 16, 100, torch.int8)
    with pytest.raises(ValueError, match="cache dtype"):
        pa.default_partition_size(128, 16, torch.float64, 4)
    with pytest.raises(ValueError, match="cache dtype"):
        pa.partition_span(4, 8, 2, 128, 16, 1, 512, torch.int32)
