"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host with the documented status
codes and a message. Every call here fails validation (or is the documented
num_seqs == 0 no-op), so nothing is ever enqueued on a device.
"""
import ctypes
import glob
import os
import re

import pytest
import torch

import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 40  # a 16-byte aligned, never dereferenced address


@pytest.fixture(scope="module", autouse=True)
def built():
    pa.ensure_built()


def declared_symbols():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        names += re.findall(r"PA_API\s+[\w\s\*]+?\b(\w+)\s*\(", open(h).read())
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for n in ("paged_attn_v2_partition", "paged_attn_v2_reduce", "paged_attn_decode",
              "paged_attn_last_error", "paged_attn_abi_version",
              "paged_attn_default_partition_size", "paged_attn_partition_span",
              "paged_attn_plan_partition_size"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for n in declared_symbols():
        assert hasattr(lib, n), n


def test_ceiling_library_exports_its_symbols():
    """libpa_ceiling.so (the benchmark's read-only page-gather instrument)
    exports what include/pa_ceiling.h declares, and rejects bad sizes on the
    host (nothing is launched)."""
    from paged_kv_cache_v2_amd import ceiling
    text = open(os.path.join(ROOT, "include", "pa_ceiling.h")).read()
    names = re.findall(r"PA_CEILING_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)
    assert sorted(names) == ["pa_gather_ceiling", "pa_gather_ceiling_sink_words", "pa_gather_units"]
    L = ceiling.lib()
    for n in names:
        assert hasattr(L, n), n
    W = ceiling.sink_words()
    assert W > 0
    assert L.pa_gather_ceiling(FAKE, 1, FAKE, FAKE, FAKE, 10, 2, 4096, 10, None) == -2  # sink
    assert L.pa_gather_ceiling(FAKE, W, FAKE, FAKE, FAKE, 10, 2, 3000, 10, None) == -2  # page
    assert L.pa_gather_ceiling(None, W, FAKE, FAKE, FAKE, 10, 2, 4096, 10, None) == -1
    assert L.pa_gather_ceiling(FAKE, W, FAKE + 4, FAKE, FAKE, 10, 2, 4096, 10, None) == -4
    assert L.pa_gather_ceiling(FAKE, W, FAKE, FAKE, FAKE, -1, 2, 4096, 10, None) == -2
    assert L.pa_gather_ceiling(FAKE, W, FAKE, FAKE, FAKE, 0, 2, 4096, 10, None) == 0  # no-op
    bt = torch.tensor([[3, 1, 7, -1], [5, -1, -1, -1], [0, 0, 0, 0]], dtype=torch.int32)
    sl = torch.tensor([40, 16, 0], dtype=torch.int32)
    assert ceiling.page_list(bt, sl, 16).tolist() == [3, 1, 7, 5]
    # the unit-structured gather: host-side rejections, nothing launched
    assert L.pa_gather_units(FAKE, 8, FAKE, FAKE, FAKE, FAKE, 0, 10, 4096, 2, None) == 0  # no-op
    assert L.pa_gather_units(FAKE, 8, FAKE, FAKE, FAKE, FAKE, -1, 10, 4096, 2, None) == -2
    assert L.pa_gather_units(FAKE, 8, FAKE, FAKE, FAKE, FAKE, 2, 10, 4096, 0, None) == -2  # wgs
    assert L.pa_gather_units(FAKE, 8, FAKE, FAKE, FAKE, FAKE, 2, 0, 4096, 2, None) == -2  # pages
    assert L.pa_gather_units(None, 8, FAKE, FAKE, FAKE, FAKE, 2, 10, 4096, 2, None) == -1
    assert L.pa_gather_units(FAKE, 8, FAKE, FAKE, None, FAKE, 2, 10, 4096, 2, None) == -1
    assert L.pa_gather_units(FAKE, 8, FAKE + 4, FAKE, FAKE, FAKE, 2, 10, 4096, 2, None) == -4
    assert L.pa_gather_units(FAKE, 7, FAKE, FAKE, FAKE, FAKE, 2, 10, 4096, 2, None) == -2  # sink
    assert L.pa_gather_units(FAKE, 8, FAKE, FAKE, FAKE, FAKE, 2, 10, 16384, 2, None) == -2  # page
    # units: (sequence, span of 2 pages) pairs by page count, then kv head
    pages, off, n = ceiling.unit_pages(bt, sl, 16, 2, 2)
    assert n == 6 and off.tolist() == [0, 2, 4, 5, 6, 7, 8]
    assert pages.tolist() == [3 * 2, 1 * 2, 3 * 2 + 1, 1 * 2 + 1, 5 * 2, 5 * 2 + 1, 7 * 2, 7 * 2 + 1]


def test_abi_version_and_default_partition_size():
    assert pa.abi_version() == 2
    for D, BS, dt, G in [(128, 16, torch.bfloat16, 4), (256, 32, torch.float16, 1),
                         (64, 16, torch.float32, 1), (128, 16, torch.bfloat16, 32)]:
        ps = pa.default_partition_size(D, BS, dt, G)
        assert ps > 0 and ps % BS == 0
    with pytest.raises(RuntimeError):
        pa.default_partition_size(96, 16, torch.float16, 1)


def test_plan_partition_size():
    """The longest partition (4096 tokens, 2048 for 8-bit caches) whose units
    (sequences x kv heads x partitions) fill every resident workgroup, no
    longer than the longest sequence needs, at least 128. (On a host without a
    device the plan assumes two workgroups per CU and 256 CUs: 512 slots.)"""
    bf, f16, f32, f8 = torch.bfloat16, torch.float16, torch.float32, torch.float8_e4m3fn
    plan = pa.plan_partition_size
    assert plan(128, 32, 8, 128, 16, 4096, bf) == 4096     # 1024 units
    assert plan(8, 64, 8, 128, 16, 32768, bf) == 4096      # 8 x 8 x 8 = 512 units
    assert plan(128, 32, 8, 128, 16, 4096, f8) == 2048     # 8-bit caches stop at 2048
    assert plan(1, 32, 8, 128, 16, 32768, bf) == 512       # 8 x 64 = 512 units
    assert plan(1, 8, 1, 128, 16, 1 << 20, bf) == 2048     # 512 partitions of 2048
    assert plan(1, 8, 1, 128, 16, 1000, bf) == 128         # too few units at any size
    assert plan(64, 32, 32, 128, 16, 2048, f16) == 2048    # one partition covers 2048
    assert plan(32, 16, 16, 256, 32, 8192, f16) == 4096
    assert plan(2, 4, 4, 64, 16, 100, f32) == 128          # never below 128
    assert plan(0, 4, 4, 64, 16, 0, f32) == 128
    for args in [(4, 32, 8, 96, 16, 100, bf), (4, 32, 8, 128, 64, 100, bf),
                 (4, 32, 4, 64, 16, 100, f32)]:                 # G = 8 with fp32
        with pytest.raises(RuntimeError, match="unsupported|group"):
            plan(*args)
    for args in [(4, 30, 8, 128, 16, 100, bf), (-1, 32, 8, 128, 16, 100, bf),
                 (4, 32, 8, 128, 16, -1, bf)]:
        with pytest.raises(RuntimeError, match="bad sizes"):
            plan(*args)


def test_planned_sizes_are_accepted_by_the_launch_plan():
    """Every size the planner returns is one the launchers take: a multiple of
    the block size, at most 256 pages, and a launch plan that passes every
    check a decode call makes (the LDS of a partition's parked state, the
    32-bit workspace offsets) for ceil(max_seq_len / size) partitions, on this
    host's device limits (64 KiB of LDS per workgroup without a device)."""
    dts = [torch.float32, torch.float16, torch.bfloat16, torch.float8_e4m3fn]
    for S in (0, 1, 7, 128, 4096):
        for H, KH in ((4, 4), (32, 8), (64, 1)):
            for D in (64, 128, 256):
                for BS in (16, 32):
                    for L in (0, 1, 100, 4096, 100_000):
                        for dt in dts:
                            if dt == torch.float32 and H // KH > 4:
                                continue
                            qdt = torch.bfloat16 if dt == torch.float8_e4m3fn else dt
                            try:
                                ps = pa.plan_partition_size(S, H, KH, D, BS, L, dt)
                            except RuntimeError as e:
                                # a geometry no partition size makes fit this device's
                                # LDS: the decode call rejects it the same way
                                assert "LDS" in str(e) and S > 0, e
                                with pytest.raises(RuntimeError, match="LDS"):
                                    pa.decode_plan(S, 1, H, KH, D, BS, max(1, -(-L // 128)),
                                                   128, qdt, dt)
                                continue
                            assert 128 <= ps <= 4096 and ps % BS == 0 and ps // BS <= 256
                            assert ps <= 2048 or dt != torch.float8_e4m3fn
                            P = max(1, -(-L // ps))
                            span = pa.partition_span(S, H, KH, D, BS, P, ps, dt)
                            assert span in (1, 2, 4, 8)
                            if S > 0:  # the whole launch check a decode call makes
                                plan = pa.decode_plan(S, 1, H, KH, D, BS, P, ps, qdt, dt)
                                assert plan["span"] in (1, 2, 4, 8) and plan["entries"] >= 1


def test_partition_span_plan():
    """Spans of up to 8 partitions and 2 MiB of K+V while the grid keeps two
    workgroups per resident slot; 1 for small grids or long partitions. (On a
    host without a device the plan assumes two workgroups per CU, 256 CUs and
    the 64 KiB per-workgroup LDS fallback.)"""
    bf, f16, f32 = torch.bfloat16, torch.float16, torch.float32
    assert pa.partition_span(128, 32, 8, 128, 16, 8, 512, bf) == 4     # GQA (LDS caps 8 here)
    assert pa.partition_span(8, 64, 8, 128, 16, 64, 512, bf) == 2      # long context: LDS
    assert pa.partition_span(128, 32, 8, 128, 16, 4, 1024, bf) == 4    # 4096 tokens, 2 MiB
    assert pa.partition_span(128, 32, 8, 128, 16, 2, 2048, bf) == 2
    assert pa.partition_span(32, 16, 16, 256, 32, 16, 512, f16) == 4   # 2 MiB, D = 256
    assert pa.partition_span(64, 32, 32, 128, 16, 4, 512, f16) == 4    # MHA: all 4 partitions
    assert pa.partition_span(2, 4, 4, 64, 16, 2, 64, f32) == 1         # small grid
    assert pa.partition_span(128, 8, 8, 64, 16, 4, 64, f32) == 4
    # 32 query heads per kv head: two column tiles, whose parked state for two
    # partitions would exceed the LDS cap
    assert pa.partition_span(128, 64, 2, 128, 16, 8, 512, bf) == 1
    with pytest.raises(RuntimeError):
        pa.partition_span(2, 4, 3, 64, 16, 2, 64, f32)                  # H % KH
    with pytest.raises(RuntimeError):
        pa.partition_span(2, 4, 4, 96, 16, 2, 64, f32)                  # head size


# Valid baseline: bf16, S=2, H=8, KH=2, D=128, BS=16, B=64, MB=8, P=1, PS=512
BASE = dict(S=2, H=8, KH=2, D=128, BS=16, B=64, MB=8, P=1, PS=512, dt=binding.PA_BF16)


def part(ptrs=None, **kw):
    a = dict(BASE, **kw)
    p = [FAKE] * 8 if ptrs is None else ptrs
    return pa.lib().paged_attn_v2_partition(*p, a["S"], a["H"], a["KH"], a["D"], a["BS"], a["B"],
                                            a["MB"], a["P"], a["PS"], 0.125, a["dt"], None)


def decode(odt, **kw):
    a = dict(BASE, **kw)
    return pa.lib().paged_attn_decode(*([FAKE] * 9), a["S"], a["H"], a["KH"], a["D"], a["BS"],
                                      a["B"], a["MB"], a["P"], a["PS"], 0.125, a["dt"], odt, None)


def reduce(ptrs=None, S=2, H=8, D=128, P=1, PS=512, odt=binding.PA_F32):
    p = [FAKE] * 5 if ptrs is None else ptrs
    return pa.lib().paged_attn_v2_reduce(*p, S, H, D, P, PS, odt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(S=-1), binding.PA_ERR_SHAPE),
    (dict(H=6, KH=4), binding.PA_ERR_SHAPE),
    (dict(D=100), binding.PA_ERR_SHAPE),               # 100 % 8 != 0
    (dict(PS=500), binding.PA_ERR_SHAPE),              # 500 % 16 != 0
    (dict(PS=0), binding.PA_ERR_SHAPE),
    (dict(P=0), binding.PA_ERR_SHAPE),
    (dict(MB=0), binding.PA_ERR_SHAPE),
    (dict(B=0), binding.PA_ERR_SHAPE),
    (dict(D=96), binding.PA_ERR_UNSUPPORTED),
    (dict(D=512), binding.PA_ERR_UNSUPPORTED),
    (dict(BS=8, PS=512), binding.PA_ERR_UNSUPPORTED),
    (dict(dt=7), binding.PA_ERR_UNSUPPORTED),
    (dict(H=16, KH=2, dt=binding.PA_F32), binding.PA_ERR_UNSUPPORTED),  # fp32, G = 8
    (dict(H=64, KH=2, dt=binding.PA_F32), binding.PA_ERR_UNSUPPORTED),  # fp32, G = 32
    (dict(PS=16 * 512), binding.PA_ERR_UNSUPPORTED),   # PS / BS > 256
])
def test_partition_rejects(kw, code):
    assert part(**kw) == code
    assert pa.last_error() != ""


@pytest.mark.parametrize("which", range(8))
def test_partition_null_pointer(which):
    ptrs = [FAKE] * 8
    ptrs[which] = None
    assert part(ptrs) == binding.PA_ERR_NULL
    assert "NULL" in pa.last_error()


@pytest.mark.parametrize("which", [0, 3, 4, 5])  # tmp_output, query, key_cache, value_cache
def test_partition_misaligned(which):
    ptrs = [FAKE] * 8
    ptrs[which] = FAKE + 2
    assert part(ptrs) == binding.PA_ERR_ALIGN


def test_num_seqs_zero_is_noop_even_with_null_pointers():
    assert part([None] * 8, S=0) == binding.PA_OK
    assert pa.last_error() == ""
    assert reduce([None] * 5, S=0) == binding.PA_OK
    assert pa.lib().paged_attn_decode(*([None] * 9), 0, 8, 2, 128, 16, 64, 8, 1, 512, 0.125,
                                      binding.PA_BF16, binding.PA_F32, None) == binding.PA_OK


def part_fp8(q_dtype=binding.PA_BF16, k_scale=1.0, v_scale=1.0, **kw):
    a = dict(BASE, **kw)
    return pa.lib().paged_attn_v2_partition_fp8(*([FAKE] * 8), a["S"], a["H"], a["KH"], a["D"],
                                                a["BS"], a["B"], a["MB"], a["P"], a["PS"], 0.125,
                                                k_scale, v_scale, q_dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q_dtype=binding.PA_F32), binding.PA_ERR_UNSUPPORTED),
    (dict(q_dtype=binding.PA_FP8_E4M3), binding.PA_ERR_UNSUPPORTED),
    (dict(k_scale=float("inf")), binding.PA_ERR_SHAPE),
    (dict(v_scale=float("nan")), binding.PA_ERR_SHAPE),
    (dict(D=72), binding.PA_ERR_SHAPE),                # 72 % 16 != 0 (x = 16 for 8-bit)
    (dict(D=96), binding.PA_ERR_UNSUPPORTED),          # head size, also with an 8-bit cache
])
def test_fp8_partition_rejects(kw, code):
    assert part_fp8(**kw) == code
    assert pa.last_error() != ""


def part_mq(M=2, q_dtype=binding.PA_BF16, kv_dtype=binding.PA_BF16, **kw):
    a = dict(BASE, **kw)
    return pa.lib().paged_attn_v2_partition_mq(*([FAKE] * 8), a["S"], M, a["H"], a["KH"], a["D"],
                                               a["BS"], a["B"], a["MB"], a["P"], a["PS"], 0.125,
                                               1.0, 1.0, q_dtype, kv_dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), binding.PA_ERR_SHAPE),
    (dict(M=2, H=64, KH=2, D=96), binding.PA_ERR_UNSUPPORTED),  # group 32, unknown head size
    (dict(q_dtype=binding.PA_F32, kv_dtype=binding.PA_F32), binding.PA_ERR_UNSUPPORTED),
    (dict(q_dtype=binding.PA_F16, kv_dtype=binding.PA_BF16), binding.PA_ERR_UNSUPPORTED),
])
def test_multi_token_rejects(kw, code):
    assert part_mq(**kw) == code
    assert pa.last_error() != ""


def test_plain_calls_reject_8bit_cache():
    assert part(dt=binding.PA_FP8_E4M3) == binding.PA_ERR_UNSUPPORTED
    assert decode(binding.PA_F32, dt=binding.PA_FP8_E4M3) == binding.PA_ERR_UNSUPPORTED
    assert "fp8" in pa.last_error()


def test_decode_out_dtype_must_be_f32_or_kv():
    assert decode(binding.PA_F16) == binding.PA_ERR_UNSUPPORTED
    assert decode(binding.PA_BF16, D=96) == binding.PA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(S=-2), binding.PA_ERR_SHAPE),
    (dict(H=0), binding.PA_ERR_SHAPE),
    (dict(P=0), binding.PA_ERR_SHAPE),
    (dict(PS=0), binding.PA_ERR_SHAPE),
    (dict(D=96), binding.PA_ERR_UNSUPPORTED),
    (dict(odt=9), binding.PA_ERR_UNSUPPORTED),
])
def test_reduce_rejects(kw, code):
    assert reduce(**kw) == code


def test_reduce_null_and_align():
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert reduce(ptrs) == binding.PA_ERR_NULL
    ptrs = [FAKE] * 5
    ptrs[0] = FAKE + 4
    assert reduce(ptrs) == binding.PA_ERR_ALIGN


def test_binding_rejects_host_tensors():
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    kc = torch.zeros(4, 2, 16, 16, 8, dtype=torch.bfloat16)
    vc = torch.zeros(4, 2, 128, 16, dtype=torch.bfloat16)
    bt = torch.zeros(2, 8, dtype=torch.int32)
    sl = torch.zeros(2, dtype=torch.int32)
    tmp, es, ml = (torch.zeros(2, 8, 1, 128), torch.zeros(2, 8, 1), torch.zeros(2, 8, 1))
    with pytest.raises(ValueError):
        pa.paged_attn_v2_partition(tmp, es, ml, q, kc, vc, bt, sl, 0.1, 512)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(binding, "_LIB", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libpaged_attn.so")
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


def reduce_lse(lse=FAKE, ptrs=None, S=2, M=1):
    ptrs = ptrs or [FAKE] * 5
    return pa.lib().paged_attn_v2_reduce_lse(ptrs[0], lse, *ptrs[1:], S, M, 8, 128, 4, 512,
                                             binding.PA_F32, None)


def test_reduce_lse_rejects():
    assert reduce_lse(lse=None) == binding.PA_ERR_NULL
    assert reduce_lse(lse=FAKE + 2) == binding.PA_ERR_ALIGN
    assert reduce_lse(M=0) == binding.PA_ERR_SHAPE
    ptrs = [FAKE] * 5
    ptrs[1] = None
    assert reduce_lse(ptrs=ptrs) == binding.PA_ERR_NULL
    assert reduce_lse(lse=None, ptrs=[None] * 5, S=0) == binding.PA_OK


def test_decode_lse_rejects():
    lib = pa.lib()
    args = lambda lse, M=1, qdt=binding.PA_BF16, kvdt=binding.PA_BF16: (
        FAKE, lse, *([FAKE] * 8), 2, M, 8, 2, 128, 16, 64, 8, 1, 512, 0.125, 1.0, 1.0, qdt, kvdt,
        binding.PA_F32, None)
    assert lib.paged_attn_decode_lse(*args(None)) == binding.PA_ERR_NULL
    assert lib.paged_attn_decode_lse(*args(FAKE + 1)) == binding.PA_ERR_ALIGN
    assert lib.paged_attn_decode_lse(*args(FAKE, M=2, qdt=binding.PA_F32, kvdt=binding.PA_F32)) \
        == binding.PA_ERR_UNSUPPORTED  # several query tokens need a 16-bit query
    assert lib.paged_attn_decode_lse(*args(FAKE, qdt=binding.PA_F32)) == binding.PA_ERR_UNSUPPORTED


def merge(ptrs=None, rows=4, D=128, dt=binding.PA_BF16):
    ptrs = ptrs or [FAKE] * 6
    return pa.lib().paged_attn_merge_states(*ptrs, rows, D, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), binding.PA_ERR_SHAPE),
    (dict(D=-64), binding.PA_ERR_SHAPE),
    (dict(D=96), binding.PA_ERR_UNSUPPORTED),
    (dict(dt=binding.PA_FP8_E4M3), binding.PA_ERR_UNSUPPORTED),
    (dict(ptrs=[FAKE, FAKE, None, FAKE, FAKE, FAKE]), binding.PA_ERR_NULL),
    (dict(ptrs=[FAKE, FAKE, FAKE, FAKE, FAKE, None]), binding.PA_ERR_NULL),
    (dict(ptrs=[FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE]), binding.PA_ERR_ALIGN),
    (dict(ptrs=[FAKE, FAKE, FAKE, FAKE + 2, FAKE, FAKE]), binding.PA_ERR_ALIGN),
    (dict(ptrs=[FAKE, FAKE + 1, FAKE, FAKE, FAKE, FAKE]), binding.PA_ERR_ALIGN),
])
def test_merge_states_rejects(kw, code):
    assert merge(**kw) == code
    assert pa.last_error() != ""


def test_merge_states_zero_rows_is_noop():
    assert merge(ptrs=[None] * 6, rows=0) == binding.PA_OK
    assert pa.last_error() == ""


def test_ex_entries_reject_misaligned_alibi_and_lse():
    lib = pa.lib()
    part_args = lambda al: (*([FAKE] * 8), 2, 1, 8, 2, 128, 16, 64, 8, 1, 512, 0.125, 1.0, 1.0,
                            al, binding.PA_BF16, binding.PA_BF16, None)
    assert lib.paged_attn_v2_partition_ex(*part_args(FAKE + 2)) == binding.PA_ERR_ALIGN
    assert "alibi" in pa.last_error()
    dec_args = lambda lse, al: (FAKE, lse, *([FAKE] * 8), 2, 1, 8, 2, 128, 16, 64, 8, 1, 512,
                                0.125, 1.0, 1.0, al, binding.PA_BF16, binding.PA_BF16,
                                binding.PA_F32, None)
    assert lib.paged_attn_decode_ex(*dec_args(FAKE + 1, None)) == binding.PA_ERR_ALIGN
    assert lib.paged_attn_decode_ex(*dec_args(None, FAKE + 1)) == binding.PA_ERR_ALIGN
    assert lib.paged_attn_decode_ex(*dec_args(None, None)[:10], 2, 2, 64, 2, 96,
                                    *dec_args(None, None)[15:]) \
        == binding.PA_ERR_UNSUPPORTED  # two query tokens, group 32, unknown head size


def test_size_limits_are_rejected_before_launch():
    """Shapes whose 32-bit offsets or launch grids would overflow fail on the host."""
    # one launch's tmp_output rows past 2 GiB (32-bit buffer offsets): G * P * D * 4 bytes
    assert part(H=8, KH=2, D=256, P=600_000) == binding.PA_ERR_UNSUPPORTED
    assert "2 GiB" in pa.last_error()
    # more than 2^31 - 1 workgroups (2^30 sequences, each at least one span)
    assert part(S=1 << 30, H=1, KH=1, D=64, P=2048) == binding.PA_ERR_UNSUPPORTED
    assert "work units" in pa.last_error()
    # more than 2^31 - 1 (query token, head) columns per kv head
    assert part_mq(M=1 << 30) == binding.PA_ERR_UNSUPPORTED
    assert "columns" in pa.last_error()
    # more than 2^31 - 1 reduce rows
    assert reduce(S=1 << 20, H=4096) == binding.PA_ERR_UNSUPPORTED
    assert "rows" in pa.last_error()
