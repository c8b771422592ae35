"""Thin Python binding of libpaged_attn.so (the C ABI in include/paged_attn.h).

Argument marshalling only: shapes are read off torch tensors, pointers and
the current HIP stream are passed through, and a nonzero status becomes a
RuntimeError carrying the library's message. Every step of the computation
runs in the HIP kernels; there is no other implementation to fall back on,
and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (load torch's HIP runtime first so both share one runtime)

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_ALIGN, PA_ERR_HIP = 0, -1, -2, -3, -4, -5
_DT = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
_CACHE_DT = {**_DT, torch.float8_e4m3fn: PA_FP8_E4M3}

# PAGED_ATTN_LIB: load another build of the same sources (e.g. one whose host
# code is instrumented by sanitizers) instead of the in-tree library.
LIB_PATH = os.environ.get("PAGED_ATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpaged_attn.so")
_LIB = None

_P, _I32, _I64, _F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "paged_attn_v2_partition": [_P, _P, _P, _P, _P, _P, _P, _P] + [_I32] * 9 + [_F32, _I32, _P],
    "paged_attn_v2_reduce": [_P, _P, _P, _P, _P] + [_I32] * 6 + [_P],
    "paged_attn_decode": [_P, _P, _P, _P, _P, _P, _P, _P, _P] + [_I32] * 9 + [_F32, _I32, _I32, _P],
    "paged_attn_last_error": [],
    "paged_attn_abi_version": [],
    "paged_attn_default_partition_size": [_I32, _I32, _I32, _I32],
    "paged_attn_partition_span": [_I32] * 8,
    "paged_attn_plan_partition_size": [_I32] * 7,
    "paged_attn_decode_plan": [_I32] * 10 + [_P],
    "paged_attn_decode_noalloc": [_P] * 7 + [_I32] * 10 + [_F32, _F32, _F32, _P, _I32, _I32,
                                                          _I32, _P],
    "paged_attn_v2_partition_fp8": [_P] * 8 + [_I32] * 9 + [_F32, _F32, _F32, _I32, _P],
    "paged_attn_decode_fp8": [_P] * 9 + [_I32] * 9 + [_F32, _F32, _F32, _I32, _I32, _P],
    "paged_attn_v2_partition_mq": [_P] * 8 + [_I32] * 10 + [_F32, _F32, _F32, _I32, _I32, _P],
    "paged_attn_v2_reduce_mq": [_P] * 5 + [_I32] * 7 + [_P],
    "paged_attn_decode_mq": [_P] * 9 + [_I32] * 10 + [_F32, _F32, _F32, _I32, _I32, _I32, _P],
    "paged_attn_v2_reduce_lse": [_P] * 6 + [_I32] * 7 + [_P],
    "paged_attn_decode_lse": [_P] * 10 + [_I32] * 10 + [_F32, _F32, _F32, _I32, _I32, _I32, _P],
    "paged_attn_merge_states": [_P] * 6 + [_I64, _I32, _I32, _P],
    "paged_attn_v2_partition_ex": [_P] * 8 + [_I32] * 10 + [_F32, _F32, _F32, _P, _I32, _I32, _P],
    "paged_attn_decode_ex": [_P] * 10 + [_I32] * 10 + [_F32, _F32, _F32, _P, _I32, _I32, _I32,
                                                        _P],
}


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m paged_kv_cache_v2_amd.build`. "
                "There is no fallback implementation.")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "paged_attn_last_error" else ctypes.c_int
        _LIB = L
    return _LIB


def last_error() -> str:
    return lib().paged_attn_last_error().decode()


def abi_version() -> int:
    return lib().paged_attn_abi_version()


def _cache_dt(dtype: torch.dtype) -> int:
    _need(dtype in _CACHE_DT, f"cache dtype must be float32, float16, bfloat16 or "
          f"float8_e4m3fn, got {dtype}")
    return _CACHE_DT[dtype]


def default_partition_size(head_size: int, block_size: int, dtype: torch.dtype, group: int) -> int:
    rc = lib().paged_attn_default_partition_size(head_size, block_size, _cache_dt(dtype), group)
    if rc < 0:
        raise RuntimeError(f"paged_attn_default_partition_size: {last_error()} (code {rc})")
    return rc


def plan_partition_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                        block_size: int, max_seq_len: int, dtype: torch.dtype) -> int:
    """Partition size for this batch (see paged_attn_plan_partition_size)."""
    rc = lib().paged_attn_plan_partition_size(num_seqs, num_heads, num_kv_heads, head_size,
                                              block_size, max_seq_len, _cache_dt(dtype))
    if rc < 0:
        raise RuntimeError(f"paged_attn_plan_partition_size: {last_error()} (code {rc})")
    return rc


def partition_span(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                   block_size: int, max_num_partitions: int, partition_size: int,
                   dtype: torch.dtype) -> int:
    """Partitions per workgroup the launchers use for these sizes (plan inspection)."""
    rc = lib().paged_attn_partition_span(num_seqs, num_heads, num_kv_heads, head_size, block_size,
                                         max_num_partitions, partition_size, _cache_dt(dtype))
    if rc < 0:
        raise RuntimeError(f"paged_attn_partition_span: {last_error()} (code {rc})")
    return rc


def decode_plan(num_seqs: int, num_queries: int, num_heads: int, num_kv_heads: int,
                head_size: int, block_size: int, max_num_partitions: int, partition_size: int,
                q_dtype: torch.dtype, kv_dtype: torch.dtype) -> dict:
    """The one-call decode's launch plan for these sizes (host-side query):
    span (partitions per workgroup), roll (ring slots of the rolling merge, 0:
    none), entries (span entries per row; 1: no reduce), launches (column
    launches)."""
    _need(q_dtype in _DT, f"query dtype must be float32, float16 or bfloat16, got {q_dtype}")
    out = (ctypes.c_int32 * 4)()
    _check("paged_attn_decode_plan",
           lib().paged_attn_decode_plan(num_seqs, num_queries, num_heads, num_kv_heads,
                                        head_size, block_size, max_num_partitions,
                                        partition_size, _DT[q_dtype], _cache_dt(kv_dtype), out))
    return dict(span=out[0], roll=out[1], entries=out[2], launches=out[3])


def _check(name: str, rc: int) -> None:
    if rc != PA_OK:
        raise RuntimeError(f"{name}: {last_error()} (code {rc})")


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _device(t: torch.Tensor):
    """Make the tensors' device current for the call (the library launches on the
    current device, on a stream of that device)."""
    return torch.cuda.device(t.device)


def _one_device(*tensors) -> None:
    _need(len({t.device for t in tensors if t is not None}) == 1,
          "all tensors of a call must be on one device")


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _kv_geometry(query, key_cache, value_cache, block_tables, seq_lens, fp8: bool = False):
    _need(query.dim() == 3 and key_cache.dim() == 5 and value_cache.dim() == 4,
          "query [S,H,D], key_cache [B,KH,D/x,BS,x], value_cache [B,KH,D,BS] expected")
    if fp8:
        _need(query.dtype in (torch.float16, torch.bfloat16) and
              key_cache.dtype == torch.float8_e4m3fn and value_cache.dtype == torch.float8_e4m3fn,
              "the fp8 calls take an f16/bf16 query and float8_e4m3fn key/value caches")
    else:
        _need(query.dtype in _DT and key_cache.dtype == query.dtype and
              value_cache.dtype == query.dtype,
              "query, key_cache and value_cache must share one dtype (f32, f16 or bf16); "
              "float8_e4m3fn caches go through the *_fp8 calls")
    _need(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32,
          "block_tables and seq_lens must be int32")
    for t in (query, key_cache, value_cache, block_tables, seq_lens):
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
    S, H, D = query.shape
    B, KH, Dx, BS, x = key_cache.shape
    _need(x == 16 // key_cache.element_size() and Dx * x == D,
          "key_cache packing must be x = 16/sizeof(cache element)")
    _need(tuple(value_cache.shape) == (B, KH, D, BS), "value_cache shape mismatch")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S and seq_lens.shape == (S,),
          "block_tables [S, MB] and seq_lens [S] expected")
    return S, H, KH, D, BS, B, block_tables.shape[1]


def _stats_geometry(tmp_output, exp_sums, max_logits, S, H, D):
    _need(all(t.dtype == torch.float32 and t.is_cuda and t.is_contiguous()
              for t in (tmp_output, exp_sums, max_logits)),
          "tmp_output, exp_sums, max_logits must be contiguous fp32 device tensors")
    _need(tmp_output.dim() == 4 and tuple(tmp_output.shape[:2]) == (S, H) and tmp_output.shape[3] == D,
          "tmp_output must be [S, H, P, D]")
    P = tmp_output.shape[2]
    _need(tuple(exp_sums.shape) == (S, H, P) and tuple(max_logits.shape) == (S, H, P),
          "exp_sums and max_logits must be [S, H, P]")
    return P


def paged_attn_v2_partition(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                            block_tables, seq_lens, scale: float, partition_size: int,
                            stream=None) -> None:
    """Phase 1: per-partition attention into tmp_output / exp_sums / max_logits."""
    S, H, KH, D, BS, B, MB = _kv_geometry(query, key_cache, value_cache, block_tables, seq_lens)
    P = _stats_geometry(tmp_output, exp_sums, max_logits, S, H, D)
    _one_device(tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                seq_lens)
    with _device(query):
        rc = lib().paged_attn_v2_partition(
            tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(), query.data_ptr(),
            key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), S, H, KH, D, BS, B, MB, P, partition_size, float(scale),
            _DT[query.dtype], _stream(query, stream))
    _check("paged_attn_v2_partition", rc)


def paged_attn_v2_reduce(out, tmp_output, exp_sums, max_logits, seq_lens, partition_size: int,
                         stream=None) -> None:
    """Phase 2: cross-partition log-sum-exp combine into out [S, H, D]."""
    _need(out.dim() == 3 and out.dtype in _DT and out.is_cuda and out.is_contiguous(),
          "out must be a contiguous [S, H, D] f32/f16/bf16 device tensor")
    S, H, D = out.shape
    P = _stats_geometry(tmp_output, exp_sums, max_logits, S, H, D)
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_cuda and seq_lens.shape == (S,),
          "seq_lens must be an int32 [S] device tensor")
    _one_device(out, tmp_output, exp_sums, max_logits, seq_lens)
    with _device(out):
        rc = lib().paged_attn_v2_reduce(
            out.data_ptr(), tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(),
            seq_lens.data_ptr(), S, H, D, P, partition_size, _DT[out.dtype], _stream(out, stream))
    _check("paged_attn_v2_reduce", rc)


def paged_attn_decode(out, tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                      block_tables, seq_lens, scale: float, partition_size: int,
                      stream=None) -> None:
    """Phase 1 then phase 2 on one stream."""
    S, H, KH, D, BS, B, MB = _kv_geometry(query, key_cache, value_cache, block_tables, seq_lens)
    P = _stats_geometry(tmp_output, exp_sums, max_logits, S, H, D)
    _need(out.dim() == 3 and tuple(out.shape) == (S, H, D) and out.dtype in _DT and out.is_cuda
          and out.is_contiguous(), "out must be a contiguous [S, H, D] device tensor")
    _one_device(out, tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                seq_lens)
    with _device(query):
        rc = lib().paged_attn_decode(
            out.data_ptr(), tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(),
            query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), S, H, KH, D, BS, B, MB, P, partition_size, float(scale),
            _DT[query.dtype], _DT[out.dtype], _stream(query, stream))
    _check("paged_attn_decode", rc)


def paged_attn_v2_partition_fp8(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                                block_tables, seq_lens, scale: float, k_scale: float,
                                v_scale: float, partition_size: int, stream=None) -> None:
    """Phase 1 over float8_e4m3fn caches (key = byte * k_scale, value = byte * v_scale)."""
    S, H, KH, D, BS, B, MB = _kv_geometry(query, key_cache, value_cache, block_tables, seq_lens,
                                          fp8=True)
    P = _stats_geometry(tmp_output, exp_sums, max_logits, S, H, D)
    _one_device(tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                seq_lens)
    with _device(query):
        rc = lib().paged_attn_v2_partition_fp8(
            tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(), query.data_ptr(),
            key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), S, H, KH, D, BS, B, MB, P, partition_size, float(scale),
            float(k_scale), float(v_scale), _DT[query.dtype], _stream(query, stream))
    _check("paged_attn_v2_partition_fp8", rc)


def paged_attn_decode_fp8(out, tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                          block_tables, seq_lens, scale: float, k_scale: float, v_scale: float,
                          partition_size: int, stream=None) -> None:
    """Phase 1 then phase 2 over float8_e4m3fn caches, on one stream."""
    S, H, KH, D, BS, B, MB = _kv_geometry(query, key_cache, value_cache, block_tables, seq_lens,
                                          fp8=True)
    P = _stats_geometry(tmp_output, exp_sums, max_logits, S, H, D)
    _need(out.dim() == 3 and tuple(out.shape) == (S, H, D) and out.dtype in _DT and out.is_cuda
          and out.is_contiguous(), "out must be a contiguous [S, H, D] device tensor")
    _one_device(out, tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                seq_lens)
    with _device(query):
        rc = lib().paged_attn_decode_fp8(
            out.data_ptr(), tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(),
            query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), S, H, KH, D, BS, B, MB, P, partition_size, float(scale),
            float(k_scale), float(v_scale), _DT[query.dtype], _DT[out.dtype],
            _stream(query, stream))
    _check("paged_attn_decode_fp8", rc)


def _mq_geometry(query, key_cache, value_cache, block_tables, seq_lens):
    """(S, M, H, KH, D, BS, B, MB) for a [S, M, H, D] query."""
    _need(query.dim() == 4, "query [S, M, H, D] expected (M query tokens per sequence)")
    S, M, H, D = query.shape
    q3 = query.view(S * M, H, D)
    cache8 = key_cache.dtype == torch.float8_e4m3fn
    _, _, KH, _, BS, B, MB = _kv_geometry(q3[:S], key_cache, value_cache, block_tables,
                                          seq_lens, fp8=cache8)
    return S, M, H, KH, D, BS, B, MB


def _mq_stats_geometry(tmp_output, exp_sums, max_logits, S, M, H, D):
    _need(all(t.dtype == torch.float32 and t.is_cuda and t.is_contiguous()
              for t in (tmp_output, exp_sums, max_logits)),
          "tmp_output, exp_sums, max_logits must be contiguous fp32 device tensors")
    _need(tmp_output.dim() == 5 and tuple(tmp_output.shape[:3]) == (S, M, H) and
          tmp_output.shape[4] == D, "tmp_output must be [S, M, H, P, D]")
    P = tmp_output.shape[3]
    _need(tuple(exp_sums.shape) == (S, M, H, P) and tuple(max_logits.shape) == (S, M, H, P),
          "exp_sums and max_logits must be [S, M, H, P]")
    return P


def paged_attn_v2_partition_mq(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                               block_tables, seq_lens, scale: float, partition_size: int,
                               k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """Phase 1 for M query tokens per sequence (the last M positions, causal)."""
    S, M, H, KH, D, BS, B, MB = _mq_geometry(query, key_cache, value_cache, block_tables,
                                             seq_lens)
    P = _mq_stats_geometry(tmp_output, exp_sums, max_logits, S, M, H, D)
    _one_device(tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                seq_lens)
    with _device(query):
        rc = lib().paged_attn_v2_partition_mq(
            tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(), query.data_ptr(),
            key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), S, M, H, KH, D, BS, B, MB, P, partition_size, float(scale),
            float(k_scale), float(v_scale), _DT[query.dtype], _CACHE_DT[key_cache.dtype],
            _stream(query, stream))
    _check("paged_attn_v2_partition_mq", rc)


def paged_attn_v2_reduce_mq(out, tmp_output, exp_sums, max_logits, seq_lens, partition_size: int,
                            stream=None) -> None:
    """Phase 2 for M query tokens per sequence: out [S, M, H, D]."""
    _need(out.dim() == 4 and out.dtype in _DT and out.is_cuda and out.is_contiguous(),
          "out must be a contiguous [S, M, H, D] f32/f16/bf16 device tensor")
    S, M, H, D = out.shape
    P = _mq_stats_geometry(tmp_output, exp_sums, max_logits, S, M, H, D)
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_cuda and seq_lens.shape == (S,),
          "seq_lens must be an int32 [S] device tensor")
    _one_device(out, tmp_output, exp_sums, max_logits, seq_lens)
    with _device(out):
        rc = lib().paged_attn_v2_reduce_mq(
            out.data_ptr(), tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(),
            seq_lens.data_ptr(), S, M, H, D, P, partition_size, _DT[out.dtype],
            _stream(out, stream))
    _check("paged_attn_v2_reduce_mq", rc)


def paged_attn_decode_mq(out, tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                         block_tables, seq_lens, scale: float, partition_size: int,
                         k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """Phase 1 then phase 2 for M query tokens per sequence, on one stream."""
    S, M, H, KH, D, BS, B, MB = _mq_geometry(query, key_cache, value_cache, block_tables,
                                             seq_lens)
    P = _mq_stats_geometry(tmp_output, exp_sums, max_logits, S, M, H, D)
    _need(out.dim() == 4 and tuple(out.shape) == (S, M, H, D) and out.dtype in _DT and
          out.is_cuda and out.is_contiguous(), "out must be a contiguous [S, M, H, D] tensor")
    _one_device(out, tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                seq_lens)
    with _device(query):
        rc = lib().paged_attn_decode_mq(
            out.data_ptr(), tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(),
            query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), S, M, H, KH, D, BS, B, MB, P, partition_size, float(scale),
            float(k_scale), float(v_scale), _DT[query.dtype], _CACHE_DT[key_cache.dtype],
            _DT[out.dtype], _stream(query, stream))
    _check("paged_attn_decode_mq", rc)


def _rows4(t, name):
    """A [S, H, ...] single-query tensor as its [S, 1, H, ...] view (M = 1); 4-D+ as is."""
    return t.unsqueeze(1) if t.dim() == {"query": 3, "out": 3, "tmp": 4, "stats": 3}[name] else t


def _lse_arg(lse, out4):
    _need(lse.dtype == torch.float32 and lse.is_cuda and lse.is_contiguous() and
          lse.numel() == out4.shape[0] * out4.shape[1] * out4.shape[2],
          "lse must be a contiguous fp32 device tensor shaped like out without its last dim")
    return lse.data_ptr()


def paged_attn_v2_reduce_lse(out, lse, tmp_output, exp_sums, max_logits, seq_lens,
                             partition_size: int, stream=None) -> None:
    """Phase 2 plus each row's log-sum-exp: lse[...] = ln sum_t exp(s_t) (-inf: no keys).
    Single-query ([S, H, D] out, [S, H, P, D] stats) or M-token ([S, M, H, D]) shapes."""
    _need(out.dim() in (3, 4) and out.dtype in _DT and out.is_cuda and out.is_contiguous(),
          "out must be a contiguous [S, (M,) H, D] f32/f16/bf16 device tensor")
    o4 = _rows4(out, "out")
    t4, e4, m4 = _rows4(tmp_output, "tmp"), _rows4(exp_sums, "stats"), _rows4(max_logits, "stats")
    S, M, H, D = o4.shape
    P = _mq_stats_geometry(t4, e4, m4, S, M, H, D)
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_cuda and seq_lens.shape == (S,),
          "seq_lens must be an int32 [S] device tensor")
    _one_device(out, lse, tmp_output, exp_sums, max_logits, seq_lens)
    with _device(out):
        rc = lib().paged_attn_v2_reduce_lse(
            out.data_ptr(), _lse_arg(lse, o4), tmp_output.data_ptr(), exp_sums.data_ptr(),
            max_logits.data_ptr(), seq_lens.data_ptr(), S, M, H, D, P, partition_size,
            _DT[out.dtype], _stream(out, stream))
    _check("paged_attn_v2_reduce_lse", rc)


def paged_attn_decode_lse(out, lse, tmp_output, exp_sums, max_logits, query, key_cache,
                          value_cache, block_tables, seq_lens, scale: float, partition_size: int,
                          k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """Decode (any supported query / cache dtype pair, one or M query tokens) that also
    writes each row's log-sum-exp into lse (shaped like out without its last dim)."""
    _need(query.dim() in (3, 4), "query [S, H, D] or [S, M, H, D] expected")
    q4 = _rows4(query, "query")
    S, M, H, KH, D, BS, B, MB = _mq_geometry(q4, key_cache, value_cache, block_tables, seq_lens)
    o4 = _rows4(out, "out") if out.dim() == query.dim() else out
    t4, e4, m4 = _rows4(tmp_output, "tmp"), _rows4(exp_sums, "stats"), _rows4(max_logits, "stats")
    P = _mq_stats_geometry(t4, e4, m4, S, M, H, D)
    _need(out.dim() == query.dim() and tuple(o4.shape) == (S, M, H, D) and out.dtype in _DT and
          out.is_cuda and out.is_contiguous(), "out must be a contiguous tensor shaped like query")
    _one_device(out, lse, tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                block_tables, seq_lens)
    with _device(query):
        rc = lib().paged_attn_decode_lse(
            out.data_ptr(), _lse_arg(lse, o4), tmp_output.data_ptr(), exp_sums.data_ptr(),
            max_logits.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            block_tables.data_ptr(), seq_lens.data_ptr(), S, M, H, KH, D, BS, B, MB, P,
            partition_size, float(scale), float(k_scale), float(v_scale), _DT[query.dtype],
            _CACHE_DT[key_cache.dtype], _DT[out.dtype], _stream(query, stream))
    _check("paged_attn_decode_lse", rc)


def _slopes_arg(alibi_slopes, H):
    if alibi_slopes is None:
        return None
    _need(alibi_slopes.dtype == torch.float32 and alibi_slopes.is_cuda and
          alibi_slopes.is_contiguous() and tuple(alibi_slopes.shape) == (H,),
          "alibi_slopes must be a contiguous fp32 [num_heads] device tensor")
    return alibi_slopes.data_ptr()


def paged_attn_v2_partition_ex(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                               block_tables, seq_lens, scale: float, partition_size: int,
                               k_scale: float = 1.0, v_scale: float = 1.0, alibi_slopes=None,
                               stream=None) -> None:
    """Phase 1, general form: [S, H, D] or [S, M, H, D] query, any supported cache
    dtype, optional ALiBi slopes [H] (slope * (key position - query position))."""
    _need(query.dim() in (3, 4), "query [S, H, D] or [S, M, H, D] expected")
    q4 = _rows4(query, "query")
    S, M, H, KH, D, BS, B, MB = _mq_geometry(q4, key_cache, value_cache, block_tables, seq_lens)
    t4, e4, m4 = _rows4(tmp_output, "tmp"), _rows4(exp_sums, "stats"), _rows4(max_logits, "stats")
    P = _mq_stats_geometry(t4, e4, m4, S, M, H, D)
    _one_device(tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                seq_lens, alibi_slopes)
    with _device(query):
        rc = lib().paged_attn_v2_partition_ex(
            tmp_output.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(), query.data_ptr(),
            key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), S, M, H, KH, D, BS, B, MB, P, partition_size, float(scale),
            float(k_scale), float(v_scale), _slopes_arg(alibi_slopes, H), _DT[query.dtype],
            _CACHE_DT[key_cache.dtype], _stream(query, stream))
    _check("paged_attn_v2_partition_ex", rc)


def paged_attn_decode_ex(out, tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                         block_tables, seq_lens, scale: float, partition_size: int,
                         k_scale: float = 1.0, v_scale: float = 1.0, alibi_slopes=None,
                         lse=None, stream=None) -> None:
    """Both phases, general form (see paged_attn_v2_partition_ex); lse (shaped like
    out without its last dim) receives each row's log-sum-exp when given."""
    _need(query.dim() in (3, 4), "query [S, H, D] or [S, M, H, D] expected")
    q4 = _rows4(query, "query")
    S, M, H, KH, D, BS, B, MB = _mq_geometry(q4, key_cache, value_cache, block_tables, seq_lens)
    t4, e4, m4 = _rows4(tmp_output, "tmp"), _rows4(exp_sums, "stats"), _rows4(max_logits, "stats")
    P = _mq_stats_geometry(t4, e4, m4, S, M, H, D)
    _need(out.dim() == query.dim() and tuple(out.shape) == tuple(query.shape) and
          out.dtype in _DT and out.is_cuda and out.is_contiguous(),
          "out must be a contiguous tensor shaped like query")
    lse_ptr = _lse_arg(lse, _rows4(out, "out")) if lse is not None else None
    _one_device(out, lse, tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                block_tables, seq_lens, alibi_slopes)
    with _device(query):
        rc = lib().paged_attn_decode_ex(
            out.data_ptr(), lse_ptr, tmp_output.data_ptr(), exp_sums.data_ptr(),
            max_logits.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            block_tables.data_ptr(), seq_lens.data_ptr(), S, M, H, KH, D, BS, B, MB, P,
            partition_size, float(scale), float(k_scale), float(v_scale),
            _slopes_arg(alibi_slopes, H), _DT[query.dtype], _CACHE_DT[key_cache.dtype],
            _DT[out.dtype], _stream(query, stream))
    _check("paged_attn_decode_ex", rc)


def paged_attn_decode_noalloc(out, query, key_cache, value_cache, block_tables, seq_lens,
                              scale: float, partition_size: int, max_num_partitions: int,
                              k_scale: float = 1.0, v_scale: float = 1.0, alibi_slopes=None,
                              lse=None, stream=None) -> None:
    """paged_attn_decode_ex with the library's static per-GPU scratch as the
    workspace: allocates nothing (calls that overlap on one GPU race)."""
    _need(query.dim() in (3, 4), "query [S, H, D] or [S, M, H, D] expected")
    q4 = _rows4(query, "query")
    S, M, H, KH, D, BS, B, MB = _mq_geometry(q4, key_cache, value_cache, block_tables, seq_lens)
    _need(out.dim() == query.dim() and tuple(out.shape) == tuple(query.shape) and
          out.dtype in _DT and out.is_cuda and out.is_contiguous(),
          "out must be a contiguous tensor shaped like query")
    lse_ptr = _lse_arg(lse, _rows4(out, "out")) if lse is not None else None
    _one_device(out, lse, query, key_cache, value_cache, block_tables, seq_lens, alibi_slopes)
    with _device(query):
        rc = lib().paged_attn_decode_noalloc(
            out.data_ptr(), lse_ptr, query.data_ptr(), key_cache.data_ptr(),
            value_cache.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), S, M, H, KH,
            D, BS, B, MB, int(max_num_partitions), partition_size, float(scale), float(k_scale),
            float(v_scale), _slopes_arg(alibi_slopes, H), _DT[query.dtype],
            _CACHE_DT[key_cache.dtype], _DT[out.dtype], _stream(query, stream))
    _check("paged_attn_decode_noalloc", rc)


def paged_attn_merge_states(out, out_lse, a, lse_a, b, lse_b, stream=None) -> None:
    """Merge two attention states over disjoint key sets (rows [..., D] plus their
    log-sum-exps [...]) into out / out_lse (out_lse may be None; out may be a or b)."""
    _need(a.dtype in _DT and b.dtype == a.dtype and out.dtype == a.dtype,
          "a, b and out must share one dtype (f32, f16 or bf16)")
    _need(a.dim() >= 1 and tuple(b.shape) == tuple(a.shape) and tuple(out.shape) == tuple(a.shape),
          "a, b and out must have one shape [..., D]")
    lse_shape = tuple(a.shape[:-1])
    lses = [lse_a, lse_b] + ([out_lse] if out_lse is not None else [])
    _need(all(t.dtype == torch.float32 and tuple(t.shape) == lse_shape for t in lses),
          "lse tensors must be fp32 and shaped like a without its last dim")
    for t in [out, a, b] + lses:
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")
    D = a.shape[-1]
    rows = a.numel() // D if D else 0
    _one_device(out, out_lse, a, lse_a, b, lse_b)
    with _device(a):
        rc = lib().paged_attn_merge_states(
            out.data_ptr(), out_lse.data_ptr() if out_lse is not None else None, a.data_ptr(),
            lse_a.data_ptr(), b.data_ptr(), lse_b.data_ptr(), rows, D, _DT[a.dtype],
            _stream(a, stream))
    _check("paged_attn_merge_states", rc)


def workspace(num_seqs: int, num_heads: int, head_size: int, max_num_partitions: int,
              device) -> tuple:
    """Allocate (tmp_output, exp_sums, max_logits) for a decode call (torch memory)."""
    tmp = torch.empty(num_seqs, num_heads, max_num_partitions, head_size, dtype=torch.float32,
                      device=device)
    es = torch.empty(num_seqs, num_heads, max_num_partitions, dtype=torch.float32, device=device)
    ml = torch.empty(num_seqs, num_heads, max_num_partitions, dtype=torch.float32, device=device)
    return tmp, es, ml


def ensure_built() -> str:
    """Build the library if no built copy exists (tests, smoke and bench use this)."""
    if not os.path.exists(LIB_PATH):
        from . import build
        build.build()
    return LIB_PATH
