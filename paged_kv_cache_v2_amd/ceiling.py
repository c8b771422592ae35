"""Binding of libpa_ceiling.so (include/pa_ceiling.h): the read-only page-gather
kernel that measures the bandwidth ceiling of a paged K/V read. A measuring
instrument for the benchmark; the decode path does not use it."""
from __future__ import annotations

import ctypes
import os

import torch

from .binding import _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_ceiling.so")
_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_v2_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.pa_gather_ceiling_sink_words.argtypes = [ctypes.c_int32] * 3
        L.pa_gather_ceiling_sink_words.restype = ctypes.c_int64
        L.pa_gather_ceiling.argtypes = ([ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 4 +
                                        [ctypes.c_int32] * 6 + [ctypes.c_void_p])
        L.pa_gather_ceiling.restype = ctypes.c_int
        _LIB = L
    return _LIB


def sink_words(num_seqs: int, num_kv_heads: int, max_blocks_per_seq: int) -> int:
    return int(lib().pa_gather_ceiling_sink_words(num_seqs, num_kv_heads, max_blocks_per_seq))


def gather_ceiling(sink: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                   block_tables: torch.Tensor, seq_lens: torch.Tensor, stream=None) -> None:
    """Read every used (block, kv head) page of both caches once."""
    B, KH = key_cache.shape[0], key_cache.shape[1]
    page = key_cache[0, 0].numel() * key_cache.element_size()
    S, MB = block_tables.shape
    BS = value_cache.shape[-1]
    rc = lib().pa_gather_ceiling(sink.data_ptr(), sink.numel(), key_cache.data_ptr(),
                                 value_cache.data_ptr(), block_tables.data_ptr(),
                                 seq_lens.data_ptr(), S, KH, page, BS, B, MB,
                                 _stream(key_cache, stream))
    if rc != 0:
        raise RuntimeError(f"pa_gather_ceiling failed with status {rc}")
