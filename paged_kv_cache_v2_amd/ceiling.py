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
        L.pa_gather_ceiling_sink_words.argtypes = []
        L.pa_gather_ceiling_sink_words.restype = ctypes.c_int64
        L.pa_gather_ceiling.argtypes = ([ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 3 +
                                        [ctypes.c_int64] + [ctypes.c_int32] * 3 +
                                        [ctypes.c_void_p])
        L.pa_gather_ceiling.restype = ctypes.c_int
        L.pa_gather_units.argtypes = ([ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 4 +
                                      [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p])
        L.pa_gather_units.restype = ctypes.c_int
        _LIB = L
    return _LIB


def sink_words() -> int:
    return int(lib().pa_gather_ceiling_sink_words())


def page_list(block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int) -> torch.Tensor:
    """The used blocks of every sequence, in sequence order (a flat int32 list)."""
    nb = (seq_lens.to(torch.int64) + block_size - 1) // block_size
    cols = torch.arange(block_tables.shape[1], device=block_tables.device)
    return block_tables[cols[None, :] < nb[:, None]].to(torch.int32).contiguous()


def gather_ceiling(sink: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                   blocks: torch.Tensor, stream=None) -> None:
    """Read the K and V page of every (block in `blocks`, kv head) once."""
    B, KH = key_cache.shape[0], key_cache.shape[1]
    page = key_cache[0, 0].numel() * key_cache.element_size()
    rc = lib().pa_gather_ceiling(sink.data_ptr(), sink.numel(), key_cache.data_ptr(),
                                 value_cache.data_ptr(), blocks.data_ptr(), blocks.numel(), KH,
                                 page, B, _stream(key_cache, stream))
    if rc != 0:
        raise RuntimeError(f"pa_gather_ceiling failed with status {rc}")


def unit_pages(block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
               num_kv_heads: int, span_pages: int):
    """The decode's work units as page lists, on the host: one unit per
    (sequence, span of span_pages pages, kv head), pairs (sequence, span)
    ranked by page count, descending, ties in index order (span-major, as the
    decode ranks them), kv head fastest. Returns (pages int32, unit_off int32,
    num_units); page = block * num_kv_heads + kv head."""
    import numpy as np
    bt = block_tables.cpu().numpy().astype(np.int64)
    nb = ((seq_lens.cpu().numpy().astype(np.int64) + block_size - 1) // block_size)
    S = len(nb)
    spans = int(max(1, -(-int(nb.max(initial=0)) // span_pages)))
    pairs = []  # (-pages, index, s, ch)
    for ch in range(spans):
        for s in range(S):
            n = int(min(max(nb[s] - ch * span_pages, 0), span_pages))
            if n:
                pairs.append((-n, ch * S + s, s, ch))
    pairs.sort()
    lists = []
    for _, _, s, ch in pairs:
        blks = bt[s, ch * span_pages: min((ch + 1) * span_pages, nb[s])]
        for kh in range(num_kv_heads):
            lists.append(blks * num_kv_heads + kh)
    off = np.zeros(len(lists) + 1, dtype=np.int64)
    if lists:
        off[1:] = np.cumsum([len(x) for x in lists])
    pages = np.concatenate(lists) if lists else np.zeros(0, dtype=np.int64)
    return (torch.from_numpy(pages.astype(np.int32)), torch.from_numpy(off.astype(np.int32)),
            len(lists))


def gather_units(sink: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                 pages: torch.Tensor, unit_off: torch.Tensor, num_units: int,
                 workgroups_per_cu: int, stream=None) -> None:
    """Read every unit's K and V pages, one workgroup per unit, at most
    workgroups_per_cu workgroups per CU."""
    B, KH = key_cache.shape[0], key_cache.shape[1]
    page = key_cache[0, 0].numel() * key_cache.element_size()
    rc = lib().pa_gather_units(sink.data_ptr(), sink.numel(), key_cache.data_ptr(),
                               value_cache.data_ptr(), pages.data_ptr(), unit_off.data_ptr(),
                               num_units, B * KH, page, workgroups_per_cu,
                               _stream(key_cache, stream))
    if rc != 0:
        raise RuntimeError(f"pa_gather_units failed with status {rc}")
