"""fp64 CPU oracle for paged V2 decode attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package.
It builds ``liboracle.so`` from ``paged_decode_oracle.c`` with gcc when no
built copy exists, and takes torch CPU tensors or numpy arrays in the layouts
of the Triton PagedAttention V2 page's problem statement. Results are numpy
float64 arrays. Every function here is marshalling only; the arithmetic is in
the C file, whose header states the definitions it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "paged_decode_oracle.c")
# PA_ORACLE_LIB: load another build of the same source instead (the sanitizer
# test points it at an AddressSanitizer / UndefinedBehaviorSanitizer build).
_LIB_PATH = os.environ.get("PA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_LIB = None

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def compile_source(src: str, out: str, sanitize: bool = False) -> str:
    """gcc a C source of the oracle into a shared library (IEEE semantics: no
    fast-math); with sanitize, instrumented by AddressSanitizer and
    UndefinedBehaviorSanitizer (load it with the sanitizer runtime preloaded)."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall",
           "-Wno-unused-function", *(SANITIZE_FLAGS if sanitize else []), src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source (not when PA_ORACLE_LIB names another build)."""
    if os.environ.get("PA_ORACLE_LIB"):
        return _LIB_PATH
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        build(force=not os.path.exists(_LIB_PATH))
        _LIB = _bind(_LIB_PATH)
    return _LIB


class using_library:
    """Context manager: route every call through another build of the oracle source
    (the mutation tests compile deliberately altered copies into a temp dir)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _LIB
        _lib()
        self.saved = _LIB
        _LIB = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _LIB
        _LIB = self.saved
        return False


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.oracle_decode_binary16.restype = ctypes.c_double
    lib.oracle_decode_binary16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bfloat16.restype = ctypes.c_double
    lib.oracle_decode_bfloat16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_e4m3.restype = ctypes.c_double
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_array.restype = None
    lib.oracle_decode_array.argtypes = [P, P, I64, ctypes.c_int]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, F32,
                                     I32, P, I32, I32]
    lib.oracle_partition_stats.restype = ctypes.c_int
    lib.oracle_partition_stats.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32,
                                           I32, I32, I32, F32, I32, P, I32, I32]
    lib.oracle_attention_ex.restype = ctypes.c_int
    lib.oracle_attention_ex.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                        F32, I32, I32, F32, F32, P, I32, I32]
    lib.oracle_partition_stats_ex.restype = ctypes.c_int
    lib.oracle_partition_stats_ex.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32,
                                              I32, I32, I32, I32, F32, I32, I32, F32, F32, P,
                                              I32, I32]
    lib.oracle_combine_ex.restype = None
    lib.oracle_combine_ex.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32]
    lib.oracle_attention_lse.restype = ctypes.c_int
    lib.oracle_attention_lse.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                         F32, I32, I32, F32, F32, P, I32, I32]
    lib.oracle_attention_full.restype = ctypes.c_int
    lib.oracle_attention_full.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                          F32, I32, I32, F32, F32, P, P, I32, I32]
    lib.oracle_partition_stats_full.restype = ctypes.c_int
    lib.oracle_partition_stats_full.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32,
                                                I32, I32, I32, I32, F32, I32, I32, F32, F32, P, P,
                                                I32, I32]
    lib.oracle_merge_states.restype = None
    lib.oracle_merge_states.argtypes = [P, P, P, P, P, P, I64, I32]
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32]
    lib.oracle_gather_indices.restype = I64
    lib.oracle_gather_indices.argtypes = [P, P, P, P, I32, I32, I32]
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _np(t) -> np.ndarray:
    """Contiguous host numpy view of a torch CPU tensor or numpy array (16-bit as uint16)."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype in (torch.float16, torch.bfloat16):
                return t.view(torch.int16).numpy().view(np.uint16)
            if t.dtype == torch.float8_e4m3fn:
                return t.view(torch.uint8).numpy()
            return t.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(t)


def _dtype_code(q) -> int:
    import torch
    m = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float8_e4m3fn: 3}
    return m[q.dtype]


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode an array of stored 8/16-bit patterns (or float32) to float64."""
    a = np.ascontiguousarray(bits)
    out = np.empty(a.size, dtype=np.float64)
    _lib().oracle_decode_array(_ptr(out), _ptr(a), a.size, DTYPE_CODES[dtype])
    return out.reshape(a.shape)


def _seq_arg(seqs: Optional[Sequence[int]]):
    if seqs is None:
        return None, 0, None
    arr = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int32))
    return _ptr(arr), arr.size, arr


def _query_rows(q):
    """(S, M, H, D) of a [S, H, D] (one query token) or [S, M, H, D] query."""
    if q.ndim == 3:
        S, H, D = q.shape
        return S, 1, H, D
    return q.shape


def _slopes(alibi_slopes, H):
    """(pointer or None, keep-alive array) of fp32 ALiBi slopes [H]."""
    if alibi_slopes is None:
        return None, None
    a = np.ascontiguousarray(_np(alibi_slopes), dtype=np.float32)
    assert a.shape == (H,), "alibi_slopes must be [num_heads]"
    return _ptr(a), a


def attention_lse(query, key_cache, value_cache, block_tables, seq_lens, scale: float,
                  seqs: Optional[Sequence[int]] = None, nthreads: Optional[int] = None,
                  k_scale: float = 1.0, v_scale: float = 1.0,
                  alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray]:
    """``attention`` plus the log-sum-exp of each row's scores: (out, lse), lse
    shaped like out without its last dim (-inf for a row with no keys)."""
    q, kc, vc = _np(query), _np(key_cache), _np(value_cache)
    bt, sl = _np(block_tables).astype(np.int32, copy=False), _np(seq_lens).astype(np.int32, copy=False)
    S, M, H, D = _query_rows(q)
    KH, BS = kc.shape[1], kc.shape[3]
    MB = bt.shape[1]
    out = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:-1], np.nan)
    sp, ns, keep = _seq_arg(seqs)
    ap, akeep = _slopes(alibi_slopes, H)
    rc = _lib().oracle_attention_full(_ptr(out), _ptr(lse), _ptr(q), _ptr(kc), _ptr(vc),
                                      _ptr(bt), _ptr(sl), S, M, H, KH, D, BS, MB,
                                      float(np.float32(scale)), _dtype_code(query),
                                      _dtype_code(key_cache), float(np.float32(k_scale)),
                                      float(np.float32(v_scale)), ap, sp, ns,
                                      nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attention: unsupported shape")
    del keep, akeep
    return out, lse


def attention(query, key_cache, value_cache, block_tables, seq_lens, scale: float,
              seqs: Optional[Sequence[int]] = None, nthreads: Optional[int] = None,
              k_scale: float = 1.0, v_scale: float = 1.0, alibi_slopes=None) -> np.ndarray:
    """Dense softmax attention over the block-table-gathered tokens, float64.

    query [S, H, D] gives out [S, H, D]; query [S, M, H, D] (M query tokens per
    sequence, the last M positions, causal) gives out [S, M, H, D]. Rows of
    sequences not in ``seqs`` are NaN. The query dtype and the cache dtype are
    read off the tensors; an e4m3fn cache stands for its decoded values times
    ``k_scale`` / ``v_scale``. ``alibi_slopes`` [H] adds slope * (key position
    - query position) to each score.
    """
    return attention_lse(query, key_cache, value_cache, block_tables, seq_lens, scale, seqs,
                         nthreads, k_scale, v_scale, alibi_slopes)[0]


def merge_states(a, lse_a, b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Merge two attention results over disjoint key sets: (out, out_lse), float64.
    a, b: [..., D]; lse_a, lse_b: [...]."""
    a = np.ascontiguousarray(np.asarray(a, np.float64))
    b = np.ascontiguousarray(np.asarray(b, np.float64))
    la = np.ascontiguousarray(np.asarray(lse_a, np.float64))
    lb = np.ascontiguousarray(np.asarray(lse_b, np.float64))
    assert a.shape == b.shape and la.shape == lb.shape == a.shape[:-1]
    out = np.empty_like(a)
    lse = np.empty_like(la)
    _lib().oracle_merge_states(_ptr(out), _ptr(lse), _ptr(a), _ptr(la), _ptr(b), _ptr(lb),
                               la.size, a.shape[-1])
    return out, lse


def partition_stats(query, key_cache, value_cache, block_tables, seq_lens, scale: float,
                    max_num_partitions: int, partition_size: int,
                    seqs: Optional[Sequence[int]] = None,
                    nthreads: Optional[int] = None, k_scale: float = 1.0,
                    v_scale: float = 1.0,
                    alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Phase-1 intermediates: tmp_output [rows, H, P, D], exp_sums and max_logits
    [rows, H, P], with rows = [S] or [S, M] as for ``attention``."""
    q, kc, vc = _np(query), _np(key_cache), _np(value_cache)
    bt, sl = _np(block_tables).astype(np.int32, copy=False), _np(seq_lens).astype(np.int32, copy=False)
    S, M, H, D = _query_rows(q)
    KH, BS = kc.shape[1], kc.shape[3]
    MB = bt.shape[1]
    P = max_num_partitions
    lead = q.shape[:-2]
    tmp = np.full(lead + (H, P, D), np.nan)
    es = np.full(lead + (H, P), np.nan)
    ml = np.full(lead + (H, P), np.nan)
    sp, ns, keep = _seq_arg(seqs)
    ap, akeep = _slopes(alibi_slopes, H)
    rc = _lib().oracle_partition_stats_full(
        _ptr(tmp), _ptr(es), _ptr(ml), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(sl), S, M, H,
        KH, D, BS, MB, P, partition_size, float(np.float32(scale)), _dtype_code(query),
        _dtype_code(key_cache), float(np.float32(k_scale)), float(np.float32(v_scale)), ap, sp,
        ns, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_partition_stats: unsupported shape or length > P*PS")
    del keep, akeep
    return tmp, es, ml


def combine(tmp: np.ndarray, exp_sums: np.ndarray, max_logits: np.ndarray, seq_lens,
            partition_size: int) -> np.ndarray:
    """Phase-2 log-sum-exp combine of the partition intermediates, float64:
    tmp [S, H, P, D] gives out [S, H, D]; tmp [S, M, H, P, D] gives [S, M, H, D]."""
    tmp = np.ascontiguousarray(tmp, dtype=np.float64)
    es = np.ascontiguousarray(exp_sums, dtype=np.float64)
    ml = np.ascontiguousarray(max_logits, dtype=np.float64)
    sl = _np(seq_lens).astype(np.int32, copy=False)
    if tmp.ndim == 4:
        S, H, P, D = tmp.shape
        M = 1
    else:
        S, M, H, P, D = tmp.shape
    out = np.empty(tmp.shape[:-2] + (D,))
    _lib().oracle_combine_ex(_ptr(out), _ptr(tmp), _ptr(es), _ptr(ml), _ptr(sl), S, M, H, D, P,
                             partition_size)
    return out


def gather_indices(block_tables, seq_lens, block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """(physical block, slot) of every token t < L_s, sequences in order."""
    bt, sl = _np(block_tables).astype(np.int32, copy=False), _np(seq_lens).astype(np.int32, copy=False)
    n = int(sl.astype(np.int64).sum())
    blk = np.empty(max(n, 1), np.int32)
    slot = np.empty(max(n, 1), np.int32)
    m = _lib().oracle_gather_indices(_ptr(blk), _ptr(slot), _ptr(bt), _ptr(sl), bt.shape[0],
                                     bt.shape[1], block_size)
    assert m == n
    return blk[:n], slot[:n]
