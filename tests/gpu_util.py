"""Helpers for the GPU parity tests: run the HIP path, compare with the oracle.

The comparison bar is the one the measurements are quoted against:
|gpu - oracle| <= 1e-3 + 1e-3 * |oracle| elementwise on fp32 results, exact
sentinels for empty partitions, bit-exact integer / index work.
"""
from __future__ import annotations

import math
import sys
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import oracle
import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import workloads as W

ATOL = 1e-3
RTOL = 1e-3
DEV = "cuda"


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (survives a crash of the step)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: Dict[str, object]) -> Dict[str, object]:
    out = dict(inp)
    for k in ("query", "key_cache", "value_cache", "block_tables", "seq_lens"):
        out[k] = inp[k].to(DEV)
    return out


def num_partitions(inp, PS: int) -> int:
    return max(1, -(-int(inp["seq_lens"].max()) // PS))


def run_decode(dinp: Dict[str, object], PS: Optional[int] = None, P: Optional[int] = None,
               out_dtype=torch.float32, split: bool = False) -> Dict[str, torch.Tensor]:
    """One batch through the C ABI; workspaces pre-filled with NaN. Host copies back.

    split=True: paged_attn_v2_partition then paged_attn_v2_reduce only.
    split=False: the same two calls (phase 1's per-partition rows and
    statistics are what `tmp`, `es` and `ml` hold, and their output is
    `out_split`), then paged_attn_decode on its own NaN-filled workspace:
    `out` is the one-call result, which combines partitions inside the kernel
    and leaves its workspace unspecified (`ws_tmp`, `ws_es`, `ws_ml`)."""
    q = dinp["query"]
    S, H, D = q.shape
    PS = PS or dinp["partition_size"]
    P = P or max(dinp["max_num_partitions"] if PS == dinp["partition_size"] else 1,
                 num_partitions(dinp, PS))

    def ws():
        return (torch.full((S, H, P, D), float("nan"), device=DEV),
                torch.full((S, H, P), float("nan"), device=DEV),
                torch.full((S, H, P), float("nan"), device=DEV))

    def new_out():
        return torch.full((S, H, D), float("nan"), device=DEV).to(out_dtype)

    args = (q, dinp["key_cache"], dinp["value_cache"], dinp["block_tables"], dinp["seq_lens"])
    fp8 = dinp["key_cache"].dtype == torch.float8_e4m3fn
    ks, vs = dinp.get("k_scale", 1.0), dinp.get("v_scale", 1.0)
    tmp, es, ml = ws()
    out_s = new_out()
    if fp8:
        pa.paged_attn_v2_partition_fp8(tmp, es, ml, *args, dinp["scale"], ks, vs, PS)
    else:
        pa.paged_attn_v2_partition(tmp, es, ml, *args, dinp["scale"], PS)
    pa.paged_attn_v2_reduce(out_s, tmp, es, ml, dinp["seq_lens"], PS)
    res = dict(tmp=tmp, es=es, ml=ml, P=P, PS=PS)
    if split:
        res["out"] = out_s
    else:
        wt, we, wm = ws()
        out = new_out()
        if fp8:
            pa.paged_attn_decode_fp8(out, wt, we, wm, *args, dinp["scale"], ks, vs, PS)
        else:
            pa.paged_attn_decode(out, wt, we, wm, *args, dinp["scale"], PS)
        res.update(out=out, out_split=out_s, ws_tmp=wt, ws_es=we, ws_ml=wm)
    torch.cuda.synchronize()
    return {k: v.cpu() if isinstance(v, torch.Tensor) else v for k, v in res.items()}


def assert_close(name: str, got, ref, atol: float = ATOL, rtol: float = RTOL) -> float:
    got = np.asarray(got.double().numpy() if isinstance(got, torch.Tensor) else got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    lim = atol + rtol * np.abs(ref)
    bad = ~(err <= lim)  # NaN counts as bad
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err - lim, -np.inf)), bad.shape)
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} outside tolerance; worst at "
                             f"{idx}: gpu={got[idx]!r} ref={ref[idx]!r}")
    return float(np.max(err / lim)) if err.size else 0.0


def check_against_oracle(inp: Dict[str, object], res: Dict[str, torch.Tensor],
                         seqs: Optional[Sequence[int]] = None, label: str = "") -> Dict[str, float]:
    """Compare out (and out_split) and the partition intermediates of `seqs` (all if
    None) with the oracle; returns the worst err/limit ratio per quantity (< 1 passes)."""
    S = inp["query"].shape[0]
    rows = list(range(S)) if seqs is None else sorted(set(int(s) for s in seqs))
    args = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
            inp["seq_lens"], inp["scale"])
    sc = dict(k_scale=inp.get("k_scale", 1.0), v_scale=inp.get("v_scale", 1.0))
    ref = oracle.attention(*args, seqs=rows, **sc)
    worst = {"out": assert_close(f"{label} out", res["out"][rows].float(), ref[rows])}
    if "out_split" in res:
        worst["out_split"] = assert_close(f"{label} out (two calls)",
                                          res["out_split"][rows].float(), ref[rows])
    tmp, es, ml = oracle.partition_stats(*args, res["P"], res["PS"], seqs=rows, **sc)
    sl = inp["seq_lens"].tolist()
    ml_w = es_w = tmp_w = 0.0
    for s in rows:
        n = -(-sl[s] // res["PS"]) if sl[s] > 0 else 0
        if n:
            ml_w = max(ml_w, assert_close(f"{label} max_logits s={s}", res["ml"][s, :, :n],
                                          ml[s, :, :n]))
            es_w = max(es_w, assert_close(f"{label} exp_sums s={s}", res["es"][s, :, :n],
                                          es[s, :, :n]))
            tmp_w = max(tmp_w, assert_close(f"{label} tmp_output s={s}", res["tmp"][s, :, :n],
                                            tmp[s, :, :n]))
        # empty partitions: exact sentinels, tmp_output untouched (still NaN)
        assert torch.all(res["ml"][s, :, n:] == -math.inf), f"{label} sentinel max s={s}"
        assert torch.all(res["es"][s, :, n:] == 0), f"{label} sentinel sum s={s}"
        assert torch.all(torch.isnan(res["tmp"][s, :, n:])), f"{label} tmp written s={s}"
    worst.update(max_logits=ml_w, exp_sums=es_w, tmp_output=tmp_w)
    note(f"{label}: worst err/limit " + " ".join(f"{k}={v:.3g}" for k, v in worst.items()))
    return worst


def small_config(name: str) -> W.DecodeConfig:
    """A reduced-size version of a named workload: same heads, dims, dtype and
    block/partition geometry; fewer and shorter sequences (several tiles,
    several partitions and a ragged tail each)."""
    cfg = W.CONFIGS[name]
    if name == "tiny_f32_d64":
        return cfg
    if name == "mha_f16_d128":
        return cfg.replace(num_seqs=5, len_lo=1, len_hi=1100)
    if name == "gqa_bf16_g4":
        return cfg.replace(num_seqs=6, len_lo=1, len_hi=1600)
    if name == "longctx_bf16_g8":
        return cfg.replace(num_seqs=2, fixed_lens=(2500, 1300))
    if name == "wide_f16_d256":
        return cfg.replace(num_seqs=3, len_lo=100, len_hi=1800)
    if name == "gqa_fp8_g4":
        return cfg.replace(num_seqs=6, len_lo=1, len_hi=1600)
    if name == "longctx_fp8_g8":
        return cfg.replace(num_seqs=2, fixed_lens=(2500, 1300))
    if name == "mha_fp8_d128":
        return cfg.replace(num_seqs=5, len_lo=1, len_hi=1100)
    raise KeyError(name)
