#!/usr/bin/env python3
"""Benchmark of paged single-query decode attention (V2 split, GQA) on one MI355X.

One step is the whole hot path over one batch: paged_attn_v2_partition then
paged_attn_v2_reduce on one stream, inputs already resident in HBM. W warmup
steps, then exactly K timed steps between two torch.cuda.synchronize() calls.
Prints ONE JSON line:

  value      = algorithmic K+V bytes per step / step time (GB/s), the metric's
               "achieved HBM GB/s", at the workload's configured partition
               size; the line also carries the % of the 8 TB/s peak and
               query-heads x tokens / s.
  tuned      = the same batch through paged_attn_decode at the partition size
               the library plans for it (paged_attn_plan_partition_size);
               same K+V bytes, same output up to rounding.
  roofline   = the dominant kernel (the partition kernel): algorithmic K+V
               bytes per launch / its average duration, measured with a HIP event
               pair on the launch stream around every partition launch of a
               second pass of the same K steps; `traffic` = HBM bytes per launch
               from the committed
               rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was taken on the
               current kernel source (else null).
  cpu_baseline = the fp64 oracle (partition stats + combine) timed on this
               host's cores over the same workload: one warm run, then the
               median of at least three timed runs (at least 10 s in all).
  flushed    = the same two calls timed one by one with their own event
               pairs after a 512 MiB scratch write (evicts the Infinity
               Cache): median and p10 / p90 over 100 calls.
  copy_context = a 1 GiB device-to-device copy's bandwidth (context for the
               8 TB/s peak).
  merge_states = paged_attn_merge_states timed with HIP events: on the
               batch's own rows (two query-dtype states of every (sequence,
               query token, head) row, as a cascade merges them) and on a
               2^20-row stream that shows the kernel's bandwidth; bytes are
               2 inputs + 1 output row plus 3 lse words per row.

Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "decode attention achieved HBM GB/s (% of peak) + query-heads×tokens/s, GQA cfg"
DEFAULT_WORKLOAD = "gqa_bf16_g4"
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "*hbm_traffic*.md")


def source_hash() -> str:
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "paged_kv_cache_v2_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, kernel: str):
    """HBM bytes per launch from a committed counter summary taken on this source."""
    want = source_hash()
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        text = open(path).read()
        fields = dict(re.findall(r"^- (\w+): `?([^`\n]+)`?$", text, re.M))
        if (fields.get("kernel_source_hash") == want and fields.get("workload") == workload
                and fields.get("kernel") == kernel and "traffic_bytes_per_launch" in fields):
            return int(float(fields["traffic_bytes_per_launch"])), os.path.relpath(path, ROOT)
    return None, None


def cpu_baseline(inp, W, min_seconds: float):
    import oracle
    import torch  # noqa: F401
    threads = oracle.default_threads()
    args = (inp["query"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
            inp["seq_lens"], inp["scale"])
    P, PS = inp["max_num_partitions"], inp["partition_size"]

    def one():
        t0 = time.perf_counter()
        tmp, es, ml = oracle.partition_stats(*args, P, PS, nthreads=threads,
                                             k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                                             alibi_slopes=inp.get("alibi_slopes"))
        oracle.combine(tmp, es, ml, inp["seq_lens"], PS)
        return time.perf_counter() - t0

    one()  # warm run (page-in, thread start)
    times = []
    while len(times) < 3 or sum(times) < min_seconds:
        times.append(one())
    per_run = sorted(times)[len(times) // 2]
    return {
        "value": round(W.kv_bytes(inp) / per_run / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"whole workload ({inp['num_seqs']} sequences, "
                   f"{int(inp['seq_lens'].sum())} tokens), fp64 partition stats + combine: "
                   f"1 warm run, median of {len(times)} timed runs, {per_run:.2f} s per run"),
    }


def merge_bench(pa, torch, dev, stream, rows: int, D: int, dtype, K: int) -> dict:
    """Average duration and algorithmic GB/s of paged_attn_merge_states."""
    def one(R):
        g = torch.Generator(device=dev).manual_seed(R)
        a = torch.randn(R, D, device=dev, generator=g).to(dtype)
        b = torch.randn(R, D, device=dev, generator=g).to(dtype)
        la = torch.randn(R, device=dev, generator=g)
        lb = torch.randn(R, device=dev, generator=g)
        out, lse = torch.empty_like(a), torch.empty_like(la)
        for _ in range(3):
            pa.paged_attn_merge_states(out, lse, a, la, b, lb, stream)
        # K back-to-back launches between two events: a small merge takes a few
        # microseconds, less than an event pair between every launch would add
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(K):
            pa.paged_attn_merge_states(out, lse, a, la, b, lb, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        avg_s = ev[0].elapsed_time(ev[1]) / K / 1e3
        nbytes = R * (3 * D * a.element_size() + 3 * 4)
        return nbytes, avg_s

    nb, t = one(rows)
    nb_s, t_s = one(1 << 20)
    return {
        "dtype": str(dtype).replace("torch.", ""), "head_size": D,
        "rows": rows, "bytes_per_launch": nb, "avg_us": round(t * 1e6, 3),
        "achieved": round(nb / t / 1e9, 2), "frac": round(nb / t / 1e9 / PEAK_HBM_GBS, 4),
        "stream_rows": 1 << 20, "stream_bytes_per_launch": nb_s,
        "stream_avg_us": round(t_s * 1e6, 3), "stream_achieved": round(nb_s / t_s / 1e9, 2),
        "stream_frac": round(nb_s / t_s / 1e9 / PEAK_HBM_GBS, 4), "unit": "GB/s",
    }


def flushed_calls(torch, dev, stream, partition, reduce, tmp, es, ml, PS, kvb, n) -> dict:
    """Each call timed by its own event pairs (partition, reduce) after a
    512 MiB scratch write that evicts the 256 MB Infinity Cache (outside the
    events): median and p10 / p90 of the step and of each kernel."""
    scratch = torch.empty(1 << 27, dtype=torch.float32, device=dev)  # 512 MiB
    steps, parts, reds = [], [], []
    for i in range(n + 10):
        scratch.fill_(float(i))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        partition(tmp, es, ml, PS)
        e[1].record(stream)
        reduce(tmp, es, ml, PS)
        e[2].record(stream)
        torch.cuda.synchronize()
        if i >= 10:  # 10 warm-up calls
            parts.append(e[0].elapsed_time(e[1]) * 1e3)
            reds.append(e[1].elapsed_time(e[2]) * 1e3)
            steps.append(e[0].elapsed_time(e[2]) * 1e3)
    del scratch

    def q(v, f):
        v = sorted(v)
        return round(v[min(len(v) - 1, int(f * len(v)))], 3)

    med = q(steps, 0.5)
    return {"calls": n, "step_median_us": med, "step_p10_us": q(steps, 0.1),
            "step_p90_us": q(steps, 0.9), "partition_median_us": q(parts, 0.5),
            "reduce_median_us": q(reds, 0.5), "value": round(kvb / med / 1e3, 2), "unit": "GB/s",
            "pct_of_peak_hbm": round(100.0 * kvb / med / 1e3 / PEAK_HBM_GBS, 2)}


def copy_bandwidth(torch, dev, stream) -> dict:
    """A 1 GiB device-to-device copy (torch copy_): read + write bytes / time."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 10 / 1e3
    del a, b
    return {"bytes": 2 * 4 * n, "us": round(t * 1e6, 2), "value": round(2 * 4 * n / t / 1e9, 1),
            "unit": "GB/s", "pct_of_peak_hbm": round(100.0 * 2 * 4 * n / t / 1e9 / PEAK_HBM_GBS, 2)}


def run(args) -> dict:
    import torch

    import paged_kv_cache_v2_amd as pa
    from paged_kv_cache_v2_amd import workloads as W

    pa.ensure_built()
    cfg = W.CONFIGS[args.workload]
    seed = W.workload_seed(args.workload)
    inp = W.make_inputs(cfg, seed=seed)
    PS = args.partition_size or cfg.partition_size
    P = max(1, -(-int(inp["seq_lens"].max()) // PS))
    P = max(P, cfg.max_num_partitions) if PS == cfg.partition_size else P
    dev = torch.device("cuda", 0)
    q, kc, vc = (inp[k].to(dev) for k in ("query", "key_cache", "value_cache"))
    bt, sl = inp["block_tables"].to(dev), inp["seq_lens"].to(dev)
    MQ = cfg.num_queries
    S, H, D = q.shape[0], q.shape[-2], q.shape[-1]
    lead = (S,) if MQ == 1 else (S, MQ)

    def work(P_):
        return (torch.empty(*lead, H, P_, D, dtype=torch.float32, device=dev),
                torch.empty(*lead, H, P_, dtype=torch.float32, device=dev),
                torch.empty(*lead, H, P_, dtype=torch.float32, device=dev))

    out = torch.empty(*lead, H, D, dtype=torch.float32, device=dev)
    tmp, es, ml = work(P)
    stream = torch.cuda.current_stream(dev)

    fp8 = cfg.dtype == "fp8"
    ks, vs = inp["k_scale"], inp["v_scale"]
    al = inp["alibi_slopes"].to(dev) if cfg.alibi else None

    def partition(tmp_, es_, ml_, PS_):
        if al is not None:
            pa.paged_attn_v2_partition_ex(tmp_, es_, ml_, q, kc, vc, bt, sl, inp["scale"], PS_,
                                          ks, vs, al, stream)
        elif MQ > 1:
            pa.paged_attn_v2_partition_mq(tmp_, es_, ml_, q, kc, vc, bt, sl, inp["scale"], PS_,
                                          ks, vs, stream)
        elif fp8:
            pa.paged_attn_v2_partition_fp8(tmp_, es_, ml_, q, kc, vc, bt, sl, inp["scale"], ks, vs,
                                           PS_, stream)
        else:
            pa.paged_attn_v2_partition(tmp_, es_, ml_, q, kc, vc, bt, sl, inp["scale"], PS_,
                                       stream)

    def reduce(tmp_, es_, ml_, PS_):
        if MQ > 1:
            pa.paged_attn_v2_reduce_mq(out, tmp_, es_, ml_, sl, PS_, stream)
        else:
            pa.paged_attn_v2_reduce(out, tmp_, es_, ml_, sl, PS_, stream)

    def step():
        partition(tmp, es, ml, PS)
        reduce(tmp, es, ml, PS)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # Timed region: exactly K whole-path steps between two synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Kernel timing: the same K steps again, with a HIP event pair on the launch
    # stream around every partition launch (events inside the timed region above
    # would add their own gaps to the step time).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        partition(tmp, es, ml, PS)
        ev[i][1].record(stream)
        reduce(tmp, es, ml, PS)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    part_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    red_ms = sorted(e[1].elapsed_time(e[2]) for e in ev)
    part_avg_s = sum(part_ms) / len(part_ms) / 1e3
    red_avg_s = sum(red_ms) / len(red_ms) / 1e3

    # The same batch through paged_attn_decode (one ABI call, partition +
    # reduce) at the partition size the library plans for this batch;
    # out does not depend on the partition size beyond rounding.
    PS_t = pa.plan_partition_size(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, D,
                                  cfg.block_size, cfg.max_len, W.DTYPES[cfg.dtype])
    P_t = max(1, -(-cfg.max_len // PS_t))
    tmp_t, es_t, ml_t = work(P_t)

    def step_tuned():
        if al is not None:
            pa.paged_attn_decode_ex(out, tmp_t, es_t, ml_t, q, kc, vc, bt, sl, inp["scale"], PS_t,
                                    ks, vs, al, stream=stream)
        elif MQ > 1:
            pa.paged_attn_decode_mq(out, tmp_t, es_t, ml_t, q, kc, vc, bt, sl, inp["scale"], PS_t,
                                    ks, vs, stream=stream)
        elif fp8:
            pa.paged_attn_decode_fp8(out, tmp_t, es_t, ml_t, q, kc, vc, bt, sl, inp["scale"], ks,
                                     vs, PS_t, stream=stream)
        else:
            pa.paged_attn_decode(out, tmp_t, es_t, ml_t, q, kc, vc, bt, sl, inp["scale"], PS_t,
                                 stream=stream)

    for _ in range(args.warmup):
        step_tuned()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step_tuned()
    torch.cuda.synchronize()
    tuned_s = (time.perf_counter() - t0) / K
    del tmp_t, es_t, ml_t

    kvb = W.kv_bytes(inp)
    step_s = elapsed / K
    gbs = kvb / step_s / 1e9
    achieved = kvb / part_avg_s / 1e9
    kernel = ("partition_mfma_kernel"
              if (cfg.query_dtype != "f32" and (cfg.group >= 4 or MQ > 1))
              else "partition_vec_kernel")
    traffic, traffic_src = committed_traffic(args.workload, kernel)
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype if not fp8 else f"fp8_e4m3 cache, {cfg.query_dtype} query",
        "data": "synthetic",
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "qheads_tokens_per_s": round(W.qhead_tokens(inp) / step_s, 1),
        "config": {
            "workload": args.workload, "num_seqs": S, "num_heads": H,
            "num_kv_heads": cfg.num_kv_heads, "head_size": D, "block_size": cfg.block_size,
            "partition_size": PS, "max_num_partitions": P,
            "seq_lens": (f"fixed {list(cfg.fixed_lens)[:2]}..." if cfg.fixed_lens else
                         f"uniform[{cfg.len_lo},{cfg.len_hi}] seed {seed}"),
            "total_tokens": int(inp["seq_lens"].sum()), "kv_bytes_per_step": kvb,
            "num_blocks": inp["num_blocks"],
            **({"k_scale": inp["k_scale"], "v_scale": inp["v_scale"]} if fp8 else {}),
            **({"num_queries": MQ} if MQ > 1 else {}),
            **({"alibi": "slopes 2^(-8(h+1)/H)"} if al is not None else {}),
        },
        "tuned": {
            "entry": ("paged_attn_decode_ex" if al is not None else
                      "paged_attn_decode_mq" if MQ > 1 else
                      "paged_attn_decode_fp8" if fp8 else "paged_attn_decode"),
            "partition_size": PS_t, "max_num_partitions": P_t,
            "partition_span": (None if MQ > 1 else
                               pa.partition_span(S, H, cfg.num_kv_heads, D, cfg.block_size, P_t,
                                                 PS_t, W.DTYPES[cfg.dtype])),
            "ms_per_step": round(tuned_s * 1e3, 5), "value": round(kvb / tuned_s / 1e9, 2),
            "unit": "GB/s", "pct_of_peak_hbm": round(100.0 * kvb / tuned_s / 1e9 / PEAK_HBM_GBS, 2),
            "qheads_tokens_per_s": round(W.qhead_tokens(inp) / tuned_s, 1),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": kernel, "kernel_avg_us": round(part_avg_s * 1e6, 3),
            "kernel_p10_us": round(part_ms[len(part_ms) // 10] * 1e3, 3),
            "kernel_p90_us": round(part_ms[(9 * len(part_ms)) // 10] * 1e3, 3),
            "bytes_per_launch": kvb, "traffic_source": traffic_src,
            "kernel_source_hash": source_hash(),
            "reduce_avg_us": round(red_avg_s * 1e6, 3),
            "partition_span": (None if MQ > 1 else
                               pa.partition_span(S, H, cfg.num_kv_heads, D, cfg.block_size, P,
                                                 PS, W.DTYPES[cfg.dtype])),
        },
    }
    res["merge_states"] = merge_bench(pa, torch, dev, stream, S * MQ * H, D,
                                      W.DTYPES[cfg.query_dtype], K)
    if args.flushed_calls > 0:
        res["flushed"] = flushed_calls(torch, dev, stream, partition, reduce, tmp, es, ml, PS,
                                       kvb, args.flushed_calls)
    res["copy_context"] = copy_bandwidth(torch, dev, stream)
    if args.calibrate_copy:
        n = 1 << 28  # 1 GiB of fp32: FETCH_SIZE / WRITE_SIZE calibration for the counters
        a = torch.ones(n, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 4 * n
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, W, args.cpu_min_seconds)
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--flushed-calls", type=int, default=100,
                    help="calls timed one by one after an Infinity Cache flush")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)",
              file=sys.stderr)
        return 2
    res = run(args)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
