#!/usr/bin/env python3
"""Benchmark of paged single-query decode attention (V2 split, GQA) on one MI355X.

One step is the whole hot path over one batch: one paged_attn_decode call at
the workload's configured partition size (512 tokens for the GQA batch),
inputs already resident in HBM. Every 512-token partition is computed on its
own and the partitions are combined with the log-sum-exp rule, inside the
partition kernel where one workgroup holds all of a row's partitions (the GQA
batch: no reduce launch, no per-partition rows), else by the reduce over the
workgroups' span entries. W warmup steps, then exactly K timed steps between
two torch.cuda.synchronize() calls. Prints ONE JSON line:

  value      = algorithmic K+V bytes per step / step time (GB/s), steps back to
               back; also as % of the 8 TB/s peak and query-heads x tokens / s.
  flushed    = the protocol the metric is defined on: each call timed by its
               own HIP event pair after a 512 MiB scratch write that evicts
               the 256 MB Infinity Cache (outside the events); median and
               p10 / p90 over the calls, as GB/s and % of peak.
  roofline   = the decode call's kernels (the partition kernel, plus the reduce
               when a row spans several workgroups): K+V bytes / their average
               duration, from one HIP event pair on the launch stream around a
               second pass of K back-to-back calls (the timed region / K); the
               per-call distribution from an event pair around each call of a
               third pass (event_pair_*: each pair also times its launch);
               `traffic` = HBM bytes per call from the committed rocprofv3
               FETCH_SIZE / WRITE_SIZE summary when it was taken on the current
               kernel source (else null).
  two_call   = the same batch through paged_attn_v2_partition + paged_attn_v2_reduce
               (every partition's row stored, then reduced): step time, and the
               two kernels' event-timed averages.
  tuned      = the same batch through paged_attn_decode at the partition size
               the library plans for it (paged_attn_plan_partition_size).
  workloads  = the same measurements (value, flushed, roofline, tuned, ceiling)
               for the other configurations named by --also (the long-context
               GQA batch by default), each after 0.1 s of untimed calls (the
               clocks ramp up again after the idle gap of building the batch).
  ceiling    = a read-only kernel that gathers the same K/V pages through the
               same block tables with the same loads and computes nothing
               (libpa_ceiling.so): the page-gather read bandwidth of this chip.
  ceiling_units = (16-bit MFMA workloads) the same reads with the decode's work
               structure: one workgroup per (sequence, span, kv head) unit of
               the one-call plan, largest first, wavefronts taking every fourth
               page, two workgroups per CU as the 16-bit MFMA decode runs.
  copy_context = a 1 GiB device-to-device copy's bandwidth.
  merge_states = paged_attn_merge_states on the batch's own rows and on a
               2^20-row stream.
  cpu_baseline = the fp64 oracle (partition statistics + combine) timed on this
               host's cores over the whole headline batch: one warm run, then
               the median of at least three timed runs (at least 10 s in all).

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
DEFAULT_ALSO = "longctx_bf16_g8"
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "*hbm_traffic*.md")


def source_hash() -> str:
    """Hash of the decode path's kernel and launch sources (csrc/, without the
    read-ceiling instrument gather_ceiling.hip): a counter summary taken on
    other sources no longer describes these kernels."""
    h = hashlib.sha256()
    files = sorted(f for f in glob.glob(os.path.join(ROOT, "paged_kv_cache_v2_amd", "csrc", "*"))
                   if os.path.basename(f) != "gather_ceiling.hip")
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, kernel: str):
    """HBM bytes per call from a committed counter summary taken on this source."""
    want = source_hash()
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        text = open(path).read()
        fields = dict(re.findall(r"^- (\w+): `?([^`\n]+)`?$", text, re.M))
        if (fields.get("kernel_source_hash") == want and fields.get("workload") == workload
                and fields.get("kernel") == kernel and "traffic_bytes_per_launch" in fields):
            return int(float(fields["traffic_bytes_per_launch"])), os.path.relpath(path, ROOT)
    return None, None


def kv_bytes(inp) -> int:
    """Algorithmic K+V bytes of one step: each token's K and V row of each kv
    head read once, 2 * D * sizeof bytes per (token, kv head)."""
    esz = inp["key_cache"].element_size()
    return int(inp["seq_lens"].to("cpu").long().sum()) * inp["num_kv_heads"] * 2 * \
        inp["head_size"] * esz


def qhead_tokens(inp) -> int:
    """(query token, query head, key) triples one step scores: with M query
    tokens per sequence (its last M positions), token m sees L - M + m + 1 keys."""
    M = inp.get("num_queries", 1)
    lens = [int(x) for x in inp["seq_lens"].tolist()]
    keys = sum(max(0, min(L, L - M + m + 1)) for L in lens for m in range(M))
    return keys * inp["num_heads"]


def cpu_baseline(inp, min_seconds: float):
    import oracle
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
        "value": round(kv_bytes(inp) / per_run / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"whole workload ({inp['num_seqs']} sequences, "
                   f"{int(inp['seq_lens'].sum())} tokens), fp64 partition stats + combine: "
                   f"1 warm run, median of {len(times)} timed runs, {per_run:.2f} s per run"),
    }


def quantile(v, f):
    v = sorted(v)
    return v[min(len(v) - 1, int(f * len(v)))]


def pct(gbs):
    return round(100.0 * gbs / PEAK_HBM_GBS, 2)


class Batch:
    """One workload's inputs on the GPU and its launch forms."""

    def __init__(self, name, pa, W, torch, PS=None):
        self.name, self.pa, self.torch = name, pa, torch
        cfg = W.CONFIGS[name]
        self.cfg = cfg
        self.seed = W.workload_seed(name)
        inp = W.make_inputs(cfg, seed=self.seed)
        self.inp = inp
        self.PS = PS or cfg.partition_size
        P = max(1, -(-int(inp["seq_lens"].max()) // self.PS))
        self.P = max(P, cfg.max_num_partitions) if self.PS == cfg.partition_size else P
        dev = torch.device("cuda", 0)
        self.dev = dev
        self.q, self.kc, self.vc = (inp[k].to(dev) for k in ("query", "key_cache", "value_cache"))
        self.bt, self.sl = inp["block_tables"].to(dev), inp["seq_lens"].to(dev)
        self.MQ = cfg.num_queries
        self.S, self.H, self.D = self.q.shape[0], self.q.shape[-2], self.q.shape[-1]
        self.lead = (self.S,) if self.MQ == 1 else (self.S, self.MQ)
        self.out = torch.empty(*self.lead, self.H, self.D, dtype=torch.float32, device=dev)
        self.ws = self.work(self.P)
        self.stream = torch.cuda.current_stream(dev)
        self.fp8 = cfg.dtype == "fp8"
        self.al = inp["alibi_slopes"].to(dev) if cfg.alibi else None
        self.kvb = kv_bytes(inp)
        self.qht = qhead_tokens(inp)
        self.PS_t = pa.plan_partition_size(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads,
                                           self.D, cfg.block_size, cfg.max_len,
                                           W.DTYPES[cfg.dtype])
        self.P_t = max(1, -(-cfg.max_len // self.PS_t))
        self.ws_t = self.work(self.P_t)
        self.dtype_name = W.DTYPES[cfg.dtype]

    def work(self, P_):
        t, dev = self.torch, self.dev
        return (t.empty(*self.lead, self.H, P_, self.D, dtype=t.float32, device=dev),
                t.empty(*self.lead, self.H, P_, dtype=t.float32, device=dev),
                t.empty(*self.lead, self.H, P_, dtype=t.float32, device=dev))

    def entry(self):
        return ("paged_attn_decode_ex" if self.al is not None else
                "paged_attn_decode_mq" if self.MQ > 1 else
                "paged_attn_decode_fp8" if self.fp8 else "paged_attn_decode")

    def decode(self, ws=None, PS=None):
        pa, i = self.pa, self.inp
        tmp, es, ml = ws or self.ws
        PS = PS or self.PS
        a = (self.q, self.kc, self.vc, self.bt, self.sl, i["scale"])
        if self.al is not None:
            pa.paged_attn_decode_ex(self.out, tmp, es, ml, *a, PS, i["k_scale"], i["v_scale"],
                                    self.al, stream=self.stream)
        elif self.MQ > 1:
            pa.paged_attn_decode_mq(self.out, tmp, es, ml, *a, PS, i["k_scale"], i["v_scale"],
                                    stream=self.stream)
        elif self.fp8:
            pa.paged_attn_decode_fp8(self.out, tmp, es, ml, *a, i["k_scale"], i["v_scale"], PS,
                                     stream=self.stream)
        else:
            pa.paged_attn_decode(self.out, tmp, es, ml, *a, PS, stream=self.stream)

    def partition(self):
        pa, i = self.pa, self.inp
        tmp, es, ml = self.ws
        a = (self.q, self.kc, self.vc, self.bt, self.sl, i["scale"])
        if self.al is not None:
            pa.paged_attn_v2_partition_ex(tmp, es, ml, *a, self.PS, i["k_scale"], i["v_scale"],
                                          self.al, self.stream)
        elif self.MQ > 1:
            pa.paged_attn_v2_partition_mq(tmp, es, ml, *a, self.PS, i["k_scale"], i["v_scale"],
                                          self.stream)
        elif self.fp8:
            pa.paged_attn_v2_partition_fp8(tmp, es, ml, *a, i["k_scale"], i["v_scale"], self.PS,
                                           self.stream)
        else:
            pa.paged_attn_v2_partition(tmp, es, ml, *a, self.PS, self.stream)

    def reduce(self):
        tmp, es, ml = self.ws
        if self.MQ > 1:
            self.pa.paged_attn_v2_reduce_mq(self.out, tmp, es, ml, self.sl, self.PS, self.stream)
        else:
            self.pa.paged_attn_v2_reduce(self.out, tmp, es, ml, self.sl, self.PS, self.stream)

    # ---- timing
    def back_to_back(self, fn, K, W_):
        """Seconds per step of K back-to-back steps between two synchronisations."""
        torch = self.torch
        for _ in range(W_):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / K

    def region(self, fn, K):
        """Microseconds per call of K back-to-back calls of `fn`, from one HIP
        event pair on the launch stream around them."""
        torch = self.torch
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        e0.record(self.stream)
        for _ in range(K):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    def events(self, fns, K):
        """K rounds of the calls in `fns`, a HIP event pair on the launch stream
        around each call: per call, the list of K durations in microseconds."""
        torch = self.torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
              for _ in range(K)]
        for k in range(K):
            ev[k][0].record(self.stream)
            for j, fn in enumerate(fns):
                fn()
                ev[k][j + 1].record(self.stream)
        torch.cuda.synchronize()
        return [[ev[k][j].elapsed_time(ev[k][j + 1]) * 1e3 for k in range(K)]
                for j in range(len(fns))]

    def flushed(self, n):
        """Each decode call timed by its own event pair after a 512 MiB scratch
        write (outside the events) that evicts the Infinity Cache; 10 warm-up
        calls, then n."""
        torch = self.torch
        scratch = torch.empty(1 << 27, dtype=torch.float32, device=self.dev)  # 512 MiB
        times = []
        for i in range(n + 10):
            scratch.fill_(float(i))
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record(self.stream)
            self.decode()
            e1.record(self.stream)
            torch.cuda.synchronize()
            if i >= 10:
                times.append(e0.elapsed_time(e1) * 1e3)
        del scratch
        med = quantile(times, 0.5)
        gbs = self.kvb / med / 1e3
        return {"calls": n, "step_median_us": round(med, 3),
                "step_p10_us": round(quantile(times, 0.1), 3),
                "step_p90_us": round(quantile(times, 0.9), 3),
                "value": round(gbs, 2), "unit": "GB/s", "pct_of_peak_hbm": pct(gbs),
                "qheads_tokens_per_s": round(self.qht / med * 1e6, 1)}

    def plan(self, P, PS):
        """The one-call decode's launch plan (span, ring slots, span entries per row)."""
        c = self.cfg
        return self.pa.decode_plan(self.S, self.MQ, self.H, c.num_kv_heads, self.D, c.block_size,
                                   P, PS, self.torch_dtype(c.query_dtype), self.dtype_name)

    def torch_dtype(self, name):
        from paged_kv_cache_v2_amd import workloads as W
        return W.DTYPES[name]

    def kernel_name(self):
        c = self.cfg
        return ("partition_mfma_kernel" if c.query_dtype != "f32" and (c.group >= 4 or self.MQ > 1)
                else "partition_vec_kernel")

    def settle(self, seconds):
        """Untimed decode calls for at least `seconds`: the GPU's clocks ramp up
        over the first ~20 ms of load after an idle gap (the 8-bit batches, whose
        kernels issue more instructions per byte, run ~10 % slower until then)."""
        torch = self.torch
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                self.decode()
            torch.cuda.synchronize()

    def measure(self, K, W_, flushed_calls, two_call=True):
        """value (back to back), roofline (events), flushed, tuned; two_call optional."""
        step_s = self.back_to_back(self.decode, K, W_)
        call_avg = self.region(self.decode, K)
        call_us = self.events([self.decode], K)[0]
        gbs = self.kvb / step_s / 1e9
        achieved = self.kvb / call_avg / 1e3
        traffic, traffic_src = committed_traffic(self.name, self.kernel_name())
        c = self.cfg
        res = {
            "value": round(gbs, 2), "unit": "GB/s", "ms_per_step": round(step_s * 1e3, 5),
            "pct_of_peak_hbm": pct(gbs),
            "qheads_tokens_per_s": round(self.qht / step_s, 1),
            "entry": self.entry(), "partition_size": self.PS, "max_num_partitions": self.P,
            "plan": self.plan(self.P, self.PS),
            "roofline": {
                "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": self.kernel_name(), "call_avg_us": round(call_avg, 3),
                "event_pair_avg_us": round(sum(call_us) / len(call_us), 3),
                "event_pair_p10_us": round(quantile(call_us, 0.1), 3),
                "event_pair_p90_us": round(quantile(call_us, 0.9), 3),
                "bytes_per_launch": self.kvb, "traffic_source": traffic_src,
                "kernel_source_hash": source_hash(),
            },
        }
        if flushed_calls > 0:
            res["flushed"] = self.flushed(flushed_calls)
        if two_call:
            two_s = self.back_to_back(lambda: (self.partition(), self.reduce()), K, W_)
            part_us, red_us = self.events([self.partition, self.reduce], K)
            pavg = sum(part_us) / len(part_us)
            res["two_call"] = {
                "entries": "paged_attn_v2_partition + paged_attn_v2_reduce",
                "ms_per_step": round(two_s * 1e3, 5),
                "value": round(self.kvb / two_s / 1e9, 2),
                "pct_of_peak_hbm": pct(self.kvb / two_s / 1e9),
                "partition_avg_us": round(pavg, 3),
                "partition_frac": round(self.kvb / pavg / 1e3 / PEAK_HBM_GBS, 4),
                "reduce_avg_us": round(sum(red_us) / len(red_us), 3),
            }
        tuned_s = self.back_to_back(lambda: self.decode(self.ws_t, self.PS_t), K, W_)
        res["tuned"] = {
            "entry": self.entry(), "partition_size": self.PS_t, "max_num_partitions": self.P_t,
            "plan": self.plan(self.P_t, self.PS_t),
            "ms_per_step": round(tuned_s * 1e3, 5), "value": round(self.kvb / tuned_s / 1e9, 2),
            "unit": "GB/s", "pct_of_peak_hbm": pct(self.kvb / tuned_s / 1e9),
            "qheads_tokens_per_s": round(self.qht / tuned_s, 1),
        }
        res["config"] = {
            "workload": self.name, "num_seqs": self.S, "num_heads": self.H,
            "num_kv_heads": c.num_kv_heads, "head_size": self.D, "block_size": c.block_size,
            "partition_size": self.PS, "max_num_partitions": self.P,
            "seq_lens": (f"fixed {list(c.fixed_lens)[:2]}..." if c.fixed_lens else
                         f"uniform[{c.len_lo},{c.len_hi}] seed {self.seed}"),
            "total_tokens": int(self.inp["seq_lens"].sum()), "kv_bytes_per_step": self.kvb,
            "num_blocks": self.inp["num_blocks"],
            **({"k_scale": self.inp["k_scale"], "v_scale": self.inp["v_scale"]}
               if self.fp8 else {}),
            **({"num_queries": self.MQ} if self.MQ > 1 else {}),
            **({"alibi": "slopes 2^(-8(h+1)/H)"} if self.al is not None else {}),
        }
        res["dtype"] = (c.dtype if not self.fp8 else f"fp8_e4m3 cache, {c.query_dtype} query")
        return res


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
        for _ in range(K):
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


def gather_ceiling(pa, torch, b: Batch, K: int) -> dict:
    """The read-only page-gather kernel over the batch's own pages: GB/s."""
    from paged_kv_cache_v2_amd import ceiling
    sink = torch.empty(ceiling.sink_words(), dtype=torch.int32, device=b.dev)
    blocks = ceiling.page_list(b.bt, b.sl, b.cfg.block_size)

    def run():
        ceiling.gather_ceiling(sink, b.kc, b.vc, blocks, stream=b.stream)

    for _ in range(5):
        run()
    avg = b.region(run, K)
    gbs = b.kvb / avg / 1e3
    return {"kernel": "gather_ceiling_kernel", "workload": b.name, "avg_us": round(avg, 3),
            "value": round(gbs, 2), "unit": "GB/s", "pct_of_peak_hbm": pct(gbs)}


# Workgroups per CU of the 16-bit MFMA decode kernel (the host caps it there).
MFMA16_WGS_PER_CU = 2


def units_ceiling(pa, torch, b: Batch, K: int) -> dict:
    """The read-only gather with the one-call decode's work units (same spans,
    same largest-first order, same residency): GB/s."""
    from paged_kv_cache_v2_amd import ceiling
    span = b.plan(b.P, b.PS)["span"]
    span_pages = span * b.PS // b.cfg.block_size
    pages, off, n = ceiling.unit_pages(b.inp["block_tables"], b.inp["seq_lens"],
                                       b.cfg.block_size, b.cfg.num_kv_heads, span_pages)
    pages, off = pages.to(b.dev), off.to(b.dev)
    sink = torch.empty(max(1, 4 * n), dtype=torch.int32, device=b.dev)

    def run():
        ceiling.gather_units(sink, b.kc, b.vc, pages, off, n, MFMA16_WGS_PER_CU, stream=b.stream)

    for _ in range(5):
        run()
    avg = b.region(run, K)
    gbs = b.kvb / avg / 1e3
    return {"kernel": "gather_units_kernel", "workload": b.name, "units": n,
            "span_pages": span_pages, "workgroups_per_cu": MFMA16_WGS_PER_CU,
            "avg_us": round(avg, 3), "value": round(gbs, 2), "unit": "GB/s",
            "pct_of_peak_hbm": pct(gbs)}


def mfma16(b: Batch) -> bool:
    return b.kernel_name() == "partition_mfma_kernel" and not b.fp8


def run(args) -> dict:
    import torch

    import paged_kv_cache_v2_amd as pa
    from paged_kv_cache_v2_amd import workloads as W

    pa.ensure_built()
    K, W_ = args.steps, args.warmup
    b = Batch(args.workload, pa, W, torch, args.partition_size)
    # Timed region: exactly K whole-path steps (one decode call each) between
    # two synchronisations, inside Batch.measure.
    m = b.measure(K, W_, args.flushed_calls, two_call=True)
    res = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W_,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic",
        "pct_of_peak_hbm": m["pct_of_peak_hbm"],
        "qheads_tokens_per_s": m["qheads_tokens_per_s"],
        "config": m["config"],
        "entry": m["entry"],
        "plan": m["plan"],
        "roofline": m["roofline"],
    }
    for k in ("flushed", "two_call", "tuned"):
        if k in m:
            res[k] = m[k]
    if not args.no_ceiling:
        res["ceiling"] = gather_ceiling(pa, torch, b, K)
        if mfma16(b):
            res["ceiling_units"] = units_ceiling(pa, torch, b, K)
    if not args.no_extras:
        res["merge_states"] = merge_bench(pa, torch, b.dev, b.stream, b.S * b.MQ * b.H, b.D,
                                          W.DTYPES[b.cfg.query_dtype], K)
        res["copy_context"] = copy_bandwidth(torch, b.dev, b.stream)
    if args.calibrate_copy:
        n = 1 << 28  # 1 GiB of fp32: FETCH_SIZE / WRITE_SIZE calibration for the counters
        a = torch.ones(n, device=b.dev)
        c = torch.empty_like(a)
        for _ in range(3):
            c.copy_(a)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 4 * n
    host_inp = b.inp
    del b
    torch.cuda.empty_cache()
    also = [w for w in (args.also.split(",") if args.also else []) if w and w != args.workload]
    if also:
        res["workloads"] = {}
        for name in also:
            o = Batch(name, pa, W, torch)
            o.settle(0.1)  # (building the batch left the GPU idle for seconds)
            r = o.measure(K, W_, args.flushed_calls, two_call=False)
            if not args.no_ceiling:
                r["ceiling"] = gather_ceiling(pa, torch, o, K)
                if mfma16(o):
                    r["ceiling_units"] = units_ceiling(pa, torch, o, K)
            res["workloads"][name] = r
            del o
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(host_inp, args.cpu_min_seconds)
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="comma-separated further workloads measured into `workloads` ('' for none)")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip merge_states and copy_context")
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
