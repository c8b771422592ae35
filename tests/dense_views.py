"""Independent views of a paged cache for pinning the oracle (test helpers).

These reach the gathered K/V by a different route than the oracle's explicit
index arithmetic: torch ``permute``/``reshape`` of the whole cache into a
token-major layout, then advanced indexing by the block table. The attention
itself is then a library routine (fp64 ``softmax`` and ``matmul`` on the CPU).
"""
from __future__ import annotations

import math
from typing import Dict, List, Tuple

import torch


def token_major(key_cache: torch.Tensor, value_cache: torch.Tensor, k_scale: float = 1.0,
                v_scale: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """[B, KH, D/x, BS, x] and [B, KH, D, BS] -> two [B, BS, KH, D] float64 tensors
    (torch's own casts decode the stored dtype; 8-bit caches are then scaled)."""
    B, KH, Dx, BS, x = key_cache.shape
    k = key_cache.permute(0, 3, 1, 2, 4).reshape(B, BS, KH, Dx * x).to(torch.float64)
    v = value_cache.permute(0, 3, 1, 2).to(torch.float64)
    return k * float(k_scale), v * float(v_scale)


def gathered(inp: Dict[str, object], s: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Dense [L, KH, D] float64 K and V of sequence s via the block table."""
    k, v = token_major(inp["key_cache"], inp["value_cache"], inp.get("k_scale", 1.0),
                       inp.get("v_scale", 1.0))
    BS = k.shape[1]
    L = int(inp["seq_lens"][s])
    nb = -(-L // BS)
    blocks = inp["block_tables"][s, :nb].to(torch.int64)
    KH, D = k.shape[2], k.shape[3]
    return (k[blocks].reshape(nb * BS, KH, D)[:L], v[blocks].reshape(nb * BS, KH, D)[:L])


def library_attention(inp: Dict[str, object], scale: float) -> torch.Tensor:
    """out[S, H, D] float64 from torch softmax/matmul over repeat_interleave'd kv heads."""
    q = inp["query"].to(torch.float64)
    S, H, D = q.shape
    KH = inp["key_cache"].shape[1]
    G = H // KH
    out = torch.zeros(S, H, D, dtype=torch.float64)
    for s in range(S):
        K, V = gathered(inp, s)
        if K.shape[0] == 0:
            continue
        Kh = K.repeat_interleave(G, dim=1).permute(1, 0, 2)  # [H, L, D]
        Vh = V.repeat_interleave(G, dim=1).permute(1, 0, 2)
        scores = torch.matmul(Kh, q[s].unsqueeze(-1)).squeeze(-1) * float(scale)  # [H, L]
        w = torch.softmax(scores, dim=-1)
        out[s] = torch.matmul(w.unsqueeze(1), Vh).squeeze(1)
    return out


def library_partitions(inp: Dict[str, object], scale: float, P: int, PS: int):
    """Phase-1 intermediates from torch ops: tmp[S,H,P,D] (NaN if empty), es, ml."""
    q = inp["query"].to(torch.float64)
    S, H, D = q.shape
    KH = inp["key_cache"].shape[1]
    G = H // KH
    tmp = torch.full((S, H, P, D), float("nan"), dtype=torch.float64)
    es = torch.zeros(S, H, P, dtype=torch.float64)
    ml = torch.full((S, H, P), -math.inf, dtype=torch.float64)
    for s in range(S):
        K, V = gathered(inp, s)
        L = K.shape[0]
        Kh = K.repeat_interleave(G, dim=1).permute(1, 0, 2)
        Vh = V.repeat_interleave(G, dim=1).permute(1, 0, 2)
        scores = torch.matmul(Kh, q[s].unsqueeze(-1)).squeeze(-1) * float(scale)
        for p in range(P):
            t0, t1 = p * PS, min((p + 1) * PS, L)
            if t0 >= L:
                continue
            sc = scores[:, t0:t1]
            m = sc.max(dim=-1).values
            e = torch.exp(sc - m[:, None])
            l = e.sum(dim=-1)
            ml[s, :, p] = m
            es[s, :, p] = l
            tmp[s, :, p] = torch.matmul(e.unsqueeze(1), Vh[:, t0:t1]).squeeze(1) / l[:, None]
    return tmp, es, ml


def brute_force_attention(inp: Dict[str, object], scale: float) -> List[List[List[float]]]:
    """Pure-Python loops on tiny inputs: nested lists, math.exp and math.fsum."""
    q = inp["query"].to(torch.float64).tolist()
    kc = (inp["key_cache"].to(torch.float64) * float(inp.get("k_scale", 1.0))).tolist()
    vc = (inp["value_cache"].to(torch.float64) * float(inp.get("v_scale", 1.0))).tolist()
    bt = inp["block_tables"].tolist()
    sl = inp["seq_lens"].tolist()
    S, H, D = len(q), len(q[0]), len(q[0][0])
    KH = len(kc[0])
    BS = len(kc[0][0][0])
    x = len(kc[0][0][0][0])
    G = H // KH
    out = []
    for s in range(S):
        rows = []
        for h in range(H):
            kh = h // G
            toks = [(bt[s][t // BS], t % BS) for t in range(sl[s])]
            if not toks:
                rows.append([0.0] * D)
                continue
            sc = [scale * math.fsum(q[s][h][d] * kc[b][kh][d // x][o][d % x] for d in range(D))
                  for b, o in toks]
            m = max(sc)
            w = [math.exp(a - m) for a in sc]
            z = math.fsum(w)
            rows.append([math.fsum(wi * vc[b][kh][d][o] for wi, (b, o) in zip(w, toks)) / z
                         for d in range(D)])
        out.append(rows)
    return out
