// gfx950 kernels for paged single-query decode attention, V2 split.
//
// Method: "paged_attention_v2_triton.py -- Triton PagedAttention V2 for
// BI-V100", phase-1 partition kernel (paged gather, scaled q.k scores, online
// softmax, normalised partition output with its max logit and exp sum,
// sentinels for empty partitions) and phase-2 reduce kernel (cross-partition
// log-sum-exp combine). That page's kernel is organised for its own GPU:
// one program per (sequence, query head, partition), K/V gathered per query
// head. Here a workgroup owns one (sequence, kv head, span of partitions) unit
// and all the query heads (and query tokens) of a launch's columns share every
// K/V fetch.
//
// Work unit and layout
//  - A workgroup owns a span of C consecutive partitions p0 .. p0+C-1 of one
//    (sequence, kv head); blockIdx.x = r * KH + kh, and the (sequence, span)
//    pair of rank r is either pair r in index order (q * S + s, p0 = q * C:
//    partition span slowest, so the last-dispatched workgroups are the cheap
//    tail/empty partitions) or, where the host asks for it, the pair of rank r
//    by page count, largest first (lpt_pair). Each partition is still
//    computed and stored on its own (outputs do not depend on C or the
//    order); spanning amortises the unit's prologue (length and block-table
//    loads) and epilogue (LDS merge, stores) over C partitions, lets the
//    stores of adjacent partitions (adjacent rows of tmp_output) go out
//    together, and retires the empty partitions of a sequence in the same
//    workgroup as its last used one.
//  - Partition p covers pages [p*PS/BS, ceil(min((p+1)*PS, L)/BS)); PS % BS
//    == 0 so partition edges are page edges, and the used pages of a span are
//    contiguous. The span's block-table slice is loaded together with the
//    sequence length (no dependent round trip) and hoisted into LDS; NW
//    wavefronts take the span's pages wave, wave+NW, ... and park their
//    running state in LDS each time they cross into the next partition.
//  - The page is the unit of fetch and compute; it is BS/16 sub-tiles of 16
//    tokens. K sub-tile: lane l holds token l%16 and d-chunks c = 4j + l/16
//    (16-byte dwordx4 loads; each 16 lanes read 256 contiguous bytes per chunk
//    row). That register image is exactly the A operand of a 16x16x32 MFMA
//    with the token as row. All of a page's loads are issued together, so the
//    two halves of every cache line of a 32-token page are requested
//    back to back.
//  - K/V loads carry the non-temporal hint: every byte is read exactly once,
//    and streaming them past the caches measured ~12 % faster on MI355X than
//    letting them allocate normally.
//  - Each wavefront keeps its own running (max, sum, unnormalised accumulator)
//    in the log2 domain (scores pre-multiplied by scale*log2(e)); at the end the
//    NW partial states of every partition are merged through LDS with the same
//    log-sum-exp rule the reduce uses, normalised, and stored with max_logits
//    back in natural units. Keeping the accumulator unnormalised and dividing once is the
//    partition kernel's normalised recurrence in exact arithmetic.
//  - Masked tokens (t >= seq_len in the last page) are selected out: score
//    -inf and value 0, never multiplied by a zero weight, so NaN in unread
//    cache slots cannot leak.
//  - The one-call decode (PartitionArgs::fuse) computes every partition the
//    same way but does not store it: the workgroup combines its span's
//    partitions with the reduce's log-sum-exp rule, either at the end from
//    the parked states (combine_store) or as the span streams, one partition
//    at a time (park_roll, the ROLL instantiations), and writes the output
//    itself when the span is the whole row, else one span entry per row for
//    the reduce.
#pragma once

#include <type_traits>

#include "pa_device.h"

namespace pa {

// Compile-time tuning (measured on MI355X).
#ifndef PA_WAVES
#define PA_WAVES 4           // wavefronts per partition workgroup
#endif
#ifndef PA_PREFETCH
#define PA_PREFETCH 1        // pages in flight ahead of the one being computed
#endif
#ifndef PA_PF_REG_BUDGET
#define PA_PF_REG_BUDGET 32  // prefetch only if a page fits in this many VGPRs
#endif
#ifndef PA_MIN_WAVES
#define PA_MIN_WAVES 0       // >0: ask the compiler for this many waves per SIMD
#endif
#if PA_MIN_WAVES > 0
#define PA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(PA_MIN_WAVES)))
#else
#define PA_OCCUPANCY
#endif
#ifndef PA_STEADY
#define PA_STEADY 1          // pipeline: branch-free steady-state rounds before the guarded drain
#endif
#ifndef PA_PIN_PREFETCH
#define PA_PIN_PREFETCH 1    // scheduling barrier between prefetch issue and compute
#endif
// MFMA path: the P high part and residual in one 16x16x32 PV MFMA (1: with
// 16-bit caches; 2: also 8-bit ones, whose 4-wavefront budget then spills a
// few registers; 0: two 16x16x16 MFMAs everywhere). Measured: neutral to
// 0.7 % faster on the 16-bit workloads, neutral on 8-bit ones.
#ifndef PA_PV32
#define PA_PV32 1
#endif
#ifndef PA_NT_LOADS
#define PA_NT_LOADS 1        // K/V loads carry the non-temporal (streaming) hint
#endif
constexpr int kWaves = PA_WAVES;

template <typename T>
__device__ __forceinline__ T stream_load(const void* p) {
#if PA_NT_LOADS
  return __builtin_nontemporal_load((const T*)p);
#else
  return *(const T*)p;
#endif
}
// The same through a global-memory (address space 1) pointer.
typedef const __attribute__((address_space(1))) uint8_t* gbytes;
template <typename T>
__device__ __forceinline__ T stream_load(gbytes p) {
  typedef const __attribute__((address_space(1))) T* gT;
#if PA_NT_LOADS
  return __builtin_nontemporal_load((gT)p);
#else
  return *(gT)p;
#endif
}

// Software pipeline over a wavefront's pages: fetch(i, buf) is issued PF pages
// ahead of process(i, buf); buffers rotate through a ring whose indices are
// compile-time constants after unrolling, so they stay in registers. pre(i)
// runs before page i + PF is fetched (page i is then already in flight and
// the ring slot of page i + PF still free: the fewest registers are live).
template <int PF, typename Buf, typename Fetch, typename Process, typename Pre>
__device__ __forceinline__ void pipeline(int n, Buf (&buf)[PF + 1], Fetch&& fetch,
                                         Process&& process, Pre&& pre) {
  constexpr int NB = PF + 1;
#pragma unroll
  for (int b = 0; b < PF; ++b)
    if (b < n) fetch(b, buf[b]);
  int t0 = 0;
#if PA_STEADY
  // Steady state: every fetch of the round is in range, so none sits under a
  // branch (a conditional fetch joins its registers with the old contents,
  // and the copies that join needs wait for the loads just issued).
  for (; PF > 0 && t0 + NB + PF <= n; t0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      pre(t0 + b);
      fetch(t0 + b + PF, buf[(b + PF) % NB]);
#if PA_PIN_PREFETCH
      __builtin_amdgcn_sched_barrier(0);
#endif
      process(t0 + b, buf[b]);
    }
  }
#endif
  for (; t0 < n; t0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int t = t0 + b;
      if (t < n) {
        pre(t);
        if (t + PF < n) fetch(t + PF, buf[(b + PF) % NB]);
#if PA_PIN_PREFETCH
        // Keep the prefetch loads ahead of this page's compute: left free, the
        // scheduler may sink them past it, which serialises load and compute.
        __builtin_amdgcn_sched_barrier(0);
#endif
        process(t, buf[b]);
      }
    }
  }
}

constexpr int prefetch_for(int page_regs) {
  return page_regs <= PA_PF_REG_BUDGET ? PA_PREFETCH : 0;
}

// cand(h) for a lane-varying h in [0, N) as a tree of selects over scalars.
// Every candidate is evaluated unconditionally first: cand() reads other lanes
// (v_readlane, a convergent operation), so a short-circuit `b ? cand(1) :
// cand(0)` would become a divergent branch. Candidates are kept in scalars,
// not an array, which the compiler could fold into an indexed stack load.
template <int N, typename F>
__device__ __forceinline__ float pick(int h, F&& cand) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "pick: N in {1, 2, 4, 8}");
  const bool b0 = h & 1, b1 = h & 2, b2 = h & 4;
  if constexpr (N == 1) {
    return cand(0);
  } else if constexpr (N == 2) {
    const float c0 = cand(0), c1 = cand(1);
    return b0 ? c1 : c0;
  } else if constexpr (N == 4) {
    const float c0 = cand(0), c1 = cand(1), c2 = cand(2), c3 = cand(3);
    const float lo = b0 ? c1 : c0, hi = b0 ? c3 : c2;
    return b1 ? hi : lo;
  } else {
    const float c0 = cand(0), c1 = cand(1), c2 = cand(2), c3 = cand(3);
    const float c4 = cand(4), c5 = cand(5), c6 = cand(6), c7 = cand(7);
    const float c01 = b0 ? c1 : c0, c23 = b0 ? c3 : c2, c45 = b0 ? c5 : c4, c67 = b0 ? c7 : c6;
    const float lo = b1 ? c23 : c01, hi = b1 ? c67 : c45;
    return b2 ? hi : lo;
  }
}

struct PartitionArgs {
  float* tmp_out;
  float* exp_sums;
  float* max_logits;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* sl;
  int S, H, KH, MB, P, PS;
  int NB;          // physical blocks; block-table entries are clamped into [0, NB)
  // Columns: a unit's Mq * G (query token m, query head kh*G + h) pairs, column
  // m*G + h; one launch covers columns c0 .. c0 + NC - 1 (NC = G, c0 = 0 for
  // single-query decode).
  int Mq;          // query tokens per sequence in the tensors (query [S, Mq, H, D])
  int NC, c0;      // columns of this launch, first one
  int C;           // consecutive partitions per workgroup (span), 1 .. kMaxSpan
  int through;     // 1: tmp_output stores with device-scope (sc1) policy
  float qk_scale;  // scale * log2(e) (times k_scale for an 8-bit cache)
  float v_scale;   // 1, or v_scale for an 8-bit cache (applied once, at the merge)
  const float* alibi;  // [H] ALiBi slopes (read by the AL kernels only)
  int lpt;             // 1: workgroups take units largest first (see lpt_pair)
  // One-call decode (combine_store): the workgroup combines its span's
  // partitions itself instead of storing a row per partition.
  int fuse;            // 0: a row per partition (phase 1 alone); 1: combine the span
  int Pq;              // fuse: span entries per row, ceil(P / C); 1: the span is the row
  void* out;           // fuse, Pq == 1: out [S * Mq * H, D] in odt
  float* lse;          // fuse, Pq == 1: optional [S * Mq * H] row log-sum-exp (NULL: none)
  int odt;             // DT_F32, DT_F16 or DT_BF16
  int roll;            // fuse, MFMA kernel: 0 (combine_store) or R = 1, 2 ring slots of
                       // the rolling merge (see roll_layout)
  int lds_bytes;       // dynamic LDS of the launch: a kernel whose layout needs more
                       // returns at once, writing nothing (a host planning error)
};

// ALiBi: a query at position i adds slope_h * (j - i) to its scaled score for
// the key at position j (Press, Smith and Lewis, "Train Short, Test Long",
// ICLR 2022; the page's launcher only names the slopes). The bias is split as
// slope * (j - T0) + slope * (T0 - i), T0 the first key of j's partition: the
// first part enters each score (at most slope * PS in magnitude, so fp32
// keeps the scores' absolute precision however far the partition lies from
// the query); the second is the same for the whole partition, cancels in its
// exp sum and normalised output, and is added to its max logit at the store.

constexpr int kMaxSpan = 8;

// LDS carve-up shared by both partition kernels (byte offsets): the span's
// block-table slice, then per (partition of the span, wavefront, head) the
// parked running max, sum and accumulator.
struct LdsLayout {
  int bt_off, m_off, l_off, acc_off, total;
};
// NC = columns of a unit (query heads x query tokens).
__host__ __device__ inline LdsLayout lds_layout(int PS, int BS, int NC, int D, int C) {
  LdsLayout o;
  auto up16 = [](int v) { return (v + 15) & ~15; };
  o.bt_off = 0;
  o.m_off = up16(C * (PS / BS) * 4);
  o.l_off = o.m_off + up16(C * kWaves * NC * 4);
  o.acc_off = o.l_off + up16(C * kWaves * NC * 4);
  o.total = o.acc_off + C * kWaves * NC * D * 4;
  return o;
}

// LDS of the rolling merge (the MFMA kernel's one-call decode, a.roll = R):
// the span's block-table slice; R ring slots, each holding per wavefront and
// column tile its 16 columns' running max and exp sum, then, per owning
// wavefront, source wavefront (the three others), column tile and owned
// d-block, the source's 64 lanes x 16 bytes of accumulator; then each
// wavefront's running rows (per tile and owned d-block, 64 lanes x 16 bytes).
// A wavefront owns D / 64 of the D / 16 d-blocks of 16 rows.
struct RollLayout {
  int bt_off, slot_off, slot_bytes, stat_bytes, run_off, total;
};
__host__ __device__ inline RollLayout roll_layout(int PS, int BS, int CT, int D, int C, int R) {
  RollLayout o;
  const int VQ = D / 64;
  o.bt_off = 0;
  o.slot_off = (C * (PS / BS) * 4 + 15) & ~15;
  o.stat_bytes = kWaves * CT * 16 * 4 * 2;
  o.slot_bytes = o.stat_bytes + kWaves * 3 * CT * VQ * 1024;
  o.run_off = o.slot_off + R * o.slot_bytes;
  o.total = o.run_off + kWaves * CT * VQ * 1024;
  return o;
}

// Stores of the partition outputs (written once, read once by the reduce).
// Interleaved with the streaming K/V reads, written-back tmp lines cost
// several times their size in read bandwidth. Device-scope (sc1) stores
// measured up to ~6 % faster where each row has many partitions (64: long
// context, 16: 256-wide heads, or 16 columns per unit: 4x the rows) and up
// to ~2.5 % slower where it has few (4-8 partitions of 4 single-query heads:
// ragged GQA batches), so the host picks the policy per launch (`through`).
constexpr int kRsrcFlags = 0x00020000;  // raw buffer resource: 32-bit format, no swizzle
constexpr int kStoreThrough = 16;       // buffer-instruction cache policy: sc1
__device__ __forceinline__ void store_row(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v,
                                          bool through) {
  const u32x4 w = __builtin_bit_cast(u32x4, v);
  if (through)
    __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, kStoreThrough);
  else
    __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, 0);
}

// Slot of (partition j of the span, wavefront w, column c) in the parked state.
__device__ __forceinline__ int slot(int j, int w, int c, int NC) { return (j * kWaves + w) * NC + c; }

// Merge the NW parked states of each of the span's ne used partitions
// (log2-domain max m, sum l, unnormalised accumulator) and store the
// normalised outputs. Local column c of the launch is column a.c0 + c = m*G + h
// of the unit: query token m (of Mq) and query head kh*G + h; its output rows
// are ((s*Mq + m)*H + kh*G + h) of the [S*Mq*H, P] statistics and
// [S*Mq*H, P, D] tmp_output. Two steps with a barrier between them:
//  1. one thread per (column, partition) forms the partition's max Mx over
//     the wavefronts, its exp sum Z = sum_w e^(m_w - Mx) l_w and its
//     statistics, and each wavefront's row weight e^(m_w - Mx) v_scale / Z,
//     which it writes over that wavefront's parked max (a thread touches only
//     its own slots);
//  2. threads walk (column, partition, d) in memory order, so the rows of
//     adjacent partitions of one head are written together; a row is the
//     weighted sum of the wavefronts' accumulators.
// A column whose causal prefix ends before a used partition merges to max
// -inf, sum 0 and a zero row (the empty-partition sentinels).
// The caller has synchronised the workgroup after parking; all its threads
// call this (it contains a barrier).
template <int D, bool AL>
__device__ __forceinline__ void merge_store(const PartitionArgs& a, float* s_m, const float* s_l,
                                            const float* s_acc, int s, int kh, int p0, int ne,
                                            int G, int NC, int L) {
  constexpr int D4 = D / 4;
  const int per_col = ne * D4;
  const int mf = a.c0 / G, ml = (a.c0 + NC - 1) / G;  // first and last query token here
  const size_t row0 = ((size_t)s * a.Mq + mf) * a.H + kh * G;  // row of (mf, head kh*G)
  for (int i = late_tid(); i < NC * ne; i += kWaves * 64) {
    const int c = i / ne, j = i - c * ne;
    const int m = (a.c0 + c) / G, h = a.c0 + c - m * G;
    float mw[kWaves];
    float Mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = s_m[slot(j, w, c, NC)];
      Mx = fmaxf(Mx, mw[w]);
    }
    const float Mu = Mx == kNegInf ? 0.0f : Mx;  // a column with no keys here: all weights 0
    float e[kWaves];
    float Z = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      e[w] = fast_exp2(mw[w] - Mu);  // 0 for a wavefront with no tokens
      Z += e[w] * s_l[slot(j, w, c, NC)];
    }
    const float f = Z > 0.0f ? a.v_scale / Z : 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s_m[slot(j, w, c, NC)] = e[w] * f;
    float mx = Mx;
    if constexpr (AL) {  // the partition's share of the ALiBi bias (see PartitionArgs)
      const float slope2 = a.alibi[kh * G + h] * kLog2e;
      mx += slope2 * (float)((p0 + j) * a.PS - (L - a.Mq + m));
    }
    const size_t row = (row0 + (m - mf) * a.H + h) * a.P + p0 + j;
    a.exp_sums[row] = Z;
    a.max_logits[row] = mx * kLn2;
  }
  __syncthreads();
  // The launch's rows of tmp_output (query tokens mf..ml x heads x P), 32-bit offsets.
  const __amdgpu_buffer_rsrc_t tmp = __builtin_amdgcn_make_buffer_rsrc(
      a.tmp_out + row0 * a.P * D, (short)0, ((ml - mf) * a.H + G) * a.P * D * 4, kRsrcFlags);
  for (int i = late_tid(); i < NC * per_col; i += kWaves * 64) {
    const int c = i / per_col, rem = i - c * per_col;
    const int j = rem / D4, d4 = rem - j * D4;
    const int m = (a.c0 + c) / G, h = a.c0 + c - m * G;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int k = slot(j, w, c, NC);
      o += s_m[k] * *(const f32x4*)&s_acc[k * D + 4 * d4];
    }
    const int hrow = (m - mf) * a.H + h;  // row of this column relative to row0
    store_row(tmp, (uint32_t)(((hrow * a.P + p0 + j) * D + 4 * d4) * 4), o, a.through);
  }
}

// Store four fp32 values of an output row in the output dtype (round to
// nearest even for the 16-bit types).
__device__ __forceinline__ void store_out4(void* out, int odt, size_t off, f32x4 v) {
  if (odt == DT_F32) {
    *(f32x4*)((float*)out + off) = v;
  } else if (odt == DT_F16) {
    *(u32x2*)((uint16_t*)out + off) =
        u32x2{codec<DT_F16>::pack(v[0], v[1]), codec<DT_F16>::pack(v[2], v[3])};
  } else {
    *(u32x2*)((uint16_t*)out + off) =
        u32x2{codec<DT_BF16>::pack(v[0], v[1]), codec<DT_BF16>::pack(v[2], v[3])};
  }
}

// One-call decode epilogue. Each of the span's ne used partitions is merged
// over the wavefronts as merge_store does it -- partition j's max m_j (log2
// units, plus its share of the ALiBi bias), exp sum l_j and normalised row
// o_j = sum_w e^(m_jw - max_w m_jw) acc_jw / l_j -- and the partitions are
// combined with the reduce's log-sum-exp rule: M = max_j m_j,
// Z = sum_j e^(m_j - M) l_j, row = sum_j (e^(m_j - M) l_j / Z) o_j. The two
// weights of a wavefront's accumulator are folded into one,
// e^(m_jw - max_w m_jw) e^(m_j - M) v_scale / Z, in three steps separated by
// barriers, each thread touching only its own parked slots until the last:
//  1. one thread per (column, partition): the partition's maxima, l_j and m_j
//     (kept in its first two exp-sum slots) and the wavefront factors
//     e^(m_jw - max_w m_jw) (over the parked maxima);
//  2. the same threads: M and Z of the column from every partition's l_j and
//     m_j, and the factors scaled by e^(m_j - M) v_scale / Z; one thread per
//     column stores the span's statistics;
//  3. threads walk (column, d) and sum the weighted accumulators.
// When the span holds every partition of the row (Pq == 1) that row is the
// attention output: it goes to `out` in its dtype, with lse = M + ln Z if
// asked for, and nothing is written to the workspace. Otherwise the span's
// (M, Z, row) is entry q = p0 / C of a [rows, Pq] workspace, which the reduce
// combines exactly like partitions of C * PS tokens. A column with no keys in
// the span (several query tokens, causal prefix ended earlier) gets M = -inf,
// Z = 0 and a zero row. The caller has synchronised the workgroup after
// parking; all its threads call this (it contains barriers).
template <int D, bool AL>
__device__ __forceinline__ void combine_store(const PartitionArgs& a, float* s_m, float* s_l,
                                              const float* s_acc, int s, int kh, int p0, int ne,
                                              int G, int NC, int L) {
  constexpr int D4 = D / 4;
  const int q = p0 / a.C;
  const int mf = a.c0 / G, ml = (a.c0 + NC - 1) / G;  // first and last query token here
  const size_t row0 = ((size_t)s * a.Mq + mf) * a.H + kh * G;  // row of (mf, head kh*G)
  for (int i = late_tid(); i < NC * ne; i += kWaves * 64) {
    const int c = i / ne, j = i - c * ne;
    float mw[kWaves];
    float Mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = s_m[slot(j, w, c, NC)];
      Mx = fmaxf(Mx, mw[w]);
    }
    const float mu = Mx == kNegInf ? 0.0f : Mx;  // 0 if no wavefront saw a key
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2(mw[w] - mu);
      l += e * s_l[slot(j, w, c, NC)];
      s_m[slot(j, w, c, NC)] = e;
    }
    float mx = Mx;
    if constexpr (AL) {
      const int m = (a.c0 + c) / G, h = a.c0 + c - m * G;
      mx += a.alibi[kh * G + h] * kLog2e * (float)((p0 + j) * a.PS - (L - a.Mq + m));
    }
    s_l[slot(j, 0, c, NC)] = l;
    s_l[slot(j, 1, c, NC)] = mx;
  }
  __syncthreads();
  for (int i = late_tid(); i < NC * ne; i += kWaves * 64) {
    const int c = i / ne, j = i - c * ne;
    float M = kNegInf;
    for (int k = 0; k < ne; ++k) M = fmaxf(M, s_l[slot(k, 1, c, NC)]);
    const float Mu = M == kNegInf ? 0.0f : M;
    float Z = 0.0f;
    for (int k = 0; k < ne; ++k) {
      const float lk = s_l[slot(k, 0, c, NC)];
      Z += lk > 0.0f ? fast_exp2(s_l[slot(k, 1, c, NC)] - Mu) * lk : 0.0f;
    }
    // (a partition without keys for this column has weight 0)
    const float lj = s_l[slot(j, 0, c, NC)];
    const float f = lj > 0.0f ? fast_exp2(s_l[slot(j, 1, c, NC)] - Mu) * a.v_scale / Z : 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s_m[slot(j, w, c, NC)] *= f;
    if (j == 0) {
      const int m = (a.c0 + c) / G, h = a.c0 + c - m * G;
      const size_t row = row0 + (m - mf) * a.H + h;
      if (a.Pq == 1) {
        if (a.lse) a.lse[row] = Z > 0.0f ? fmaf(__builtin_amdgcn_logf(Z), kLn2, M * kLn2) : kNegInf;
      } else {
        a.exp_sums[row * a.Pq + q] = Z;
        a.max_logits[row * a.Pq + q] = M * kLn2;
      }
    }
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t tmp = __builtin_amdgcn_make_buffer_rsrc(
      a.tmp_out + row0 * a.Pq * D, (short)0, ((ml - mf) * a.H + G) * a.Pq * D * 4, kRsrcFlags);
  for (int i = late_tid(); i < NC * D4; i += kWaves * 64) {
    const int c = i / D4, d4 = i - c * D4;
    const int m = (a.c0 + c) / G, h = a.c0 + c - m * G;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < ne; ++j) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int k = slot(j, w, c, NC);
        o += s_m[k] * *(const f32x4*)&s_acc[k * D + 4 * d4];
      }
    }
    const int hrow = (m - mf) * a.H + h;  // row of this column relative to row0
    if (a.Pq == 1)
      store_out4(a.out, a.odt, (row0 + hrow) * D + 4 * d4, o);
    else
      store_row(tmp, (uint32_t)(((hrow * a.Pq + q) * D + 4 * d4) * 4), o, a.through);
  }
}

// A work unit: sequence s, kv head kh, partitions p0 .. p0+nparts-1.
struct Unit {
  int s, kh, p0, nparts, G, L, pg0;
  int NC;          // columns of this launch
  int npages;      // used pages of the span (contiguous from its first page)
  int ne;          // used partitions of the span
  int32_t bt_val;  // this thread's entry of the span's block-table slice
};

// Pages of span ch (partitions ch*C .. ch*C + C - 1) of a length-L sequence.
template <int BS>
__device__ __forceinline__ int span_pages(const PartitionArgs& a, int L, int ch) {
  const int cap = min(a.C, a.P - ch * a.C) * a.PS;
  const int n = min(max(L - ch * a.C * a.PS, 0), cap);
  return (n + BS - 1) / BS;
}

// LDS bytes lpt_pair needs (host and device).
__host__ __device__ inline int lpt_lds_bytes(int S, int P, int PS, int BS, int C) {
  const int pmax = C * PS / BS, pairs = S * ((P + C - 1) / C);
  return ((4 * (pmax + 1) + 15) & ~15) + ((2 * pairs + 15) & ~15) + 16;
}

// Largest-first work order. With ragged lengths the units (sequence, span)
// range from empty to full; dispatched in index order, the last workgroups of
// a launch are a random mix of sizes and a few long ones finish alone. Here
// every workgroup ranks all (sequence, span) pairs by their page count,
// descending (a counting sort; ties keep index order), and takes the pair of
// its own rank, so full spans run first, partial ones by size after them and
// empty ones (sentinel writes only) last. The order depends only on the
// lengths, so every workgroup derives the same one; each unit is still
// computed exactly as before, so results do not depend on the order.
// Uses LDS from `smem` (lpt_lds_bytes) before the unit's own use of it.
template <int BS>
__device__ __forceinline__ int lpt_pair(const PartitionArgs& a, uint8_t* smem) {
  const int pmax = a.C * a.PS / BS;
  const int pairs = a.S * ((a.P + a.C - 1) / a.C);
  int* hist = (int*)smem;  // [pmax + 1] pairs per page count
  uint16_t* keys = (uint16_t*)(smem + ((4 * (pmax + 1) + 15) & ~15));  // [pairs] page counts
  int* res = (int*)((uint8_t*)keys + ((2 * pairs + 15) & ~15));
  for (int k = threadIdx.x; k <= pmax; k += kWaves * 64) hist[k] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < pairs; i += kWaves * 64) {  // pair i = span ch of sequence s
    const int ch = i / a.S, s = i - ch * a.S;
    const int key = span_pages<BS>(a, a.sl[s], ch);
    keys[i] = (uint16_t)key;
    atomicAdd(&hist[key], 1);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int r = blockIdx.x / a.KH;  // this workgroup's rank among the pairs
    if (lane == 0) res[0] = r;         // (index order if the search below finds nothing)
    // Page counts in descending order d = pmax - k; lane owns d in [lane*W, lane*W + W).
    const int W = (pmax + 64) / 64;
    int sum = 0;
    for (int e = 0; e < W; ++e) {
      const int d = lane * W + e;
      if (d <= pmax) sum += hist[pmax - d];
    }
    int incl = sum;  // inclusive scan over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int excl = incl - sum;
    const uint64_t own = __builtin_amdgcn_ballot_w64(r >= excl && r < incl);
    const int owner = own ? __builtin_ctzll(own) : 0;
    int key = -1, j = 0;
    if (lane == owner && own) {
      int before = excl;
      for (int e = 0; e < W && lane * W + e <= pmax; ++e) {
        const int k = pmax - (lane * W + e);
        if (r < before + hist[k]) {
          key = k;
          j = r - before;
          break;
        }
        before += hist[k];
      }
    }
    key = __builtin_amdgcn_readlane(key, owner);
    j = __builtin_amdgcn_readlane(j, owner);
    // The j-th pair (in index order) whose page count is key.
    for (int base = 0; base < pairs; base += 64) {
      const int i = base + lane;
      const bool m = i < pairs && keys[i] == key;
      const uint64_t mb = __builtin_amdgcn_ballot_w64(m);
      const int c = __builtin_popcountll(mb);
      if (j < c) {
        if (m && __builtin_popcountll(mb & ((1ull << lane) - 1)) == j) res[0] = i;
        break;
      }
      j -= c;
    }
  }
  __syncthreads();
  return min(max(res[0], 0), pairs - 1);
}

// Decode the unit and issue its first loads together: the sequence length and
// the block-table slice of the whole span (clamped to the row, so always in
// bounds; entries past the sequence's last block are loaded but never used).
// Nothing here waits on the length, so the loads overlap.
template <int BS>
__device__ __forceinline__ void unit_begin(const PartitionArgs& a, Unit& u, uint8_t* smem) {
  u.kh = blockIdx.x % a.KH;
  // (uniform; read out of lane 0 so that the unit's indices live in scalar
  // registers rather than vector ones)
  const int pair =
      __builtin_amdgcn_readfirstlane(a.lpt ? lpt_pair<BS>(a, smem) : (int)(blockIdx.x / a.KH));
  u.s = pair % a.S;
  u.p0 = (pair / a.S) * a.C;
  u.nparts = min(a.C, a.P - u.p0);
  u.G = a.H / a.KH;
  u.NC = a.NC;
  const int pps = a.PS / BS;
  u.pg0 = u.p0 * pps;
  const int nspec = min(u.nparts * pps, a.MB - u.pg0);
  u.bt_val = (int)threadIdx.x < nspec ? a.bt[(size_t)u.s * a.MB + u.pg0 + threadIdx.x] : 0;
  u.L = a.sl[u.s];
}

// After unit_begin: sentinels (max -inf, sum 0) for the span's empty
// partitions; false if the whole span is empty, otherwise publish the span's
// block-table slice to LDS for the whole workgroup.
template <int BS, int D>
__device__ __forceinline__ bool unit_hoist(const PartitionArgs& a, int32_t* s_bt, Unit& u) {
  u.L = __builtin_amdgcn_readfirstlane(u.L);  // (uniform, as the unit's indices)
  const int t0 = u.p0 * a.PS;
  if (!a.fuse) {
    if ((int)threadIdx.x < u.nparts * u.NC) {
      const int j = threadIdx.x / u.NC, c = a.c0 + threadIdx.x % u.NC;
      const int m = c / u.G, h = c - m * u.G;
      if ((u.p0 + j) * a.PS >= u.L) {
        const size_t row =
            (((size_t)u.s * a.Mq + m) * a.H + u.kh * u.G + h) * a.P + u.p0 + j;
        a.max_logits[row] = kNegInf;
        a.exp_sums[row] = 0.0f;
      }
    }
  } else if (t0 >= u.L) {
    // An empty span of the one-call decode: the sentinel entry (Pq > 1), or,
    // when the span is the whole row (an empty sequence), out = 0, lse = -inf.
    for (int i = threadIdx.x; i < u.NC * (a.Pq > 1 ? 1 : D / 4); i += kWaves * 64) {
      const int ci = a.Pq > 1 ? i : i / (D / 4), d4 = a.Pq > 1 ? 0 : i % (D / 4);
      const int c = a.c0 + ci, m = c / u.G, h = c - m * u.G;
      const size_t row = ((size_t)u.s * a.Mq + m) * a.H + u.kh * u.G + h;
      if (a.Pq > 1) {
        a.max_logits[row * a.Pq + u.p0 / a.C] = kNegInf;
        a.exp_sums[row * a.Pq + u.p0 / a.C] = 0.0f;
      } else {
        store_out4(a.out, a.odt, row * D + 4 * d4, f32x4{0.f, 0.f, 0.f, 0.f});
        if (a.lse && d4 == 0) a.lse[row] = kNegInf;
      }
    }
  }
  if (t0 >= u.L) return false;
  const int t1 = min(t0 + u.nparts * a.PS, u.L);
  u.npages = (t1 - t0 + BS - 1) / BS;
  u.ne = (t1 - t0 + a.PS - 1) / a.PS;
  if ((int)threadIdx.x < u.npages) s_bt[threadIdx.x] = u.bt_val;
  __syncthreads();
  return true;
}

// =====================================================================
// MFMA path: 16-bit query, columns (query token, query head) of a kv head in
// CT tiles of 16 (a launch covers up to 16*CT of them); the cache is 16-bit
// (KV8 = false) or OCP E4M3 bytes converted to the query's type in registers
// (KV8 = true). The column tiles share every K and V operand: CT = 2 reads the
// pages once for up to 32 columns.
// QK^T per 16-token sub-tile and column tile: D/32 MFMA 16x16x32, token rows x
// columns (columns past the launch's are zero-padded). The fp32 C tile (lane l: tokens 4*(l/16)+r,
// head l%16) is exactly the B operand layout of a 16x16x16 MFMA with tokens as
// k, so P feeds PV without any data movement. V is read as 4 tokens of one d
// (8 bytes, or 4 bytes for an 8-bit cache) that form the matching A operand.
// P is split into a 16-bit high part and a 16-bit residual so the
// probabilities keep ~16 bits of mantissa instead of bf16's 8; both enter one
// 16x16x32 PV MFMA (16-bit caches) or two 16x16x16 ones (8-bit caches).
// K k-steps: a 16-bit cache chunk is 8 d of one token (one k-step per 16-byte
// load); an 8-bit chunk is 16 d (two k-steps per load: its low and high 8 d).
// The query B operand follows the same d assignment, so the contraction over
// d is unchanged.
// =====================================================================
template <bool KV8, int SUB, int D> struct MfmaPage {
  u32x4 k[SUB][D / 32];  // 16-bit K: one 16-byte load per k-step
  u32x2 v[SUB][D / 16];  // 16-bit V: 4 tokens x 2 bytes per d-block
};
template <int SUB, int D> struct MfmaPage<true, SUB, D> {
  u32x4 k[SUB][D / 64];  // 8-bit K: one 16-byte load per two k-steps
  u32x4 v[SUB][D / 64];  // 8-bit V: 16 tokens of one d per 16-byte load (see v_words)
};

// 8-bit V operands. The PV A operand of d-block mb wants, in lane (g, r)
// (g = lane % 16, r = lane / 16), tokens 4r .. 4r+3 of d-row 16 mb + g: four
// bytes. Loading those directly takes one 4-byte load per d-block; instead
// lane (g, r) loads all 16 tokens of d-row 16 (4q + r) + g with one 16-byte
// load (words w0..w3 = tokens 0-3 .. 12-15), and a 4 x 4 transpose across
// the four 16-lane rows (gfx950's v_permlane32_swap then v_permlane16_swap:
// the former swaps the upper half of its first operand with the lower half of
// its second, the latter the odd rows of the first with the even rows of the
// second) leaves in lane (g, r) word r of each of d-blocks 4q .. 4q+3.
__device__ __forceinline__ void v_words(u32x4 w, uint32_t (&out)[4]) {
  const auto a02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
  const auto a13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
  const auto b01 = __builtin_amdgcn_permlane16_swap(a02[0], a13[0], false, false);
  const auto b23 = __builtin_amdgcn_permlane16_swap(a02[1], a13[1], false, false);
  out[0] = b01[0];
  out[1] = b01[1];
  out[2] = b23[0];
  out[3] = b23[1];
}

// Pages in flight for an 8-bit cache page of `page_regs` VGPRs. An 8-bit page
// carries twice the arithmetic per byte of a 16-bit one, so occupancy matters
// more than depth (three pages ahead at 2 wavefronts per SIMD measured ~20 %
// slower than one page ahead at 3 or 4): one page ahead for small pages,
// none for larger ones.
#ifndef PA_PREFETCH_FP8
#define PA_PREFETCH_FP8 1
#endif
constexpr int prefetch_fp8(int page_regs) { return page_regs <= 16 ? PA_PREFETCH_FP8 : 0; }

// Wavefronts per SIMD the 8-bit MFMA kernel is register-budgeted for: its
// pages carry twice the arithmetic per byte of a 16-bit cache's, so latency
// hiding needs more resident wavefronts (D = 128, BS = 16: 4 per SIMD
// measured ~10 % faster than 3 and ~25 % faster than 2). Larger pages need
// more registers; the budget shrinks so that nothing spills (the ALiBi
// variant's two extra per-lane values tip the smallest page over 4).
#ifndef PA_FP8_WAVES
#define PA_FP8_WAVES 0  // measurement builds: >0 overrides the budget below
#endif
constexpr int fp8_waves(int D, int BS, bool AL) {
  return PA_FP8_WAVES > 0 ? PA_FP8_WAVES : D * BS <= 2048 && !AL ? 4 : D <= 128 ? 3 : 2;
}
// Wavefronts per SIMD of the 8-bit rolling-merge kernel (one column tile): its
// running combination and merge do not fit the plain 8-bit kernel's budget.
#ifndef PA_FP8_ROLL_WAVES
#define PA_FP8_ROLL_WAVES 2
#endif
// Register budget (wavefronts per SIMD) of the MFMA kernel: 2 for 16-bit
// caches (one or two column tiles; left unbounded, the one-tile kernel at head
// size 128 took 288 registers, one wavefront per SIMD, and ran ~1 % slower on
// the GQA and long-context batches than at 2) except the largest page (head
// size 256, 32-token blocks), which would spill at 2; the 8-bit budgets above
// otherwise.
constexpr int mfma_waves(int D, int BS, bool KV8, bool AL, int CT, bool ROLL) {
  return CT > 1 ? 2
         : KV8  ? (ROLL ? (PA_FP8_ROLL_WAVES < fp8_waves(D, BS, AL) ? PA_FP8_ROLL_WAVES
                                                                     : fp8_waves(D, BS, AL))
                        : fp8_waves(D, BS, AL))
                : (PA_MIN_WAVES > 0 ? PA_MIN_WAVES : D * BS <= 4096 ? 2 : 1);
}

// Pages in flight for the rolling-merge kernels: as the others, except with
// two column tiles, whose registers (two accumulators, two query operands,
// the merge) only fit two wavefronts per SIMD without a page of prefetch.
#ifndef PA_ROLL_CT2_PREFETCH
#define PA_ROLL_CT2_PREFETCH 0
#endif
template <bool ROLL, int CT>
constexpr int roll_prefetch(int pf) {
  return ROLL && CT > 1 ? (pf < PA_ROLL_CT2_PREFETCH ? pf : PA_ROLL_CT2_PREFETCH) : pf;
}

// ROLL: the one-call decode's rolling merge (see park_roll), a separate
// instantiation so that the other kernels carry none of its code or registers.
template <int DT, int D, int BS, bool KV8, bool AL, int CT, bool ROLL>
__global__ void __launch_bounds__(kWaves * 64)
__attribute__((amdgpu_waves_per_eu(mfma_waves(D, BS, KV8, AL, CT, ROLL))))
partition_mfma_kernel(PartitionArgs a) {
  static_assert(CT == 1 || CT == 2, "one or two column tiles");
  constexpr int SUB = BS / 16;  // 16-token sub-tiles per page
  constexpr int KS = D / 32;    // QK k-steps (32 d each) per sub-tile
  constexpr int KL = KV8 ? D / 64 : D / 32;  // K 16-byte loads per lane per sub-tile
  constexpr int VB = D / 16;    // PV d-blocks (16 d each)
  constexpr int ESZ = KV8 ? 1 : 2;
  constexpr size_t PAGE = (size_t)D * BS * ESZ;  // bytes of one (block, kv head) page
  constexpr int PREGS = SUB * (KL * 4 + VB * (KV8 ? 1 : 2));
  constexpr int PF = KV8 ? prefetch_fp8(PREGS) : roll_prefetch<ROLL, CT>(prefetch_for(PREGS));
  using C = codec<DT>;
  using M = mma<DT>;
  using Page = MfmaPage<KV8, SUB, D>;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Unit u;
  unit_begin<BS>(a, u, smem);
  const int G = u.G, NC = u.NC;
  const int lane = threadIdx.x & 63;
  // (read out of lane 0: the compiler then knows it is wavefront-uniform, so
  // the page index and the branches on it are scalar)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15, grp = lane >> 4;  // g: this lane's column in a tile (and token row)
  // Column 16t + g of the launch (tile t) is column a.c0 + 16t + g = qm*G + h
  // of the unit: query head kh*G + h of query token qm, which sees tokens
  // t < lim (the causal prefix; L for single-query decode). Padding columns
  // (>= NC) take the launch's first column with a zero query, so their
  // running max stays put like a live column's.
  int lim[CT];
  // The smallest of the launch's limits: that of its first column's query
  // token (the padding columns take the first column too).
  const int lim_lo = min(u.L, max(0, u.L - a.Mq + a.c0 / G + 1));
  float slope2[CT];  // ALiBi slope of the column, log2 units
  int qpos[CT];      // the column's query position (ALiBi, rolling merge)
  u32x4 qb[CT][KS];  // Q columns as the QK B operand
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const bool live = 16 * t + g < NC;
    const int c = a.c0 + (live ? 16 * t + g : 0);
    const int qm = c / G, h = c - qm * G;
    lim[t] = min(u.L, max(0, u.L - a.Mq + qm + 1));
    qpos[t] = u.L - a.Mq + qm;
    slope2[t] = AL && live ? a.alibi[u.kh * G + h] * kLog2e : 0.0f;
    // k-step mk: lane holds 8 consecutive d of its column, d = 32mk + 8*grp
    // (16-bit cache) or 16*(4*(mk/2) + grp) + 8*(mk%2) (8-bit).
    const uint16_t* qrow =
        (const uint16_t*)a.q + (((size_t)u.s * a.Mq + qm) * a.H + u.kh * G + h) * D;
#pragma unroll
    for (int mk = 0; mk < KS; ++mk) {
      const int d0 = KV8 ? 16 * (4 * (mk / 2) + grp) + 8 * (mk % 2) : 32 * mk + 8 * grp;
      u32x4 v = *(const u32x4*)(qrow + d0);
      qb[t][mk] = live ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const LdsLayout lay = lds_layout(a.PS, BS, NC, D, a.C);
  if ((ROLL ? roll_layout(a.PS, BS, CT, D, a.C, a.roll == 2 ? 2 : 1).total : lay.total) >
      a.lds_bytes)
    return;  // (uniform: the launch's LDS does not hold this kernel's layout)
  if (!unit_hoist<BS, D>(a, (int32_t*)smem, u)) return;
  const int32_t* s_bt = (const int32_t*)(smem + lay.bt_off);
  float* s_m = (float*)(smem + lay.m_off);
  float* s_l = (float*)(smem + lay.l_off);
  float* s_acc = (float*)(smem + lay.acc_off);
  const int pps = a.PS / BS;

  const size_t head_off = (size_t)u.kh * PAGE;
  const size_t blk_stride = (size_t)a.KH * PAGE;
  const uint8_t* kbase = (const uint8_t*)a.kc + head_off;
  const uint8_t* vbase = (const uint8_t*)a.vc + head_off;
  // K: chunk c = 4j + grp of token g at (c*BS + g)*16 bytes (+ st*256).
  const uint32_t k_lane = (uint32_t)(grp * BS + g) * 16;
  // V: d-row 16*mb + g, tokens 16*st + 4*grp .. +3 (16-bit); 8-bit: d-row
  // 16*(4q + grp) + g, tokens 16*st .. +15 (v_words).
  const uint32_t v_lane = KV8 ? (uint32_t)(16 * grp + g) * BS : (uint32_t)(g * BS + 4 * grp) * ESZ;

  const int npg = u.npages > wave ? (u.npages - wave + kWaves - 1) / kWaves : 0;

  float m[CT];     // running max (log2 domain), uniform over a column
  float lsum[CT];  // this lane's share of the running exp sum
  f32x4 acc[CT][VB];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    m[t] = kNegInf;
    lsum[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < VB; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Park this wavefront's state of partition jcur of the span in LDS and
  // start the next partition empty (wavefront-uniform control flow).
  int jcur = 0, next_edge = pps;  // next_edge: first page of partition jcur + 1
  auto park = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      const float ls = rows_sum(lsum[t]);
      if (16 * t + g < NC) {
        const int k = slot(jcur, wave, 16 * t + g, NC);
        if (grp == 0) {
          s_m[k] = m[t];
          s_l[k] = ls;
        }
        float* dst = s_acc + k * D + 4 * grp;
#pragma unroll
        for (int mb = 0; mb < VB; ++mb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[16 * mb + r] = acc[t][mb][r];
        }
      }
      m[t] = kNegInf;
      lsum[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < VB; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    ++jcur;
    next_edge += pps;
  };

  // Rolling merge (one-call decode, a.roll = R ring slots; roll_layout). At
  // each partition edge every wavefront hands the three quarters of its
  // accumulator that it does not own (d-blocks mb with mb / VQ != wave) to
  // their owners through LDS, with its columns' max and exp sum; after a
  // barrier each wavefront merges its own quarter of the partition over the
  // four wavefronts -- the partition's max logit, exp sum and normalised row,
  // exactly what the plain epilogue stores for it -- and folds that into its
  // running combination of the span's partitions with the log-sum-exp rule
  // (running max rM, sum rZ = sum_j e^(m_j - rM) l_j, rows sum_j e^(m_j - rM)
  // l_j o_j in LDS; the span's row is their ratio). With one slot, a second
  // barrier keeps the next partition's writes behind this one's merge; with
  // two, the next edge's barrier does. Every wavefront parks every used
  // partition of the span once, so all reach the same barriers.
  constexpr int VQ = VB / 4;
  static_assert(kWaves == 4 && VB % 4 == 0, "the rolling merge splits d-blocks over 4 wavefronts");
  float rM[CT], rZ[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    rM[t] = kNegInf;
    rZ[t] = 0.0f;
  }
  const int R = a.roll == 2 ? 2 : 1;  // ring slots (the host plans 1 or 2)
  const RollLayout rl = roll_layout(a.PS, BS, CT, D, a.C, R);
  f32x4* s_run = (f32x4*)(smem + rl.run_off) + wave * CT * VQ * 64 + lane;  // [t][mbl] x 64 lanes
  auto park_roll = [&]() __attribute__((always_inline)) {
    uint8_t* slotp = smem + rl.slot_off + (R == 2 ? (jcur & 1) : 0) * rl.slot_bytes;
    float* st_m = (float*)slotp;                 // [wave][t][16]
    float* st_l = st_m + kWaves * CT * 16;
    f32x4* xch = (f32x4*)(slotp + rl.stat_bytes);  // [owner][source 0..2][t][mbl][64 lanes]
    if (R == 1 && jcur > 0) __syncthreads();  // the slot's last merge is done
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      const float ls = rows_sum(lsum[t]);
      if (grp == 0) {
        st_m[(wave * CT + t) * 16 + g] = m[t];
        st_l[(wave * CT + t) * 16 + g] = ls;
      }
#pragma unroll
      for (int mb = 0; mb < VB; ++mb) {
        const int owner = mb / VQ;
        if (owner != wave)  // source index of this wavefront as the owner counts them
          xch[(((owner * 3 + ((wave - owner - 1) & 3)) * CT + t) * VQ + mb % VQ) * 64 + lane] =
              acc[t][mb];
      }
    }
    __syncthreads();  // the partition's four wavefront states are in the slot
    // The merge of this wavefront's quarter; WQ = wave as a compile-time
    // constant, so the accumulator's d-blocks are selected by register name
    // (a runtime index would put the accumulator in scratch memory).
    auto merge_quarter = [&](auto WQ) __attribute__((always_inline)) {
      constexpr int wq = decltype(WQ)::value;
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        // (statistics are re-read from LDS where needed rather than held in
        // registers: this runs with a page in flight and one being computed)
        float Mx = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, st_m[(w * CT + t) * 16 + g]);
        const float mu = Mx == kNegInf ? 0.0f : Mx;
        float Z = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)  // 0 for a wavefront with no keys
          Z += fast_exp2(st_m[(w * CT + t) * 16 + g] - mu) * st_l[(w * CT + t) * 16 + g];
        // The partition's max logit (log2 units, with its share of the bias)
        // and its weight in the running combination; a column with no keys
        // in it (Z = 0) leaves the running state as it is.
        float mj = Mx;
        if constexpr (AL) mj += slope2[t] * (float)((u.p0 + jcur) * a.PS - qpos[t]);
        const bool has = Z > 0.0f;
        const float nM = has ? fmaxf(rM[t], mj) : rM[t];
        const float al = has ? fast_exp2(rM[t] - nM) : 1.0f;
        const float be = has ? fast_exp2(mj - nM) * Z : 0.0f;
        const float inv = has ? a.v_scale / Z : 0.0f;
        rM[t] = nM;
        rZ[t] = rZ[t] * al + be;
#pragma unroll
        for (int mbl = 0; mbl < VQ; ++mbl) {
          f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {  // sources in wavefront order
            const f32x4 v =
                w == wq ? acc[t][wq * VQ + mbl]
                        : xch[(((wq * 3 + ((w - wq - 1) & 3)) * CT + t) * VQ + mbl) * 64 + lane];
            o += fast_exp2(st_m[(w * CT + t) * 16 + g] - mu) * v;
          }
          const f32x4 oj = o * inv;  // the partition's normalised row (this lane's 4 d)
          f32x4* r = s_run + (t * VQ + mbl) * 64;
          *r = (jcur == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : *r * al) + be * oj;
        }
      }
    };
    switch (wave) {
      case 0: merge_quarter(std::integral_constant<int, 0>{}); break;
      case 1: merge_quarter(std::integral_constant<int, 1>{}); break;
      case 2: merge_quarter(std::integral_constant<int, 2>{}); break;
      default: merge_quarter(std::integral_constant<int, 3>{}); break;
    }
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      m[t] = kNegInf;
      lsum[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < VB; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    ++jcur;
    next_edge += pps;
  };

  // The page's base is wavefront-uniform (scalar registers) and each lane adds
  // a 32-bit offset: the loads take the scalar-base form, with no per-page
  // 64-bit address arithmetic in vector registers.
  auto fetch = [&](int i, Page& pg) {
    const int blk = min(max(__builtin_amdgcn_readfirstlane(s_bt[wave + i * kWaves]), 0), a.NB - 1);
    gbytes kpage = (gbytes)(kbase + (size_t)blk * blk_stride);
    gbytes vpage = (gbytes)(vbase + (size_t)blk * blk_stride);
    // (opaque scalar values from here: the compiler would otherwise fold the
    // lane offsets into the base once, outside the loop, and redo the page
    // arithmetic per lane)
    asm volatile("" : "+s"(kpage), "+s"(vpage));
#pragma unroll
    for (int j = 0; j < KL; ++j) {
#pragma unroll
      for (int st = 0; st < SUB; ++st)
        pg.k[st][j] = stream_load<u32x4>(kpage + (k_lane + (uint32_t)(j * 4 * BS * 16 + st * 256)));
    }
#pragma unroll
    for (int mb = 0; mb < VB; ++mb) {
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
        if constexpr (KV8) {
          if (mb % 4 == 0)
            pg.v[st][mb / 4] =
                stream_load<u32x4>(vpage + (v_lane + (uint32_t)(mb * 16 * BS + st * 16)));
        } else {
          pg.v[st][mb] = stream_load<u32x2>(vpage + (v_lane + (uint32_t)(mb * 16 * BS * 2 + st * 32)));
        }
      }
    }
  };

  // A operand of QK k-step mk of sub-tile st (8-bit: low or high 8 d of a chunk).
  auto k_operand = [&](const Page& pg, int st, int mk) -> u32x4 {
    if constexpr (KV8) {
      using F = fp8cvt<DT>;
      const u32x4 w = pg.k[st][mk / 2];
      const uint32_t w0 = (mk % 2) ? w[2] : w[0], w1 = (mk % 2) ? w[3] : w[1];
      return u32x4{F::template pair<false>(w0), F::template pair<true>(w0),
                   F::template pair<false>(w1), F::template pair<true>(w1)};
    } else {
      return pg.k[st][mk];
    }
  };
  using VWord = typename std::conditional<KV8, uint32_t, u32x2>::type;
  auto v_operand = [&](VWord w) -> u32x2 {
    if constexpr (KV8) {
      using F = fp8cvt<DT>;
      return u32x2{F::template pair<false>(w), F::template pair<true>(w)};
    } else {
      return w;
    }
  };

  auto process = [&](int i, const Page& pg) {
    const int page = wave + i * kWaves;  // page of the span
    while (page >= next_edge) park();  // (the rolling merge has parked in pre)
    const int tok0 = (u.pg0 + page) * BS;  // first token of the page
    const bool full = tok0 + BS <= lim_lo;
    float s2[CT][SUB][4];
#pragma unroll
    for (int st = 0; st < SUB; ++st) {
      f32x4 sc[CT];
#pragma unroll
      for (int t = 0; t < CT; ++t) sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mk = 0; mk < KS; ++mk) {
        const u32x4 ko = k_operand(pg, st, mk);
#pragma unroll
        for (int t = 0; t < CT; ++t) sc[t] = M::qk(ko, qb[t][mk], sc[t]);
      }
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        // score of row 4*grp+r (log2 units, with this page's share of the bias)
        auto score = [&](int r) {
          if constexpr (AL) {  // position relative to the page's partition start
            const float base =
                slope2[t] * (float)(tok0 + 16 * st + 4 * grp - (u.p0 + jcur) * a.PS);
            return fmaf(sc[t][r], a.qk_scale, fmaf(slope2[t], (float)r, base));
          } else {
            return sc[t][r] * a.qk_scale;
          }
        };
#pragma unroll
        for (int r = 0; r < 4; ++r) s2[t][st][r] = score(r);
      }
    }
    // Rows past a column's limit (the sequence's end, or a query token's causal
    // prefix): only on pages that reach a limit (wavefront-uniform branch).
    if (!full) {
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          const int nvalid = lim[t] - (tok0 + 16 * st + 4 * grp);  // row 4*grp+r valid iff r < nvalid
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r >= nvalid) s2[t][st][r] = kNegInf;
        }
      }
    }
    u32x2 phi[CT][SUB], plo[CT][SUB];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      float mt = max_raw(max3_raw(s2[t][0][0], s2[t][0][1], s2[t][0][2]), s2[t][0][3]);
#pragma unroll
      for (int st = 1; st < SUB; ++st)
        mt = max3_raw(mt, max3_raw(s2[t][st][0], s2[t][st][1], s2[t][st][2]), s2[t][st][3]);
      const float mn = rows_max_with(mt, m[t]);
      const float mu = mn == kNegInf ? 0.0f : mn;
      const float alpha = fast_exp2(m[t] - mu);
      m[t] = mn;
      float psum = 0.0f;  // (the first term is assigned, not added to 0: the same value, one add fewer)
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(s2[t][st][r] - mu);
        const float ps = (pr[0] + pr[1]) + (pr[2] + pr[3]);
        psum = st == 0 ? ps : psum + ps;
        const uint32_t h01 = C::pack(pr[0], pr[1]), h23 = C::pack(pr[2], pr[3]);
        phi[t][st] = u32x2{h01, h23};
        plo[t][st] = u32x2{C::pack(pr[0] - C::lo(h01), pr[1] - C::hi(h01)),
                           C::pack(pr[2] - C::lo(h23), pr[3] - C::hi(h23))};
      }
      lsum[t] = lsum[t] * alpha + psum;
      // Rescale the accumulator only if some column's running max moved: alpha
      // is exactly 1 otherwise, so skipping is bit-identical and saves 4*VB
      // multiplies on most pages.
      if (any_lane(alpha != 1.0f)) {
#pragma unroll
        for (int mb = 0; mb < VB; ++mb) acc[t][mb] *= alpha;
      }
    }
    // V tail slots past the sequence end are zeroed (selected, never multiplied
    // by a zero weight: they may hold NaN). Only the last page of a sequence is
    // partial, so the masking is a separate, wavefront-uniform branch.
    VWord vw[SUB][VB];
#pragma unroll
    for (int st = 0; st < SUB; ++st) {
      if constexpr (KV8) {
#pragma unroll
        for (int q = 0; q < VB / 4; ++q) {
          uint32_t w[4];
          v_words(pg.v[st][q], w);
#pragma unroll
          for (int j = 0; j < 4; ++j) vw[st][4 * q + j] = w[j];
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < VB; ++mb) vw[st][mb] = pg.v[st][mb];
      }
    }
    if (tok0 + BS > u.L) {
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
        const int nv = u.L - (tok0 + 16 * st + 4 * grp);  // valid among this lane's 4 tokens
#pragma unroll
        for (int mb = 0; mb < VB; ++mb) {
          if constexpr (KV8)
            vw[st][mb] = keep_first_bytes(vw[st][mb], nv);
          else
            vw[st][mb] = keep_first(vw[st][mb], nv);
        }
      }
    }
    if constexpr (PA_PV32 == 2 || (PA_PV32 == 1 && !KV8)) {
      // One 16x16x32 MFMA per d-block and sub-tile: lane row grp holds k-slots
      // 8grp .. 8grp+7 = (its 4 tokens' P high parts, the same tokens'
      // residuals) in B and its 4 V values twice in A, so the contraction is
      // sum_t v_t * (hi_t + lo_t), both parts in one instruction.
      u32x4 pp[CT][SUB];
#pragma unroll
      for (int t = 0; t < CT; ++t) {
#pragma unroll
        for (int st = 0; st < SUB; ++st)
          pp[t][st] = u32x4{phi[t][st][0], phi[t][st][1], plo[t][st][0], plo[t][st][1]};
      }
#pragma unroll
      for (int mb = 0; mb < VB; ++mb) {
#pragma unroll
        for (int st = 0; st < SUB; ++st) {
          const u32x2 v = v_operand(vw[st][mb]);
          const u32x4 vv = {v[0], v[1], v[0], v[1]};
#pragma unroll
          for (int t = 0; t < CT; ++t) acc[t][mb] = M::qk(vv, pp[t][st], acc[t][mb]);
        }
      }
    } else {  // two 16x16x16 MFMAs (high part, then residual)
#pragma unroll
      for (int mb = 0; mb < VB; ++mb) {
#pragma unroll
        for (int st = 0; st < SUB; ++st) {
          const u32x2 v = v_operand(vw[st][mb]);
#pragma unroll
          for (int t = 0; t < CT; ++t) {
            acc[t][mb] = M::pv(v, phi[t][st], acc[t][mb]);
            acc[t][mb] = M::pv(v, plo[t][st], acc[t][mb]);
          }
        }
      }
    }
  };

  // The rolling merge parks before the next page's fetch is issued, so that
  // its merge runs with one page fewer of registers live.
  auto pre = [&](int i) __attribute__((always_inline)) {
    if constexpr (ROLL) {
      const int page = wave + i * kWaves;
      while (page >= next_edge) park_roll();
    }
  };
  Page ring[PF + 1];
  pipeline<PF>(npg, ring, fetch, process, pre);
  if constexpr (ROLL) {
    while (jcur < u.ne) park_roll();
    // Each wavefront writes its quarter of every live column's combined row.
    const int q = u.p0 / a.C;
    const int mf = a.c0 / G;
    const size_t row0 = ((size_t)u.s * a.Mq + mf) * a.H + u.kh * G;
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      const int cl = 16 * t + g;
      if (cl >= NC) continue;
      const int c = a.c0 + cl, qm = c / G, h = c - qm * G;
      const size_t row = row0 + (size_t)(qm - mf) * a.H + h;
      const bool has = rZ[t] > 0.0f;
      const float inv = has ? 1.0f / rZ[t] : 0.0f;
#pragma unroll
      for (int mbl = 0; mbl < VQ; ++mbl) {
        const f32x4 o = s_run[(t * VQ + mbl) * 64] * inv;
        const int d = 16 * (wave * VQ + mbl) + 4 * grp;
        if (a.Pq == 1)
          store_out4(a.out, a.odt, row * D + d, o);
        else
          *(f32x4*)(a.tmp_out + (row * a.Pq + q) * D + d) = o;
      }
      if (wave == 0 && grp == 0) {
        if (a.Pq == 1) {
          if (a.lse)
            a.lse[row] = has ? fmaf(__builtin_amdgcn_logf(rZ[t]), kLn2, rM[t] * kLn2) : kNegInf;
        } else {
          a.exp_sums[row * a.Pq + q] = rZ[t];
          a.max_logits[row * a.Pq + q] = rM[t] * kLn2;
        }
      }
    }
    return;
  }
  while (jcur < u.ne) park();
  __syncthreads();
  if (a.fuse)
    combine_store<D, AL>(a, s_m, s_l, s_acc, u.s, u.kh, u.p0, u.ne, G, NC, u.L);
  else
    merge_store<D, AL>(a, s_m, s_l, s_acc, u.s, u.kh, u.p0, u.ne, G, NC, u.L);
}

// =====================================================================
// Vector path: any kv dtype, G <= GM query heads per kv head (GM in 1, 2, 4).
// An 8-bit cache (KV8) has 16 elements per 16-byte chunk: K words are
// converted to the query's 16-bit pairs for v_dot2, V bytes to fp32.
// QK: each lane dots its d-chunks of one token with the packed query
// (v_dot2 for 16-bit, fma for fp32), then a sum across the four 16-lane rows.
// PV: lane l owns X consecutive tokens (one 16-byte V chunk) of one d; the
// page's probabilities are read out of lanes 0..15 with v_readlane
// (wavefront-uniform) and each lane selects the X of its chunk.
// =====================================================================
template <int DT> struct vec_elem {
  static constexpr int X = 8;
};
template <> struct vec_elem<DT_F32> {
  static constexpr int X = 4;
};

template <int DT, int D, int BS, int GM, bool KV8, bool AL>
__global__ void __launch_bounds__(kWaves * 64) PA_OCCUPANCY
partition_vec_kernel(PartitionArgs a) {
  constexpr int X = KV8 ? 16 : vec_elem<DT>::X;  // cache elements per 16-byte chunk
  constexpr int ESZ = 16 / X;                     // cache element bytes
  constexpr int QSZ = DT == DT_F32 ? 4 : 2;       // query element bytes
  constexpr int QW = X * QSZ / 4;                 // query words per K chunk
  constexpr int SUB = BS / 16;       // 16-token sub-tiles per page
  constexpr int KJ = D / X / 4;      // K chunks per lane per sub-tile (c = 4j + row)
  constexpr int CPS = 16 / X;        // V chunks per d-row of one sub-tile
  constexpr int CPR = SUB * CPS;     // V chunks per d-row of a page
  constexpr int DPL = 64 / CPR;      // d distance between one lane's V chunks
  constexpr int VJ = D / DPL;        // V chunks per lane per page
  constexpr size_t PAGE = (size_t)D * BS * ESZ;
  constexpr int PREGS = (SUB * KJ + VJ) * 4;
  constexpr int PF = KV8 ? prefetch_fp8(PREGS) : prefetch_for(PREGS);

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Unit u;
  unit_begin<BS>(a, u, smem);
  const int G = u.G;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (uniform, scalar)
  const int t = lane & 15, grp = lane >> 4;     // K: token, chunk row
  const int h = lane % CPR, dl = lane / CPR;    // V: token chunk, d offset

  // Query d-chunks c = 4j + grp of each head (the d of K chunk c), as raw
  // 32-bit words: 16 bytes per chunk, or 32 for an 8-bit cache's 16-d chunks.
  uint32_t qw[GM][KJ][QW];
#pragma unroll
  for (int gg = 0; gg < GM; ++gg) {
    const int hh = gg < G ? gg : 0;
    const uint8_t* qrow = (const uint8_t*)a.q + (((size_t)u.s * a.H + u.kh * G + hh) * D) * QSZ;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
#pragma unroll
      for (int q4 = 0; q4 < QW / 4; ++q4) {
        const u32x4 v = *(const u32x4*)(qrow + (4 * j + grp) * X * QSZ + 16 * q4);
#pragma unroll
        for (int w = 0; w < 4; ++w) qw[gg][j][4 * q4 + w] = gg < G ? v[w] : 0u;
      }
    }
  }
  // ALiBi slopes of the lane's heads, log2 units.
  float slope2[GM];
#pragma unroll
  for (int gg = 0; gg < GM; ++gg) slope2[gg] = AL && gg < G ? a.alibi[u.kh * G + gg] * kLog2e : 0.0f;
  const LdsLayout lay = lds_layout(a.PS, BS, G, D, a.C);
  if (lay.total > a.lds_bytes) return;  // (uniform: the launch's LDS does not hold the layout)
  if (!unit_hoist<BS, D>(a, (int32_t*)smem, u)) return;
  const int32_t* s_bt = (const int32_t*)(smem + lay.bt_off);
  float* s_m = (float*)(smem + lay.m_off);
  float* s_l = (float*)(smem + lay.l_off);
  float* s_acc = (float*)(smem + lay.acc_off);
  const int pps = a.PS / BS;

  const size_t head_off = (size_t)u.kh * PAGE;
  const size_t blk_stride = (size_t)a.KH * PAGE;
  const uint8_t* kbase = (const uint8_t*)a.kc + head_off;
  const uint8_t* vbase = (const uint8_t*)a.vc + head_off;
  const uint32_t k_lane = (uint32_t)(grp * BS + t) * 16;
  const uint32_t v_lane = (uint32_t)(dl * BS + h * X) * ESZ;

  const int npg = u.npages > wave ? (u.npages - wave + kWaves - 1) / kWaves : 0;

  float m[GM], lpart[GM], acc[GM][VJ];
#pragma unroll
  for (int gg = 0; gg < GM; ++gg) {
    m[gg] = kNegInf;
    lpart[gg] = 0.0f;
#pragma unroll
    for (int j = 0; j < VJ; ++j) acc[gg][j] = 0.0f;
  }

  // Park this wavefront's state of partition jcur of the span in LDS and
  // start the next partition empty (wavefront-uniform control flow).
  int jcur = 0, next_edge = pps;  // next_edge: first page of partition jcur + 1
  auto park = [&]() {
#pragma unroll
    for (int gg = 0; gg < GM; ++gg) {
      const float ls = row16_sum(lpart[gg]);
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
        float v = acc[gg][j];
#pragma unroll
        for (int x = 1; x < CPR; x <<= 1) v += __shfl_xor(v, x, 64);
        acc[gg][j] = v;
      }
      if (gg < G) {
        const int k = slot(jcur, wave, gg, G);
        if (lane == 0) {
          s_m[k] = m[gg];
          s_l[k] = ls;
        }
        if (h == 0) {
#pragma unroll
          for (int j = 0; j < VJ; ++j) s_acc[k * D + j * DPL + dl] = acc[gg][j];
        }
      }
      m[gg] = kNegInf;
      lpart[gg] = 0.0f;
#pragma unroll
      for (int j = 0; j < VJ; ++j) acc[gg][j] = 0.0f;
    }
    ++jcur;
    next_edge += pps;
  };

  struct Page {
    u32x4 k[SUB][KJ];
    u32x4 v[VJ];
  };
  auto fetch = [&](int i, Page& pg) {
    const int blk = min(max(__builtin_amdgcn_readfirstlane(s_bt[wave + i * kWaves]), 0), a.NB - 1);
    const uint8_t* kp = kbase + (size_t)blk * blk_stride + k_lane;
    const uint8_t* vp = vbase + (size_t)blk * blk_stride + v_lane;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
#pragma unroll
      for (int st = 0; st < SUB; ++st)
        pg.k[st][j] = stream_load<u32x4>(kp + j * 4 * BS * 16 + st * 256);
    }
#pragma unroll
    for (int j = 0; j < VJ; ++j) pg.v[j] = stream_load<u32x4>(vp + j * DPL * BS * ESZ);
  };

  auto process = [&](int i, const Page& pg) {
    const int page = wave + i * kWaves;  // page of the span
    while (page >= next_edge) park();
    const int tok0 = (u.pg0 + page) * BS;  // first token of the page
    const bool tail = tok0 + BS > u.L;     // the sequence's last page (uniform)
    float p[GM][SUB];
#pragma unroll
    for (int gg = 0; gg < GM; ++gg) {
      float s2[SUB];
      float mt = kNegInf;
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (KV8) {
              // word w holds d 4w .. 4w+3 of the chunk: two 16-bit pairs
              const uint32_t kw = pg.k[st][j][w];
              dot = codec<DT>::dot2(fp8cvt<DT>::template pair<false>(kw), qw[gg][j][2 * w], dot);
              dot = codec<DT>::dot2(fp8cvt<DT>::template pair<true>(kw), qw[gg][j][2 * w + 1], dot);
            } else if constexpr (DT == DT_F32) {
              dot = fmaf(__uint_as_float(pg.k[st][j][w]), __uint_as_float(qw[gg][j][w]), dot);
            } else {
              dot = codec<DT>::dot2(pg.k[st][j][w], qw[gg][j][w], dot);
            }
          }
        }
        dot = rows_sum(dot);
        const int tk = tok0 + 16 * st + t;  // this lane's token
        if constexpr (AL)  // position relative to the page's partition start
          s2[st] = fmaf(dot, a.qk_scale, slope2[gg] * (float)(tk - (u.p0 + jcur) * a.PS));
        else
          s2[st] = dot * a.qk_scale;
      }
      // Tokens past the sequence's end: only on its last page (wavefront-uniform branch).
      if (tail) {
#pragma unroll
        for (int st = 0; st < SUB; ++st)
          if (tok0 + 16 * st + t >= u.L) s2[st] = kNegInf;
      }
#pragma unroll
      for (int st = 0; st < SUB; ++st) mt = max_raw(mt, s2[st]);
      mt = row16_max(mt);
      const float mn = max_raw(m[gg], mt);
      const float mu = mn == kNegInf ? 0.0f : mn;
      const float alpha = fast_exp2(m[gg] - mu);
      float ps = 0.0f;
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
        p[gg][st] = fast_exp2(s2[st] - mu);
        ps = st == 0 ? p[gg][st] : ps + p[gg][st];
      }
      lpart[gg] = lpart[gg] * alpha + ps;
      m[gg] = mn;
      if (any_lane(alpha != 1.0f)) {  // skipping a multiply by exactly 1 is bit-identical
#pragma unroll
        for (int j = 0; j < VJ; ++j) acc[gg][j] *= alpha;
      }
    }
    // V tail slots past the sequence's end are zeroed (not multiplied by a zero
    // weight: they may hold NaN), only on its last page.
    u32x4 vw[VJ];
#pragma unroll
    for (int j = 0; j < VJ; ++j) vw[j] = pg.v[j];
    if (tail) {
      const int nv = u.L - (tok0 + h * X);  // valid tokens among this lane's X
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
#pragma unroll
        for (int w = 0; w < 4; ++w) vw[j][w] = keep_first_elems<ESZ>(vw[j][w], nv - w * (4 / ESZ));
      }
    }
#pragma unroll
    for (int gg = 0; gg < GM; ++gg) {
      // p of page token 16*st + k sits in lane k (rows repeat it); this lane
      // needs tokens h*X .. h*X+X-1, i.e. chunk h of the page row.
      float pw[X];
#pragma unroll
      for (int e = 0; e < X; ++e) {
        pw[e] = pick<CPR>(h, [&](int hh) {
          return lane_value(p[gg][hh / CPS], (hh % CPS) * X + e);
        });
      }
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
        float sum = acc[gg][j];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (KV8) {
            const f32x2 lo = fp8_pair_f32<false>(vw[j][w]), hi = fp8_pair_f32<true>(vw[j][w]);
            sum = fmaf(pw[4 * w], lo[0], sum);
            sum = fmaf(pw[4 * w + 1], lo[1], sum);
            sum = fmaf(pw[4 * w + 2], hi[0], sum);
            sum = fmaf(pw[4 * w + 3], hi[1], sum);
          } else if constexpr (DT == DT_F32) {
            sum = fmaf(pw[w], __uint_as_float(vw[j][w]), sum);
          } else {
            sum = fmaf(pw[2 * w], codec<DT>::lo(vw[j][w]), sum);
            sum = fmaf(pw[2 * w + 1], codec<DT>::hi(vw[j][w]), sum);
          }
        }
        acc[gg][j] = sum;
      }
    }
  };

  Page ring[PF + 1];
  pipeline<PF>(npg, ring, fetch, process, [](int) {});
  while (jcur < u.ne) park();
  __syncthreads();
  if (a.fuse)
    combine_store<D, AL>(a, s_m, s_l, s_acc, u.s, u.kh, u.p0, u.ne, G, G, u.L);
  else
    merge_store<D, AL>(a, s_m, s_l, s_acc, u.s, u.kh, u.p0, u.ne, G, G, u.L);
}

// =====================================================================
// Reduce: the page's phase-2 log-sum-exp combine over the n = ceil(L / PS)
// partitions a row's keys use (L: the sequence length, or a query token's
// causal prefix when there are several per sequence), for one (sequence,
// query token, query head) row per WPI
// wavefronts (WPI = 1, 2 or 4, from the partition count, so that long
// sequences spread their rows over a whole workgroup).
//  - First round trip: the sequence length and the first 64 partitions'
//    statistics (lane i holds partition i); every wavefront of the row forms
//    the global max M and sum Z itself.
//  - Second round trip: the rows of the used partitions only (never the
//    unspecified rows of empty ones), 16 bytes per lane, D/4 lanes per row,
//    kU rows per lane in flight. Row r of a 64-partition chunk belongs to
//    wavefront (r / R) % WPI; its weight e^(m_r - M) l_r / Z is read from lane
//    r with a cross-lane permute.
//  - The per-lane sums are folded over the rows of a load with xor shuffles
//    and over the WPI wavefronts through LDS, in a fixed order (the result is
//    run-to-run identical).
// =====================================================================
struct ReduceArgs {
  void* out;
  const float* tmp_out;
  const float* exp_sums;
  const float* max_logits;
  const int32_t* sl;
  int S, H, P, PS;
  int M;    // query tokens per sequence (rows are (sequence, query token, head))
  int WPI;  // wavefronts per row: 1, 2 or 4
  float* lse;  // optional [rows]: log-sum-exp of each row's scores (NULL: not written)
};

// Partition rows per lane in flight. 4 keeps the kernel at 59 VGPRs, so 8
// wavefronts per SIMD (8 rows in flight at 86 VGPRs held it to 5): measured
// reduce times, 8 -> 4: 16384 rows (GQA, 4 query tokens) 15.5 -> 12.9 us, GQA
// 7.5 -> 7.1, long context 8.1 -> 7.9, wide heads 6.9 -> 6.6, MHA equal.
constexpr int kReduceU = 4;

// Wavefronts per row for a given partition count and head size (host side).
__host__ __device__ constexpr int reduce_waves_per_row(int P, int D) {
  const int rows_per_wave = (256 / D) * kReduceU;
  const int p = P < 64 ? P : 64;
  return p <= rows_per_wave ? 1 : p <= 2 * rows_per_wave ? 2 : 4;
}

template <int D, int ODT>
__global__ void __launch_bounds__(kWaves * 64) reduce_kernel(ReduceArgs a) {
  constexpr int LPR = D / 4;   // lanes per row, one f32x4 each
  constexpr int R = 64 / LPR;  // rows per wavefront load
  __shared__ f32x4 s_part[kWaves][LPR];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int WPI = a.WPI;
  const int sh = blockIdx.x * (kWaves / WPI) + wave / WPI;
  const int wi = wave % WPI;
  const int sub = lane / LPR, c4 = lane % LPR;
  const bool live = sh < a.S * a.M * a.H;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = kNegInf;  // row log-sum-exp, natural units; -inf when the row has no keys
  if (live) {
    const int sm = sh / a.H;               // query row: sequence s, query token qm
    const int s = sm / a.M, qm = sm - s * a.M;
    const float* mlr = a.max_logits + (size_t)sh * a.P;
    const float* esr = a.exp_sums + (size_t)sh * a.P;
    const float* trow = a.tmp_out + (size_t)sh * a.P * D + 4 * c4;
    // Independent loads: length and the first 64 partitions' statistics.
    const int L0 = a.sl[s];
    // keys query token qm sees: the causal prefix (L0 for single-query decode)
    const int L = min(L0, max(0, L0 - a.M + qm + 1));
    float mi = lane < a.P ? mlr[lane] : kNegInf;
    float li = lane < a.P ? esr[lane] : 0.0f;
    const int n = L > 0 ? min((L - 1) / a.PS + 1, a.P) : 0;  // P bounds a length past P*PS
    if (n > 0) {
      if (lane >= n) {
        mi = kNegInf;
        li = 0.0f;
      }
      float M = mi;
      for (int i = lane + 64; i < n; i += 64) M = fmaxf(M, mlr[i]);
      M = wave_max(M);
      float Z = lane < n ? fast_exp2((mi - M) * kLog2e) * li : 0.0f;
      for (int i = lane + 64; i < n; i += 64) Z += fast_exp2((mlr[i] - M) * kLog2e) * esr[i];
      Z = wave_sum(Z);
      // Z >= 1 (the partition holding the row's max contributes its l >= 1)
      lse = fmaf(__builtin_amdgcn_logf(Z), kLn2, M);
      for (int base = 0; base < n; base += 64) {
        // Weight of partition base + lane.
        float wl;
        if (base == 0) {
          wl = lane < n ? fast_exp2((mi - M) * kLog2e) * li / Z : 0.0f;
        } else {
          const int i = base + lane;
          wl = i < n ? fast_exp2((mlr[i] - M) * kLog2e) * esr[i] / Z : 0.0f;
        }
        const int cnt = min(64, n - base);
        const float* crow = trow + (size_t)base * D;
        for (int k0 = 0; (k0 * WPI + wi) * R < cnt; k0 += kReduceU) {
          f32x4 v[kReduceU];
#pragma unroll
          for (int k = 0; k < kReduceU; ++k) {
            const int r = ((k0 + k) * WPI + wi) * R + sub;
            v[k] = r < cnt ? *(const f32x4*)(crow + (size_t)r * D) : f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int k = 0; k < kReduceU; ++k) {
            const int r = ((k0 + k) * WPI + wi) * R + sub;
            const float w = __shfl(wl, r & 63, 64);
            if (r < cnt) acc += w * v[k];
          }
        }
      }
    }
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += shfl_xor(acc[e], x);
    }
  }
  if (WPI > 1) {  // uniform over the workgroup
    if (sub == 0) s_part[wave][c4] = acc;
    __syncthreads();
    if (sub == 0 && wi == 0) {
      for (int w = 1; w < WPI; ++w) acc += s_part[wave + w][c4];
    }
  }
  if (a.lse && live && wi == 0 && lane == 0) a.lse[sh] = lse;
  if (live && wi == 0 && sub == 0) {
    const size_t o = (size_t)sh * D + 4 * c4;
    if constexpr (ODT == DT_F32) {
      *(f32x4*)((float*)a.out + o) = acc;
    } else {
      using Cd = codec<ODT>;
      *(u32x2*)((uint16_t*)a.out + o) = u32x2{Cd::pack(acc[0], acc[1]), Cd::pack(acc[2], acc[3])};
    }
  }
}

// The same combine when every row has one partition (P = 1): its normalised
// row is the output (weight e^(m - m) l / l = 1, so out = tmp exactly) and the
// row's lse is m + ln l. The length, the statistics and the row are loaded
// together, one round trip; 256 / D rows per wavefront (D / 4 lanes each, one
// 16-byte piece per lane). A row with no keys (the partition left unwritten)
// gives out = 0 and lse = -inf.
template <int D, int ODT>
__global__ void __launch_bounds__(kWaves * 64) reduce_one_kernel(ReduceArgs a) {
  constexpr int LPR = D / 4;   // lanes per row
  constexpr int R = 64 / LPR;  // rows per wavefront
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, c4 = lane % LPR;
  const long long sh = ((long long)blockIdx.x * kWaves + wave) * R + sub;
  if (sh >= (long long)a.S * a.M * a.H) return;
  const int sm = (int)(sh / a.H);
  const int s = sm / a.M, qm = sm - s * a.M;
  const int L0 = a.sl[s];
  const f32x4 v = *(const f32x4*)(a.tmp_out + sh * D + 4 * c4);
  float m = 0.0f, l = 1.0f;
  if (a.lse && c4 == 0) {
    m = a.max_logits[sh];
    l = a.exp_sums[sh];
  }
  const int L = min(L0, max(0, L0 - a.M + qm + 1));  // keys query token qm sees
  const f32x4 acc = L > 0 ? v : f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.lse && c4 == 0) a.lse[sh] = L > 0 ? fmaf(__builtin_amdgcn_logf(l), kLn2, m) : kNegInf;
  const size_t o = (size_t)sh * D + 4 * c4;
  if constexpr (ODT == DT_F32) {
    *(f32x4*)((float*)a.out + o) = acc;
  } else {
    using Cd = codec<ODT>;
    *(u32x2*)((uint16_t*)a.out + o) = u32x2{Cd::pack(acc[0], acc[1]), Cd::pack(acc[2], acc[3])};
  }
}

// ---------------------------------------------------------------- merge states
// Two attention results of the same rows over disjoint key sets, each with its
// rows' log-sum-exps, merge into one: with Mx = max(la, lb), w = e^(l - Mx),
// out = (wa a + wb b) / (wa + wb), out_lse = Mx + ln(wa + wb); both -inf gives
// out = 0, out_lse = -inf. This is the V2 reduce's combine for two parts whose
// (max, exp-sum) pairs are already folded into one number each.
//
// Streaming and HBM-bound: each lane moves one 16-byte chunk of a, b and out;
// a row's D values take TPR = D * esize / 16 lanes (4..64, a power of two),
// so a row never straddles a wavefront. Every lane of a row reads the row's
// two lse words (cache broadcasts) and the row's first lane writes out_lse;
// within a wavefront all loads are issued before the dependent stores, so out
// may be a or b and out_lse may be lse_a or lse_b (exactly, not offset).
struct MergeArgs {
  void* out;
  float* out_lse;  // NULL: not written
  const void* a;
  const float* lse_a;
  const void* b;
  const float* lse_b;
  long long chunks;  // rows * TPR
  int tpr_shift;     // log2(TPR)
};

template <int DT>
__global__ void __launch_bounds__(256) merge_states_kernel(MergeArgs g) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= g.chunks) return;
  const long long r = i >> g.tpr_shift;
  const float la = g.lse_a[r], lb = g.lse_b[r];
  const float mx = fmaxf(la, lb);
  const u32x4 va = ((const u32x4*)g.a)[i];
  const u32x4 vb = ((const u32x4*)g.b)[i];
  float pa = 0.0f, pb = 0.0f, ol = kNegInf;
  if (mx != kNegInf) {
    const float wa = fast_exp2((la - mx) * kLog2e), wb = fast_exp2((lb - mx) * kLog2e);
    const float inv = 1.0f / (wa + wb);  // wa + wb in [1, 2]
    pa = wa * inv;
    pb = wb * inv;
    ol = mx + __builtin_amdgcn_logf(wa + wb) * kLn2;
  }
  // A side with lse -inf (no keys) is selected out, not multiplied by its zero
  // weight: its row is unspecified and may hold NaN.
  const bool ua = la != kNegInf, ub = lb != kNegInf;
  auto mix = [&](float x, float y) {
    return (ua ? pa * x : 0.0f) + (ub ? pb * y : 0.0f);
  };
  u32x4 vo;
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vo[e] = __float_as_uint(mix(__uint_as_float(va[e]), __uint_as_float(vb[e])));
  } else {
    using Cd = codec<DT>;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vo[e] = Cd::pack(mix(Cd::lo(va[e]), Cd::lo(vb[e])), mix(Cd::hi(va[e]), Cd::hi(vb[e])));
  }
  ((u32x4*)g.out)[i] = vo;
  if (g.out_lse && (i & ((1 << g.tpr_shift) - 1)) == 0) g.out_lse[r] = ol;
}

}  // namespace pa
