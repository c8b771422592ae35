// gfx950 kernels for paged single-query decode attention, V2 split.
//
// Method: "paged_attention_v2_triton.py -- Triton PagedAttention V2 for
// BI-V100", phase-1 partition kernel (paged gather, scaled q.k scores, online
// softmax, normalised partition output with its max logit and exp sum,
// sentinels for empty partitions) and phase-2 reduce kernel (cross-partition
// log-sum-exp combine). That page's kernel is organised for its own GPU:
// one program per (sequence, query head, partition), K/V gathered per query
// head. Here a workgroup owns one (sequence, kv head, partition) unit and all
// G query heads of the group share every K/V fetch.
//
// Work unit and layout
//  - blockIdx.x = (p * S + s) * KH + kh: kv head fastest, partition slowest, so
//    the last-dispatched workgroups are the cheap tail/empty partitions.
//  - A unit covers pages [p*PS/BS, ceil(min((p+1)*PS, L)/BS)); PS % BS == 0 so
//    partition edges are page edges. The unit's block-table slice is hoisted
//    into LDS once; NW wavefronts take pages wave, wave+NW, ...
//  - A page is processed as BS/16 tiles of 16 tokens. K tile: lane l holds
//    token l%16 and d-chunks c = 4j + l/16 (16-byte dwordx4 loads; each 16 lanes
//    read 256 contiguous bytes per chunk row). That register image is exactly
//    the A operand of a 16x16x32 MFMA with the token as row.
//  - Each wavefront keeps its own running (max, sum, unnormalised accumulator)
//    in the log2 domain (scores pre-multiplied by scale*log2(e)); at the end the
//    NW partial states are merged through LDS with the same log-sum-exp rule
//    the reduce uses, normalised, and stored with max_logits back in natural
//    units. Keeping the accumulator unnormalised and dividing once is the
//    partition kernel's normalised recurrence in exact arithmetic.
//  - Masked tokens (t >= seq_len in the last page) are selected out: score
//    -inf and value 0, never multiplied by a zero weight, so NaN in unread
//    cache slots cannot leak.
#pragma once

#include "pa_device.h"

namespace pa {

constexpr int kWaves = 4;  // wavefronts per partition workgroup

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
  float qk_scale;  // scale * log2(e)
};

// LDS carve-up shared by both partition kernels (byte offsets).
struct LdsLayout {
  int bt_off, m_off, l_off, acc_off, total;
};
__host__ __device__ inline LdsLayout lds_layout(int PS, int BS, int G, int D) {
  LdsLayout o;
  auto up16 = [](int v) { return (v + 15) & ~15; };
  o.bt_off = 0;
  o.m_off = up16((PS / BS) * 4);
  o.l_off = o.m_off + up16(kWaves * G * 4);
  o.acc_off = o.l_off + up16(kWaves * G * 4);
  o.total = o.acc_off + kWaves * G * D * 4;
  return o;
}

// Empty partition: the sentinels of the page's partition kernel.
__device__ __forceinline__ void write_sentinels(const PartitionArgs& a, int s, int kh, int p,
                                                int G) {
  if ((int)threadIdx.x < G) {
    const size_t row = ((size_t)s * a.H + kh * G + threadIdx.x) * a.P + p;
    a.max_logits[row] = kNegInf;
    a.exp_sums[row] = 0.0f;
  }
}

// Merge the NW per-wavefront states (log2-domain max m, sum l, unnormalised
// accumulators acc[w][g][D]) and store the unit's normalised outputs.
template <int D>
__device__ __forceinline__ void merge_store(const PartitionArgs& a, const float* s_m,
                                            const float* s_l, const float* s_acc, int s, int kh,
                                            int p, int G) {
  constexpr int D4 = D / 4;
  for (int i = threadIdx.x; i < G * D4; i += kWaves * 64) {
    const int g = i / D4, d4 = i % D4;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w * G + g]);
    float Z = 0.0f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2(s_m[w * G + g] - M);  // 0 for a wavefront with no tokens
      Z += e * s_l[w * G + g];
      const f32x4 v = *(const f32x4*)&s_acc[(w * G + g) * D + 4 * d4];
      o += e * v;
    }
    const float inv = 1.0f / Z;
    const size_t row = ((size_t)s * a.H + kh * G + g) * a.P + p;
    *(f32x4*)&a.tmp_out[row * D + 4 * d4] = o * inv;
    if (d4 == 0) {
      a.exp_sums[row] = Z;
      a.max_logits[row] = M * kLn2;
    }
  }
}

// Decode the unit index and hoist the block-table slice. Returns false for an
// empty partition (after writing its sentinels).
struct Unit {
  int s, kh, p, G, L, pg0, npages;
};
template <int BS>
__device__ __forceinline__ bool unit_setup(const PartitionArgs& a, int32_t* s_bt, Unit& u) {
  const int unit = blockIdx.x;
  u.kh = unit % a.KH;
  const int rest = unit / a.KH;
  u.s = rest % a.S;
  u.p = rest / a.S;
  u.G = a.H / a.KH;
  u.L = a.sl[u.s];
  const int t0 = u.p * a.PS;
  if (t0 >= u.L) {
    write_sentinels(a, u.s, u.kh, u.p, u.G);
    return false;
  }
  const int t1 = min(t0 + a.PS, u.L);
  u.pg0 = t0 / BS;
  u.npages = (t1 - t0 + BS - 1) / BS;
  const int32_t* row = a.bt + (size_t)u.s * a.MB + u.pg0;
  for (int i = threadIdx.x; i < u.npages; i += kWaves * 64) s_bt[i] = row[i];
  __syncthreads();
  return true;
}

// =====================================================================
// MFMA path: 16-bit K/V, G in [4, 16] query heads per kv head.
// QK^T per tile: D/32 MFMA 16x16x32, token rows x head columns (heads >= G are
// zero-padded). The fp32 C tile (lane l: tokens 4*(l/16)+r, head l%16) is
// exactly the B operand layout of a 16x16x16 MFMA with tokens as k, so P
// feeds PV without any data movement. V is read as 8-byte pieces (4 tokens
// of one d) that form the matching A operand. P is split into a 16-bit high
// part and a 16-bit residual (two PV MFMAs) so the probabilities keep ~16
// bits of mantissa instead of bf16's 8.
// =====================================================================
template <int DT, int D, int BS>
__global__ void __launch_bounds__(kWaves * 64)
partition_mfma_kernel(PartitionArgs a) {
  constexpr int KJ = D / 32;  // K dwordx4 per lane per tile = QK k-steps
  constexpr int VB = D / 16;  // V dwordx2 per lane per tile = PV d-blocks
  constexpr int TPP = BS / 16;
  constexpr size_t PAGE = (size_t)D * BS * 2;  // bytes of one (block, kv head) page
  using C = codec<DT>;
  using M = mma<DT>;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Unit u;
  if (!unit_setup<BS>(a, (int32_t*)smem, u)) return;
  const int G = u.G;
  const LdsLayout lay = lds_layout(a.PS, BS, G, D);
  const int32_t* s_bt = (const int32_t*)(smem + lay.bt_off);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane & 15, grp = lane >> 4;

  // Q group as the QK B operand: lane holds q[head g][32j + 8*grp .. +7].
  u32x4 qb[KJ];
  {
    const uint16_t* qrow =
        (const uint16_t*)a.q + ((size_t)u.s * a.H + u.kh * G + (g < G ? g : 0)) * D;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      u32x4 v = *(const u32x4*)(qrow + 32 * j + 8 * grp);
      qb[j] = g < G ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const size_t head_off = (size_t)u.kh * PAGE;
  const size_t blk_stride = (size_t)a.KH * PAGE;
  const uint8_t* kbase = (const uint8_t*)a.kc + head_off;
  const uint8_t* vbase = (const uint8_t*)a.vc + head_off;
  const uint32_t k_lane = (uint32_t)(grp * BS + g) * 16;          // + j*4*BS*16 + tt*256
  const uint32_t v_lane = (uint32_t)(g * BS + 4 * grp) * 2;       // + mb*16*BS*2 + tt*32

  const int my_pages = u.npages > wave ? (u.npages - wave + kWaves - 1) / kWaves : 0;
  const int ntiles = my_pages * TPP;

  float m = kNegInf;  // running max (log2 domain), uniform over a head column
  float lsum = 0.0f;  // this lane's share of the running exp sum
  f32x4 acc[VB];
#pragma unroll
  for (int i = 0; i < VB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](int ti, u32x4(&kr)[KJ], u32x2(&vr)[VB]) {
    const int pi = wave + (ti / TPP) * kWaves;
    const int tt = ti % TPP;
    const int blk = __builtin_amdgcn_readfirstlane(s_bt[pi]);
    const uint8_t* kp = kbase + (size_t)blk * blk_stride + tt * 256 + k_lane;
    const uint8_t* vp = vbase + (size_t)blk * blk_stride + tt * 32 + v_lane;
#pragma unroll
    for (int j = 0; j < KJ; ++j) kr[j] = *(const u32x4*)(kp + j * 4 * BS * 16);
#pragma unroll
    for (int mb = 0; mb < VB; ++mb) vr[mb] = *(const u32x2*)(vp + mb * 16 * BS * 2);
  };

  auto process = [&](int ti, const u32x4(&kr)[KJ], const u32x2(&vr)[VB]) {
    const int pi = wave + (ti / TPP) * kWaves;
    const int tt = ti % TPP;
    const int tok = (u.pg0 + pi) * BS + tt * 16 + 4 * grp;  // token of row 4*grp
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KJ; ++j) sc = M::qk(kr[j], qb[j], sc);
    const int nvalid = u.L - tok;  // rows 4*grp+r valid iff r < nvalid
    float s2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s2[r] = r < nvalid ? sc[r] * a.qk_scale : kNegInf;
    float mt = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mt = rows_max(mt);
    const float mn = fmaxf(m, mt);
    const float mu = mn == kNegInf ? 0.0f : mn;
    const float alpha = fast_exp2(m - mu);
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(s2[r] - mu);
    lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = mn;
    const uint32_t h01 = C::pack(pr[0], pr[1]), h23 = C::pack(pr[2], pr[3]);
    const u32x2 phi = {h01, h23};
    const u32x2 plo = {C::pack(pr[0] - C::lo(h01), pr[1] - C::hi(h01)),
                       C::pack(pr[2] - C::lo(h23), pr[3] - C::hi(h23))};
    const bool partial = (u.pg0 + pi) * BS + tt * 16 + 16 > u.L;  // wavefront-uniform
#pragma unroll
    for (int mb = 0; mb < VB; ++mb) {
      const u32x2 v = partial ? keep_first(vr[mb], nvalid) : vr[mb];
      acc[mb] *= alpha;
      acc[mb] = M::pv(v, phi, acc[mb]);
      acc[mb] = M::pv(v, plo, acc[mb]);
    }
  };

  u32x4 kA[KJ], kB[KJ];
  u32x2 vA[VB], vB[VB];
  if (ntiles > 0) fetch(0, kA, vA);
  int ti = 0;
  for (; ti + 1 < ntiles; ti += 2) {
    fetch(ti + 1, kB, vB);
    process(ti, kA, vA);
    if (ti + 2 < ntiles) fetch(ti + 2, kA, vA);
    process(ti + 1, kB, vB);
  }
  if (ti < ntiles) process(ti, kA, vA);

  lsum = rows_sum(lsum);
  float* s_m = (float*)(smem + lay.m_off);
  float* s_l = (float*)(smem + lay.l_off);
  float* s_acc = (float*)(smem + lay.acc_off);
  if (g < G) {
    if (grp == 0) {
      s_m[wave * G + g] = m;
      s_l[wave * G + g] = lsum;
    }
    float* dst = s_acc + (wave * G + g) * D + 4 * grp;
#pragma unroll
    for (int mb = 0; mb < VB; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[16 * mb + r] = acc[mb][r];
    }
  }
  __syncthreads();
  merge_store<D>(a, s_m, s_l, s_acc, u.s, u.kh, u.p, G);
}

// =====================================================================
// Vector path: any kv dtype, G <= GM query heads per kv head (GM in 1, 2, 4).
// QK: each lane dots its d-chunks of one token with the packed query
// (v_dot2 for 16-bit, fma for fp32), then a sum across the four 16-lane rows.
// PV: lane l owns X consecutive tokens (one 16-byte V chunk) of one d; the
// tile's 16 probabilities are read out of lanes 0..15 with v_readlane
// (wavefront-uniform) and each lane selects the X of its chunk.
// =====================================================================
template <int DT> struct vec_elem {
  static constexpr int X = 8;
};
template <> struct vec_elem<DT_F32> {
  static constexpr int X = 4;
};

template <int DT, int D, int BS, int GM>
__global__ void __launch_bounds__(kWaves * 64)
partition_vec_kernel(PartitionArgs a) {
  constexpr int X = vec_elem<DT>::X;
  constexpr int ESZ = 16 / X;
  constexpr int KJ = D / X / 4;     // K chunks per lane per tile (c = 4j + row)
  constexpr int CPR = 16 / X;       // V chunks per d-row of a 16-token tile
  constexpr int DPL = 64 / CPR;     // d distance between one lane's V chunks
  constexpr int VJ = D / DPL;       // V chunks per lane per tile
  constexpr int TPP = BS / 16;
  constexpr size_t PAGE = (size_t)D * BS * ESZ;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Unit u;
  if (!unit_setup<BS>(a, (int32_t*)smem, u)) return;
  const int G = u.G;
  const LdsLayout lay = lds_layout(a.PS, BS, G, D);
  const int32_t* s_bt = (const int32_t*)(smem + lay.bt_off);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = lane & 15, grp = lane >> 4;     // K: token, chunk row
  const int h = lane % CPR, dl = lane / CPR;    // V: token chunk, d offset

  // Query d-chunks c = 4j + grp of each head, as raw 32-bit words.
  uint32_t qw[GM][KJ][4];
#pragma unroll
  for (int gg = 0; gg < GM; ++gg) {
    const int hh = gg < G ? gg : 0;
    const uint8_t* qrow = (const uint8_t*)a.q + (((size_t)u.s * a.H + u.kh * G + hh) * D) * ESZ;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const u32x4 v = *(const u32x4*)(qrow + (4 * j + grp) * 16);
#pragma unroll
      for (int w = 0; w < 4; ++w) qw[gg][j][w] = gg < G ? v[w] : 0u;
    }
  }

  const size_t head_off = (size_t)u.kh * PAGE;
  const size_t blk_stride = (size_t)a.KH * PAGE;
  const uint8_t* kbase = (const uint8_t*)a.kc + head_off;
  const uint8_t* vbase = (const uint8_t*)a.vc + head_off;
  const uint32_t k_lane = (uint32_t)(grp * BS + t) * 16;
  const uint32_t v_lane = (uint32_t)(dl * BS + h * X) * ESZ;

  const int my_pages = u.npages > wave ? (u.npages - wave + kWaves - 1) / kWaves : 0;
  const int ntiles = my_pages * TPP;

  float m[GM], lpart[GM], acc[GM][VJ];
#pragma unroll
  for (int gg = 0; gg < GM; ++gg) {
    m[gg] = kNegInf;
    lpart[gg] = 0.0f;
#pragma unroll
    for (int j = 0; j < VJ; ++j) acc[gg][j] = 0.0f;
  }

  auto fetch = [&](int ti, u32x4(&kr)[KJ], u32x4(&vr)[VJ]) {
    const int pi = wave + (ti / TPP) * kWaves;
    const int tt = ti % TPP;
    const int blk = __builtin_amdgcn_readfirstlane(s_bt[pi]);
    const uint8_t* kp = kbase + (size_t)blk * blk_stride + tt * 256 + k_lane;
    const uint8_t* vp = vbase + (size_t)blk * blk_stride + tt * 16 * ESZ + v_lane;
#pragma unroll
    for (int j = 0; j < KJ; ++j) kr[j] = *(const u32x4*)(kp + j * 4 * BS * 16);
#pragma unroll
    for (int j = 0; j < VJ; ++j) vr[j] = *(const u32x4*)(vp + j * DPL * BS * ESZ);
  };

  auto process = [&](int ti, const u32x4(&kr)[KJ], const u32x4(&vr)[VJ]) {
    const int pi = wave + (ti / TPP) * kWaves;
    const int tt = ti % TPP;
    const int tok0 = (u.pg0 + pi) * BS + tt * 16;  // token of tile row 0
    const bool valid = tok0 + t < u.L;
    float p[GM];
#pragma unroll
    for (int gg = 0; gg < GM; ++gg) {
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (DT == DT_F32) {
            dot = fmaf(__uint_as_float(kr[j][w]), __uint_as_float(qw[gg][j][w]), dot);
          } else {
            dot = codec<DT>::dot2(kr[j][w], qw[gg][j][w], dot);
          }
        }
      }
      dot = rows_sum(dot);
      const float s2 = valid ? dot * a.qk_scale : kNegInf;
      const float mt = row16_max(s2);
      const float mn = fmaxf(m[gg], mt);
      const float mu = mn == kNegInf ? 0.0f : mn;
      const float alpha = fast_exp2(m[gg] - mu);
      p[gg] = fast_exp2(s2 - mu);
      lpart[gg] = lpart[gg] * alpha + p[gg];
      m[gg] = mn;
#pragma unroll
      for (int j = 0; j < VJ; ++j) acc[gg][j] *= alpha;
    }
    const int nv = u.L - (tok0 + h * X);  // valid tokens among this lane's X
#pragma unroll
    for (int gg = 0; gg < GM; ++gg) {
      // p of token k sits in lane k (rows repeat it); lane picks tokens h*X .. h*X+X-1.
      float sp[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) sp[k] = lane_value(p[gg], k);
      float pw[X];
#pragma unroll
      for (int e = 0; e < X; ++e) {
        if constexpr (CPR == 2) {
          pw[e] = h ? sp[8 + e] : sp[e];
        } else {
          const float lo = (h & 1) ? sp[4 + e] : sp[e];
          const float hi = (h & 1) ? sp[12 + e] : sp[8 + e];
          pw[e] = (h & 2) ? hi : lo;
        }
      }
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
        float sum = acc[gg][j];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (DT == DT_F32) {
            const float v = e_valid(w, nv) ? __uint_as_float(vr[j][w]) : 0.0f;
            sum = fmaf(pw[w], v, sum);
          } else {
            const float v0 = e_valid(2 * w, nv) ? codec<DT>::lo(vr[j][w]) : 0.0f;
            const float v1 = e_valid(2 * w + 1, nv) ? codec<DT>::hi(vr[j][w]) : 0.0f;
            sum = fmaf(pw[2 * w], v0, sum);
            sum = fmaf(pw[2 * w + 1], v1, sum);
          }
        }
        acc[gg][j] = sum;
      }
    }
  };

  u32x4 kA[KJ], kB[KJ], vA[VJ], vB[VJ];
  if (ntiles > 0) fetch(0, kA, vA);
  int ti = 0;
  for (; ti + 1 < ntiles; ti += 2) {
    fetch(ti + 1, kB, vB);
    process(ti, kA, vA);
    if (ti + 2 < ntiles) fetch(ti + 2, kA, vA);
    process(ti + 1, kB, vB);
  }
  if (ti < ntiles) process(ti, kA, vA);

  float* s_m = (float*)(smem + lay.m_off);
  float* s_l = (float*)(smem + lay.l_off);
  float* s_acc = (float*)(smem + lay.acc_off);
#pragma unroll
  for (int gg = 0; gg < GM; ++gg) {
    const float ls = row16_sum(lpart[gg]);
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      float v = acc[gg][j];
      v += __shfl_xor(v, 1, 64);
      if constexpr (CPR == 4) v += __shfl_xor(v, 2, 64);
      acc[gg][j] = v;
    }
    if (gg < G) {
      if (lane == 0) {
        s_m[wave * G + gg] = m[gg];
        s_l[wave * G + gg] = ls;
      }
      if (h == 0) {
#pragma unroll
        for (int j = 0; j < VJ; ++j) s_acc[(wave * G + gg) * D + j * DPL + dl] = acc[gg][j];
      }
    }
  }
  __syncthreads();
  merge_store<D>(a, s_m, s_l, s_acc, u.s, u.kh, u.p, G);
}

// =====================================================================
// Reduce: one wavefront per (sequence, query head); the page's phase-2
// log-sum-exp combine over the partitions the sequence uses. Lane i computes
// the weight of partition base+i; the d-parallel accumulation reads each
// weight back with v_readlane.
// =====================================================================
struct ReduceArgs {
  void* out;
  const float* tmp_out;
  const float* exp_sums;
  const float* max_logits;
  const int32_t* sl;
  int S, H, P, PS;
};

template <int D, int ODT>
__global__ void __launch_bounds__(256) reduce_kernel(ReduceArgs a) {
  constexpr int NWR = 4;
  constexpr int DPL = D / 64;  // consecutive d per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sh = blockIdx.x * NWR + wave;
  if (sh >= a.S * a.H) return;  // whole wavefront; only wavefront-local LDS below
  const int s = sh / a.H;
  const int L = a.sl[s];
  const int n = L > 0 ? (L + a.PS - 1) / a.PS : 0;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
  if (n > 0) {
    const float* mlr = a.max_logits + (size_t)sh * a.P;
    const float* esr = a.exp_sums + (size_t)sh * a.P;
    float M = kNegInf;
    for (int i = lane; i < n; i += 64) M = fmaxf(M, mlr[i]);
    M = wave_max(M);
    float Z = 0.0f;
    for (int i = lane; i < n; i += 64) Z += fast_exp2((mlr[i] - M) * kLog2e) * esr[i];
    Z = wave_sum(Z);
    const float* trow = a.tmp_out + (size_t)sh * a.P * D + lane * DPL;
    for (int base = 0; base < n; base += 64) {
      const int i = base + lane;
      const float wl = i < n ? fast_exp2((mlr[i] - M) * kLog2e) * esr[i] / Z : 0.0f;
      const int cnt = min(64, n - base);
      int k = 0;
      for (; k + 4 <= cnt; k += 4) {
        float v[4][DPL];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float* src = trow + (size_t)(base + k + u) * D;
#pragma unroll
          for (int e = 0; e < DPL; ++e) v[u][e] = src[e];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = lane_value(wl, k + u);
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
        }
      }
      for (; k < cnt; ++k) {
        const float w = lane_value(wl, k);
        const float* src = trow + (size_t)(base + k) * D;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, src[e], acc[e]);
      }
    }
  }
  const size_t o = (size_t)sh * D + lane * DPL;
  if constexpr (ODT == DT_F32) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) ((float*)a.out)[o + e] = acc[e];
  } else {
#pragma unroll
    for (int e = 0; e < DPL; ++e) ((uint16_t*)a.out)[o + e] = codec<ODT>::one(acc[e]);
  }
}

}  // namespace pa
