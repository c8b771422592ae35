// Read-only page gather on gfx950: the bandwidth ceiling of a paged K/V read.
// A workgroup owns (sequence s, kv head kh, run of 32 blocks of s's block-table
// row); its four wavefronts take the run's blocks w, w + 4, ...; for each block
// every lane issues its 16-byte non-temporal loads of the K page and of the V
// page (two blocks' loads in flight per wavefront), and folds the words into
// one register with xor, so no load can be dropped. No arithmetic on the data,
// no LDS, no stores but four words per workgroup.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRun = 32;  // blocks per workgroup

template <int CH>  // 16-byte chunks per lane per page: page_bytes / 1024
__global__ void __launch_bounds__(256) gather_ceiling_kernel(
    int32_t* sink, const uint8_t* kc, const uint8_t* vc, const int32_t* bt, const int32_t* sl,
    int KH, int BS, int NB, int MB, int runs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kh = blockIdx.x % KH;
  const int rs = blockIdx.x / KH;
  const int r = rs % runs, s = rs / runs;
  const int L = sl[s];
  const int nb = min((L + BS - 1) / BS, MB);
  const int b0 = r * kRun, b1 = min(b0 + kRun, nb);
  const size_t page = (size_t)CH * 1024;
  const size_t stride = (size_t)KH * page;
  const int32_t* row = bt + (size_t)s * MB;
  uint32_t acc = 0;
  auto load = [&](int i, u32x4 (&k)[CH], u32x4 (&v)[CH]) {
    const int blk = min(max(__builtin_amdgcn_readfirstlane(row[i]), 0), NB - 1);
    const uint8_t* kp = kc + (size_t)blk * stride + kh * page + lane * 16;
    const uint8_t* vp = vc + (size_t)blk * stride + kh * page + lane * 16;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      k[c] = __builtin_nontemporal_load((const u32x4*)(kp + c * 1024));
      v[c] = __builtin_nontemporal_load((const u32x4*)(vp + c * 1024));
    }
  };
  auto fold = [&](const u32x4 (&k)[CH], const u32x4 (&v)[CH]) {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc ^= k[c].x ^ k[c].y ^ k[c].z ^ k[c].w ^ v[c].x ^ v[c].y ^
                                        v[c].z ^ v[c].w;
  };
  int i = b0 + wave;
  if constexpr (CH <= 8) {
    for (; i + 4 < b1; i += 8) {  // two blocks in flight (one for 16 KiB pages)
      u32x4 k0[CH], v0[CH], k1[CH], v1[CH];
      load(i, k0, v0);
      load(i + 4, k1, v1);
      fold(k0, v0);
      fold(k1, v1);
    }
  }
  for (; i + 4 < b1; i += 4) {
    u32x4 k0[CH], v0[CH];
    load(i, k0, v0);
    fold(k0, v0);
  }
  if (i < b1) {
    u32x4 k0[CH], v0[CH];
    load(i, k0, v0);
    fold(k0, v0);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) sink[(size_t)blockIdx.x * 4 + wave] = (int32_t)acc;
}

typedef void (*ceiling_fn)(int32_t*, const uint8_t*, const uint8_t*, const int32_t*,
                           const int32_t*, int, int, int, int, int);

}  // namespace

extern "C" {

int64_t pa_gather_ceiling_sink_words(int32_t num_seqs, int32_t num_kv_heads,
                                     int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_kv_heads < 1 || max_blocks_per_seq < 1) return -2;
  const int64_t runs = (max_blocks_per_seq + kRun - 1) / kRun;
  return (int64_t)num_seqs * num_kv_heads * runs * 4;
}

int pa_gather_ceiling(int32_t* sink, int64_t sink_words, const void* key_cache,
                      const void* value_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                      int32_t page_bytes, int32_t block_size, int32_t num_blocks,
                      int32_t max_blocks_per_seq, void* stream) {
  if (num_seqs < 0 || num_kv_heads < 1 || block_size < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1)
    return -2;
  if (num_seqs == 0) return 0;
  if (!sink || !key_cache || !value_cache || !block_tables || !seq_lens) return -1;
  if (((uintptr_t)key_cache | (uintptr_t)value_cache) & 15u) return -4;
  const int64_t need = pa_gather_ceiling_sink_words(num_seqs, num_kv_heads, max_blocks_per_seq);
  if (sink_words < need) return -2;
  ceiling_fn fn;
  switch (page_bytes) {
    case 1024: fn = gather_ceiling_kernel<1>; break;
    case 2048: fn = gather_ceiling_kernel<2>; break;
    case 4096: fn = gather_ceiling_kernel<4>; break;
    case 8192: fn = gather_ceiling_kernel<8>; break;
    case 16384: fn = gather_ceiling_kernel<16>; break;
    default: return -2;
  }
  const int runs = (max_blocks_per_seq + kRun - 1) / kRun;
  const int64_t grid = need / 4;
  if (grid > 0x7fffffffLL) return -2;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, sink,
                     (const uint8_t*)key_cache, (const uint8_t*)value_cache, block_tables,
                     seq_lens, num_kv_heads, block_size, num_blocks, max_blocks_per_seq, runs);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
