// Read-only page gather on gfx950: the bandwidth ceiling of a paged K/V read.
// The pages are a flat list of (block, kv head) items, item i = block
// blocks[i / KH], kv head i % KH; the launch's wavefronts split the list into
// contiguous runs, and each wavefront streams its run with the loads of four
// items in flight (two for 8 KiB pages, one for 16 KiB): every lane issues its
// 16-byte non-temporal loads of the item's K page and V page and folds the
// words into one register with xor, so no load can be dropped. No arithmetic
// on the data, no LDS, no stores but four words per workgroup. Unlike the
// decode kernels, nothing here depends on how the pages are spread over
// sequences, so ragged lengths cost it no load balance. The launch shape is
// the best of a sweep on MI355X (1024 / 2048 / 4096 workgroups x 1 / 2 / 4
// items in flight; 2, 4 and 16 KiB pages): on the 4 KiB pages of the GQA
// batch it reads 0.7-0.9 points of peak faster than 2048 x 2.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pa_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#ifndef PA_CEIL_GRID
#define PA_CEIL_GRID 4096  // workgroups: 16 per compute unit of the 256
#endif
#ifndef PA_CEIL_INFLIGHT
#define PA_CEIL_INFLIGHT 4  // items whose loads a wavefront keeps in flight (pages <= 4 KiB)
#endif
constexpr int kGrid = PA_CEIL_GRID;

template <int CH>  // 16-byte chunks per lane per page: page_bytes / 1024
__global__ void __launch_bounds__(256) gather_ceiling_kernel(
    int32_t* sink, const uint8_t* kc, const uint8_t* vc, const int32_t* blocks, long long items,
    int KH, int NB) {
  constexpr int NIF = CH <= 4 ? PA_CEIL_INFLIGHT : CH == 8 ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long waves = (long long)gridDim.x * 4;
  const long long w = (long long)blockIdx.x * 4 + wave;
  const long long per = (items + waves - 1) / waves;
  const long long i0 = w * per, i1 = i0 + per < items ? i0 + per : items;
  const size_t page = (size_t)CH * 1024;
  const size_t stride = (size_t)KH * page;
  uint32_t acc = 0;
  auto load = [&](long long i, u32x4 (&k)[CH], u32x4 (&v)[CH]) {
    const int blk = min(max(__builtin_amdgcn_readfirstlane(blocks[i / KH]), 0), NB - 1);
    const int kh = (int)(i % KH);
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
  long long i = i0;
  for (; i + NIF <= i1; i += NIF) {  // NIF items in flight
    u32x4 k[NIF][CH], v[NIF][CH];
#pragma unroll
    for (int j = 0; j < NIF; ++j) load(i + j, k[j], v[j]);
#pragma unroll
    for (int j = 0; j < NIF; ++j) fold(k[j], v[j]);
  }
  for (; i < i1; ++i) {
    u32x4 k0[CH], v0[CH];
    load(i, k0, v0);
    fold(k0, v0);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) sink[(size_t)blockIdx.x * 4 + wave] = (int32_t)acc;
}

typedef void (*ceiling_fn)(int32_t*, const uint8_t*, const uint8_t*, const int32_t*, long long,
                           int, int);

// The same reads with the decode kernels' work structure: workgroup u owns
// the pages pages[unit_off[u] .. unit_off[u + 1]) (page p = block * KH + kv
// head, p < num_cache_pages; clamped into range) and its four wavefronts take
// every fourth of them, each with two pages' K and V loads in flight. The
// dynamic LDS request (a launch argument) bounds the workgroups per CU.
template <int CH>  // 16-byte chunks per lane per page: page_bytes / 1024
__global__ void __launch_bounds__(256) gather_units_kernel(
    int32_t* sink, const uint8_t* kc, const uint8_t* vc, const int32_t* pages,
    const int32_t* unit_off, long long num_cache_pages) {
  extern __shared__ int32_t lds[];
  constexpr int NIF = 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t page = (size_t)CH * 1024;
  const int i1 = unit_off[blockIdx.x + 1];
  uint32_t acc = 0;
  auto base = [&](int i) {
    long long p = __builtin_amdgcn_readfirstlane(pages[i]);
    p = p < 0 ? 0 : (p >= num_cache_pages ? num_cache_pages - 1 : p);
    return (size_t)p * page + lane * 16;
  };
  int i = unit_off[blockIdx.x] + wave;
  for (; i + 4 * (NIF - 1) < i1; i += 4 * NIF) {
    u32x4 k[NIF][CH], v[NIF][CH];
#pragma unroll
    for (int j = 0; j < NIF; ++j) {
      const size_t off = base(i + 4 * j);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        k[j][c] = __builtin_nontemporal_load((const u32x4*)(kc + off + c * 1024));
        v[j][c] = __builtin_nontemporal_load((const u32x4*)(vc + off + c * 1024));
      }
    }
#pragma unroll
    for (int j = 0; j < NIF; ++j)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        acc ^= k[j][c].x ^ k[j][c].y ^ k[j][c].z ^ k[j][c].w ^ v[j][c].x ^ v[j][c].y ^
               v[j][c].z ^ v[j][c].w;
  }
  for (; i < i1; i += 4) {
    const size_t off = base(i);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const u32x4 k = __builtin_nontemporal_load((const u32x4*)(kc + off + c * 1024));
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)(vc + off + c * 1024));
      acc ^= k.x ^ k.y ^ k.z ^ k.w ^ v.x ^ v.y ^ v.z ^ v.w;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) {
    lds[wave] = (int32_t)acc;
    sink[(size_t)blockIdx.x * 4 + wave] = lds[wave];
  }
}

typedef void (*units_fn)(int32_t*, const uint8_t*, const uint8_t*, const int32_t*,
                         const int32_t*, long long);

}  // namespace

extern "C" {

int64_t pa_gather_ceiling_sink_words(void) { return (int64_t)kGrid * 4; }

int pa_gather_ceiling(int32_t* sink, int64_t sink_words, const void* key_cache,
                      const void* value_cache, const int32_t* blocks, int64_t num_pages,
                      int32_t num_kv_heads, int32_t page_bytes, int32_t num_blocks,
                      void* stream) {
  if (num_pages < 0 || num_kv_heads < 1 || num_blocks < 1) return -2;
  if (num_pages == 0) return 0;
  if (!sink || !key_cache || !value_cache || !blocks) return -1;
  if (((uintptr_t)key_cache | (uintptr_t)value_cache) & 15u) return -4;
  if (sink_words < pa_gather_ceiling_sink_words()) return -2;
  if (num_pages > (1LL << 40)) return -2;
  ceiling_fn fn;
  switch (page_bytes) {
    case 1024: fn = gather_ceiling_kernel<1>; break;
    case 2048: fn = gather_ceiling_kernel<2>; break;
    case 4096: fn = gather_ceiling_kernel<4>; break;
    case 8192: fn = gather_ceiling_kernel<8>; break;
    case 16384: fn = gather_ceiling_kernel<16>; break;
    default: return -2;
  }
  hipLaunchKernelGGL(fn, dim3(kGrid), dim3(256), 0, (hipStream_t)stream, sink,
                     (const uint8_t*)key_cache, (const uint8_t*)value_cache, blocks,
                     (long long)num_pages * num_kv_heads, num_kv_heads, num_blocks);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int pa_gather_units(int32_t* sink, int64_t sink_words, const void* key_cache,
                    const void* value_cache, const int32_t* pages, const int32_t* unit_off,
                    int32_t num_units, int64_t num_cache_pages, int32_t page_bytes,
                    int32_t workgroups_per_cu, void* stream) {
  if (num_units < 0 || num_cache_pages < 1 || workgroups_per_cu < 1) return -2;
  if (num_units == 0) return 0;
  if (!sink || !key_cache || !value_cache || !pages || !unit_off) return -1;
  if (((uintptr_t)key_cache | (uintptr_t)value_cache) & 15u) return -4;
  if (sink_words < (int64_t)num_units * 4) return -2;
  units_fn fn;
  switch (page_bytes) {
    case 1024: fn = gather_units_kernel<1>; break;
    case 2048: fn = gather_units_kernel<2>; break;
    case 4096: fn = gather_units_kernel<4>; break;
    case 8192: fn = gather_units_kernel<8>; break;
    default: return -2;
  }
  int dev = 0, per_cu = 0, per_block = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess ||
      hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
          hipSuccess)
    return -5;
  // the LDS share that leaves room for workgroups_per_cu workgroups on a CU
  int lds = (per_cu / workgroups_per_cu) & ~1023;
  lds = lds < 16 ? 16 : lds > per_block ? per_block : lds;
  hipLaunchKernelGGL(fn, dim3(num_units), dim3(256), lds, (hipStream_t)stream, sink,
                     (const uint8_t*)key_cache, (const uint8_t*)value_cache, pages, unit_off,
                     (long long)num_cache_pages);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
