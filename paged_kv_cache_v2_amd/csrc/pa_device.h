// Device helpers for the gfx950 paged decode kernels: element codecs,
// MFMA wrappers, wavefront reductions. wave64 only (CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };  // DT_FP8: OCP E4M3 (e4m3fn)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// threadIdx.x as a value the compiler cannot form earlier than this point (an
// empty asm statement that claims to modify it): index arithmetic of an
// epilogue that starts from it then stays after the streaming loop instead of
// being hoisted above it and holding registers through it.
__device__ __forceinline__ int late_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
// A wavefront-uniform value made opaque the same way (kept in a scalar
// register), so that arithmetic on it is not hoisted either.
__device__ __forceinline__ int late_uniform(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// ---------------------------------------------------------------- codecs
// Two 16-bit elements packed in one 32-bit word: element 0 in the low half.
template <int DT> struct codec;

template <> struct codec<DT_BF16> {
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  // Round-to-nearest-even pack of two floats.
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ uint16_t one(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
  }
  // fp32 += a.lo*b.lo + a.hi*b.hi
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
};

template <> struct codec<DT_F16> {
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ uint16_t one(float a) {
    return __builtin_bit_cast(uint16_t, (_Float16)a);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
};

// ---------------------------------------------------------------- 8-bit caches
// OCP FP8 E4M3 bytes, four per 32-bit word (element 0 in the low byte). Every
// E4M3 value (subnormals included) is exactly representable in bf16 and in
// f16, and gfx950's conversions decode exactly this format (checked on every
// code by the GPU tests), so a cache page converted to the query's 16-bit
// type feeds the same MFMA / dot2 arithmetic as a 16-bit cache.
template <int DT> struct fp8cvt;
template <> struct fp8cvt<DT_BF16> {
  // Elements 2*HI, 2*HI+1 of w -> two packed bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1).
  template <bool HI> static __device__ __forceinline__ uint32_t pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
};
template <> struct fp8cvt<DT_F16> {
  template <bool HI> static __device__ __forceinline__ uint32_t pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
};
// Elements 2*HI, 2*HI+1 of w as two floats (v_cvt_pk_f32_fp8).
template <bool HI> __device__ __forceinline__ f32x2 fp8_pair_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// ---------------------------------------------------------------- MFMA
// QK: 16x16x32 (A = 16 token rows x 32 d, B = 32 d x 16 head columns).
// PV: 16x16x16 (A = 16 d rows x 16 tokens, B = 16 tokens x 16 head columns).
// Operand layout (CDNA3/CDNA4): A[i][k] lives in lane i + 16*(k / kpl), element
// k % kpl (kpl = k-values per lane: 8 for x32, 4 for x16); B[k][j] in lane
// j + 16*(k / kpl); C[i][j] in lane j + 16*(i / 4), register i % 4.
template <int DT> struct mma;

template <> struct mma<DT_BF16> {
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
};

template <> struct mma<DT_F16> {
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// v_max_f32 / v_max3_f32 as single instructions. fmaxf makes the compiler
// quiet possible signalling NaNs first (one v_max_f32 x, x, x per operand it
// cannot prove canonical: every value that comes out of a cross-lane swap or
// a select). The scores and running maxima maxed here are products, sums and
// selects of finite values and -inf, and the instruction's result is the
// same; the quieting is dropped. (ALU instructions only; nothing is loaded.)
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Exchange across 16-lane rows with gfx950's v_permlane16_swap / v_permlane32_swap
// (register-to-register, no LDS round trip). Called with the same value in
// both operands, each returns, in every lane l, the pair (x_a, x_b) = the
// values of lanes {l, l ^ 16} (resp. {l, l ^ 32}) with a the lower of the two
// lanes -- the same operands in the same order in both lanes of the pair, so a
// reduction step gives both lanes the identical result.
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Max / sum over the four 16-lane rows of a wavefront (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_max(float v) {
  float a, b;
  pair16(v, a, b);
  pair32(max_raw(a, b), a, b);
  return max_raw(a, b);
}
// max(m, rows_max(v)) with the last step fused into one v_max3_f32.
__device__ __forceinline__ float rows_max_with(float v, float m) {
  float a, b;
  pair16(v, a, b);
  pair32(max_raw(a, b), a, b);
  return max3_raw(m, a, b);
}
__device__ __forceinline__ float rows_sum(float v) {
  float a, b;
  pair16(v, a, b);
  pair32(a + b, a, b);
  return a + b;
}
// Max / sum within each 16-lane row.
__device__ __forceinline__ float row16_max(float v) {
  v = max_raw(v, shfl_xor(v, 1));
  v = max_raw(v, shfl_xor(v, 2));
  v = max_raw(v, shfl_xor(v, 4));
  return max_raw(v, shfl_xor(v, 8));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += shfl_xor(v, 1);
  v += shfl_xor(v, 2);
  v += shfl_xor(v, 4);
  return v + shfl_xor(v, 8);
}
// Whole-wavefront max / sum.
__device__ __forceinline__ float wave_max(float v) { return rows_max(row16_max(v)); }
__device__ __forceinline__ float wave_sum(float v) { return rows_sum(row16_sum(v)); }

// Value of `v` in lane `src` (wavefront-uniform src): v_readlane into an SGPR.
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Element e of a lane's run of tokens is a real token iff e < nvalid.
__device__ __forceinline__ bool e_valid(int e, int nvalid) { return e < nvalid; }

// Zero the bytes of a word at positions >= nvalid (0..4): the 8-bit-cache form
// of keep_first.
__device__ __forceinline__ uint32_t keep_first_bytes(uint32_t w, int nvalid) {
  const uint32_t m = nvalid >= 4 ? 0xffffffffu : nvalid <= 0 ? 0u : (1u << (8 * nvalid)) - 1u;
  return w & m;
}

// Zero the elements (ESZ bytes each: 1, 2 or 4) of a word at positions >=
// nvalid; nvalid may be negative or past the word's elements.
template <int ESZ>
__device__ __forceinline__ uint32_t keep_first_elems(uint32_t w, int nvalid) {
  constexpr int N = 4 / ESZ;
  const uint32_t m = nvalid >= N ? 0xffffffffu : nvalid <= 0 ? 0u : (1u << (8 * ESZ * nvalid)) - 1u;
  return w & m;
}

// True in every lane if cond holds in any active lane (wavefront-uniform).
__device__ __forceinline__ bool any_lane(bool cond) { return __builtin_amdgcn_ballot_w64(cond) != 0; }

// Zero the 16-bit elements of a packed pair of words at positions >= nvalid (0..4).
__device__ __forceinline__ u32x2 keep_first(u32x2 v, int nvalid) {
  const uint32_t mx = nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0x0000ffffu : 0u);
  const uint32_t my = nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0x0000ffffu : 0u);
  return u32x2{v.x & mx, v.y & my};
}

}  // namespace pa
