// Device-side helpers shared by the gfx950 kernels of the paged LATENT attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Storage-type tags. Raw 16-bit patterns travel as uint16_t; conversions round
// to nearest even (the page's kernel stores with __float2half_rn /
// __float2bfloat16_rn).
struct BF16 {
  static __device__ __forceinline__ float to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
  static __device__ __forceinline__ uint32_t from_f32(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
  }
  // (a, b) rounded and packed, a in the low half: one v_cvt_pk_bf16_f32.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
  }
  // acc + lo + hi of a packed pair (one v_dot2 against (1, 1)).
  static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), bf16x2_t{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
  }
  static __device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

struct F16 {
  static __device__ __forceinline__ float to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  }
  static __device__ __forceinline__ uint32_t from_f32(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
  }
  static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pair), f16x2_t{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
  }
  static __device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

template <typename DT>
__device__ __forceinline__ void unpack8(u32x4_t v, float (&x)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = DT::to_f32(v[k] & 0xFFFFu);
    x[2 * k + 1] = DT::to_f32(v[k] >> 16);
  }
}

template <typename DT>
__device__ __forceinline__ u32x4_t pack8(const float (&x)[8]) {
  u32x4_t v;
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = DT::pack2(x[2 * k], x[2 * k + 1]);
  return v;
}

// Sequence of global token t: the first b with t < cumseq[b + 1] (the page's
// locate_token scans linearly; a binary search over the non-decreasing prefix
// sums finds the same b). Clamped to [0, B - 1].
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cumseq, int B, int64_t t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (t < (int64_t)cumseq[mid + 1]) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Rotate one 8-channel chunk [c0, c0 + 8) of a row in place (float32 math).
// Requires rotary_offset % 8 == 0 and rotary_dim % 16 == 0, so a chunk lies
// entirely inside or outside the rotary range and, non-interleaved, its
// partner chunk (c0 +- rd/2) is again a whole chunk. `row` is the row's first
// element, cos/sin are [P, rd/2] tables. Non-interleaved: channel d with
// r = d - ro < rd/2 takes x_d c_r - x_{d+rd/2} s_r, otherwise
// x_d c_{r-rd/2} + x_{d-rd/2} s_{r-rd/2}; interleaved: pairs (2i, 2i+1) take
// (x_{2i} c_i - x_{2i+1} s_i, x_{2i+1} c_i + x_{2i} s_i), i counted from ro.
template <typename DT>
__device__ __forceinline__ void rope_chunk(float (&x)[8], const uint16_t* __restrict__ row, int c0, int ro,
                                           int rd, int interleaved, int64_t pos,
                                           const uint16_t* __restrict__ cos_t,
                                           const uint16_t* __restrict__ sin_t) {
  const int half = rd >> 1;
  const int r = c0 - ro;
  if (interleaved) {
    const int64_t base = pos * half + (r >> 1);
    const u32x2_t cv = *(const u32x2_t*)(cos_t + base);
    const u32x2_t sv = *(const u32x2_t*)(sin_t + base);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t cw = cv[k >> 1], sw = sv[k >> 1];
      const float c = DT::to_f32((k & 1) ? (cw >> 16) : (cw & 0xFFFFu));
      const float s = DT::to_f32((k & 1) ? (sw >> 16) : (sw & 0xFFFFu));
      const float xe = x[2 * k], xo = x[2 * k + 1];
      x[2 * k] = xe * c - xo * s;
      x[2 * k + 1] = xo * c + xe * s;
    }
  } else {
    const bool first = r < half;
    const int i0 = first ? r : r - half;
    const int pc = first ? c0 + half : c0 - half;
    const u32x4_t pv = *(const u32x4_t*)(row + pc);
    const u32x4_t cv = *(const u32x4_t*)(cos_t + pos * half + i0);
    const u32x4_t sv = *(const u32x4_t*)(sin_t + pos * half + i0);
    float xp[8], c[8], s[8];
    unpack8<DT>(pv, xp);
    unpack8<DT>(cv, c);
    unpack8<DT>(sv, s);
    const float sign = first ? -1.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = x[k] * c[k] + sign * (xp[k] * s[k]);
  }
}

}  // namespace pa
