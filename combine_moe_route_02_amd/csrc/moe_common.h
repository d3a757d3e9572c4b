// Shared device helpers of the MoE-layer HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_WAVE 64

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Scalar format conversions (16-bit storage as uint16_t)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float32 -> bfloat16, round to nearest even (NaN stays NaN): the hardware
// conversion (v_cvt_pk_bf16_f32), which gives the same bits as rounding the
// binary32 pattern to nearest even for every non-NaN input, denormals and
// infinities included.  A software rounding with a NaN branch compiled to
// ~14 instructions per value, four of them exec-mask changes, and made the
// GEMM epilogues' staging of a 256 x 256 bf16 tile cost ~9 us.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const __bf16 h = (__bf16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// float32 -> binary16, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// OCP E4M3FN code -> float32.  Normal codes: the 7 magnitude bits placed at
// the top of a binary32 exponent/mantissa field give 1.m * 2^(e-127); scaling
// by 2^120 moves the exponent bias from 127 to 7.  Subnormal codes (exponent
// field 0) are m * 2^-9.  NaN codes are never produced by the weight encoder.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  uint32_t mag = code & 0x7fu;
  float v = (mag >= 8u) ? __uint_as_float((mag << 20) + (120u << 23))
                        : (float)mag * 0.001953125f;
  return (code & 0x80u) ? -v : v;
}

// float32 -> OCP E4M3FN code, round to nearest even, for |v| <= 448 (the
// caller's scaling guarantees it; nothing saturates).  The sign bit is kept,
// so -0 and negative values that round to zero give 0x80.  Below the
// smallest normal (2^-6) the code is the integer nearest v * 2^9 (exact
// product; 8 carries into the smallest normal); above it the 23-bit binary32
// mantissa is rounded to 3 bits, a carry out of the mantissa stepping the
// exponent field.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  uint32_t code;
  if (a < 0x3c800000u) {  // |v| < 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t e = (a >> 23) - 120u;  // biased exponent 127 -> 7
    const uint32_t keep = (a >> 20) & 7u, rem = a & 0xfffffu;
    const uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (keep & 1u));
    code = (e << 3) + keep + up;
  }
  return code | sign;
}

// Power-of-two scale exponent of an fp8 row: the smallest e with
// amax <= 448 * 2^e (448 = 0.875 * 2^9 is E4M3's largest finite value), so
// every |x| * 2^-e fits without saturation; 0 for an all-zero row.
__device__ __forceinline__ int e4m3_row_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  const float m = frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1)
  return ex - 9 + (m > 0.875f ? 1 : 0);
}

template <int DT> struct Act;
template <> struct Act<MOE_DTYPE_F32> {
  typedef float T;
  static __device__ __forceinline__ float load(T v) { return v; }
  static __device__ __forceinline__ T store(float f) { return f; }
};
template <> struct Act<MOE_DTYPE_F16> {
  typedef uint16_t T;
  static __device__ __forceinline__ float load(T v) { return f16_to_f32(v); }
  static __device__ __forceinline__ T store(float f) { return f32_to_f16(f); }
  // two values, a in the low half
  static __device__ __forceinline__ uint32_t store2(float a, float b) {
    return (uint32_t)f32_to_f16(a) | ((uint32_t)f32_to_f16(b) << 16);
  }
};
template <> struct Act<MOE_DTYPE_BF16> {
  typedef uint16_t T;
  static __device__ __forceinline__ float load(T v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ T store(float f) { return f32_to_bf16(f); }
  // two values in one packed conversion (v_cvt_pk_bf16_f32), a in the low half
  static __device__ __forceinline__ uint32_t store2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const f2 v = {a, b};
    const b2 h = __builtin_convertvector(v, b2);
    uint32_t r;
    __builtin_memcpy(&r, &h, 4);
    return r;
  }
};

// 16 bytes of a 16-bit activation row -> 8 floats.
template <int DT>
__device__ __forceinline__ void unpack8(const uint4& q, float* f) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = Act<DT>::load((uint16_t)(w[i] & 0xffffu));
    f[2 * i + 1] = Act<DT>::load((uint16_t)(w[i] >> 16));
  }
}

template <int DT>
__device__ __forceinline__ uint4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)Act<DT>::store(f[2 * i]) |
           ((uint32_t)Act<DT>::store(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// Wave primitives
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, MOE_WAVE);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (MOE_WAVE - 1); }

}  // namespace moe

// Host-side launch check used by the entry points.
#define MOE_LAUNCH_CHECK()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP; \
  } while (0)
