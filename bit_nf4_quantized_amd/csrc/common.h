// Device-side helpers shared by the HIP kernels of the QLoRA NF4 library.
// gfx950 (CDNA4) only. All kernels are compiled with -ffp-contract=off,
// correctly rounded fp32 division and IEEE denormals, so every scalar fp32
// step below rounds exactly once, as the quantisation format requires.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;     // weights per first-level constant
constexpr int kDqBlock = 256;  // first-level constants per second-level scale

// The 16 NF4 values, passed by value in the kernel argument segment.
struct NF4Table {
  float q[16];
};

// Decision thresholds of the nearest-code search: t[j] is the smallest fp32
// strictly greater than the midpoint (q[j] + q[j+1]) / 2, so that for an fp32
// x, x > midpoint  <=>  x >= t[j]; code(x) = #{ j : x >= t[j] }.
struct NF4Thresholds {
  float t[15];
};

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float((b & 0xFFFFu) << 16);
}

// OCP E4M3 ("E4M3FN") code -> fp32, exact. Exponent field 0 is subnormal
// (m * 2^-9); otherwise (1 + m/8) * 2^(e-7). The NaN codes (S.1111.111) never
// occur in buffers written by this library.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u;
  const uint32_t m = c & 7u;
  float mag = (e == 0) ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// fp32 -> E4M3 code: nearest representable value, ties to the even code,
// saturating at +-448 (never NaN); the sign bit is the input's sign bit.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 31) << 7;
  const float av = __builtin_fabsf(v);
  uint32_t code;
  if (!(av < 448.0f)) {
    code = 0x7Eu;
  } else if (av < 0x1p-6f) {
    // subnormal range, quantum 2^-9; av * 512 is exact, rint is RNE
    code = (uint32_t)__builtin_rintf(av * 512.0f);
  } else {
    const int E = (int)((bits >> 23) & 255u) - 127;                  // -6 .. 8
    const float scaled = av * __uint_as_float((uint32_t)(127 + 3 - E) << 23);  // [8, 16), exact
    const uint32_t mm = (uint32_t)__builtin_rintf(scaled);           // 8 .. 16
    code = ((uint32_t)(E + 7) << 3) + (mm - 8u);                     // carry into exponent ok
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

// Dequantised first-level constant a' = RN32(RN32(e4m3(c) * sigma) + mu).
__device__ __forceinline__ float block_scale(uint32_t c8, float sigma, float mu) {
  const float prod = e4m3_to_f32(c8) * sigma;
  return prod + mu;
}

__device__ __forceinline__ float wave_max(float v, int width) {
  for (int o = width / 2; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qlora
