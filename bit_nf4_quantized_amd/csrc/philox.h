// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC 2011) and the LoRA-dropout element rule built on it,
// shared by the kernels that regenerate the dropout mask.
//
// Element e of a row-major adapter input uses counter (lo(e/4), hi(e/4), 0,
// 0), key (lo(seed), hi(seed)) and output word e % 4; it is kept iff that word
// is at least thr = floor(p 2^32), and a kept value x becomes bf16(RN32(x c)).
#pragma once

#include "common.h"

namespace qlora {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

// Philox4x32-10 of counter (c0, c1, 0, 0) under key (k0, k1).
__device__ __forceinline__ u32x4_t philox(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
  uint32_t x0 = c0, x1 = c1, x2 = 0u, x3 = 0u;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * x0;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * x2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return u32x4_t{x0, x1, x2, x3};
}

// The four words of Philox block b (elements 4b .. 4b+3).
__device__ __forceinline__ u32x4_t philox_block(int64_t b, uint64_t seed) {
  return philox((uint32_t)b, (uint32_t)((uint64_t)b >> 32), (uint32_t)seed, (uint32_t)(seed >> 32));
}

// Two packed bf16 inputs (low half first) after dropout, given their words.
__device__ __forceinline__ uint32_t dropout_pair(uint32_t xw, uint32_t u_lo, uint32_t u_hi, uint32_t thr, float c) {
  const uint32_t lo = pack_bf16x2(__uint_as_float(xw << 16) * c, 0.0f) & 0xFFFFu;
  const uint32_t hi = pack_bf16x2(__uint_as_float(xw & 0xFFFF0000u) * c, 0.0f) & 0xFFFFu;
  return (u_lo >= thr ? lo : 0u) | ((u_hi >= thr ? hi : 0u) << 16);
}

}  // namespace qlora
