// Blockwise Int8 absmax codec for gfx950.
//
// Method (QLoRA pages, diycv.top "QLoRA 论文解读", section 方法总览 item 1):
// flatten the tensor, cut it into contiguous blocks of B elements and store
// per block its absmax a and per element round(127 / a * x) as a signed
// byte. The factor is RN32(127 / a) (IEEE division), the product rounds once
// to fp32 and the integer rounding is to nearest, ties to even; a block with
// a below 2^-120 stores zeros. Dequantisation multiplies each code by
// RN32(a / 127).
//
// Both kernels are HBM-bound streams (quantise: 4 or 2 B in, 1 B out per
// element; dequantise: 1 B in, 4 or 2 B out), so the design is about
// coalescing: every lane owns 8 consecutive elements (one or two 16-byte
// loads), a wave covers 512 contiguous elements per chunk, and the block
// absmax is a cross-lane max over the lanes that share a block (B/8 lanes
// for B <= 512; the whole wave, over B/512 chunks per lane, above that).
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int kInt8Threads = 256;            // 4 waves
constexpr float kZeroBlockBelow = 0x1p-120f;

__device__ __forceinline__ void load8(const float* __restrict__ x, int64_t e0, int64_t numel, float v[8]) {
  if (e0 + 8 <= numel) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(x + e0);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(x + e0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < numel) ? x[e0 + i] : 0.0f;
  }
}

__device__ __forceinline__ void load8(const uint16_t* __restrict__ x, int64_t e0, int64_t numel, float v[8]) {
  if (e0 + 8 <= numel) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(x + e0);
    v[0] = __uint_as_float(a.x << 16); v[1] = __uint_as_float(a.x & 0xFFFF0000u);
    v[2] = __uint_as_float(a.y << 16); v[3] = __uint_as_float(a.y & 0xFFFF0000u);
    v[4] = __uint_as_float(a.z << 16); v[5] = __uint_as_float(a.z & 0xFFFF0000u);
    v[6] = __uint_as_float(a.w << 16); v[7] = __uint_as_float(a.w & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < numel) ? bf16_to_f32(x[e0 + i]) : 0.0f;
  }
}

// round(x * c) as a signed byte: one fp32 product, round to nearest even,
// clamped to [-127, 127].
__device__ __forceinline__ uint32_t code_byte(float x, float c) {
  float v = __builtin_rintf(x * c);
  v = __builtin_fminf(__builtin_fmaxf(v, -127.0f), 127.0f);
  return (uint32_t)((int32_t)v) & 0xFFu;
}

__device__ __forceinline__ void store8(int8_t* __restrict__ codes, int64_t e0, int64_t numel, const float v[8],
                                       float c) {
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = code_byte(v[i], c);
  if (e0 + 8 <= numel) {
    u32x2_t w;
    w.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    w.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    *reinterpret_cast<u32x2_t*>(codes + e0) = w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (e0 + i < numel) codes[e0 + i] = (int8_t)b[i];
  }
}

// T = 1: blocks of B <= 512 elements, B/8 lanes per block (lanes_log2), 64/(B/8)
//        blocks per wave; T > 1: one block of 512 T elements per wave.
template <typename InT, int T>
__global__ __launch_bounds__(kInt8Threads) void int8_quant_kernel(const InT* __restrict__ x, int64_t numel,
                                                                  int lanes_log2, int8_t* __restrict__ codes,
                                                                  float* __restrict__ absmax, int64_t nb) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kInt8Threads / 64) + (threadIdx.x >> 6);
  const int64_t base = wave * (512 * T);
  float v[T][8];
  float m = 0.0f;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    load8(x, base + (int64_t)(t * 64 + lane) * 8, numel, v[t]);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[t][i]));
  }
  const int lanes = T == 1 ? (1 << lanes_log2) : 64;
  const float a = wave_max(m, lanes);
  const float c = a < kZeroBlockBelow ? 0.0f : 127.0f / a;   // RN32(127 / a); 0 for a zero block
#pragma unroll
  for (int t = 0; t < T; ++t) store8(codes, base + (int64_t)(t * 64 + lane) * 8, numel, v[t], c);
  if ((lane & (lanes - 1)) == 0) {
    const int64_t blk = T == 1 ? (base + lane * 8) >> (lanes_log2 + 3) : wave;
    if (blk < nb) absmax[blk] = a;
  }
}

// 8 elements per lane: x' = RN32(code * RN32(a / 127)), fp32 or bf16 (RNE).
template <bool BF16_OUT>
__global__ __launch_bounds__(kInt8Threads) void int8_dequant_kernel(const int8_t* __restrict__ codes,
                                                                    const float* __restrict__ absmax,
                                                                    int64_t numel, int block_log2,
                                                                    void* __restrict__ out) {
  const int64_t e0 = ((int64_t)blockIdx.x * kInt8Threads + threadIdx.x) * 8;
  if (e0 >= numel) return;
  const float d = absmax[e0 >> block_log2] / 127.0f;   // RN32(a / 127); 8 | B, so one block per lane
  float y[8];
  if (e0 + 8 <= numel) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t*>(codes + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = (float)(int8_t)((w.x >> (8 * i)) & 0xFFu) * d;
      y[4 + i] = (float)(int8_t)((w.y >> (8 * i)) & 0xFFu) * d;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (e0 + i < numel) ? (float)codes[e0 + i] * d : 0.0f;
  }
  if (BF16_OUT) {
    uint16_t* o = static_cast<uint16_t*>(out);
    if (e0 + 8 <= numel) {
      u32x4_t p = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                   pack_bf16x2(y[6], y[7])};
      *reinterpret_cast<u32x4_t*>(o + e0) = p;
    } else {
      for (int i = 0; i < 8; ++i)
        if (e0 + i < numel) o[e0 + i] = f32_to_bf16(y[i]);
    }
  } else {
    float* o = static_cast<float*>(out);
    if (e0 + 8 <= numel) {
      *reinterpret_cast<f32x4_t*>(o + e0) = f32x4_t{y[0], y[1], y[2], y[3]};
      *reinterpret_cast<f32x4_t*>(o + e0 + 4) = f32x4_t{y[4], y[5], y[6], y[7]};
    } else {
      for (int i = 0; i < 8; ++i)
        if (e0 + i < numel) o[e0 + i] = y[i];
    }
  }
}

template <typename InT>
hipError_t quant_dispatch(const InT* x, int64_t numel, int block_log2, int8_t* codes, float* absmax,
                          hipStream_t s) {
  const int64_t nb = (numel + (int64_t(1) << block_log2) - 1) >> block_log2;
  const int per_wave = block_log2 <= 9 ? 512 : (1 << block_log2);
  const int64_t waves = (numel + per_wave - 1) / per_wave;
  const dim3 grid((unsigned)((waves + 3) / 4));
  switch (block_log2) {
    case 10: hipLaunchKernelGGL((int8_quant_kernel<InT, 2>), grid, dim3(kInt8Threads), 0, s, x, numel, 6, codes, absmax, nb); break;
    case 11: hipLaunchKernelGGL((int8_quant_kernel<InT, 4>), grid, dim3(kInt8Threads), 0, s, x, numel, 6, codes, absmax, nb); break;
    case 12: hipLaunchKernelGGL((int8_quant_kernel<InT, 8>), grid, dim3(kInt8Threads), 0, s, x, numel, 6, codes, absmax, nb); break;
    default:
      hipLaunchKernelGGL((int8_quant_kernel<InT, 1>), grid, dim3(kInt8Threads), 0, s, x, numel, block_log2 - 3,
                         codes, absmax, nb);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_int8_quantize(const void* x, bool bf16_in, int64_t numel, int block_log2, int8_t* codes,
                                float* absmax, hipStream_t stream) {
  if (numel <= 0) return hipSuccess;
  return bf16_in ? quant_dispatch(static_cast<const uint16_t*>(x), numel, block_log2, codes, absmax, stream)
                 : quant_dispatch(static_cast<const float*>(x), numel, block_log2, codes, absmax, stream);
}

hipError_t launch_int8_dequantize(const int8_t* codes, const float* absmax, int64_t numel, int block_log2,
                                  void* out, bool bf16_out, hipStream_t stream) {
  if (numel <= 0) return hipSuccess;
  const dim3 grid((unsigned)((numel + 8 * kInt8Threads - 1) / (8 * kInt8Threads)));
  if (bf16_out)
    hipLaunchKernelGGL((int8_dequant_kernel<true>), grid, dim3(kInt8Threads), 0, stream, codes, absmax, numel,
                       block_log2, out);
  else
    hipLaunchKernelGGL((int8_dequant_kernel<false>), grid, dim3(kInt8Threads), 0, stream, codes, absmax, numel,
                       block_log2, out);
  return hipGetLastError();
}

}  // namespace qlora
