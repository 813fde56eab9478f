// Measurement aids for the roofline figures of the benchmark (no part of
// the method): the attainable dense bf16 MFMA rate of this GPU at the clock
// it runs under load, and the attainable HBM streaming-read rate.
//
//   mfma_probe_kernel   8 waves per workgroup, each running `iters` rounds of
//                       8 independent v_mfma_f32_32x32x16_bf16 on register
//                       operands (no memory traffic in the loop); workgroup
//                       0 records s_memtime and s_memrealtime (100 MHz)
//                       around its loop, so the caller can derive the shader
//                       clock. 8 * 32768 flops per wave per round.
//   read_probe_kernel   each thread issues 16 loads of 16 bytes (all before
//                       any use) from consecutive 4 KB-wide rows of the
//                       buffer, so a workgroup reads 64 KB and the grid
//                       reads the buffer once; the XOR of the words is
//                       stored only if it matches a value the caller's data
//                       never produces, so no load can be dropped.
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int kProbeWaves = 8;
constexpr int kReadLoads = 16;

__global__ __launch_bounds__(64 * kProbeWaves, 1) void mfma_probe_kernel(int iters, float* __restrict__ sink,
                                                                          unsigned long long* __restrict__ clocks) {
  const int tid = threadIdx.x;
  // operands that the compiler cannot fold (depend on the thread index)
  const float fa = 1.0f + (float)(tid & 7) * 0.0078125f, fb = 1.0f - (float)(tid >> 6) * 0.0078125f;
  const bf16x8_t a = {(__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb};
  const bf16x8_t b = {(__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa, (__bf16)fb, (__bf16)fa};
  f32x16_t acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[m][v] = 0.0f;
  unsigned long long t0 = 0, r0 = 0;
  if (blockIdx.x == 0 && tid == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m], 0, 0, 0);
  }
  if (blockIdx.x == 0 && tid == 0) {
    clocks[0] = __builtin_amdgcn_s_memtime() - t0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[m][v];
  sink[(int64_t)blockIdx.x * blockDim.x + tid] = s;
}

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* __restrict__ src, uint32_t never,
                                                         uint32_t* __restrict__ sink) {
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * (kReadLoads * 256);
  u32x4_t v[kReadLoads];
#pragma unroll
  for (int i = 0; i < kReadLoads; ++i) v[i] = __builtin_nontemporal_load(src + base + (int64_t)i * 256 + t);
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kReadLoads; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (x == never) sink[0] = x;
}

}  // namespace

hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, unsigned long long* clocks, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(64 * kProbeWaves), 0, stream, iters, sink,
                     clocks);
  return hipGetLastError();
}

size_t read_probe_granule() { return (size_t)kReadLoads * 256 * 16; }

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t never, uint32_t* sink, hipStream_t stream) {
  const size_t blocks = bytes / read_probe_granule();
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4_t*>(src), never, sink);
  return hipGetLastError();
}

}  // namespace qlora
