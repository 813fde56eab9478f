// Verification entry for the device number conversions the kernels use:
// fp32 -> bf16 (round to nearest even, the packed-pair conversion), fp32 ->
// OCP E4M3 (nearest, ties to the even code, saturating at +-448) and E4M3 ->
// fp32. The pages fix these formats: the first-level constants are stored
// in an 8-bit float and every product computes in bf16 (diycv.top "QLoRA
// 论文解读", section 关键公式, the dtype table). The kernel applies the
// library's own helpers to consecutive fp32 bit patterns so that a test can
// compare them with the definitions over all 2^32 patterns.
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

// Pattern first + i for i < count (mod 2^32). bf[i] holds the low half of
// pack_bf16x2(x, x); 0xFFFF (a NaN pattern, never the rounding of a finite
// value that stays finite) marks a pair whose two halves differ.
__global__ __launch_bounds__(256) void convcheck_kernel(uint32_t first, int64_t count, uint16_t* __restrict__ bf,
                                                        uint8_t* __restrict__ e8) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
    const float x = __uint_as_float(first + (uint32_t)i);
    if (bf) {
      const uint32_t pr = pack_bf16x2(x, x);
      bf[i] = (pr >> 16) == (pr & 0xFFFFu) ? (uint16_t)(pr & 0xFFFFu) : (uint16_t)0xFFFFu;
    }
    if (e8) e8[i] = (uint8_t)f32_to_e4m3(x);
  }
}

__global__ void e4m3_table_kernel(float* __restrict__ out) { out[threadIdx.x] = e4m3_to_f32(threadIdx.x); }

}  // namespace

hipError_t launch_convcheck(uint32_t first, int64_t count, uint16_t* bf, uint8_t* e8, float* table,
                            hipStream_t stream) {
  if (count > 0 && (bf || e8)) {
    int64_t blocks = (count + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(convcheck_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, first, count, bf, e8);
  }
  if (table) hipLaunchKernelGGL(e4m3_table_kernel, dim3(1), dim3(256), 0, stream, table);
  return hipGetLastError();
}

}  // namespace qlora
