// Small-M (decode-style) QLoRA forward on gfx950:
//   Y[m][n] = sum_k X[m][k] dequant(Wt)[n][k] + sum_j sT[m][j] L2[j][n],  M <= 16
// (QLoRA pages, diycv.top, section 关键公式; inference keeps the 4-bit base
// and the trained adapters, section 训练与推理流程 "推理").
//
// The weight is read once and is the only large stream, so the kernel is
// HBM-bound: each wave owns one weight row n and its 64 lanes stream that
// row's packed codes in 16-byte pieces (32 weights, half a 64-block, per
// lane per step), dequantise them exactly as the standalone dequant does
// (bf16(RN32(q[code] * a'))), and accumulate the M dot products in fp32.
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

template <int MT>
__global__ __launch_bounds__(256) void gemv_kernel(NF4View W, NF4Table tab, const uint16_t* __restrict__ X,
                                                   int64_t M, const uint16_t* __restrict__ sT,
                                                   const uint16_t* __restrict__ L2, int r,
                                                   uint16_t* __restrict__ Y) {
  __shared__ float sQ[16];
  const int tid = threadIdx.x;
  if (tid < 16) sQ[tid] = tab.q[tid];
  __syncthreads();
  const float mu = W.mean[0];
  const int64_t K = W.cols, N = W.rows;
  const int wave = tid >> 6, lane = tid & 63;

  for (int64_t n = (int64_t)blockIdx.x * 4 + wave; n < N; n += (int64_t)gridDim.x * 4) {
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    for (int64_t kc = (int64_t)lane * 32; kc < K; kc += 64 * 32) {
      const u32x4_t c = *reinterpret_cast<const u32x4_t*>(W.codes + n * (K >> 1) + (kc >> 1));
      const int64_t blk = n * (K / kBlock) + kc / kBlock;
      const float ap = block_scale(W.absmax8[blk], W.scale2[blk / kDqBlock], mu);
      const uint32_t words[4] = {c.x, c.y, c.z, c.w};
      float w[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t byte = (words[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const uint32_t pr = pack_bf16x2(sQ[byte & 15u] * ap, sQ[byte >> 4] * ap);
        w[2 * i] = __uint_as_float(pr << 16);
        w[2 * i + 1] = __uint_as_float(pr & 0xFFFF0000u);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(X + m * K + kc);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const u32x4_t xv = xp[q4];
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const int i = q4 * 8 + h * 2;
              acc[m] = __builtin_fmaf(w[i], __uint_as_float(xw[h] << 16), acc[m]);
              acc[m] = __builtin_fmaf(w[i + 1], __uint_as_float(xw[h] & 0xFFFF0000u), acc[m]);
            }
          }
        }
      }
    }
    // LoRA branch: sum_j sT[m][j] L2[j][n]
    for (int j = lane; j < r; j += 64) {
      const float l2 = bf16_to_f32(L2[(int64_t)j * N + n]);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M) acc[m] = __builtin_fmaf(bf16_to_f32(sT[m * r + j]), l2, acc[m]);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[m];
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      acc[m] = v;
    }
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M) Y[m * N + n] = f32_to_bf16(acc[m]);
    }
  }
}

}  // namespace

hipError_t launch_gemv(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M,
                       const uint16_t* sT, const uint16_t* L2, int r, uint16_t* Y, hipStream_t stream) {
  const int64_t N = W.rows;
  int64_t blocks = (N + 3) / 4;
  if (blocks > 65535) blocks = 65535;
  const dim3 grid((unsigned)blocks), block(256);
  if (M <= 1)
    hipLaunchKernelGGL(gemv_kernel<1>, grid, block, 0, stream, W, tab, X, M, sT, L2, r, Y);
  else if (M <= 2)
    hipLaunchKernelGGL(gemv_kernel<2>, grid, block, 0, stream, W, tab, X, M, sT, L2, r, Y);
  else if (M <= 4)
    hipLaunchKernelGGL(gemv_kernel<4>, grid, block, 0, stream, W, tab, X, M, sT, L2, r, Y);
  else if (M <= 8)
    hipLaunchKernelGGL(gemv_kernel<8>, grid, block, 0, stream, W, tab, X, M, sT, L2, r, Y);
  else
    hipLaunchKernelGGL(gemv_kernel<16>, grid, block, 0, stream, W, tab, X, M, sT, L2, r, Y);
  return hipGetLastError();
}

}  // namespace qlora
