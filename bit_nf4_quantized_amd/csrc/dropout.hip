// LoRA dropout on the adapter branch, for gfx950.
//
// The QLoRA pages train Guanaco with LoRA dropout 0.1 (7B/13B) or 0.05
// (33B/65B) (diycv.top "QLoRA 论文解读", section 训练与推理流程, common
// settings). The dropout acts on the adapter branch's input:
//   Y  = X Wd^T + s (Xd L1) L2,   Xd = keep ? bf16(RN32(x c)) : 0,  c = RN32(1/(1-p))
//   dX = dY Wd + keep * c * (bf16(s dY L2^T) L1^T),  dL1 = s Xd^T U,  dL2 = s (Xd L1)^T dY
// The keep mask comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): element e of the
// row-major [M][K] input uses counter (lo(e/4), hi(e/4), 0, 0), key
// (lo(seed), hi(seed)) and output word e % 4, and is kept iff that word is at
// least floor(p 2^32). Nothing is stored between the forward and the
// backward: both regenerate the mask from (seed, p).
//
// Kernels (both HBM-bound):
//   dropout_input_kernel   Xd from X, 8 elements (two Philox blocks) per thread;
//                          the large-M layer does not use it: its adapter
//                          kernels drop X in registers (skinny_gemm.hip)
//   masked_lora_kernel     D[m][k] = keep c sum_j sU[m][j] L1[k][j] on MFMA (rank r),
//                          written as fp32 (added by the dX GEMM's epilogue), or
//                          combined with an fp32 main product into bf16 dX
#include "common.h"
#include "launch.h"
#include "philox.h"

namespace qlora {

namespace {

__global__ __launch_bounds__(256) void dropout_input_kernel(const uint16_t* __restrict__ X, int64_t numel,
                                                            uint32_t thr, float c, uint64_t seed,
                                                            uint16_t* __restrict__ Xd) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= numel) return;                          // numel % 8 == 0
  const u32x4_t u0 = philox_block(e0 >> 2, seed), u1 = philox_block((e0 >> 2) + 1, seed);
  const uint32_t u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(X + e0);
  const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = dropout_pair(xw[i], u[2 * i], u[2 * i + 1], thr, c);
  *reinterpret_cast<u32x4_t*>(Xd + e0) = u32x4_t{o[0], o[1], o[2], o[3]};
}

// One wave per 16 (m) x 64 (k) block of D^T[k][m] = L1[k][:] . sU[m][:]
// (v_mfma_f32_16x16x32_bf16; A = 8 consecutive ranks of an L1 row, B = 8
// consecutive ranks of an sU row, both 16-byte loads), so that a lane holds 4
// consecutive k of one m: one Philox block, one 16-byte fp32 store.
// COMBINE: dX[m][k] = bf16(F[m][k] + D[m][k]) instead of storing D.
template <bool COMBINE>
__global__ __launch_bounds__(256) void masked_lora_kernel(const uint16_t* __restrict__ sU, int64_t ldsu,
                                                          const uint16_t* __restrict__ L1, int r, int64_t M,
                                                          int64_t K, uint32_t thr, float c, uint64_t seed,
                                                          const float* __restrict__ F, float* __restrict__ D,
                                                          uint16_t* __restrict__ dX) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row16 = lane & 15, quad = lane >> 4;
  const int64_t kt = blockIdx.x;                          // 64-column block of k
  const int64_t m = ((int64_t)blockIdx.y * 4 + wave) * 16 + row16;
  const bool m_ok = m < M;
  const int64_t mc = m_ok ? m : 0;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = 0; j0 < r; j0 += 32) {
    const int j = j0 + quad * 8;
    const bool j_ok = j < r;                              // r % 8 == 0: all 8 ranks or none
    const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(sU + mc * ldsu + (j_ok ? j : 0));
    const u32x4_t b = (j_ok && m_ok) ? bv : zero4;
    u32x4_t a[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t k = kt * 64 + t * 16 + row16;
      const u32x4_t av = *reinterpret_cast<const u32x4_t*>(L1 + k * r + (j_ok ? j : 0));
      a[t] = j_ok ? av : zero4;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[t]),
                                                       __builtin_bit_cast(bf16x8_t, b), acc[t], 0, 0, 0);
  }
  if (!m_ok) return;
  // lane holds D[m][k = 64 kt + 16 t + 4 quad + i], i = 0..3
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t k = kt * 64 + t * 16 + quad * 4;
    const int64_t e = m * K + k;                          // multiple of 4: one Philox block
    const u32x4_t u = philox_block(e >> 2, seed);
    f32x4_t d;
    d.x = u.x >= thr ? c * acc[t].x : 0.0f;
    d.y = u.y >= thr ? c * acc[t].y : 0.0f;
    d.z = u.z >= thr ? c * acc[t].z : 0.0f;
    d.w = u.w >= thr ? c * acc[t].w : 0.0f;
    if (COMBINE) {
      const f32x4_t f = *reinterpret_cast<const f32x4_t*>(F + e);
      *reinterpret_cast<u32x2_t*>(dX + e) = u32x2_t{pack_bf16x2(f.x + d.x, f.y + d.y), pack_bf16x2(f.z + d.z, f.w + d.w)};
    } else {
      *reinterpret_cast<f32x4_t*>(D + e) = d;
    }
  }
}

}  // namespace

DropoutParams dropout_params(float p, uint64_t seed) {
  DropoutParams d;
  d.thr = (uint32_t)floor((double)p * 4294967296.0);
  d.c = (float)(1.0 / (1.0 - (double)p));
  d.seed = seed;
  return d;
}

hipError_t launch_dropout_input(const uint16_t* X, int64_t numel, const DropoutParams& d, uint16_t* Xd,
                                hipStream_t stream) {
  if (numel <= 0) return hipSuccess;
  if (numel % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dropout_input_kernel, dim3((unsigned)((numel / 8 + 255) / 256)), dim3(256), 0, stream, X, numel,
                     d.thr, d.c, d.seed, Xd);
  return hipGetLastError();
}

hipError_t launch_masked_lora(const uint16_t* sU, int64_t ldsu, const uint16_t* L1, int r, int64_t M, int64_t K,
                              const DropoutParams& d, const float* F, float* D, uint16_t* dX, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (K % 64 || r % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(K / 64), (unsigned)((M + 63) / 64));
  if (F)
    hipLaunchKernelGGL(masked_lora_kernel<true>, grid, dim3(256), 0, stream, sU, ldsu, L1, r, M, K, d.thr, d.c,
                       d.seed, F, D, dX);
  else
    hipLaunchKernelGGL(masked_lora_kernel<false>, grid, dim3(256), 0, stream, sU, ldsu, L1, r, M, K, d.thr, d.c,
                       d.seed, F, D, dX);
  return hipGetLastError();
}

}  // namespace qlora
