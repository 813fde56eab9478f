// The adapters' optimiser step for gfx950: global gradient-norm clipping and
// Adam, with the optimiser state either in HBM or "paged" out to pinned host
// memory.
//
// The QLoRA pages train the adapters with Adam (beta2 = 0.999, max grad norm
// 0.3, constant learning rate; diycv.top "QLoRA 论文解读", section
// 训练与推理流程) and page the optimiser state between GPU and CPU memory with
// unified memory (section 方法总览 item 4), without measuring what paging
// costs. Here the placement is explicit: the state vectors m and v may live
// in device memory or in pinned host memory, which the update kernel reads
// and writes in place over the host link (no migration, no HBM used for the
// state). The same kernel serves both placements, so results are identical.
//
// Kernels (HBM-bound, or host-link-bound for host-resident state):
//   sumsq_partial_kernel   fixed grid of 1024 workgroups; each thread adds
//                          the squares of its strided 4-element vectors in
//                          float64, then a fixed-order LDS tree per workgroup
//   clip_finalize_kernel   one workgroup: fixed-order tree over the 1024
//                          partials, norm = sqrt(sum), coef = min(1,
//                          max_norm / (norm + 1e-6)) in float64
//   adam_kernel            4 elements per thread (16-byte accesses):
//                          g' = coef g, m = b1 m + (1-b1) g', v = b2 v + (1-b2) g'^2,
//                          theta -= lr (m/bc1 / (sqrt(v/bc2) + eps) + wd theta),
//                          and the bf16 copy of theta for the layer
// Every result is deterministic (fixed reduction order, no atomics).
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int kNormBlocks = 1024;

__device__ __forceinline__ double tree_sum_256(double v, double* s) {
  const int t = threadIdx.x;
  s[t] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) s[t] += s[t + w];
    __syncthreads();
  }
  return s[0];
}

__global__ __launch_bounds__(256) void sumsq_partial_kernel(const float* __restrict__ g, int64_t n,
                                                            double* __restrict__ part) {
  __shared__ double s[256];
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)kNormBlocks * 256;
  double acc = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(g + 4 * i);
    acc += (double)x.x * x.x;
    acc += (double)x.y * x.y;
    acc += (double)x.z * x.z;
    acc += (double)x.w * x.w;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t i = 4 * n4; i < n; ++i) acc += (double)g[i] * g[i];
  const double tot = tree_sum_256(acc, s);
  if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void clip_finalize_kernel(const double* __restrict__ part, double max_norm,
                                                             float* __restrict__ coef, double* __restrict__ norm) {
  __shared__ double s[1024];
  const int t = threadIdx.x;
  s[t] = part[t];
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) s[t] += s[t + w];
    __syncthreads();
  }
  if (t == 0) {
    const double nrm = sqrt(s[0]);
    const double c = max_norm / (nrm + 1e-6);
    if (coef) *coef = (float)(c < 1.0 ? c : 1.0);
    if (norm) *norm = nrm;
  }
}

struct AdamConsts {
  float lr, b1, b2, omb1, omb2, eps, wd, bc1, bc2;
};

__device__ __forceinline__ void adam_one(float& th, float g, float& m, float& v, float cf, const AdamConsts& k) {
  const float gc = cf * g;
  m = k.b1 * m + k.omb1 * gc;
  v = k.b2 * v + k.omb2 * (gc * gc);
  const float mh = m / k.bc1;
  const float vh = v / k.bc2;
  const float upd = mh / (__builtin_sqrtf(vh) + k.eps);
  th = th - k.lr * (upd + k.wd * th);
}

__global__ __launch_bounds__(256) void adam_kernel(float* __restrict__ theta, const float* __restrict__ g,
                                                   float* __restrict__ m, float* __restrict__ v, int64_t n,
                                                   AdamConsts k, const float* __restrict__ coef,
                                                   uint16_t* __restrict__ theta_bf16) {
  const float cf = coef ? *coef : 1.0f;
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const f32x4_t th4 = *reinterpret_cast<const f32x4_t*>(theta + 4 * i);
    const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(g + 4 * i);
    const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(m + 4 * i);
    const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(v + 4 * i);
    float th[4] = {th4.x, th4.y, th4.z, th4.w}, mm[4] = {m4.x, m4.y, m4.z, m4.w}, vv[4] = {v4.x, v4.y, v4.z, v4.w};
    const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) adam_one(th[j], gg[j], mm[j], vv[j], cf, k);
    *reinterpret_cast<f32x4_t*>(theta + 4 * i) = f32x4_t{th[0], th[1], th[2], th[3]};
    *reinterpret_cast<f32x4_t*>(m + 4 * i) = f32x4_t{mm[0], mm[1], mm[2], mm[3]};
    *reinterpret_cast<f32x4_t*>(v + 4 * i) = f32x4_t{vv[0], vv[1], vv[2], vv[3]};
    if (theta_bf16)
      *reinterpret_cast<u32x2_t*>(theta_bf16 + 4 * i) = u32x2_t{pack_bf16x2(th[0], th[1]), pack_bf16x2(th[2], th[3])};
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) {   // the last n % 4 elements
    const int64_t i = 4 * n4 + threadIdx.x;
    float th = theta[i], mm = m[i], vv = v[i];
    adam_one(th, g[i], mm, vv, cf, k);
    theta[i] = th;
    m[i] = mm;
    v[i] = vv;
    if (theta_bf16) theta_bf16[i] = f32_to_bf16(th);
  }
}

}  // namespace

hipError_t launch_clip_norm(const float* g, int64_t n, double max_norm, float* coef, double* norm, double* part,
                            hipStream_t stream) {
  hipLaunchKernelGGL(sumsq_partial_kernel, dim3(kNormBlocks), dim3(256), 0, stream, g, n, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(clip_finalize_kernel, dim3(1), dim3(1024), 0, stream, part, max_norm, coef, norm);
  return hipGetLastError();
}

hipError_t launch_adam(float* theta, const float* g, float* m, float* v, int64_t n, const AdamHyper& h,
                       const float* coef, uint16_t* theta_bf16, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  AdamConsts k;
  k.lr = h.lr; k.b1 = h.beta1; k.b2 = h.beta2; k.eps = h.eps; k.wd = h.wd;
  k.omb1 = (float)(1.0 - (double)h.beta1);
  k.omb2 = (float)(1.0 - (double)h.beta2);
  k.bc1 = (float)(1.0 - pow((double)h.beta1, (double)h.step));
  k.bc2 = (float)(1.0 - pow((double)h.beta2, (double)h.step));
  int64_t blocks = (n / 4 + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(adam_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, theta, g, m, v, n, k, coef,
                     theta_bf16);
  return hipGetLastError();
}

}  // namespace qlora
