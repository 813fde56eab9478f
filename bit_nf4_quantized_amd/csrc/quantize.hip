// NF4 blockwise quantisation with double quantisation, and the standalone
// doubleDequant to bf16, for gfx950.
//
// Method (QLoRA pages, diycv.top "QLoRA 论文解读", section 方法总览 items
// 1-3; neura.market "How It Works"): flatten the weight, cut it into
// contiguous 64-blocks, scale each block by its absmax into [-1, 1] and store
// the nearest NF4 code; then quantise the block absmax values, minus their
// mean, to an 8-bit float in groups of 256 with one fp32 scale per group.
//
// Kernels (all HBM-bound; see the launchers at the bottom):
//   quant_blocks_kernel   one workgroup per DQ group of 256 blocks
//                         (16384 weights): coalesced loads, absmax by
//                         cross-lane max over the 8 lanes of a block, codes
//                         from a 512-bucket LDS table, nibble packing, and
//                         the float64 adjacent-pair tree
//                         sum of the group's 256 absmax values in LDS.
//   tree_fold_kernel      one workgroup folds the per-group sums with the
//                         same adjacent-pair rule (first levels in
//                         registers, the rest in LDS) and writes the fp32
//                         mean.
//   dq_encode_kernel      one wave per group: a - mean, group absmax,
//                         fp32 scale, E4M3 codes.
//   dequant_kernel        4 units of 8 weights per thread: a code dword + the
//                         E4M3 constant -> bf16, one 16-byte store per unit.
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int kGroupWeights = kBlock * kDqBlock;  // 16384
constexpr int kQuantThreads = 256;                // 8 lanes per 64-block

template <typename InT>
__device__ __forceinline__ void load8(const InT* __restrict__ w, int64_t e0, int64_t numel, float v[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* __restrict__ w, int64_t e0, int64_t numel,
                                             float v[8]) {
  if (e0 + 8 <= numel) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(w + e0);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(w + e0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < numel) ? w[e0 + i] : 0.0f;
  }
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* __restrict__ w, int64_t e0,
                                                int64_t numel, float v[8]) {
  if (e0 + 8 <= numel) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(w + e0);
    v[0] = __uint_as_float(a.x << 16); v[1] = __uint_as_float(a.x & 0xFFFF0000u);
    v[2] = __uint_as_float(a.y << 16); v[3] = __uint_as_float(a.y & 0xFFFF0000u);
    v[4] = __uint_as_float(a.z << 16); v[5] = __uint_as_float(a.z & 0xFFFF0000u);
    v[6] = __uint_as_float(a.w << 16); v[7] = __uint_as_float(a.w & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < numel) ? bf16_to_f32(w[e0 + i]) : 0.0f;
  }
}

template <typename InT>
__device__ __forceinline__ void unpack8(const u32x4_t* raw, float v[8]);

template <>
__device__ __forceinline__ void unpack8<float>(const u32x4_t* raw, float v[8]) {
  v[0] = __uint_as_float(raw[0].x); v[1] = __uint_as_float(raw[0].y);
  v[2] = __uint_as_float(raw[0].z); v[3] = __uint_as_float(raw[0].w);
  v[4] = __uint_as_float(raw[1].x); v[5] = __uint_as_float(raw[1].y);
  v[6] = __uint_as_float(raw[1].z); v[7] = __uint_as_float(raw[1].w);
}

template <>
__device__ __forceinline__ void unpack8<uint16_t>(const u32x4_t* raw, float v[8]) {
  const u32x4_t a = raw[0];
  v[0] = __uint_as_float(a.x << 16); v[1] = __uint_as_float(a.x & 0xFFFF0000u);
  v[2] = __uint_as_float(a.y << 16); v[3] = __uint_as_float(a.y & 0xFFFF0000u);
  v[4] = __uint_as_float(a.z << 16); v[5] = __uint_as_float(a.z & 0xFFFF0000u);
  v[6] = __uint_as_float(a.w << 16); v[7] = __uint_as_float(a.w & 0xFFFF0000u);
}

// Nearest code by table: the normalised range is cut into 512 buckets by
// the monotone map b(x) = clamp(RN32(RN32(x + 1) * 256), 0, 511) truncated,
// which puts at most one decision threshold in any bucket for all four
// 4-bit tables (the closest thresholds, FP4 E3M0's near 0, are 4 buckets
// apart). Then every threshold in a lower bucket is below x and every one in
// a higher bucket above it, so the code is the count of thresholds in lower
// buckets plus one compare with the bucket's own threshold (+inf if none):
// the same result as a search over the thresholds, for about a third of the
// VALU work of a 4-level select search.
constexpr int kLutBuckets = 512;

__device__ __forceinline__ int lut_bucket(float x) {
  float y = (x + 1.0f) * 256.0f;
  y = __builtin_fminf(__builtin_fmaxf(y, 0.0f), (float)(kLutBuckets - 1));  // NaN -> 0
  return (int)y;
}

// One group's codes and block constants. FULL: the whole group lies inside
// the tensor, so every load and store is unconditional (per-lane bounds
// checks around the loads made the compiler wait for them where the
// branches join, one memory round trip per load).
template <typename InT, bool FULL>
__device__ __forceinline__ void quant_group(const InT* __restrict__ w, int64_t numel, int64_t nb, int64_t g,
                                            const NF4Thresholds& th, uint8_t* __restrict__ codes,
                                            float* __restrict__ absmax, float* s_a, u32x2_t* s_lut) {
  const int t = threadIdx.x;
  const int64_t gbase = g * kGroupWeights;
  float tt[15];
#pragma unroll
  for (int j = 0; j < 15; ++j) tt[j] = th.t[j];
  constexpr int kIters = kGroupWeights / (kQuantThreads * 8);
  constexpr int kWords = sizeof(InT) * 8 / 16;         // 16-byte pieces per 8 elements
  // all of this thread's full 16-byte loads first (one memory round trip per
  // group); a ragged tail is loaded element-wise in its iteration
  u32x4_t raw[kIters][kWords];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int64_t e0 = gbase + it * (kQuantThreads * 8) + t * 8;
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      const u32x4_t z = {0u, 0u, 0u, 0u};
      raw[it][q] = (FULL || e0 + 8 <= numel) ? reinterpret_cast<const u32x4_t*>(w + e0)[q] : z;
    }
  }
  // the bucket table, while the loads are in flight
#pragma unroll
  for (int b = t; b < kLutBuckets; b += kQuantThreads) {
    uint32_t below = 0u, thr = 0x7F800000u;  // +inf: no threshold in this bucket
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      const int bj = lut_bucket(tt[j]);
      below += bj < b ? 1u : 0u;
      if (bj == b) thr = __float_as_uint(tt[j]);
    }
    s_lut[b] = u32x2_t{below, thr};
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int local = it * (kQuantThreads * 8) + t * 8;  // element offset in the group
    const int64_t e0 = gbase + local;
    float v[8];
    if (FULL || e0 + 8 <= numel) {
      unpack8<InT>(raw[it], v);
    } else if (e0 < numel) {
      load8<InT>(w, e0, numel, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
    float a = wave_max(m, 8);                 // max over the 8 lanes of this block
    const bool zero_block = !(a >= 0x1p-126f);
    if (zero_block) a = 0.0f;
    const float r = zero_block ? 0.0f : 1.0f / a;  // correctly rounded RN32(1/a)
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = v[i] * r;
      const u32x2_t e = s_lut[lut_bucket(x)];
      uint32_t c = e.x + (x >= __uint_as_float(e.y) ? 1u : 0u);  // a zero block has r = 0, x = 0: the zero code
      if (!FULL && e0 + i >= numel) c = 0u;   // padding beyond the tensor
      packed |= c << (4 * i);
    }
    if (FULL || e0 < numel) {
      const int64_t byte0 = e0 >> 1;
      if (FULL || e0 + 8 <= numel) {
        *reinterpret_cast<uint32_t*>(codes + byte0) = packed;
      } else {
        const int64_t nbytes = ((numel - e0) + 1) >> 1;
        for (int64_t b = 0; b < nbytes; ++b) codes[byte0 + b] = (uint8_t)(packed >> (8 * b));
      }
    }
    if ((t & 7) == 0) {
      const int lb = local / kBlock;
      s_a[lb] = a;
      const int64_t blk = e0 / kBlock;
      if (FULL || blk < nb) absmax[blk] = a;
    }
  }
}

// The tensors of one launch: workgroup x quantises group x - gb[i] of
// tensor i, where gb[i] <= x < gb[i + 1] (gb = prefix sums of the group
// counts). Passed by value; indexed only with workgroup-uniform values.
struct QuantBatchArgs {
  int n;
  int64_t gb[kQuantBatchMax + 1];
  const void* w[kQuantBatchMax];
  int64_t numel[kQuantBatchMax];
  uint8_t* codes[kQuantBatchMax];
  float* absmax[kQuantBatchMax];
  double* gsum[kQuantBatchMax];
};

// DQ passes of the tensors that have them: sums of tensor i in sum_a[i]
// (sum_b[i] the fold's second buffer), its block absmax values in absmax[i].
struct DqBatchArgs {
  int n;
  int64_t gb[kQuantBatchMax + 1];
  const float* absmax[kQuantBatchMax];
  int64_t nb[kQuantBatchMax];
  double* sum_a[kQuantBatchMax];
  double* sum_b[kQuantBatchMax];
  float* mean[kQuantBatchMax];
  uint8_t* absmax8[kQuantBatchMax];
  float* scale2[kQuantBatchMax];
};

// The tensor that holds workgroup x (uniform: a scan over the prefix sums).
__device__ __forceinline__ int batch_item(const int64_t* gb, int n, int64_t x) {
  int i = 0;
  while (i + 1 < n && gb[i + 1] <= x) ++i;
  return __builtin_amdgcn_readfirstlane(i);
}

template <typename InT>
__global__ __launch_bounds__(kQuantThreads) void quant_blocks_kernel(QuantBatchArgs B, NF4Thresholds th) {
  __shared__ float s_a[kDqBlock];
  __shared__ double s_t[2][kDqBlock];
  __shared__ u32x2_t s_lut[kLutBuckets];  // (count of thresholds in lower buckets, the bucket's threshold bits)
  const int t = threadIdx.x;
  const int i = batch_item(B.gb, B.n, blockIdx.x);
  const int64_t g = (int64_t)blockIdx.x - B.gb[i];
  const InT* __restrict__ w = static_cast<const InT*>(B.w[i]);
  const int64_t numel = B.numel[i];
  const int64_t nb = (numel + kBlock - 1) / kBlock;
  uint8_t* __restrict__ codes = B.codes[i];
  float* __restrict__ absmax = B.absmax[i];
  if ((g + 1) * kGroupWeights <= numel)   // uniform per workgroup
    quant_group<InT, true>(w, numel, nb, g, th, codes, absmax, s_a, s_lut);
  else
    quant_group<InT, false>(w, numel, nb, g, th, codes, absmax, s_a, s_lut);
  __syncthreads();
  // float64 adjacent-pair tree over the group's valid block constants
  int n = (int)((nb - g * kDqBlock) < kDqBlock ? (nb - g * kDqBlock) : kDqBlock);
  s_t[0][t] = (t < n) ? (double)s_a[t] : 0.0;
  __syncthreads();
  int src = 0;
  while (n > 1) {
    const int half = n >> 1;
    if (t < half) s_t[src ^ 1][t] = s_t[src][2 * t] + s_t[src][2 * t + 1];
    if ((n & 1) && t == half) s_t[src ^ 1][t] = s_t[src][n - 1];
    __syncthreads();
    src ^= 1;
    n = (n + 1) >> 1;
  }
  if (t == 0) B.gsum[i][g] = s_t[src][0];
}

// Folds buf[0..n) with the adjacent-pair rule, level by level, in place
// across two halves of the workspace, then writes mean = RN32(S / nb).
// Adjacent-pair tree over the n group sums: at each level s'[i] = s[2i] +
// s[2i+1], an odd last value carried up unchanged. With n <= 32 x 1024 the
// first 5 levels run in registers (thread t folds the aligned 32 values
// [32 t, 32 t + 32); a whole run of 32 reduces exactly as inside the full
// tree, and the last, partial run ends the array at every level, so its
// carries are the tree's own), the remaining levels in LDS. Larger n fold
// level by level in the two global buffers.
__global__ __launch_bounds__(1024) void tree_fold_kernel(DqBatchArgs D) {
  constexpr int kRun = 32;
  __shared__ double s_fold[2][1024];
  const int t = threadIdx.x;
  const int item = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
  double* __restrict__ a = D.sum_a[item];
  double* __restrict__ b = D.sum_b[item];
  const int64_t nb = D.nb[item];
  int64_t n = D.gb[item + 1] - D.gb[item];       // the tensor's group count
  float* __restrict__ mean = D.mean[item];
  if (n <= (int64_t)kRun * 1024) {
    const int nruns = (int)((n + kRun - 1) / kRun);
    if (t < nruns) {
      const int64_t c0 = (int64_t)t * kRun;
      int cnt = (int)(n - c0 < kRun ? n - c0 : kRun);
      double r[kRun];
#pragma unroll
      for (int i = 0; i < kRun; ++i) r[i] = i < cnt ? a[c0 + i] : 0.0;
#pragma unroll
      for (int w = kRun; w > 1; w >>= 1) {          // one tree level: cnt values -> ceil(cnt / 2)
#pragma unroll
        for (int i = 0; i < w / 2; ++i) r[i] = (2 * i + 1 < cnt) ? r[2 * i] + r[2 * i + 1] : r[2 * i];
        cnt = (cnt + 1) >> 1;
      }
      s_fold[0][t] = r[0];
    }
    __syncthreads();
    int m = nruns, cur = 0;
    while (m > 1) {
      const int half = m >> 1;
      if (t < half) s_fold[cur ^ 1][t] = s_fold[cur][2 * t] + s_fold[cur][2 * t + 1];
      if ((m & 1) && t == 0) s_fold[cur ^ 1][half] = s_fold[cur][m - 1];
      __syncthreads();
      cur ^= 1;
      m = (m + 1) >> 1;
    }
    if (t == 0) mean[0] = (nb > 0 && n > 0) ? (float)(s_fold[cur][0] / (double)nb) : 0.0f;
    return;
  }
  double* src = a;
  double* dst = b;
  while (n > 1) {
    const int64_t half = n >> 1;
    for (int64_t i = t; i < half; i += blockDim.x) dst[i] = src[2 * i] + src[2 * i + 1];
    if ((n & 1) && t == 0) dst[half] = src[n - 1];
    __syncthreads();
    double* tmp = src;
    src = dst;
    dst = tmp;
    n = (n + 1) >> 1;
  }
  if (t == 0) {
    const double S = (n == 1) ? src[0] : 0.0;
    mean[0] = nb > 0 ? (float)(S / (double)nb) : 0.0f;
  }
}

// The E4M3 pass: one wave per DQ group of 256 block constants. Lane l holds
// blocks 4l .. 4l+3 of its group (one 16-byte load, one 4-byte store of the
// codes), so the group absmax is one cross-lane max: no LDS, no barrier.
// Each wave takes kDqGroupsPerWave consecutive groups of the batch's group
// space, all their loads issued first. Per block: d = RN32(a - mean); per
// group: sigma = RN32(max|d| / 448) (0 below 2^-126); code = E4M3 of
// RN32(d / sigma).
constexpr int kDqWaves = 4;
constexpr int kDqGroupsPerWave = 2;
__global__ __launch_bounds__(64 * kDqWaves) void dq_encode_kernel(DqBatchArgs D, int64_t total_groups) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t g0 = ((int64_t)blockIdx.x * kDqWaves + wave) * kDqGroupsPerWave;
  f32x4_t v[kDqGroupsPerWave];
  int item[kDqGroupsPerWave];
  int64_t grp[kDqGroupsPerWave];
#pragma unroll
  for (int q = 0; q < kDqGroupsPerWave; ++q) {
    const int64_t gg = g0 + q < total_groups ? g0 + q : total_groups - 1;   // clamped: loads stay unconditional
    item[q] = batch_item(D.gb, D.n, gg);
    grp[q] = gg - D.gb[item[q]];
    const int64_t nb = D.nb[item[q]];
    const int64_t b0 = grp[q] * kDqBlock + 4 * lane;
    const int64_t bl = b0 < nb ? b0 : ((nb - 1) & ~(int64_t)3);   // an aligned quad inside the padded array
    v[q] = *reinterpret_cast<const f32x4_t*>(D.absmax[item[q]] + bl);
  }
#pragma unroll
  for (int q = 0; q < kDqGroupsPerWave; ++q) {
    const int it = item[q];
    const int64_t nb = D.nb[it];
    const int64_t b0 = grp[q] * kDqBlock + 4 * lane;
    const float mu = D.mean[it][0];
    const float a[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
    float d[4];
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d[e] = (b0 + e < nb) ? a[e] - mu : 0.0f;         // RN32(a - mu)
      m = __builtin_fmaxf(m, __builtin_fabsf(d[e]));
    }
    const float A = wave_max(m, 64);
    float sigma = A / 448.0f;                            // RN32(A / 448)
    if (!(sigma >= 0x1p-126f)) sigma = 0.0f;
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t c = sigma != 0.0f ? f32_to_e4m3(d[e] / sigma) : 0u;   // RN32(d / sigma), then E4M3
      packed |= c << (8 * e);
    }
    if (g0 + q >= total_groups) continue;                // a clamped duplicate: nothing stored
    uint8_t* a8 = D.absmax8[it] + b0;
    if (b0 + 3 < nb && ((uintptr_t)D.absmax8[it] & 3u) == 0) {
      *reinterpret_cast<uint32_t*>(a8) = packed;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (b0 + e < nb) a8[e] = (uint8_t)(packed >> (8 * e));
    }
    if (lane == 0) D.scale2[it][grp[q]] = sigma;
  }
}

// Units of 8 weights (one code dword in, one 16-byte bf16 store out). A
// thread takes 4 units 256 apart, so that each load and store instruction of
// a wave covers one contiguous range, and issues their 4 code loads and block
// constants before any store. The last numel % 8 weights are done by one
// thread, one at a time.
constexpr int kDqUnits = 4;
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ absmax8,
                                                      const float* __restrict__ scale2,
                                                      const float* __restrict__ mean,
                                                      const float* __restrict__ absmax32, NF4Table tab,
                                                      int64_t numel, uint16_t* __restrict__ out) {
  __shared__ float s_q[16];
  if (threadIdx.x < 16) s_q[threadIdx.x] = tab.q[threadIdx.x];
  __syncthreads();
  const float mu = absmax32 ? 0.0f : mean[0];
  auto block_a = [&](int64_t blk) {
    return absmax32 ? absmax32[blk] : block_scale(absmax8[blk], scale2[blk / kDqBlock], mu);
  };
  const int64_t nunits = numel / 8;
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  const int64_t stride = (int64_t)gridDim.x * 256 * kDqUnits;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kDqUnits + threadIdx.x; base < nunits; base += stride) {
    uint32_t c[kDqUnits];
    float ap[kDqUnits];
#pragma unroll
    for (int u = 0; u < kDqUnits; ++u) {
      const int64_t un = base + (int64_t)u * 256;
      const int64_t uc = un < nunits ? un : nunits - 1;  // clamped: loads stay unconditional
      c[u] = cw[uc];
      ap[u] = block_a(uc >> 3);  // 8 units per 64-block
    }
#pragma unroll
    for (int u = 0; u < kDqUnits; ++u) {
      const int64_t un = base + (int64_t)u * 256;
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t byte = (c[u] >> (8 * i)) & 0xFFu;
        o[i] = pack_bf16x2(s_q[byte & 15u] * ap[u], s_q[byte >> 4] * ap[u]);
      }
      if (un < nunits) *reinterpret_cast<u32x4_t*>(out + un * 8) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t e = nunits * 8; e < numel; ++e) {
      const uint32_t byte = codes[e >> 1];
      const uint32_t q = (e & 1) ? (byte >> 4) : (byte & 15u);
      out[e] = f32_to_bf16(s_q[q] * block_a(e / kBlock));
    }
  }
}

}  // namespace

hipError_t launch_quantize_batch(const QuantItem* items, int n, bool bf16_in, const NF4Thresholds& th,
                                 hipStream_t stream) {
  if (n < 1 || n > kQuantBatchMax) return hipErrorInvalidValue;
  QuantBatchArgs B{};
  DqBatchArgs D{};
  int64_t groups = 0, dq_groups = 0;
  for (int k = 0; k < n; ++k) {
    const QuantItem& it = items[k];
    if (it.numel == 0) continue;
    const int64_t nb = (it.numel + kBlock - 1) / kBlock;
    const int64_t ng = (nb + kDqBlock - 1) / kDqBlock;
    const QuantWorkspace L = quant_workspace_layout(it.numel);
    char* base = static_cast<char*>(it.ws);
    float* absmax = it.absmax32 ? it.absmax32 : reinterpret_cast<float*>(base + L.absmax_off);
    double* sum_a = reinterpret_cast<double*>(base + L.sum_a_off);
    B.gb[B.n] = groups;
    B.w[B.n] = it.w;
    B.numel[B.n] = it.numel;
    B.codes[B.n] = it.codes;
    B.absmax[B.n] = absmax;
    B.gsum[B.n] = sum_a;
    ++B.n;
    groups += ng;
    if (!it.absmax32) {   // double quantisation: the fold and the E4M3 pass
      D.gb[D.n] = dq_groups;
      D.absmax[D.n] = absmax;
      D.nb[D.n] = nb;
      D.sum_a[D.n] = sum_a;
      D.sum_b[D.n] = reinterpret_cast<double*>(base + L.sum_b_off);
      D.mean[D.n] = it.mean;
      D.absmax8[D.n] = it.absmax8;
      D.scale2[D.n] = it.scale2;
      ++D.n;
      dq_groups += ng;
    }
  }
  B.gb[B.n] = groups;
  D.gb[D.n] = dq_groups;
  if (groups == 0) return hipSuccess;
  hipError_t e = timed(kTimeQuant, stream, [&] {
    if (bf16_in)
      hipLaunchKernelGGL(quant_blocks_kernel<uint16_t>, dim3((unsigned)groups), dim3(kQuantThreads), 0, stream, B, th);
    else
      hipLaunchKernelGGL(quant_blocks_kernel<float>, dim3((unsigned)groups), dim3(kQuantThreads), 0, stream, B, th);
    return hipGetLastError();
  });
  if (e != hipSuccess || D.n == 0) return e;
  hipLaunchKernelGGL(tree_fold_kernel, dim3((unsigned)D.n), dim3(1024), 0, stream, D);
  const int64_t per_wg = (int64_t)kDqWaves * kDqGroupsPerWave;
  hipLaunchKernelGGL(dq_encode_kernel, dim3((unsigned)((dq_groups + per_wg - 1) / per_wg)), dim3(64 * kDqWaves), 0,
                     stream, D, dq_groups);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* w, bool bf16_in, int64_t numel, const NF4Thresholds& th,
                           uint8_t* codes, uint8_t* absmax8, float* scale2, float* mean, float* absmax32,
                           void* ws, hipStream_t stream) {
  const QuantItem it{w, numel, codes, absmax8, scale2, mean, absmax32, ws};
  return launch_quantize_batch(&it, 1, bf16_in, th, stream);
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* absmax8, const float* scale2,
                             const float* mean, const float* absmax32, const NF4Table& tab, int64_t numel,
                             uint16_t* out, hipStream_t stream) {
  const int64_t nunits = numel / 8;
  int64_t blocks = (nunits + 256 * kDqUnits - 1) / (256 * kDqUnits);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return timed(kTimeDequant, stream, [&] {
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, absmax8, scale2,
                       mean, absmax32, tab, numel, out);
    return hipGetLastError();
  });
}

}  // namespace qlora
