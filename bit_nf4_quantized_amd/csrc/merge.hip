// Adapter merge into the bf16 dequantised base, for gfx950:
//
//   M[n][k] = bf16( Wd[n][k] + s * sum_j L1[k][j] L2[j][n] )
//
// with Wd the doubleDequant bf16 weight (QLoRA pages: robocikowo.com "QLoRA",
// the list of common mistakes, entry on merging: merge into the dequantised
// 16-bit base rather than the 4-bit one; diycv.top "QLoRA 论文解读", section 关键公式 for the dequant).
// Per element: Wd = bf16(RN32(q[code] * a')), t = RN32(s * D) with D the
// fp32-accumulated rank-r product, result bf16_RNE(RN32(Wd + t)).
//
// The merge writes 2 B and reads 0.516 B per weight, so it is HBM-bound; the
// rank-r product (2 r flops per weight, 51 flop/B at r = 64) is too much for
// the VALU at that rate, so it runs on MFMA. One workgroup makes a 32 x 256
// output tile; it issues all of its global loads (the L2 slab, its L1
// fragments, the codes and block constants of its outputs) first, so that it
// waits for memory once, then works in two phases:
//   1. each of the 4 waves computes a 32 (n) x 64 (k) block of D with
//      v_mfma_f32_16x16x32_bf16 in the orientation D^T[k][n] = L1[k][:] .
//      L2[:][n], whose A operand (8 consecutive j of one L1 row) is a
//      16-byte load and whose lanes end up with 4 consecutive k of one n;
//      L2's 32-column slab is staged in LDS for the B operand; the fp32
//      results go to an LDS tile [32][256];
//   2. every thread then takes 8 consecutive k of one row: 4 bytes of codes,
//      the block constant, 8 fp32 of D from LDS, and one 16-byte bf16 store,
//      so rows are read and written in 128-byte and 512-byte runs.
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeTN = 32;                    // output rows (n) per tile
constexpr int kMergeTK = 256;                   // output columns (k) per tile
constexpr int kDeltaPitch = kMergeTK + 4;       // fp32 per LDS row (16-byte aligned rows)
constexpr int kDeltaBytes = kMergeTN * kDeltaPitch * 4;

// Loads of one tile that phase 2 and the B operand need: the L2 slab
// (kL2PerThread 16-byte chunks per thread), and per output slot the codes
// word, the E4M3 byte (DQ) and the fp32 value (group scale with DQ, block
// absmax without).
template <int kL2PerThread>
struct MergeTileLoads {
  u32x4_t l2[kL2PerThread];
  uint32_t codes[kMergeTN / 8], c8[kMergeTN / 8];
  float fv[kMergeTN / 8];
};

// RPC = rank chunks of 32 (r rounded up to 32, 64, 128 or 256).
//
// Persistent: workgroup g owns the k-panel g % ktiles and walks the n-tiles
// g / ktiles, + groups, + 2 groups, ...; it loads its L1 fragments once and
// keeps them in registers, and while it computes one tile the loads of the
// next are in flight (two register sets). Every global load is
// unconditional, from a clamped address, with the value zeroed by a select
// afterwards: a load under a branch makes the compiler wait for it where the
// branches join, which would serialise the loads.
template <int RPC>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(NF4View W, NF4Table tab,
                                                              const uint16_t* __restrict__ L1,
                                                              const uint16_t* __restrict__ L2, int r, float s,
                                                              int64_t ktiles, int64_t ntiles, int64_t groups,
                                                              uint16_t* __restrict__ out) {
  constexpr int kRp = 32 * RPC;
  constexpr int kL2Chunks = kRp * 4;                                  // 16-byte chunks of the L2 slab
  constexpr int kL2PerThread = (kL2Chunks + kMergeThreads - 1) / kMergeThreads;
  __shared__ float s_q[16];
  extern __shared__ __align__(16) unsigned char s_dyn[];
  float* s_delta = reinterpret_cast<float*>(s_dyn);                    // [32][kDeltaPitch]
  uint16_t* s_l2 = reinterpret_cast<uint16_t*>(s_dyn + kDeltaBytes);  // [kRp][32]

  const int64_t N = W.rows, K = W.cols;
  const int64_t k0 = (blockIdx.x % ktiles) * kMergeTK;
  const int64_t nt_first = blockIdx.x / ktiles;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int row16 = lane & 15, quad = lane >> 4;
  const int kw = wave * 64;                    // this wave's 64 columns of the tile
  const int k8 = (tid & 31) * 8;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  // constant indices: the table values come from scalar kernel-argument
  // loads (an indexed read would be a vector load that waits for all others)
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (tid == i) s_q[i] = tab.q[i];

  // block constants without branches: with DQ an E4M3 byte, its group scale
  // and the mean; without, the fp32 absmax (read through the same pointers)
  const bool dq = W.absmax32 == nullptr;
  const uint8_t* bp = dq ? W.absmax8 : reinterpret_cast<const uint8_t*>(W.absmax32);
  const float* fp = dq ? W.scale2 : W.absmax32;
  const float mraw = *(dq ? W.mean : W.absmax32);
  const float mu = dq ? mraw : 0.0f;

  auto load_tile = [&](int64_t nt, MergeTileLoads<kL2PerThread>& d) {
    const int64_t n0 = nt * kMergeTN;
#pragma unroll
    for (int u = 0; u < kL2PerThread; ++u) {
      const int idx = tid + u * kMergeThreads;
      const int j = idx >> 2, c = (idx & 3) * 8;
      const int64_t n = n0 + c;
      const bool ok = idx < kL2Chunks && j < r && n < N;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(L2 + (ok ? (int64_t)j * N + n : 0));
      d.l2[u] = ok ? v : zero4;
    }
#pragma unroll
    for (int pass = 0; pass < kMergeTN / 8; ++pass) {
      const int64_t n = n0 + pass * 8 + (tid >> 5), k = k0 + k8;
      const int64_t e = (n < N && k < K) ? n * K + k : 0;   // an out-of-range slot reads element 0
      const int64_t blk = e / kBlock;
      d.codes[pass] = *reinterpret_cast<const uint32_t*>(W.codes + (e >> 1));
      d.c8[pass] = bp[dq ? blk : 0];
      d.fv[pass] = fp[dq ? blk / kDqBlock : blk];
    }
  };

  // this wave's L1 fragments: 64 k x kRp j, kept for every tile
  u32x4_t a[4][RPC];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < RPC; ++c) {
      const int64_t k = k0 + kw + t * 16 + row16;
      const int j0 = c * 32 + quad * 8;
      const bool ok = k < K && j0 < r;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(L1 + (ok ? k * r + j0 : 0));
      a[t][c] = ok ? v : zero4;
    }

  // one tile: stage its L2 slab, start the next tile's loads, MFMA phase,
  // dequant-add-store phase
  auto step = [&](int64_t nt, const MergeTileLoads<kL2PerThread>& cur, MergeTileLoads<kL2PerThread>& nxt,
                  int64_t nt_next) {
#pragma unroll
    for (int u = 0; u < kL2PerThread; ++u) {
      const int idx = tid + u * kMergeThreads;
      if (idx < kL2Chunks) *reinterpret_cast<u32x4_t*>(s_l2 + (idx >> 2) * kMergeTN + (idx & 3) * 8) = cur.l2[u];
    }
    load_tile(nt_next, nxt);
    __syncthreads();

    // ---- phase 1: D^T[k][n] on MFMA, 4 k-tiles x 2 n-tiles per wave ----
    f32x4_t acc[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[h][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < RPC; ++c) {
      const int j0 = c * 32 + quad * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t bw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bw[i] = (uint32_t)s_l2[(j0 + 2 * i) * kMergeTN + h * 16 + row16] |
                  ((uint32_t)s_l2[(j0 + 2 * i + 1) * kMergeTN + h * 16 + row16] << 16);
        const u32x4_t b = {bw[0], bw[1], bw[2], bw[3]};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[t][c]),
                                                              __builtin_bit_cast(bf16x8_t, b), acc[h][t], 0, 0, 0);
      }
    }
    // lane holds D[n = 16 h + row16][k = kw + 16 t + 4 quad + i], i = 0..3
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *reinterpret_cast<f32x4_t*>(s_delta + (h * 16 + row16) * kDeltaPitch + kw + t * 16 + quad * 4) =
            acc[h][t];
    __syncthreads();

    // ---- phase 2: dequantise, add, round, store ----
    const int64_t n0 = nt * kMergeTN;
#pragma unroll
    for (int pass = 0; pass < kMergeTN / 8; ++pass) {
      const int row = pass * 8 + (tid >> 5);
      const int64_t n = n0 + row, k = k0 + k8;
      const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(s_delta + row * kDeltaPitch + k8);
      const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(s_delta + row * kDeltaPitch + k8 + 4);
      const float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      const float ap = dq ? block_scale(cur.c8[pass], cur.fv[pass], mu) : cur.fv[pass];
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float wd = bf16_to_f32(f32_to_bf16(s_q[(cur.codes[pass] >> (4 * i)) & 15u] * ap));   // bf16 base
        v[i] = wd + s * d[i];
      }
      const u32x4_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7])};
      if (n < N && k < K) *reinterpret_cast<u32x4_t*>(out + n * K + k) = o;   // K % 8 == 0
    }
  };

  // two register sets used in turn, so no copies between tiles (a copy would
  // wait for the prefetch and for the previous tile's stores); a tile past
  // the end loads the last one again
  auto clamp_nt = [&](int64_t nt) { return nt < ntiles ? nt : ntiles - 1; };
  MergeTileLoads<kL2PerThread> bufA, bufB;
  load_tile(clamp_nt(nt_first), bufA);
  for (int64_t nt = nt_first; nt < ntiles; nt += 2 * groups) {
    step(nt, bufA, bufB, clamp_nt(nt + groups));
    if (nt + groups >= ntiles) break;
    step(nt + groups, bufB, bufA, clamp_nt(nt + 2 * groups));
  }
}

template <int RPC>
hipError_t launch_merge_rpc(const NF4View& W, const NF4Table& tab, const uint16_t* L1, const uint16_t* L2, int r,
                            float s, uint16_t* out, hipStream_t stream) {
  const int64_t ktiles = (W.cols + kMergeTK - 1) / kMergeTK;
  const int64_t ntiles = (W.rows + kMergeTN - 1) / kMergeTN;
  const size_t lds = kDeltaBytes + (size_t)32 * RPC * kMergeTN * 2;
  // every workgroup resident at once: CUs x workgroups per CU (queried once),
  // grouped by k-panel
  static int per_cu = 0;
  if (per_cu <= 0) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, merge_kernel<RPC>, kMergeThreads, lds) == hipSuccess) per_cu = b;
    (void)hipGetLastError();
    if (per_cu <= 0) per_cu = 1;
  }
  int64_t groups = (int64_t)device_cu_count() * per_cu / ktiles;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  hipLaunchKernelGGL(merge_kernel<RPC>, dim3((unsigned)(ktiles * groups)), dim3(kMergeThreads), lds, stream, W, tab,
                     L1, L2, r, s, ktiles, ntiles, groups, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const NF4View& W, const NF4Table& tab, const uint16_t* L1, const uint16_t* L2, int r,
                        float s, uint16_t* out, hipStream_t stream) {
  if (W.rows <= 0 || W.cols <= 0) return hipSuccess;
  if (r <= 32) return launch_merge_rpc<1>(W, tab, L1, L2, r, s, out, stream);
  if (r <= 64) return launch_merge_rpc<2>(W, tab, L1, L2, r, s, out, stream);
  if (r <= 128) return launch_merge_rpc<4>(W, tab, L1, L2, r, s, out, stream);
  return launch_merge_rpc<8>(W, tab, L1, L2, r, s, out, stream);
}

}  // namespace qlora
