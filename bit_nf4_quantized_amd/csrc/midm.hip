// Forward of the QLoRA linear layer for 16 < M <= 128 (batched decode and
// short prefill), for gfx950:
//
//   Y = X Wd^T + bf16(s X L1) L2^T-slab,   Wd = bf16(RN32(q[code] * a'))
//
// (QLoRA pages: diycv.top "QLoRA 论文解读", section 关键公式 for the
// dequantised product and section 推理 for the inference path; neura.market
// "QLoRA" for batched inference at this size.) At these M the weight stream
// (0.516 B per weight) and the 2 M flops per weight are of the same order
// (M = 128 is 496 flop/B, above the 312 flop/B ridge; M = 32 is 124), so the
// kernel streams the 4-bit weight once and reuses each dequantised value for
// all M columns on MFMA.
//
// Tiling: a workgroup owns 64 weight rows (output columns n) and all M (padded
// to MT = 32, 64 or 128) over one K-slice; the K-slices of a tile add up in a
// fixed-order reduction (midm_reduce_kernel), which also rounds to bf16.
//   - Each wave owns 16 rows. A lane loads the codes of its own MFMA A
//     operand (8 bytes per 64-k step) and dequantises them in registers, so
//     the weight never passes through LDS. Within a 64-k step, lane quad q
//     takes k = 16 q .. 16 q + 16: the first 8 feed the first
//     v_mfma_f32_16x16x32_bf16, the next 8 the second (any assignment of k to
//     lanes works as long as the X operand uses the same one).
//   - The X tile of the step (MT x 64 bf16) is staged in LDS, double
//     buffered, and shared by the 4 waves.
//   - The LoRA term is one more step per 64 adapter ranks in slice 0, with
//     L2's column n (16 ranks per lane, read strided) as the A operand and
//     bf16(s X L1) [m][j] as X.
//   - The codes of a step are loaded two steps ahead and its X tile three
//     steps ahead (staged into LDS one step ahead), each in three register
//     sets used in rotation.
//   - Every global load is unconditional, from a clamped address, zeroed by a
//     select afterwards (a load under a branch makes the compiler wait for it
//     where the branches join).
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int kMidThreads = 256;
constexpr int kMidTN = 64;   // weight rows per workgroup

// bf16 index of 16-byte chunk `chunk` (0..7) of row `row` in a [rows][64]
// LDS tile, chunks XOR-swizzled by the row so that 16 rows' reads spread
// over the banks
__device__ __forceinline__ int mid_swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

struct MidCodes {
  u32x2_t codes;      // 16 codes of this lane's row, k = 16 quad .. 16 quad + 16
  uint8_t c8;         // E4M3 byte of the row's block (DQ); widened where it is used, not at the load
  float fv;           // group scale (DQ) or block absmax (no DQ)
};

template <int MT>
struct MidX {
  u32x4_t x[MT / 32]; // this thread's 16-byte chunks of the step's X tile
};

template <int MT>
__global__ __launch_bounds__(kMidThreads) void midm_kernel(NF4View W, NF4Table tab, const uint16_t* __restrict__ X,
                                                           int M, const uint16_t* __restrict__ sT,
                                                           const uint16_t* __restrict__ L2, int r, int rp,
                                                           int64_t kslice, float* __restrict__ part,
                                                           uint16_t* __restrict__ Y) {
  constexpr int kXPer = MT / 32;           // 16-byte X chunks per thread per step (MT * 8 / 256)
  constexpr int kMT = MT / 16;             // m-tiles
  __shared__ float s_q[16];
  __shared__ __align__(16) uint16_t sX[2][MT * 64];

  const int64_t N = W.rows, K = W.cols;
  const int64_t n0 = (int64_t)blockIdx.x * kMidTN;
  const int z = blockIdx.y;
  const int64_t kb = (int64_t)z * kslice;
  const int64_t ke = kb + kslice < K ? kb + kslice : K;
  const int nmain = (int)((ke - kb) / 64);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int row16 = lane & 15, quad = lane >> 4;
  const int64_t nrow = n0 + wave * 16 + row16;          // this lane's weight row
  const bool row_ok = nrow < N;
  const int64_t nrow_c = row_ok ? nrow : 0;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (tid == i) s_q[i] = tab.q[i];   // constant indices: scalar kernel-argument loads

  const bool dq = W.absmax32 == nullptr;
  const uint8_t* bp = dq ? W.absmax8 : reinterpret_cast<const uint8_t*>(W.absmax32);
  const float* fp = dq ? W.scale2 : W.absmax32;
  const float mraw = *(dq ? W.mean : W.absmax32);
  const float mu = dq ? mraw : 0.0f;

  // Per-lane 32-bit offsets from uniform bases (the launcher checks that they
  // fit), advanced by a constant per step: a 64-bit address per load costs
  // several VALU instructions, per step and lane.
  const uint32_t e0 = (uint32_t)(nrow_c * K + kb) + (uint32_t)(quad * 16);   // first code of step 0
  const uint32_t blk0 = (uint32_t)((nrow_c * K + kb) / kBlock);            // its 64-block
  auto load_codes = [&](int st, MidCodes& d) {
    const uint32_t e = e0 + (uint32_t)st * 64u;      // 16 codes, inside one 64-block
    d.codes = *reinterpret_cast<const u32x2_t*>(W.codes + (e >> 1));
    const uint32_t blk = blk0 + (uint32_t)st;
    d.c8 = bp[dq ? blk : 0u];
    d.fv = fp[dq ? blk / (uint32_t)kDqBlock : blk];
  };
  // rows m >= M of the X tile read row 0 (finite values) and only feed
  // output columns m >= M, which are never stored: no select is needed (a
  // select after the load would make the compiler wait for it where it sinks)
  uint32_t xo[kXPer];
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    const int idx = tid + u * kMidThreads;
    const int m = idx >> 3, ch = idx & 7;
    xo[u] = (uint32_t)((m < M ? (int64_t)m * K : 0) + kb) + (uint32_t)(ch * 8);
  }
  auto load_x = [&](int st, MidX<MT>& d) {
#pragma unroll
    for (int u = 0; u < kXPer; ++u) d.x[u] = *reinterpret_cast<const u32x4_t*>(X + xo[u] + (uint32_t)st * 64u);
  };
  auto store_x = [&](const MidX<MT>& d, int buf) {
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int idx = tid + u * kMidThreads;
      *reinterpret_cast<u32x4_t*>(&sX[buf][mid_swz(idx >> 3, idx & 7)]) = d.x[u];
    }
  };

  f32x4_t acc[kMT];
#pragma unroll
  for (int t = 0; t < kMT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // A operands a0 (k = 16 quad .. +8) and a1 (+8 .. +16) times the X tile in `buf`
  auto mma = [&](const u32x4_t& a0, const u32x4_t& a1, int buf) {
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      const int m = t * 16 + row16;
      const u32x4_t b0 = *reinterpret_cast<const u32x4_t*>(&sX[buf][mid_swz(m, quad * 2)]);
      const u32x4_t b1 = *reinterpret_cast<const u32x4_t*>(&sX[buf][mid_swz(m, quad * 2 + 1)]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                       __builtin_bit_cast(bf16x8_t, b0), acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                       __builtin_bit_cast(bf16x8_t, b1), acc[t], 0, 0, 0);
    }
  };

  __syncthreads();  // s_q
  // one 64-k step st: start the loads of the codes of step st+2 and of the X
  // tile of step st+3, dequantise this lane's 16 weights (bf16(RN32(q[c]
  // a'))) and multiply them with the X tile in LDS, then stage the X tile of
  // step st+1 (loaded two steps ago) into the other LDS buffer. Loads past
  // the last step repeat the last step.
  auto clampst = [&](int st) { return st < nmain ? st : nmain - 1; };
  auto step = [&](int st, const MidCodes& cur, MidCodes& c2, MidX<MT>& x3, const MidX<MT>& x1) {
    const int buf = st & 1;
    // nothing moves across step boundaries: the scheduler would otherwise
    // hoist arithmetic on a later step's loads, and wait for them early
    __builtin_amdgcn_sched_barrier(0);
    load_codes(clampst(st + 2), c2);
    load_x(clampst(st + 3), x3);
    const float ap = dq ? block_scale(cur.c8, cur.fv, mu) : cur.fv;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = i < 4 ? cur.codes.x : cur.codes.y;
      const uint32_t byte = (word >> (8 * (i & 3))) & 0xFFu;
      w[i] = pack_bf16x2(s_q[byte & 15u] * ap, s_q[byte >> 4] * ap);
    }
    // rows n >= N dequantise row 0 and only feed outputs n >= N, never stored
    mma(u32x4_t{w[0], w[1], w[2], w[3]}, u32x4_t{w[4], w[5], w[6], w[7]}, buf);
    store_x(x1, buf ^ 1);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nmain > 0) {
    // three register sets each for the codes and the X tiles, in rotation
    // (no copies between steps: a copy would wait for the loads in flight)
    MidCodes c0, c1, c2;
    MidX<MT> x0, x1, x2;
    load_codes(0, c0);
    load_codes(clampst(1), c1);
    load_x(0, x0);
    load_x(clampst(1), x1);
    load_x(clampst(2), x2);
    store_x(x0, 0);
    __syncthreads();
    // whole rounds of three steps, then the last one or two (a loop with
    // exits between its steps makes the compiler wait for every load in
    // flight at the loop head)
    int st = 0;
    for (; st + 3 <= nmain; st += 3) {
      step(st, c0, c2, x0, x1);
      step(st + 1, c1, c0, x1, x2);
      step(st + 2, c2, c1, x2, x0);
    }
    if (st < nmain) step(st, c0, c2, x0, x1);
    if (st + 1 < nmain) step(st + 1, c1, c0, x1, x2);
  }

  // the LoRA slab in slice 0: A = L2[j .. j + 16)[n] (16 ranks of this
  // lane's column of L2, zero past r), X = bf16(s X L1)[m][j .. ] (row
  // stride rp, zero past r)
  if (z == 0) {
    for (int j0 = 0; j0 < rp; j0 += 64) {
      uint32_t lw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ja = j0 + quad * 16 + 2 * i;   // r even: ranks ja and ja+1 are both inside or both outside
        const bool ok = ja < r;
        const uint32_t lo = L2[(int64_t)(ok ? ja : 0) * N + nrow_c];
        const uint32_t hi = L2[(int64_t)(ok ? ja + 1 : 0) * N + nrow_c];
        lw[i] = ok ? (lo | (hi << 16)) : 0u;
      }
      const u32x4_t a0v = {lw[0], lw[1], lw[2], lw[3]}, a1v = {lw[4], lw[5], lw[6], lw[7]};
#pragma unroll
      for (int u = 0; u < kXPer; ++u) {
        const int idx = tid + u * kMidThreads;
        const int m = idx >> 3, ch = idx & 7;
        const bool ok = m < M && j0 + ch * 8 < r;   // r % 8 == 0: a chunk is wholly inside or outside
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sT + (ok ? (int64_t)m * rp + j0 + ch * 8 : 0));
        *reinterpret_cast<u32x4_t*>(&sX[0][mid_swz(m, ch)]) = ok ? v : zero4;
      }
      __syncthreads();
      mma(a0v, a1v, 0);
      __syncthreads();
    }
  }

  // lane holds D[n = n0 + 16 wave + 4 quad + i][m = 16 t + row16], i = 0..3
  const int64_t nn = n0 + wave * 16 + quad * 4;
#pragma unroll
  for (int t = 0; t < kMT; ++t) {
    const int m = t * 16 + row16;
    if (m >= M || nn >= N) continue;                 // N % 8 == 0: all 4 columns are inside
    if (part) {
      *reinterpret_cast<f32x4_t*>(part + ((int64_t)z * M + m) * N + nn) = acc[t];
    } else {
      const u32x2_t o = {pack_bf16x2(acc[t].x, acc[t].y), pack_bf16x2(acc[t].z, acc[t].w)};
      *reinterpret_cast<u32x2_t*>(Y + (int64_t)m * N + nn) = o;
    }
  }
}

// Y[m][n] = bf16(sum over z = 0 .. S-1 of part[z][m][n]), in that order;
// 4 columns per thread.
__global__ __launch_bounds__(256) void midm_reduce_kernel(const float* __restrict__ part, int S, int64_t MN,
                                                          uint16_t* __restrict__ Y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  f32x4_t a = *reinterpret_cast<const f32x4_t*>(part + i);
  for (int z = 1; z < S; ++z) {
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(part + (int64_t)z * MN + i);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  *reinterpret_cast<u32x2_t*>(Y + i) = u32x2_t{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w)};
}

struct MidSplit {
  int64_t tiles, S, kslice;
};

MidSplit mid_split(int64_t K, int64_t N) {
  MidSplit p;
  p.tiles = (N + kMidTN - 1) / kMidTN;
  const int64_t ksteps = K / 64;
  const int64_t target = 2 * (int64_t)device_cu_count();   // workgroups to fill the chip twice
  int64_t S = (target + p.tiles - 1) / p.tiles;
  if (S > ksteps) S = ksteps;
  if (S < 1) S = 1;
  const int64_t per = (ksteps + S - 1) / S;
  p.kslice = per * 64;
  p.S = (K + p.kslice - 1) / p.kslice;
  return p;
}

}  // namespace

size_t midm_partial_bytes(int64_t M, int64_t K, int64_t N) {
  if (M <= 16 || M > kMidMaxM || K <= 0 || N <= 0) return 0;
  const MidSplit p = mid_split(K, N);
  return p.S > 1 ? (size_t)p.S * M * N * 4 : 0;
}

bool midm_fits(int64_t M, int64_t K, int64_t N) {
  // the kernel's per-lane element offsets into the codes and X are 32-bit
  return N * K < ((int64_t)1 << 32) && M * K < ((int64_t)1 << 32);
}

hipError_t launch_midm(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M, const uint16_t* sT,
                       const uint16_t* L2, int r, int rp, float* part, uint16_t* Y, hipStream_t stream) {
  if (M <= 16 || M > kMidMaxM || (W.cols % 64) != 0 || (W.rows % 8) != 0 || (rp % 64) != 0 ||
      !midm_fits(M, W.cols, W.rows))
    return hipErrorInvalidValue;
  const MidSplit p = mid_split(W.cols, W.rows);
  float* pp = p.S > 1 ? part : nullptr;
  const dim3 grid((unsigned)p.tiles, (unsigned)p.S), block(kMidThreads);
  const int m = (int)M;
  if (M <= 32)
    hipLaunchKernelGGL(midm_kernel<32>, grid, block, 0, stream, W, tab, X, m, sT, L2, r, rp, p.kslice, pp, Y);
  else if (M <= 64)
    hipLaunchKernelGGL(midm_kernel<64>, grid, block, 0, stream, W, tab, X, m, sT, L2, r, rp, p.kslice, pp, Y);
  else
    hipLaunchKernelGGL(midm_kernel<128>, grid, block, 0, stream, W, tab, X, m, sT, L2, r, rp, p.kslice, pp, Y);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  const int64_t MN = M * W.rows;
  hipLaunchKernelGGL(midm_reduce_kernel, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, stream, part,
                     (int)p.S, MN, Y);
  return hipGetLastError();
}

}  // namespace qlora
