// Small-M (decode-style) QLoRA forward on gfx950:
//   Y[m][n] = sum_k X[m][k] dequant(Wt)[n][k] + sum_j sT[m][j] L2[j][n],  M <= 16
// (QLoRA pages, diycv.top, section 关键公式; inference keeps the 4-bit base
// and the trained adapters, section 训练与推理流程 "推理").
//
// The packed weight is the only large stream (0.52 B per weight), so these
// kernels are HBM- and latency-bound. Shared by both kernels below:
//   * one workgroup per 16 weight rows; the K axis is cut into steps of 128
//     and the waves take the steps round-robin;
//   * in a step, lane l holds weight row l%16 and the 32 consecutive k of
//     lane group l/16 (16 bytes of codes, half a 64-block): four
//     v_mfma_f32_16x16x32_bf16 multiply them with the matching 32 k of X
//     (B operand: column m = l%16; columns m >= M are never stored), so the
//     M dot products cost no VALU work;
//   * the weights are dequantised exactly as the standalone dequant does,
//     bf16(RN32(q[code] * a')), with the 16-entry codebook in LDS (16
//     distinct words: no bank conflicts);
//   * the waves' partial sums are added in a fixed order through LDS and Y
//     is rounded to bf16 once.
// gemv_kernel (the streamed kernel, used when its LDS layout fits) moves the
// codes and X through per-wave LDS rings with global_load_lds; gemv_ring_kernel
// (short or very long rows) keeps the next 4 steps of each wave in registers.
// The small-M LoRA down projection bf16(s X L1) that feeds them is at the end.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace qlora {

namespace {

constexpr int kGvRows = 16;   // weight rows per workgroup = MFMA rows
constexpr int kGvStep = 128;  // k per step: 4 lane groups x 32
constexpr int kGvDepth = 4;   // steps in flight per wave
constexpr int kGvMaxRank = 256; // largest rank the C ABI accepts

struct GvStep {
  u32x4_t codes;   // 32 codes of this lane's row
  u32x4_t x[4];    // X[m][k .. k+32) for this lane's column m
  uint32_t a8;     // E4M3 block constant
  float sigma;     // DQ scale of the block's group
  int k;           // first k of the lane's 32 (>= K: past the row, masked)
};

// ---- register-ring kernel ----------------------------------------------------
// Each wave keeps the codes, block constants and X fragments of its next 4
// steps in registers; the rank-r LoRA term is added in fp32 (sT and the 16
// columns of L2 are staged in LDS while the first code loads are in flight).
template <int kGvWaves>
__global__ __launch_bounds__(64 * kGvWaves) void gemv_ring_kernel(NF4View W, NF4Table tab, const uint16_t* __restrict__ X,
                                                          int M, const uint16_t* __restrict__ sT, int ldst,
                                                          const uint16_t* __restrict__ L2, int r,
                                                          uint16_t* __restrict__ Y) {
  __shared__ float sQ[16];
  __shared__ float red[kGvWaves][kGvRows * 16];
  __shared__ uint16_t sL2[kGvMaxRank * kGvRows];  // L2[j][n0 .. n0+16)
  __shared__ uint16_t sS[16 * kGvMaxRank];        // sT[m][j]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t K = W.cols, N = W.rows;
  const int64_t n0 = (int64_t)blockIdx.x * kGvRows;

  // Without double quantisation the fp32 block absmax is a' itself: the
  // loads below then read it in place of the DQ scale (the 8-bit load reads
  // any valid byte, unused), so that no load depends on a branch.
  const bool dq = W.absmax32 == nullptr;
  const float mu = *(dq ? W.mean : W.absmax32) * (dq ? 1.0f : 0.0f);
  const uint8_t* a8p = dq ? W.absmax8 : reinterpret_cast<const uint8_t*>(W.absmax32);
  const int row = lane & 15, grp = lane >> 4;
  int64_t n = n0 + row;
  if (n > N - 1) n = N - 1;  // rows past N are computed on a valid row and never stored
  const uint8_t* crow = W.codes + n * (K >> 1);
  const int64_t blk_row = n * (K / kBlock);
  // X column m = row; columns m >= M read row 0 and are never stored (each
  // MFMA output column depends on its own B column only)
  const uint16_t* xrow = X + (int64_t)(row < M ? row : 0) * K;
  const int nsteps = (int)((K + kGvStep - 1) / kGvStep);

  // Loads are unconditional (addresses clamped into the row) so that the
  // compiler can count them exactly; steps past the row are masked in compute.
  auto load = [&](int s, GvStep& g) {
    g.k = s * kGvStep + grp * 32;
    const int kc = g.k < K ? g.k : (int)K - 32;
    g.codes = *reinterpret_cast<const u32x4_t*>(crow + (kc >> 1));
    const int64_t blk = blk_row + (kc >> 6);
    g.a8 = a8p[blk];
    g.sigma = dq ? W.scale2[blk / kDqBlock] : W.absmax32[blk];
    const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xrow + kc);
#pragma unroll
    for (int j = 0; j < 4; ++j) g.x[j] = xp[j];
  };

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](const GvStep& g) {
    const bool valid = g.k < K;
    const float ap = valid ? (dq ? block_scale(g.a8, g.sigma, mu) : g.sigma) : 0.0f;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const uint32_t words[4] = {g.codes.x, g.codes.y, g.codes.z, g.codes.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4_t wv;
      uint32_t* wp = reinterpret_cast<uint32_t*>(&wv);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t byte = (words[j] >> (8 * i)) & 0xFFu;
        wp[i] = pack_bf16x2(sQ[byte & 15u] * ap, sQ[byte >> 4] * ap);
      }
      const u32x4_t xv = valid ? g.x[j] : z;  // zero weights times finite zeros past the row
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv),
                                                     __builtin_bit_cast(bf16x8_t, xv), acc, 0, 0, 0);
    }
  };

  // ring of kGvDepth steps: this wave's i-th step (wave + kGvWaves * i) sits
  // in slot i % kGvDepth; trailing steps past the row compute zeros
  GvStep ring[kGvDepth];
#pragma unroll
  for (int d = 0; d < kGvDepth; ++d) load(wave + kGvWaves * d, ring[d]);

  // codebook and LoRA operands into LDS while the first code loads are in flight
  constexpr int kThreads = 64 * kGvWaves;
  if (tid < 16) sQ[tid] = tab.q[tid];
  for (int i = tid; i < r * kGvRows; i += kThreads) {
    const int j = i / kGvRows, c = i % kGvRows;
    const int64_t nc = n0 + c;
    sL2[i] = nc < N ? L2[(int64_t)j * N + nc] : (uint16_t)0;
  }
  for (int i = tid; i < M * r; i += kThreads) sS[i] = sT[(int64_t)(i / r) * ldst + (i % r)];
  __syncthreads();
  for (int s0 = wave; s0 < nsteps; s0 += kGvWaves * kGvDepth) {
#pragma unroll
    for (int d = 0; d < kGvDepth; ++d) {
      compute(ring[d]);
      load(s0 + kGvWaves * (d + kGvDepth), ring[d]);
    }
  }

  // acc register i of lane l is C[row 4 (l/16) + i][column l%16] = partial Y[m][n0 + row]
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * grp + i) * 16 + row] = acc[i];
  __syncthreads();
  if (tid < kGvRows * 16) {
    const int nr = tid / 16, m = tid % 16;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kGvWaves; ++w) v += red[w][nr * 16 + m];
    if (m < M) {
      for (int j = 0; j < r; ++j) v = __builtin_fmaf(bf16_to_f32(sS[m * r + j]), bf16_to_f32(sL2[j * kGvRows + nr]), v);
      const int64_t ny = n0 + nr;
      if (ny < N) Y[(int64_t)m * N + ny] = f32_to_bf16(v);
    }
  }
}

// ---- streamed kernel ---------------------------------------------------------
//
// Every wave streams its own k-steps (steps wave, wave + W, ... of 128 k)
// through its own LDS ring of NS slots, filled by global_load_lds_dwordx4:
// a slot holds the 16 rows x 64 bytes of codes of the step (one copy) and
// the step's 128 k of the M rows of X (one copy of up to 4 rows, or four).
// Nothing a wave reads was copied by another wave, so the K loop has no
// barrier: each wave waits on its own vmcnt, with up to NS - 1 steps in
// flight and no registers held by them. 16-byte chunks are XOR-swizzled so
// that the 16 rows read by one MFMA operand hit distinct banks. Lane l of a
// step holds weight row l%16 and the 32 k of lane group l/16; it dequantises
// them through the 16-entry codebook in LDS with the block constant a' from
// a per-workgroup table and issues 4 MFMAs (two accumulators, alternated).
// The LoRA term is MFMAs on wave 0 (A = the tile's L2 columns, B = bf16(s T));
// the waves' partial sums are added in a fixed order through LDS.

typedef __attribute__((address_space(3))) void gv_lds_t;

__device__ __forceinline__ void gv_dma16(const void* gbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(gbase), "s"(m0) : "memory", "m0");
}

__device__ __forceinline__ void gv_dma4(const void* gbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(gbase), "s"(m0) : "memory", "m0");
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 40] (the count is an immediate)
__device__ __forceinline__ void gv_wait_vm(int n) {
  switch (n) {
#define GV_W(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    GV_W(1) GV_W(2) GV_W(3) GV_W(4) GV_W(5) GV_W(6) GV_W(7) GV_W(8) GV_W(9) GV_W(10) GV_W(11) GV_W(12)
    GV_W(13) GV_W(14) GV_W(15) GV_W(16) GV_W(17) GV_W(18) GV_W(19) GV_W(20) GV_W(21) GV_W(22) GV_W(23)
    GV_W(24) GV_W(25) GV_W(26) GV_W(27) GV_W(28) GV_W(29) GV_W(30) GV_W(31) GV_W(32) GV_W(33) GV_W(34)
    GV_W(35) GV_W(36) GV_W(37) GV_W(38) GV_W(39) GV_W(40)
#undef GV_W
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

struct GvLayout {
  uint32_t slot_bytes, x_off, ring_bytes, red_off, l2_off, s_off, a_off, ab_off, sc_off, total;
  int nblk_p, rp;
};

// mx: X rows held per slot (1, 4 or 16)
__host__ __device__ inline GvLayout gv_layout(int waves, int mx, int ns, int64_t K, int r) {
  GvLayout L;
  L.x_off = 1024u;                              // codes: 16 rows x 64 bytes
  L.slot_bytes = 1024u + (uint32_t)mx * 256u;   // X: mx rows x 128 k (one, four or sixteen)
  L.ring_bytes = L.slot_bytes * ns;
  const int nblk = (int)(K / kBlock);
  L.nblk_p = nblk | 1;                          // odd row pitch: rows on different banks
  L.rp = (r + 31) & ~31;                        // LoRA rank padded to the MFMA depth
  uint32_t off = L.ring_bytes * waves;
  L.a_off = off;    off += 16u * L.nblk_p * 4u;
  L.ab_off = off;   off += ((16u * nblk + 255u) / 256u) * 256u;     // the tile's absmax bytes
  L.sc_off = off;   off += 256u;                                    // its DQ scales (<= 64 groups)
  L.total = (off + 15u) & ~15u;
  // after the K loop the rings are free: LoRA operands and the partial sums
  L.l2_off = 0;                                 // L2 columns of the tile, [16][rp]
  L.s_off = 16u * L.rp * 2u;                    // bf16(s T), [16][rp], rows >= M zero
  L.red_off = 2u * 16u * L.rp * 2u;             // partial sums, [W][256] fp32 (fits: rings >= 40 KB)
  return L;
}

template <int W, int MX, int NS>
__global__ __launch_bounds__(64 * W) void gemv_kernel(NF4View Wt, NF4Table tab, const uint16_t* __restrict__ X,
                                                      int M, const uint16_t* __restrict__ sT, int ldst,
                                                      const uint16_t* __restrict__ L2, int r,
                                                      uint16_t* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gv_smem[];
  __shared__ float sQ[16];
  constexpr int kThreads = 64 * W;
  constexpr int kXCopies = MX <= 4 ? 1 : MX / 4;  // copies of X per step (4 rows each; MX = 1: 16 lanes)
  constexpr int kDma = 1 + kXCopies;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = Wt.cols, N = Wt.rows;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const GvLayout L = gv_layout(W, MX, NS, K, r);
  const int nsteps = (int)((K + 127) / 128);
  const int mysteps = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;
  unsigned char* ring = gv_smem + wave * L.ring_bytes;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(gv_lds_t*)ring;

  // copy lanes: codes lane l -> row l/4, slot chunk l%4 holding chunk (l%4) ^ ((row>>2)&3)
  const int crow = lane >> 2;
  const int cchunk = (lane & 3) ^ ((crow >> 2) & 3);
  int64_t nrow = n0 + crow;
  if (nrow > N - 1) nrow = N - 1;
  const uint32_t crow_off = (uint32_t)(nrow * (K >> 1));  // codes < 4 GB (checked by the launcher)
  // X lane l of copy t -> row 4t + l/16, slot chunk l%16 holding chunk (l%16) ^ (row & 15)
  uint32_t xrow[kXCopies], xch[kXCopies];
#pragma unroll
  for (int t = 0; t < kXCopies; ++t) {
    const int m = 4 * t + (lane >> 4);
    xch[t] = (uint32_t)((lane & 15) ^ (m & 15));
    xrow[t] = (uint32_t)((m < M ? m : 0) * K * 2);   // rows >= M: any valid row
  }
  auto issue = [&](int i) {  // this wave's i-th step into slot i % NS
    const int s = wave + W * i;
    const uint32_t sl = ring_lds + (uint32_t)(i % NS) * L.slot_bytes;
    int64_t cb = (int64_t)s * 64 + 16 * cchunk;        // this lane's 16 bytes of the step's codes
    if (cb > (K >> 1) - 16) cb = (K >> 1) - 16;        // past the row: any valid chunk (masked)
    gv_dma16(Wt.codes, crow_off + (uint32_t)cb, __builtin_amdgcn_readfirstlane(sl));
#pragma unroll
    for (int t = 0; t < kXCopies; ++t) {
      int64_t xk = (int64_t)s * 128 + 8 * xch[t];
      if (xk > K - 8) xk = K - 8;                      // past the row: any valid chunk (masked)
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(sl + L.x_off + (uint32_t)(t * 1024));
      if (MX > 1 || lane < 16) gv_dma16(X, xrow[t] + (uint32_t)(xk * 2), m0);
    }
  };

  // Shared tables. The tile's absmax bytes (16 nblk contiguous bytes) and its
  // DQ scales are copied into LDS by wave 0 ahead of its step copies, so that
  // waiting for them (an exact vmcnt) does not wait for the step copies; the
  // a' table is then built from LDS.
  float* sA = reinterpret_cast<float*>(gv_smem + L.a_off);
  uint16_t* sL2 = reinterpret_cast<uint16_t*>(gv_smem + L.l2_off);
  uint16_t* sS = reinterpret_cast<uint16_t*>(gv_smem + L.s_off);
  float* red = reinterpret_cast<float*>(gv_smem + L.red_off);
  const int nblk = (int)(K / kBlock);
  const int64_t nb_total = N * nblk, ng_total = (nb_total + kDqBlock - 1) / kDqBlock;
  const int64_t ab0 = n0 * nblk;                       // first block of the tile
  const int64_t g0 = ab0 / kDqBlock;
  const int ab_copies = (16 * nblk + 255) / 256;      // 4 bytes per lane: N % 8 == 0 makes nb_total % 8 == 0,
  if (wave == 0) {                                     // so no 4-byte piece straddles the end of the tensor
    for (int t = 0; t < ab_copies; ++t) {
      int64_t off = ab0 + 256 * t + 4 * lane;
      if (off > nb_total - 4) off = nb_total - 4;      // past the tensor (rows >= N only): any valid bytes
      gv_dma4(Wt.absmax8, (uint32_t)off, __builtin_amdgcn_readfirstlane(
                                             (uint32_t)(uintptr_t)(gv_lds_t*)(gv_smem + L.ab_off + 256 * t)));
    }
    int64_t g = g0 + lane;
    if (g > ng_total - 1) g = ng_total - 1;
    gv_dma4(Wt.scale2, (uint32_t)(g * 4), __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(gv_lds_t*)(gv_smem + L.sc_off)));
  }
  for (int i = 0; i < NS - 1 && i < mysteps; ++i) issue(i);
  if (wave == 0) gv_wait_vm((NS - 1 < mysteps ? NS - 1 : mysteps) * kDma);  // the table copies have landed
  if (tid < 16) sQ[tid] = tab.q[tid];
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // (__syncthreads would drain the copies)
  {
    const float mu = Wt.mean[0];
    const unsigned char* ab = gv_smem + L.ab_off;
    const float* sc = reinterpret_cast<const float*>(gv_smem + L.sc_off);
    for (int i = tid; i < 16 * nblk; i += kThreads) {
      int gi = (int)((ab0 + i) / kDqBlock - g0);
      if (gi > 63) gi = 63;                           // rows >= N only
      sA[(i / nblk) * L.nblk_p + i % nblk] = block_scale(ab[i], sc[gi], mu);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // a' table visible

  const int row = lane & 15, grp = lane >> 4;
  const bool xlane = row < M;                   // lanes whose X column is stored
  f32x4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  const int cread = row * 64 + 16 * (grp ^ ((row >> 2) & 3));
  const int xt = row >> 2, xread = (row & 3) * 256;        // copy and row within it
  for (int i = 0; i < mysteps; ++i) {
    const int after = mysteps - 1 - i < NS - 2 ? mysteps - 1 - i : NS - 2;  // steps issued after i
    gv_wait_vm(after * kDma);
    if (i + NS - 1 < mysteps) issue(i + NS - 1);
    const unsigned char* sl = ring + (i % NS) * L.slot_bytes;
    const int64_t k = (int64_t)(wave + W * i) * 128 + 32 * grp;
    const bool valid = k < K;
    const u32x4_t codes = *reinterpret_cast<const u32x4_t*>(sl + cread);
    const float ap = valid ? sA[row * L.nblk_p + (int)(k >> 6)] : 0.0f;
    const uint32_t words[4] = {codes.x, codes.y, codes.z, codes.w};
    // all 32 codebook reads of the step first (one LDS round trip), then the products
    float qv[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) qv[e] = sQ[(words[e >> 3] >> (4 * (e & 7))) & 15u];
    u32x4_t xf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xf[j] = z;
      if (xlane && valid)
        xf[j] = *reinterpret_cast<const u32x4_t*>(sl + L.x_off + xt * 1024 + xread + 16 * ((4 * grp + j) ^ (row & 15)));
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 36, 0);  // the LDS reads as one group
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4_t wv;
      uint32_t* wp = reinterpret_cast<uint32_t*>(&wv);
#pragma unroll
      for (int q = 0; q < 4; ++q) wp[q] = pack_bf16x2(qv[8 * j + 2 * q] * ap, qv[8 * j + 2 * q + 1] * ap);
      const u32x4_t xv = xf[j];
      if (j & 1)
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv),
                                                        __builtin_bit_cast(bf16x8_t, xv), acc1, 0, 0, 0);
      else
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv),
                                                        __builtin_bit_cast(bf16x8_t, xv), acc0, 0, 0, 0);
    }
  }
  f32x4_t acc = acc0 + acc1;

  // LoRA term on wave 0: A = the tile's L2 columns (rows n), B = bf16(s T)^T
  __syncthreads();  // every wave is done with its ring
  for (int i = tid; i < 16 * L.rp; i += kThreads) {
    const int c = i / L.rp, j = i % L.rp;
    const int64_t nc = n0 + c;
    sL2[i] = (j < r && nc < N) ? L2[(int64_t)j * N + nc] : (uint16_t)0;
    sS[i] = (j < r && c < M) ? sT[(int64_t)c * ldst + j] : (uint16_t)0;
  }
  __syncthreads();
  if (wave == 0) {
    for (int j0 = 0; j0 < L.rp; j0 += 32) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(sL2 + row * L.rp + j0 + 8 * grp);
      const u32x4_t b = *reinterpret_cast<const u32x4_t*>(sS + row * L.rp + j0 + 8 * grp);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                     acc, 0, 0, 0);
    }
  }

  // acc register i of lane l: Y[m = l%16][n0 + 4 (l/16) + i], partial over this wave's k
#pragma unroll
  for (int q = 0; q < 4; ++q) red[wave * 256 + (4 * grp + q) * 16 + row] = acc[q];
  __syncthreads();
  if (tid < 256) {
    const int nr = tid / 16, m = tid % 16;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += red[w * 256 + nr * 16 + m];
    const int64_t ny = n0 + nr;
    if (m < M && ny < N) Y[(int64_t)m * N + ny] = f32_to_bf16(v);
  }
}

constexpr uint32_t kGvMaxLds = 160u * 1024u - 64u;  // dynamic part (the codebook is static)

// Returns false (nothing launched) when the LDS layout does not fit.
template <int W, int MX, int NS>
bool launch_streamed(const NF4View& Wt, const NF4Table& tab, const uint16_t* X, int M, const uint16_t* sT,
                     const uint16_t* L2, int r, uint16_t* Y, int64_t tiles, hipStream_t stream, hipError_t* err) {
  const GvLayout L = gv_layout(W, MX, NS, Wt.cols, r);
  if (L.total > kGvMaxLds || L.red_off + 1024u * W > L.ring_bytes * W) return false;
  static bool attr_set = false;  // raise the dynamic-LDS limit once per instantiation (idempotent)
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<W, MX, NS>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGvMaxLds);
    (void)hipGetLastError();  // a refusal shows up as a launch error below
    attr_set = true;
  }
  hipLaunchKernelGGL((gemv_kernel<W, MX, NS>), dim3((unsigned)tiles), dim3(64 * W), L.total, stream, Wt, tab, X, M,
                     sT, r, L2, r, Y);
  *err = hipGetLastError();
  return true;
}

// ---- byte-table kernel ---------------------------------------------------------
//
// Within one 64-block of a row every weight carries the same constant a', so
// the row's dot product with an X column is  sum_blocks a' * sum_k q[c_k] x_k.
// This kernel computes the inner sums with MFMAs whose A operand is bf16(q[c])
// and applies a' afterwards, in fp32, four FMAs per block and lane. The K loop
// then does no per-weight arithmetic beyond one LDS lookup per code byte: a
// 256-entry table maps a byte (two codes, low nibble first) straight to the
// packed pair bf16(q[lo]) | bf16(q[hi]) << 16. The table is replicated 32 times,
// copy c in LDS bank c, and lane l reads copy l % 32, so lookups never conflict.
// The effective weight is bf16(q)·a' rather than bf16(q·a'): both round once
// to bf16 precision, and the result differs from the dequantised product only
// at that rounding level.
//
// Layout of a step (128 k = two 64-blocks of a row): lane l loads 16 bytes of
// row l%16 (one 16-byte load per lane: 8-byte loads reach only about 70 % of
// the streaming rate), and a cross-half lane swap (v_permlane32_swap) gives
// every lane 16 codes of each block. MFMA h (h = 0, 1) of a block takes the
// lane's codes 8h .. 8h+8 and the matching 8 k of X, so each MFMA sums one
// block only.
// The codes of the next D steps of a wave are in flight in registers; X is
// staged once in LDS when it fits (XL), else its fragments ride with the codes.
// Each wave computes the block constants of its own next D steps into a
// private LDS ring, so the only workgroup barrier before the K loop waits for
// the table and the staged X. The LoRA term (operands loaded first) is added
// by wave 0 after its K loop, and the waves' partial sums are added in a
// fixed order through LDS.
// Fused variants (FT > 0) also take over the last step of the adapter's down
// projection: instead of reading bf16(s T) written by a separate reduction,
// each wave loads the K-slice partials of T = X L1 of its slices first in the
// prologue, sums them in slice order and leaves the sums in LDS before the
// barrier; after the K loop wave 0 adds the waves' sums in wave order, rounds
// bf16(s T) for its MFMA operand, and workgroup 0 writes bf16(T) when asked.

constexpr int kLutCopies = 32;
constexpr uint32_t kLutBytes = 256u * kLutCopies * 4u;   // 32 KB

struct GlLayout {
  uint32_t a_off, lora_off, x_off, xpitch, q_off, total;
};

// waves, ring depth, X rows staged in LDS (0 when X rides in registers),
// bytes of the per-wave sums of the adapter's slice partials (0 unless fused)
__host__ __device__ inline GlLayout gl_layout(int64_t K, int waves, int depth, int mx_lds, uint32_t q_bytes) {
  GlLayout L;
  uint32_t off = kLutBytes;                      // the table; partial sums reuse it at the end
  L.a_off = off; off += (uint32_t)(waves * depth) * 128u;  // per wave: a' [slot][block][16 rows] fp32
  // wave 0's packed LoRA fragments: the L2 operand [2 rank chunks][64 lanes]
  // x 16 B, then (unless fused) the sT operand in the same layout
  L.lora_off = off; off += q_bytes ? 2048u : 4096u;
  L.xpitch = (uint32_t)K * 2u;                   // X rows back to back (staged only for M <= 2 in practice)
  L.x_off = off; off += (uint32_t)mx_lds * L.xpitch;
  L.q_off = off; off += q_bytes;                 // [wave][M r] fp32
  L.total = off;
  return L;
}

// The adapter's last reduction folded into the GEMV (the slice partials of
// X L1 summed in the kernel instead of a separate launch): P = [Z][M][r] fp32
// slice partials, s the LoRA scale, T_out optional bf16(X L1) [M][r].
struct FuseT {
  const float* P;
  int Z;
  float s;
  uint16_t* T_out;
};
// Fused variants FT = F: lane l loads the 16-byte chunks f 64 + l (f < F)
// of each of its wave's slices, so M r <= 256 F; a wave takes at most
// ft_slices(F) slices (the loads stay within 12 registers of 16 bytes).
constexpr int ft_slices(int F) { return F == 1 ? 4 : 12 / F; }

template <int D, bool XL>
struct GlSlot {
  u32x4_t c;                       // 16 bytes of codes: row l%16, bytes 16 (l/16) .. +16 of the step
  u32x4_t x[XL ? 1 : 2][2];        // X fragments (register path only)
};

template <int W, int D, bool XL, int FT>
__global__ __launch_bounds__(64 * W) void gemv_lut_kernel(NF4View Wt, NF4Table tab, const uint16_t* __restrict__ X,
                                                          int M, const uint16_t* __restrict__ sT, int ldst,
                                                          const uint16_t* __restrict__ L2, int r,
                                                          uint16_t* __restrict__ Y, FuseT ft) {
  static_assert(D % 4 == 0, "a round of D steps gives each lane D/4 (row, step) block-constant pairs");
  extern __shared__ __attribute__((aligned(16))) unsigned char gl_smem[];
  constexpr int kThreads = 64 * W;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Sizes fit 32-bit arithmetic (the launcher checks the byte extents), so each
  // load is a uniform 64-bit base plus a 32-bit per-lane byte offset, and the
  // products are 24-bit multiplies: a 64-bit address costs several quarter-rate
  // VALU instructions, which the prologue of every wave would pay.
  const int K = (int)Wt.cols, N = (int)Wt.rows;
  const int n0 = (int)blockIdx.x * 16;
  const int nblk = K / kBlock;
  const int mr = M * r;
  const GlLayout L = gl_layout(K, W, D, XL ? M : 0, FT ? (uint32_t)(W * mr) * 4u : 0u);
  const int nsteps = nblk / 2;                   // K % 128 == 0
  const int mysteps = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;
  const int row = lane & 15, grp = lane >> 4;
  const int xm = row < M ? row : 0;              // X column of this lane (unused columns repeat row 0)
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const int nrow = n0 + row < N ? n0 + row : N - 1;  // rows past N are computed on a valid row, never stored
  auto ld16 = [](const void* base, uint32_t off) { return *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(base) + off); };

  // ---- loads, in the order they are needed: they complete in issue order ----
  // Fused adapter reduction: the slice partials first (the prologue sums
  // them before its barrier). Lane l reads the 16-byte chunks f 64 + l of the
  // [M][r] slab of slices z = wave, wave + W, ...; missing slices and chunks
  // read offset 0 and are not used.
  constexpr int kSl = FT ? ft_slices(FT) : 1;
  f32x4_t pz[FT ? kSl * FT : 1];
  if constexpr (FT > 0) {
#pragma unroll
    for (int i = 0; i < kSl; ++i)
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const int z = wave + W * i, q = 4 * (64 * f + lane);
        const bool ok = z < ft.Z && q < mr;
        const uint32_t off = ok ? (__umul24((uint32_t)z, (uint32_t)mr) + (uint32_t)q) * 4u : 0u;
        pz[i * FT + f] = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const char*>(ft.P) + off);
      }
  }
  // LoRA operands for wave 0 (ranks <= 64; the term is added after the K loop):
  // A = L2[j][n0 + row], B = sT[row][j], rank chunks of 32. The prologue loads
  // are unconditional (addresses in bounds): a load under a branch makes the
  // compiler wait for it where the branch joins.
  constexpr int kLoraChunks = 2;
  uint32_t la[kLoraChunks][8];
  u32x4_t lb[kLoraChunks];
  const int rp = (r + 31) & ~31;
#pragma unroll
  for (int c = 0; c < kLoraChunks; ++c) {
    const int j0 = 32 * c + 8 * grp;
    const int jb = j0 < r ? j0 : 0;              // r % 8 == 0: a chunk of 8 is all in or all out
    const uint32_t o = (__umul24((uint32_t)jb, (uint32_t)N) + (uint32_t)nrow) * 2u;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      la[c][e] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(L2) + o + (uint32_t)(e * N) * 2u);
    if constexpr (FT == 0) lb[c] = ld16(sT, (__umul24((uint32_t)xm, (uint32_t)ldst) + (uint32_t)jb) * 2u);
  }
  // Block constants, one round of D steps ahead: lane l computes a' of row l%16
  // for the wave's steps base + l/16 + 4k (both 64-blocks of the step).
  // Without double quantisation (Wt.absmax32 set) a' is the fp32 block
  // absmax: sg0/sg1 then read it for the two blocks and the 16-bit load reads
  // any valid bytes (unused); with DQ both scale loads read the group's DQ
  // scale. No load depends on a branch.
  constexpr int kAPairs = D / 4;
  const bool dq = Wt.absmax32 == nullptr;
  const void* a8p = dq ? static_cast<const void*>(Wt.absmax8) : static_cast<const void*>(Wt.absmax32);
  const void* sgp = dq ? static_cast<const void*>(Wt.scale2) : static_cast<const void*>(Wt.absmax32);
  uint32_t a16[kAPairs];
  float sg0[kAPairs], sg1[kAPairs];
  const uint32_t arow = __umul24((uint32_t)nrow, (uint32_t)nblk);  // first block of this lane's row
  auto load_a = [&](int base) {
#pragma unroll
    for (int k = 0; k < kAPairs; ++k) {
      int s = wave + W * (base + grp + 4 * k);
      if (s >= nsteps) s = 0;                    // past the row: any valid step (not used)
      const uint32_t b = arow + 2u * (uint32_t)s;  // blocks 2s, 2s+1 share a DQ group (256 is even)
      a16[k] = *reinterpret_cast<const uint16_t*>(static_cast<const char*>(a8p) + b);
      const uint32_t so = dq ? (b >> 8) * 4u : b * 4u;
      sg0[k] = *reinterpret_cast<const float*>(static_cast<const char*>(sgp) + so);
      sg1[k] = *reinterpret_cast<const float*>(static_cast<const char*>(sgp) + so + (dq ? 0u : 4u));
    }
  };
  load_a(0);
  const float mu = *reinterpret_cast<const float*>(dq ? static_cast<const void*>(Wt.mean) : sgp) * (dq ? 1.0f : 0.0f);
  // X chunks of 8 (staged path), row-major: chunk c is bytes 16c .. 16c+16 of X
  constexpr int kXPer = 4;                       // the launcher stages X only when M K / 8 <= kXPer threads
  const int xchunks = XL ? M * (K / 8) : 0;
  u32x4_t xv[kXPer];
  if constexpr (XL) {
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      int c = tid + u * kThreads;
      if (c > xchunks - 1) c = xchunks - 1;      // past the staged rows: a repeated chunk (not stored)
      xv[u] = ld16(X, 16u * (uint32_t)c);
    }
  }
  // codes (and X fragments) of this wave's first D steps
  const uint32_t crow = __umul24((uint32_t)nrow, (uint32_t)(K >> 1)) + 16u * (uint32_t)grp;
  const int kb = 32 * (grp & 1) + 16 * (grp >> 1);  // k-offset in a block of this lane's 16 codes (see compute)
  const uint32_t xrow = (__umul24((uint32_t)xm, (uint32_t)K) + (uint32_t)kb) * 2u;
  auto load = [&](int i, GlSlot<D, XL>& sl) {
    int s = wave + W * i;
    if (s >= nsteps) s = wave < nsteps ? wave : 0;  // past the row: any valid step (not computed)
    sl.c = ld16(Wt.codes, crow + 64u * (uint32_t)s);
    if constexpr (!XL) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int h = 0; h < 2; ++h) sl.x[b][h] = ld16(X, xrow + 2u * (uint32_t)(128 * s + 64 * b + 8 * h));
    }
  };
  GlSlot<D, XL> ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, ring[d]);
  // keep every use of the loaded values below the last load, so that no wait
  // for an early load delays the issue of the code loads (the empty asm
  // statements after the table build take the loaded registers, and no memory
  // access moves across them)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");

  // ---- tables in LDS ----
  const uint32_t lane4 = (uint32_t)(lane & 31) << 2;
  if (tid < 256) {  // entry tid: the pair (low nibble, high nibble), 32 copies
    // lane j of qv holds bf16(q[j]) (written from the scalar arguments; no
    // indexed access to the argument segment), then two cross-lane reads
    uint32_t qv = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t u = __float_as_uint(tab.q[j]);       // finite: round to nearest even in scalar integer ops
      const uint32_t b = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(qv) : "s"(b), "i"(j));
    }
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute((tid & 15) << 2, (int)qv);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((tid >> 4) << 2, (int)qv);
    const uint32_t v = (lo & 0xFFFFu) | (hi << 16);
    const u32x4_t v4 = {v, v, v, v};
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(gl_smem + (uint32_t)tid * (kLutCopies * 4u));
#pragma unroll
    for (int q = 0; q < kLutCopies / 4; ++q) dst[q] = v4;
  }
#pragma unroll
  for (int c = 0; c < kLoraChunks; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(la[c][e]) :: "memory");
    if constexpr (FT == 0) asm volatile("" : "+v"(lb[c]) :: "memory");
  }
#pragma unroll
  for (int k = 0; k < kAPairs; ++k) asm volatile("" : "+v"(a16[k]), "+v"(sg0[k]), "+v"(sg1[k]) :: "memory");
  if constexpr (XL) {
#pragma unroll
    for (int u = 0; u < kXPer; ++u) asm volatile("" : "+v"(xv[u]) :: "memory");
  }
  if (wave == 0) {  // packed LoRA fragments, read back by the same lanes after the K loop
    u32x4_t* lp = reinterpret_cast<u32x4_t*>(gl_smem + L.lora_off) + lane;
#pragma unroll
    for (int c = 0; c < kLoraChunks; ++c) {
      const bool in = 32 * c + 8 * grp < r;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      const u32x4_t a = {la[c][0] | (la[c][1] << 16), la[c][2] | (la[c][3] << 16), la[c][4] | (la[c][5] << 16),
                         la[c][6] | (la[c][7] << 16)};
      lp[c * 64] = in ? a : z;
      if constexpr (FT == 0) lp[128 + c * 64] = in ? lb[c] : z;
    }
  }
  if constexpr (XL) {  // the staged X rows (the launcher keeps them within one round of loads)
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int c = tid + u * kThreads;
      if (c < xchunks) *reinterpret_cast<u32x4_t*>(gl_smem + L.x_off + 16u * (uint32_t)c) = xv[u];
    }
  }
  // this wave's a' ring: [slot][block][16 rows]; written and read by this wave only
  float* aw = reinterpret_cast<float*>(gl_smem + L.a_off + (uint32_t)wave * (D * 128u));
  auto store_a = [&]() {
#pragma unroll
    for (int k = 0; k < kAPairs; ++k) {
      const int slot = grp + 4 * k;
      aw[(slot * 2 + 0) * 16 + row] = dq ? block_scale(a16[k] & 0xFFu, sg0[k], mu) : sg0[k];
      aw[(slot * 2 + 1) * 16 + row] = dq ? block_scale((a16[k] >> 8) & 0xFFu, sg1[k], mu) : sg1[k];
    }
  };
  if constexpr (FT > 0) {  // this wave's slices, summed in ascending order, for wave 0 after the K loop
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      f32x4_t v = pz[f];
#pragma unroll
      for (int i = 1; i < kSl; ++i)
        if (wave + W * i < ft.Z) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += pz[i * FT + f][e];
        }
      const int q = 4 * (64 * f + lane);
      if (q < mr && wave < ft.Z) *reinterpret_cast<f32x4_t*>(gl_smem + L.q_off + (uint32_t)(wave * mr + q) * 4u) = v;
    }
  }
  store_a();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // table and X visible; code loads stay in flight

  // ---- K loop ----
  auto lut = [&](uint32_t w, int t) -> uint32_t {
    const uint32_t sh = t == 0 ? (w << 7) : (w >> (8 * t - 7));
    return *reinterpret_cast<const uint32_t*>(gl_smem + ((sh & 0x7F80u) | lane4));
  };
  f32x4_t acc = zero4;
  auto compute = [&](int i, const GlSlot<D, XL>& sl) {  // K % 128 == 0: both blocks of a step are in the row
    const int s = wave + W * i;
    // Lanes 0-31 loaded block 0 of the step (k 0-31 in lanes 0-15, k 32-63 in
    // lanes 16-31), lanes 32-63 block 1. Swapping dwords 0,1 of the upper half
    // with dwords 2,3 of the lower half leaves every lane with 16 codes of each
    // block: lane group g holds k kb(g) .. kb(g)+16, kb = 0, 32, 16, 48.
    const auto p02 = __builtin_amdgcn_permlane32_swap(sl.c.x, sl.c.z, false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap(sl.c.y, sl.c.w, false, false);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int blk = 2 * s + b;
      const u32x2_t cw = {b == 0 ? p02[0] : p02[1], b == 0 ? p13[0] : p13[1]};
      const u32x4_t a0 = {lut(cw.x, 0), lut(cw.x, 1), lut(cw.x, 2), lut(cw.x, 3)};
      const u32x4_t a1 = {lut(cw.y, 0), lut(cw.y, 1), lut(cw.y, 2), lut(cw.y, 3)};
      u32x4_t x0, x1;
      if constexpr (XL) {
        const unsigned char* xp = gl_smem + L.x_off + (uint32_t)xm * L.xpitch + (uint32_t)(64 * blk + kb) * 2u;
        x0 = *reinterpret_cast<const u32x4_t*>(xp);
        x1 = *reinterpret_cast<const u32x4_t*>(xp + 16);
      } else {
        x0 = sl.x[b][0];
        x1 = sl.x[b][1];
      }
      f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                          __builtin_bit_cast(bf16x8_t, x0), zero4, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), __builtin_bit_cast(bf16x8_t, x1),
                                                  p, 0, 0, 0);
      // register q of lane l is row 4 (l/16) + q of the tile
      const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(aw + ((i % D) * 2 + b) * 16 + 4 * grp);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(s4[q], p[q], acc[q]);
    }
  };
  // full rounds (one basic block each, so the waits stay exact), then the last
  int base = 0;
  for (; base + D < mysteps; base += D) {
    load_a(base + D);  // the next round's block constants, ahead of its code loads
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(base + d, ring[d]);
      load(base + D + d, ring[d]);
      __builtin_amdgcn_sched_barrier(0);  // slot by slot: each waits only for its own loads
    }
    store_a();  // this round's constants are consumed
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (base + d < mysteps) compute(base + d, ring[d]);

  // ---- LoRA term (wave 0): acc += sum_j L2[j][n] sT[m][j] ----
  if (wave == 0) {
    const u32x4_t* lp = reinterpret_cast<const u32x4_t*>(gl_smem + L.lora_off) + lane;
#pragma unroll
    for (int c = 0; c < kLoraChunks; ++c) {
      if (32 * c < rp) {
        u32x4_t b;
        if constexpr (FT > 0) {  // T[m][j0 .. j0+8] = the waves' sums added in order; B = bf16(s T)
          const int j0 = 32 * c + 8 * grp;
          const bool in = j0 < r;
          const int nw = ft.Z < W ? ft.Z : W;
          float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
          const unsigned char* qp = gl_smem + L.q_off + (uint32_t)(xm * r + (in ? j0 : 0)) * 4u;
          for (int w = 0; w < nw; ++w) {
            const f32x4_t t0 = *reinterpret_cast<const f32x4_t*>(qp + (uint32_t)(w * mr) * 4u);
            const f32x4_t t1 = *reinterpret_cast<const f32x4_t*>(qp + (uint32_t)(w * mr) * 4u + 16u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] += t0[e];
              v[4 + e] += t1[e];
            }
          }
          uint32_t h[8], t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            h[e] = f32_to_bf16(ft.s * v[e]);
            t[e] = f32_to_bf16(v[e]);
          }
          const u32x4_t zb = {0u, 0u, 0u, 0u};
          const u32x4_t hb = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
          b = in ? hb : zb;
          if (ft.T_out != nullptr && blockIdx.x == 0 && row < M && in) {
            const u32x4_t tb = {t[0] | (t[1] << 16), t[2] | (t[3] << 16), t[4] | (t[5] << 16), t[6] | (t[7] << 16)};
            *reinterpret_cast<u32x4_t*>(ft.T_out + row * r + j0) = tb;
          }
        } else {
          b = lp[128 + c * 64];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lp[c * 64]),
                                                       __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
      }
    }
    for (int j0 = 32 * kLoraChunks; j0 < rp; j0 += 32) {  // ranks above 64
      const int jj = j0 + 8 * grp;
      const bool in = jj < r;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      u32x4_t b = {0u, 0u, 0u, 0u};
      if (in) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)L2[(int64_t)(jj + 2 * e) * N + nrow] | ((uint32_t)L2[(int64_t)(jj + 2 * e + 1) * N + nrow] << 16);
        b = *reinterpret_cast<const u32x4_t*>(sT + (int64_t)xm * ldst + jj);
      }
      const u32x4_t a = {w[0], w[1], w[2], w[3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                     acc, 0, 0, 0);
    }
  }

  // ---- fixed-order sum of the waves' partials ----
  float* red = reinterpret_cast<float*>(gl_smem);   // reuses the table
  __syncthreads();
  // acc register q of lane l: Y[m = l%16][n0 + 4 (l/16) + q]
#pragma unroll
  for (int q = 0; q < 4; ++q) red[wave * 256 + (4 * grp + q) * 16 + row] = acc[q];
  __syncthreads();
  if (tid < 256) {
    const int nr = tid / 16, m = tid % 16;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += red[w * 256 + nr * 16 + m];
    const int64_t ny = n0 + nr;
    if (m < M && ny < N) Y[(int64_t)m * N + ny] = f32_to_bf16(v);
  }
}

template <int W, int D, bool XL, int FT>
hipError_t launch_lut(const NF4View& Wt, const NF4Table& tab, const uint16_t* X, int M, const uint16_t* sT,
                      const uint16_t* L2, int r, uint16_t* Y, const FuseT& ft, int64_t tiles, uint32_t lds,
                      hipStream_t stream) {
  static bool attr_set = false;  // raise the dynamic-LDS limit once per instantiation (idempotent)
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_lut_kernel<W, D, XL, FT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGvMaxLds);
    (void)hipGetLastError();  // a refusal shows up as a launch error below
    attr_set = true;
  }
  hipLaunchKernelGGL((gemv_lut_kernel<W, D, XL, FT>), dim3((unsigned)tiles), dim3(64 * W), lds, stream, Wt, tab, X, M,
                     sT, r, L2, r, Y, ft);
  return hipGetLastError();
}

// The byte-table kernel's configuration for a shape: every workgroup of the
// launch resident at once (LDS budget per workgroup = LDS per CU / workgroups
// per CU), 4 waves when a CU holds three or more workgroups, else 8; X staged
// in LDS when it fits. With fusion asked for, the adapter's slice partials
// are summed in the kernel (fuse = F of the fused variant) when r <= 64,
// M r <= 256 F (F = 1, or 4 with 8-wave workgroups), each wave has at most
// ft_slices(F) slices and their per-wave sums fit the same budget. waves == 0: the kernel does not
// apply.
struct LutPlan {
  int waves = 0;
  bool xl = false;
  int fuse = 0;
  uint32_t lds = 0;
};

// the small-M LoRA down projection's slices (its kernels are below)
constexpr int kTsWaves = 16;
constexpr int kTsRows = 32;                  // L1 rows per wave
constexpr int kTsK = kTsWaves * kTsRows;     // k per slice

LutPlan lut_plan(const NF4View& W, int64_t M, int r, bool want_fuse) {
  LutPlan p;
  const int64_t N = W.rows, K = W.cols;
  const int64_t tiles = (N + kGvRows - 1) / kGvRows;
  const bool fits32 = N < (1 << 24) && K < (1 << 24) && N * K / 2 < ((int64_t)1 << 32) &&
                      M * K * 2 < ((int64_t)1 << 32) && (int64_t)r * N * 2 < ((int64_t)1 << 32);
  if (K % 128 != 0 || !fits32) return p;  // 32-bit byte offsets and 24-bit products in the kernel
  static int cus = 0;  // compute units of the device (the same on every device this library runs on)
  if (cus <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cus = n;
    (void)hipGetLastError();
    if (cus <= 0) cus = 256;
  }
  int64_t per_cu = (tiles + cus - 1) / cus;
  if (per_cu > 4) per_cu = 4;
  const uint32_t budget = (uint32_t)(160 * 1024 / per_cu) - 1024u;
  const int waves = per_cu >= 3 ? 4 : 8;
  const int m = (int)M;
  const int64_t xchunks = M * K / 8;   // X staged by one round of kXPer (4) loads per thread
  const GlLayout xl = gl_layout(K, waves, 4, m, 0u), xr = gl_layout(K, waves, 4, 0, 0u);
  if (xl.total <= budget && xchunks <= 4 * 64 * waves) p.xl = true;
  else if (xr.total > budget) return p;
  p.waves = waves;
  p.lds = p.xl ? xl.total : xr.total;
  const int64_t Z = (K + kTsK - 1) / kTsK;
  // four chunks per lane only with one workgroup per CU: with 4-wave
  // workgroups (more tiles than two per CU) their longer prologue cost more
  // than the separate reduction saves (LLaMA-7B 4096 -> 11008, M = 16: 26.0
  // against 25.6 us per call; 11008 -> 4096: 22.9 against 25.5)
  const int F = M * r <= 256 ? 1 : (M * r <= 1024 && waves == 8) ? 4 : 0;
  if (want_fuse && r <= 64 && F > 0 && Z <= (int64_t)ft_slices(F) * waves) {
    const uint32_t lf = gl_layout(K, waves, 4, p.xl ? m : 0, (uint32_t)(waves * m * r) * 4u).total;
    if (lf <= budget) {
      p.fuse = F;
      p.lds = lf;
    }
  }
  return p;
}

// ---- small-M LoRA down projection -------------------------------------------
//
// T = X L1 for M <= 128 rows, in two short kernels:
//   * partial sums over k-slices of 512: one workgroup of 16 waves per slice,
//     64 columns and 16 rows of X (blockIdx.z); wave w multiplies its 32 rows of the slice with
//     v_mfma_f32_16x16x32_bf16 (A = the rows of X, B = the columns of L1,
//     zero rows beyond M), and the 16 waves' sums are added in a fixed order
//     through LDS;
//   * a fixed-order sum over the (K/512) slices that writes bf16(s T)
//     for the second adapter product, and bf16(T) when asked.


__global__ __launch_bounds__(64 * kTsWaves) void small_t_partial_kernel(const uint16_t* __restrict__ X, int M,
                                                                        int64_t K, const uint16_t* __restrict__ L1,
                                                                        int r, float* __restrict__ P) {
  // wave w: the 32 rows kw .. kw+32 of the slice, 4 MFMA column tiles of 16;
  // A = X rows (lane l: row l%16, k 8 (l/16) .. +8), B = L1 columns (lane l:
  // column l%16 of the tile, the same 8 k)
  __shared__ float red[kTsWaves][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t kw = (int64_t)blockIdx.x * kTsK + wave * kTsRows + 8 * (lane >> 4);
  const int row = lane & 15;
  const int j0 = blockIdx.y * 64;
  const int mb = blockIdx.z * 16;   // this workgroup's 16 rows of X
  u32x4_t xa = {0u, 0u, 0u, 0u};
  if (mb + row < M && kw < K) xa = *reinterpret_cast<const u32x4_t*>(X + (int64_t)(mb + row) * K + kw);  // K % 64 == 0
  uint32_t h[4][8];  // all 32 loads first (one round trip)
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const int j = j0 + 16 * jt + row;
    const bool in = j < r && kw < K;
    const uint16_t* lp = L1 + (in ? kw * r + j : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) h[jt][i] = lp[in ? (int64_t)i * r : 0];
    if (!in) {
#pragma unroll
      for (int i = 0; i < 8; ++i) h[jt][i] = 0u;
    }
  }
  f32x4_t acc[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const u32x4_t b = {h[jt][0] | (h[jt][1] << 16), h[jt][2] | (h[jt][3] << 16), h[jt][4] | (h[jt][5] << 16),
                       h[jt][6] | (h[jt][7] << 16)};
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa), __builtin_bit_cast(bf16x8_t, b),
                                                       zero, 0, 0, 0);
  }
  // acc[jt] register i of lane l: T[m = mb + 4 (l/16) + i][j = j0 + 16 jt + l%16]
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][16 * jt + row] = acc[jt][i];
  __syncthreads();
  const int m = wave;  // thread (m, lane) of the first 16 waves sums the waves in order
  float v = 0.0f;
#pragma unroll
  for (int w = 0; w < kTsWaves; ++w) v += red[w][m][lane];
  if (mb + m < M && j0 + lane < r) P[((int64_t)blockIdx.x * M + mb + m) * r + j0 + lane] = v;
}

__global__ __launch_bounds__(256) void small_t_reduce_kernel(const float* __restrict__ P, int Z, int M, int r, float s,
                                                             uint16_t* __restrict__ sT, int64_t ldst,
                                                             uint16_t* __restrict__ T_out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * r) return;
  float v = 0.0f;
  int z = 0;
  for (; z + 8 <= Z; z += 8) {  // loads of 8 slices in flight, added in order
    float p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = P[(int64_t)(z + u) * M * r + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += p[u];
  }
  for (; z < Z; ++z) v += P[(int64_t)z * M * r + i];
  const int m = i / r, j = i % r;
  sT[(int64_t)m * ldst + j] = f32_to_bf16(s * v);
  if (T_out) T_out[(int64_t)m * r + j] = f32_to_bf16(v);
}

}  // namespace

size_t small_t_partial_bytes(int64_t M, int64_t K, int r) {
  return (size_t)((K + kTsK - 1) / kTsK) * (size_t)M * (size_t)r * 4;
}

int small_t_slices(int64_t K) { return (int)((K + kTsK - 1) / kTsK); }

hipError_t launch_small_t_partial(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, float* part,
                                  hipStream_t stream) {
  if (M < 1 || M > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(small_t_partial_kernel,
                     dim3((unsigned)small_t_slices(K), (unsigned)((r + 63) / 64), (unsigned)((M + 15) / 16)),
                     dim3(64 * kTsWaves), 0, stream, X, (int)M, K, L1, r, part);
  return hipGetLastError();
}

hipError_t launch_small_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, float s,
                                  uint16_t* sT, int64_t ldst, uint16_t* T_out, float* part, hipStream_t stream) {
  hipError_t e = launch_small_t_partial(X, M, K, L1, r, part, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(small_t_reduce_kernel, dim3((unsigned)((M * r + 255) / 256)), dim3(256), 0, stream, part,
                     small_t_slices(K), (int)M, r, s, sT, ldst, T_out);
  return hipGetLastError();
}

bool gemv_fuses_t(const NF4View& W, int64_t M, int r) {
  return M >= 1 && M <= 16 && r <= kGvMaxRank && W.cols % kBlock == 0 && lut_plan(W, M, r, true).fuse > 0;
}

static hipError_t launch_gemv_impl(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M,
                                   const uint16_t* sT, const uint16_t* L2, int r, uint16_t* Y, const FuseT* ft,
                                   hipStream_t stream) {
  if (M < 1 || M > 16 || r > kGvMaxRank || (W.cols % kBlock) != 0) return hipErrorInvalidValue;
  const int64_t N = W.rows, K = W.cols;
  const int64_t tiles = (N + kGvRows - 1) / kGvRows;
  const int m = (int)M;
  const LutPlan p = lut_plan(W, M, r, ft != nullptr);
  if (ft != nullptr && p.fuse == 0) return hipErrorInvalidValue;  // callers ask gemv_fuses_t first
  if (p.waves > 0) {
    const FuseT f = ft ? *ft : FuseT{nullptr, 0, 0.0f, nullptr};
    const int F = ft ? p.fuse : 0;
    auto go = [&](auto w, auto xl) -> hipError_t {
      constexpr int kW = decltype(w)::value;
      constexpr bool kXL = decltype(xl)::value;
      if (F == 1) return launch_lut<kW, 4, kXL, 1>(W, tab, X, m, sT, L2, r, Y, f, tiles, p.lds, stream);
      if (F == 4) return launch_lut<kW, 4, kXL, 4>(W, tab, X, m, sT, L2, r, Y, f, tiles, p.lds, stream);
      return launch_lut<kW, 4, kXL, 0>(W, tab, X, m, sT, L2, r, Y, f, tiles, p.lds, stream);
    };
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    using T = std::true_type;
    using Fa = std::false_type;
    if (p.waves == 4) return p.xl ? go(I4{}, T{}) : go(I4{}, Fa{});
    return p.xl ? go(I8{}, T{}) : go(I8{}, Fa{});
  }
  // streamed kernel (double quantisation only): 4 waves when there are
  // enough row tiles for two or more workgroups per CU, else 8
  if (W.absmax32 == nullptr && K >= 128 && K <= 32768 && N * K / 2 < ((int64_t)1 << 32)) {
    hipError_t e = hipSuccess;
    bool done;
    if (tiles >= 512)
      done = m <= 1   ? launch_streamed<4, 1, 8>(W, tab, X, m, sT, L2, r, Y, tiles, stream, &e)
             : m <= 4 ? launch_streamed<4, 4, 5>(W, tab, X, m, sT, L2, r, Y, tiles, stream, &e)
                      : launch_streamed<4, 16, 2>(W, tab, X, m, sT, L2, r, Y, tiles, stream, &e);
    else
      done = m <= 1   ? launch_streamed<8, 1, 8>(W, tab, X, m, sT, L2, r, Y, tiles, stream, &e)
             : m <= 4 ? launch_streamed<8, 4, 6>(W, tab, X, m, sT, L2, r, Y, tiles, stream, &e)
                      : launch_streamed<8, 16, 3>(W, tab, X, m, sT, L2, r, Y, tiles, stream, &e);
    if (done) return e;
  }
  // register-ring kernel: short rows, very long rows, or layouts beyond the LDS
  if (tiles >= 512)
    hipLaunchKernelGGL(gemv_ring_kernel<4>, dim3((unsigned)tiles), dim3(256), 0, stream, W, tab, X, m, sT, r, L2, r, Y);
  else
    hipLaunchKernelGGL(gemv_ring_kernel<8>, dim3((unsigned)tiles), dim3(512), 0, stream, W, tab, X, m, sT, r, L2, r, Y);
  return hipGetLastError();
}

hipError_t launch_gemv(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M,
                       const uint16_t* sT, const uint16_t* L2, int r, uint16_t* Y, hipStream_t stream) {
  return launch_gemv_impl(W, tab, X, M, sT, L2, r, Y, nullptr, stream);
}

hipError_t launch_gemv_fused_t(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M,
                               const float* part, int Z, float s, uint16_t* T_out, const uint16_t* L2, int r,
                               uint16_t* Y, hipStream_t stream) {
  const FuseT ft{part, Z, s, T_out};
  return launch_gemv_impl(W, tab, X, M, nullptr, L2, r, Y, &ft, stream);
}

}  // namespace qlora
