// Skinny adapter products of the QLoRA linear on gfx950 (rank r <= 64):
//
//   forward   T   = X L1           [M][r]   (reduction over K)
//   backward  U   = dY L2^T        [M][r]   (reduction over N)
//             dL1 = s X^T U        [K][r]   (reduction over the M tokens)
//             dL2 = s (X L1)^T dY  [r][N]   (reduction over the M tokens)
//
// (QLoRA pages, diycv.top, section 问题背景 LoRA equation and section
// 关键公式.) Each product reads one large activation (X or dY, 64-180 MB at
// 8192 tokens) once and a small rank-r operand, so it is HBM-bound; the
// kernels stream the large operand with coalesced 16-byte loads, keep the
// whole rank dimension (padded to 64) in one tile, and use
// v_mfma_f32_32x32x16_bf16 for the products. The reduction is split over
// blockIdx.z into fp32 partials that skinny_reduce_kernel sums in a fixed
// order, so results are deterministic.
//
// skinny_nt_kernel:  C[z][m][j] = sum_{k in slice z} A[m][k] B[j][k]
//   A [M][K] and B [64][K] (rows j >= r are zero) are both K-contiguous and
//   are copied global -> LDS by global_load_lds_dwordx4; 128 rows x 64 j per
//   workgroup, 4 waves of 32 rows, K-stages of 64, 3-stage ring. With LoRA
//   dropout (DROP) A is the adapter input X, and every A fragment is
//   dropped in registers after its LDS read (each A element is read by
//   exactly one lane), from the Philox words of its element indices.
// skinny_tn_dma_kernel:  C[z][c][j] = sum_{m in slice z} L[m][c] S[m][j]
//   the reduction runs down the rows of both operands; both are copied
//   global -> LDS in their memory layout into a 3-stage ring, and the MFMA
//   fragments (consecutive m of one column) are read with the LDS transpose
//   read; 128 columns c x 64 j per workgroup, M-stages of 64.
// skinny_tn_kernel<true>:  the same product with LoRA dropout on the large
//   operand (the adapter input X): each thread loads two rows x 8 columns,
//   drops them in registers from the Philox words of their element indices
//   m W + c, and writes them to LDS transposed as (m, m+1) pairs, so the
//   dropped copy of X is never written to memory.
#include "common.h"
#include "launch.h"
#include "philox.h"

namespace qlora {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

constexpr int SK = 64;     // reduction per stage (elements)
constexpr int SJ = 64;     // rank columns per tile (r padded)
constexpr int SM = 128;    // large-operand rows (nt) or columns (tn) per tile
constexpr int kSkThreads = 256;

// 16-byte chunk c of LDS row `row` lives at c ^ sk_swz(row): (row >> 1) keeps
// the fragment reads of 16 consecutive rows on distinct bank groups, and
// (row >> 4) separates the rows that 8 neighbouring threads write at the
// same reduction index when a tile is transposed into LDS.
__device__ __forceinline__ int sk_swz(int row) { return ((row >> 1) ^ (row >> 4)) & 7; }
__device__ __forceinline__ int sk_off(int row, int chunk) { return row * SK + ((chunk ^ sk_swz(row)) << 3); }

// ---- NT: both operands contiguous in the reduction -----------------------------

constexpr int kNtStages = 3;

struct NtArgs {
  const uint16_t* A;  // [M][lda]
  const uint16_t* B;  // [SJ][ldb]  (64 rows; rows >= r zero)
  float* C;           // [Z][M][SJ]
  int64_t lda, ldb, M, K, k_split;
  uint32_t thr;       // DROP: keep iff the element's Philox word >= thr; kept values scaled by c
  float c;
  uint64_t seed;
};

template <bool DROP>
__global__ __launch_bounds__(kSkThreads) void skinny_nt_kernel(NtArgs p) {
  __shared__ __attribute__((aligned(1024))) uint16_t sA[kNtStages][SM * SK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB[kNtStages][SJ * SK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * SM;
  const int64_t kz0 = (int64_t)blockIdx.z * p.k_split;
  const int64_t kz1 = (kz0 + p.k_split < p.K) ? kz0 + p.k_split : p.K;
  const int nk = kz0 < kz1 ? (int)((kz1 - kz0) / SK) : 0;

  // per-lane 32-bit offsets of the direct-to-LDS copies (8 rows x 128 B per instruction)
  const int lr = lane >> 3;
  uint32_t offA[4], offB[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // A: 128 rows = 16 instructions, 4 per wave
    const int rloc = (wave * 4 + j) * 8 + lr;
    int64_t r = m0 + rloc;
    if (r > p.M - 1) r = p.M - 1;
    offA[j] = (uint32_t)((r * p.lda + (((lane & 7) ^ sk_swz(rloc)) * 8)) * 2);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // B: 64 rows = 8 instructions, 2 per wave
    const int rloc = (wave * 2 + j) * 8 + lr;
    offB[j] = (uint32_t)((rloc * p.ldb + (((lane & 7) ^ sk_swz(rloc)) * 8)) * 2);
  }
  // The copies are issued from inline assembly (uniform base in SGPRs, the
  // lane's offset in a VGPR): with the compiler builtin for them, the
  // generated code waited for every copy in flight, the next stages'
  // included, before the first LDS read of each stage, so no copy overlapped
  // the MFMAs. The explicit vmcnt before each stage's barrier is the only
  // wait on them.
  auto copy = [&](const char* base, uint32_t off, const uint16_t* lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
  };
  auto issue = [&](int st, int buf) {
    const int64_t k0 = kz0 + (int64_t)st * SK;
    const char* a = reinterpret_cast<const char*>(p.A + k0);
    const char* b = reinterpret_cast<const char*>(p.B + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) copy(a, offA[j], sA[buf] + (wave * 4 + j) * 8 * SK);
#pragma unroll
    for (int j = 0; j < 2; ++j) copy(b, offB[j], sB[buf] + (wave * 2 + j) * 8 * SK);
  };

  f32x16_t acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;

#pragma unroll
  for (int s = 0; s < kNtStages - 1; ++s)
    if (s < nk) issue(s, s);
  for (int st = 0; st < nk; ++st) {
    const int buf = st % kNtStages;
    if (st + 1 < nk) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");  // stage st+1 (6 loads) may stay in flight
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st + kNtStages - 1 < nk) issue(st + kNtStages - 1, (st + kNtStages - 1) % kNtStages);
#pragma unroll
    for (int kk = 0; kk < SK / 16; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sA[buf] + sk_off(wave * 32 + (lane & 31), ch));
      if constexpr (DROP) {
        // element indices of the 8 values: row m of X (row length lda), columns k .. k+7
        const int64_t e0 = (m0 + wave * 32 + (lane & 31)) * p.lda + kz0 + (int64_t)st * SK + ch * 8;
        const u32x4_t u0 = philox_block(e0 >> 2, p.seed), u1 = philox_block((e0 >> 2) + 1, p.seed);
        const u32x4_t v = __builtin_bit_cast(u32x4_t, a);
        a = __builtin_bit_cast(bf16x8_t, u32x4_t{dropout_pair(v.x, u0.x, u0.y, p.thr, p.c),
                                                 dropout_pair(v.y, u0.z, u0.w, p.thr, p.c),
                                                 dropout_pair(v.z, u1.x, u1.y, p.thr, p.c),
                                                 dropout_pair(v.w, u1.z, u1.w, p.thr, p.c)});
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(sB[buf] + sk_off(t * 32 + (lane & 31), ch));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
  }
  // C[z][m][j]: lane l, register v -> row (v%4) + 4(l/32) + 8(v/4), column l%32
  float* Cz = p.C + (int64_t)blockIdx.z * p.M * SJ;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = t * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = m0 + wave * 32 + (v & 3) + 4 * (lane >> 5) + 8 * (v >> 2);
      if (m < p.M) Cz[m * SJ + j] = acc[t][v];
    }
  }
}

// ---- TN: both operands run the reduction down their rows ----------------------------

struct TnArgs {
  const uint16_t* L;  // [M][ldl]  large operand (X or dY)
  const uint16_t* S;  // [M][lds]  small operand (U or T), r columns valid
  float* C;           // [Z][W][SJ]
  int64_t ldl, lds, M, W, r, m_split;
  uint32_t thr;       // DROP: keep iff the element's Philox word >= thr; kept values scaled by c
  float c;
  uint64_t seed;
};

template <bool DROP>
__global__ __launch_bounds__(kSkThreads) void skinny_tn_kernel(TnArgs p) {
  __shared__ __attribute__((aligned(1024))) uint16_t sL[SM * SK];  // [c][m]
  __shared__ __attribute__((aligned(1024))) uint16_t sS[SJ * SK];  // [j][m]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * SM;
  const int64_t mz0 = (int64_t)blockIdx.z * p.m_split;
  const int64_t mz1 = (mz0 + p.m_split < p.M) ? mz0 + p.m_split : p.M;

  // staging roles: L tile = 64 rows x 128 columns -> thread: row pair rp, two 8-column chunks
  const int l_cq = tid & 7, l_rp = tid >> 3;              // 8 threads per row pair, 32 row pairs
  // S tile = 64 rows x 64 columns -> thread: row pair, one 8-column chunk (first 256 threads)
  const int s_cq = tid & 7, s_rp = tid >> 3;

  f32x16_t acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;

  u32x4_t lv[2][2], sv[2];
  auto load = [&](int64_t ms) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t m = ms + 2 * l_rp + h;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t c = c0 + (l_cq * 2 + q) * 8;
        lv[h][q] = (m < mz1 && c < p.W) ? *reinterpret_cast<const u32x4_t*>(p.L + m * p.ldl + c)
                                        : u32x4_t{0, 0, 0, 0};
      }
      const int64_t cs = s_cq * 8;
      sv[h] = (m < mz1 && cs < p.r) ? *reinterpret_cast<const u32x4_t*>(p.S + m * p.lds + cs) : u32x4_t{0, 0, 0, 0};
    }
  };
  // write (m, m+1) pairs of column c as one dword at [c][m]
  auto put_pairs = [&](uint16_t* T, int cbase, const u32x4_t& r0, const u32x4_t& r1, int mloc) {
    const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
    const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xFFFFu);
      const uint32_t b = (e & 1) ? (w1[e >> 1] >> 16) : (w1[e >> 1] & 0xFFFFu);
      const int row = cbase + e;
      *reinterpret_cast<uint32_t*>(T + sk_off(row, mloc >> 3) + (mloc & 7)) = a | (b << 16);
    }
  };

  // DROP: the staged rows of L (row-major [M][W], W % 64 == 0) after dropout;
  // out-of-range values were loaded as 0 and stay 0
  auto drop = [&](int64_t ms) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t m = ms + 2 * l_rp + h;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t e0 = m * p.W + c0 + (l_cq * 2 + q) * 8;  // multiple of 8: two Philox blocks
        const u32x4_t u0 = philox_block(e0 >> 2, p.seed), u1 = philox_block((e0 >> 2) + 1, p.seed);
        u32x4_t& v = lv[h][q];
        v = u32x4_t{dropout_pair(v.x, u0.x, u0.y, p.thr, p.c), dropout_pair(v.y, u0.z, u0.w, p.thr, p.c),
                    dropout_pair(v.z, u1.x, u1.y, p.thr, p.c), dropout_pair(v.w, u1.z, u1.w, p.thr, p.c)};
      }
    }
  };

  if (mz0 < mz1) load(mz0);
  for (int64_t ms = mz0; ms < mz1; ms += SK) {
    __syncthreads();  // previous stage's fragment reads are done
    if constexpr (DROP) drop(ms);
    const int mloc = 2 * l_rp;
#pragma unroll
    for (int q = 0; q < 2; ++q) put_pairs(sL, (l_cq * 2 + q) * 8, lv[0][q], lv[1][q], mloc);
    put_pairs(sS, s_cq * 8, sv[0], sv[1], 2 * s_rp);
    __syncthreads();
    if (ms + SK < mz1) load(ms + SK);  // next stage's global loads overlap the MFMAs
#pragma unroll
    for (int kk = 0; kk < SK / 16; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sL + sk_off(wave * 32 + (lane & 31), ch));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(sS + sk_off(t * 32 + (lane & 31), ch));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
  }
  float* Cz = p.C + (int64_t)blockIdx.z * p.W * SJ;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = t * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t c = c0 + wave * 32 + (v & 3) + 4 * (lane >> 5) + 8 * (v >> 2);
      if (c < p.W) Cz[c * SJ + j] = acc[t][v];
    }
  }
}

// skinny_tn_dma_kernel: the product of skinny_tn_kernel without dropout, with both
// operands copied global -> LDS by global_load_lds_dwordx4 in their memory
// layout (rows of 128 L columns and of 64 S columns, m running down the rows)
// into a ring of kTnStages stages, so that the copies of two stages are in
// flight while a third is multiplied. The MFMA fragments (8 consecutive m of
// one column) are read with the transpose read ds_read_b64_tr_b16: in each
// group of 16 lanes, lane i receives element i % 4 of the 8 bytes that lane
// 4e + i / 4 addresses, as its element e. If lane j of the group addresses
// row m0 + j / 4, columns cb + 4 (j % 4) .. +3, lane i receives rows
// m0 .. m0 + 3 of column cb + i. Two such reads make one 8-element fragment.
// Rows outside the slice and S columns at or beyond r are copied from a
// zeroed 16-byte block, L columns at or beyond W from clamped (valid)
// addresses: their outputs are never stored. The results equal the
// register-staged kernel's bit for bit (the same MFMAs in the same order).
constexpr int kTnStages = 3;
constexpr int kTnLRow = SM * 2;                       // bytes per staged L row (128 columns)
constexpr int kTnSRow = SJ * 2;                       // bytes per staged S row (64 columns)
constexpr int kTnLBytes = SK * kTnLRow;               // 16 KB
constexpr int kTnStageBytes = kTnLBytes + SK * kTnSRow;  // 24 KB

__device__ __attribute__((aligned(16))) uint32_t g_tn_zero[4];  // zero-initialised copy source

// 16-byte chunk q of staged row m sits at chunk q ^ swz(m). L rows are 256 B
// (one row per pass of the 64 banks): the four rows that one transpose read
// of 32 lanes touches (m0 .. m0 + 3, four chunks each) land on 16 distinct
// chunk positions. S rows are 128 B (two rows per pass): rows m0 and m0 + 2
// are moved apart.
__device__ __forceinline__ int tn_lswz(int m) { return (m & 3) << 2; }
__device__ __forceinline__ int tn_sswz(int m) { return ((m >> 1) & 1) << 2; }

typedef short tn_v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ tn_v4i16 tn_read_tr(const char* lds_byte) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tn_v4i16*)(lds_void_t*)lds_byte);
}

__global__ __launch_bounds__(kSkThreads) void skinny_tn_dma_kernel(TnArgs p) {
  __shared__ __attribute__((aligned(1024))) char ring[kTnStages * kTnStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * SM;
  const int64_t mz0 = (int64_t)blockIdx.z * p.m_split;
  const int64_t mz1 = (mz0 + p.m_split < p.M) ? mz0 + p.m_split : p.M;
  const int ns = mz0 < mz1 ? (int)((mz1 - mz0 + SK - 1) / SK) : 0;
  const char* zero = reinterpret_cast<const char*>(g_tn_zero);

  // Copy roles. L: instruction i of wave w moves rows 4 (4w + i) .. +3, lane
  // -> row 4 (4w + i) + lane / 16, chunk position lane % 16. S: instruction i
  // moves rows 8 (2w + i) .. +7, lane -> row 8 (2w + i) + lane / 8, position
  // lane % 8. The column parts of the source addresses are fixed per lane.
  int64_t l_col[4], s_col[2];
  bool s_in[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (4 * wave + i) + (lane >> 4);
    int64_t c = c0 + 8 * ((lane & 15) ^ tn_lswz(row));
    if (c > p.W - 8) c = p.W - 8;  // W % 8 == 0
    l_col[i] = c;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (2 * wave + i) + (lane >> 3);
    const int j = 8 * ((lane & 7) ^ tn_sswz(row));
    s_in[i] = j < p.r;
    s_col[i] = s_in[i] ? j : 0;
  }
  auto copy = [&](const char* src, char* lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "s"(m0) : "memory", "m0");
  };
  auto issue = [&](int st) {  // the 6 copy instructions of this wave for stage st
    const int64_t ms = mz0 + (int64_t)st * SK;
    char* buf = ring + (st % kTnStages) * kTnStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (4 * wave + i) + (lane >> 4);
      const int64_t m = ms + row;
      const char* src = m < mz1 ? reinterpret_cast<const char*>(p.L + m * p.ldl + l_col[i]) : zero;
      copy(src, buf + (4 * wave + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 8 * (2 * wave + i) + (lane >> 3);
      const int64_t m = ms + row;
      const char* src = (m < mz1 && s_in[i]) ? reinterpret_cast<const char*>(p.S + m * p.lds + s_col[i]) : zero;
      copy(src, buf + kTnLBytes + (2 * wave + i) * 1024);
    }
  };

  f32x16_t acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;

  // Transpose-read addresses, relative to a stage buffer and k-step: lane j
  // of its group addresses row (lane / 32) * 8 + 4 h + j / 4 (+16 kk),
  // columns cb + 4 (j % 4) .. +3 with cb = 16 ((lane / 16) % 2) + the wave's
  // (L) or the tile's (S) first column.
  const int jl = lane & 15;
  const int rbase = 8 * (lane >> 5) + (jl >> 2);
  const int cl = wave * 32 + 16 * ((lane >> 4) & 1) + 4 * (jl & 3);  // L column (within the tile)
  const int cs = 16 * ((lane >> 4) & 1) + 4 * (jl & 3);              // S column within a 32-wide tile
  auto loff = [&](int row) { return row * kTnLRow + ((((cl >> 3) ^ tn_lswz(row))) << 4) + ((cl & 7) << 1); };
  auto soff = [&](int row, int t) {
    const int c = 32 * t + cs;
    return kTnLBytes + row * kTnSRow + (((c >> 3) ^ tn_sswz(row)) << 4) + ((c & 7) << 1);
  };

#pragma unroll
  for (int st = 0; st < kTnStages - 1; ++st)
    if (st < ns) issue(st);
  for (int st = 0; st < ns; ++st) {
    // this wave's copies of stage st are complete (those of st + 1 may not be)
    if (st + 1 < ns) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's copies of stage st are visible; stage st-1's reads are done
    if (st + kTnStages - 1 < ns) issue(st + kTnStages - 1);  // into stage st-1's buffer
    const char* buf = ring + (st % kTnStages) * kTnStageBytes;
#pragma unroll
    for (int kk = 0; kk < SK / 16; ++kk) {
      const int r0 = 16 * kk + rbase;
      const tn_v4i16 a0 = tn_read_tr(buf + loff(r0)), a1 = tn_read_tr(buf + loff(r0 + 4));
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const tn_v4i16 b0 = tn_read_tr(buf + soff(r0, t)), b1 = tn_read_tr(buf + soff(r0 + 4, t));
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
  }
  float* Cz = p.C + (int64_t)blockIdx.z * p.W * SJ;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = t * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t c = c0 + wave * 32 + (v & 3) + 4 * (lane >> 5) + 8 * (v >> 2);
      if (c < p.W) Cz[c * SJ + j] = acc[t][v];
    }
  }
}

// out = alpha * sum_z P[z] over a [rows][SJ] slab, columns j < r:
//   mode 0: out[m][j] (row stride ldo; columns [r, ldo) zero) in bf16, plus
//           optional out2[m][j] = bf16(alpha2 * sum) with row stride r
//   mode 1: out[m][j] fp32 or bf16, row stride r
// Four consecutive columns per thread (r % 8 == 0 and ldo % 4 == 0, so a
// group of four is all below r or all at or above it): 16-byte partial loads,
// the sum over z in order, 8- or 16-byte stores.
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ P, int Z, int64_t rows, int r,
                                                            float alpha, int mode, int out_bf16, void* __restrict__ out,
                                                            int64_t ldo, float alpha2, uint16_t* __restrict__ out2) {
  const int64_t width = (mode == 0) ? ldo : r;
  const int64_t w4 = width / 4;
  const int64_t total = rows * w4;
  const int64_t slab = rows * SJ;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / w4, j = (i - m * w4) * 4;
    const int64_t o = m * width + j;
    if (j >= r) {
      *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + o) = u32x2_t{0u, 0u};
      continue;
    }
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int z = 0; z < Z; ++z) acc += *reinterpret_cast<const f32x4_t*>(P + (int64_t)z * slab + m * SJ + j);
    const f32x4_t v = {alpha * acc.x, alpha * acc.y, alpha * acc.z, alpha * acc.w};
    if (out_bf16)
      *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + o) = u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    else
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + o) = v;
    if (mode == 0 && out2)
      *reinterpret_cast<u32x2_t*>(out2 + m * r + j) =
          u32x2_t{pack_bf16x2(alpha2 * acc.x, alpha2 * acc.y), pack_bf16x2(alpha2 * acc.z, alpha2 * acc.w)};
  }
}

// Transposed reduction: out[j][c] = alpha * sum_z P[z][c][j] for j < r, c < W,
// output row stride W. One workgroup per 64 columns c and 16 ranks j (so
// that even W = 4096 gives 256 workgroups): each thread sums 4 ranks of one
// column over the Z partial tiles in a fixed z order (16-byte loads), the
// 64 x 16 result is transposed through LDS, and each output row segment is
// written 4 columns per thread.
__global__ __launch_bounds__(256) void skinny_reduce_t_kernel(const float* __restrict__ P, int Z, int64_t W, int r,
                                                              float alpha, int out_bf16, void* __restrict__ out) {
  __shared__ float tile[64][16 + 1];
  const int t = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int j0 = blockIdx.y * 16;
  if (j0 >= r) return;                         // uniform per workgroup
  const int cl = t >> 2, jq = (t & 3) * 4;     // column c0 + cl, ranks j0 + jq .. +4
  const int64_t c = c0 + cl;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (c < W) {
    const int64_t slab = W * SJ;
    for (int z = 0; z < Z; ++z) acc += *reinterpret_cast<const f32x4_t*>(P + (int64_t)z * slab + c * SJ + j0 + jq);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) tile[cl][jq + e] = acc[e];
  __syncthreads();
  const int jl = t >> 4, cq = (t & 15) * 4;   // rank j0 + jl, columns c0 + cq .. +4
  const int j = j0 + jl;
  if (j < r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t cc = c0 + cq + e;
      if (cc < W) {
        const float v = alpha * tile[cq + e][jl];
        if (out_bf16) static_cast<uint16_t*>(out)[(int64_t)j * W + cc] = f32_to_bf16(v);
        else static_cast<float*>(out)[(int64_t)j * W + cc] = v;
      }
    }
  }
}

int64_t sk_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t sk_grid(int64_t total) {
  int64_t b = sk_cdiv(total, 256);
  if (b > 8192) b = 8192;
  return b < 1 ? 1 : b;
}

}  // namespace

// Number of reduction slices for a skinny product with `tiles` output tiles
// over a reduction of length klen (multiples of 64): about 512 workgroups
// stream the large operand, or, with fit > 0, at most max(fit, tiles) of
// them (the workgroups that fit on the device at once), so that none waits
// for a second round.
SkinnySplit skinny_split(int64_t tiles, int64_t klen, int64_t fit) {
  const int64_t steps = sk_cdiv(klen, SK);
  if (steps < 1) return SkinnySplit{1, SK};
  int64_t z = fit > 0 ? fit / (tiles < 1 ? 1 : tiles) : sk_cdiv(512, tiles < 1 ? 1 : tiles);
  if (z > 32) z = 32;
  if (z > steps) z = steps;
  if (z < 1) z = 1;
  const int64_t per = sk_cdiv(steps, z);
  SkinnySplit s;
  s.len = per * SK;
  s.Z = (int)sk_cdiv(steps, per);
  if (s.Z < 1) s.Z = 1;
  return s;
}

size_t skinny_partial_bytes(int64_t M, int64_t K, int64_t N) {
  const SkinnySplit a = skinny_split(sk_cdiv(M, SM), K);
  const SkinnySplit b = skinny_split(sk_cdiv(M, SM), N);
  const SkinnySplit c = skinny_split(sk_cdiv(K, SM), M);
  const SkinnySplit d = skinny_split(sk_cdiv(N, SM), M);
  size_t m = (size_t)a.Z * M;
  if ((size_t)b.Z * M > m) m = (size_t)b.Z * M;
  if ((size_t)c.Z * K > m) m = (size_t)c.Z * K;
  if ((size_t)d.Z * N > m) m = (size_t)d.Z * N;
  return m * SJ * sizeof(float);
}

// C = A B^T over K with B [64][ldb] (rows >= r zero), then reduce.
hipError_t skinny_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t K, int r,
                     float* part, float alpha, uint16_t* out, int64_t ldo, float alpha2, uint16_t* out2,
                     hipStream_t stream, const DropoutParams* dr) {
  if (dr && lda != K) return hipErrorInvalidValue;  // the mask indexes a contiguous [M][K] input
  // 72 KB of LDS: two workgroups per CU
  const SkinnySplit sp = skinny_split(sk_cdiv(M, SM), K, 2 * (int64_t)device_cu_count());
  NtArgs a;
  a.A = A; a.B = B; a.C = part; a.lda = lda; a.ldb = ldb; a.M = M; a.K = K; a.k_split = sp.len;
  a.thr = dr ? dr->thr : 0u; a.c = dr ? dr->c : 1.0f; a.seed = dr ? dr->seed : 0u;
  const dim3 grid((unsigned)sk_cdiv(M, SM), 1, (unsigned)sp.Z);
  if (dr)
    hipLaunchKernelGGL(skinny_nt_kernel<true>, grid, dim3(kSkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(skinny_nt_kernel<false>, grid, dim3(kSkThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)sk_grid(M * ldo / 4)), dim3(256), 0, stream, part, sp.Z, M, r,
                     alpha, 0, 1, (void*)out, ldo, alpha2, out2);
  return hipGetLastError();
}

// C[c][j] = sum_m L[m][c] S[m][j], then reduce to out (transposed if `transpose`).
hipError_t skinny_tn(const uint16_t* L, int64_t ldl, int64_t W, const uint16_t* S, int64_t lds, int64_t M, int r,
                     float* part, float alpha, bool transpose, bool out_bf16, void* out, hipStream_t stream,
                     const DropoutParams* dr) {
  if (dr && (ldl != W || W % 64)) return hipErrorInvalidValue;  // the mask indexes a contiguous [M][W] input
  // the copy-ring kernel (72 KB of LDS) fits two workgroups per CU
  const SkinnySplit sp = skinny_split(sk_cdiv(W, SM), M, dr ? 0 : 2 * (int64_t)device_cu_count());
  TnArgs a;
  a.L = L; a.S = S; a.C = part; a.ldl = ldl; a.lds = lds; a.M = M; a.W = W; a.r = r; a.m_split = sp.len;
  a.thr = dr ? dr->thr : 0u; a.c = dr ? dr->c : 1.0f; a.seed = dr ? dr->seed : 0u;
  const dim3 grid((unsigned)sk_cdiv(W, SM), 1, (unsigned)sp.Z);
  if (dr)
    hipLaunchKernelGGL(skinny_tn_kernel<true>, grid, dim3(kSkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(skinny_tn_dma_kernel, grid, dim3(kSkThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (transpose)
    hipLaunchKernelGGL(skinny_reduce_t_kernel, dim3((unsigned)sk_cdiv(W, 64), SJ / 16), dim3(256), 0, stream, part, sp.Z, W, r,
                       alpha, out_bf16 ? 1 : 0, out);
  else
    hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)sk_grid(W * (int64_t)r / 4)), dim3(256), 0, stream, part, sp.Z,
                       W, r, alpha, 1, out_bf16 ? 1 : 0, out, (int64_t)r, 0.0f, (uint16_t*)nullptr);
  return hipGetLastError();
}

}  // namespace qlora
