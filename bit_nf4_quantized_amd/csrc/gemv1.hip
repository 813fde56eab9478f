// Single-token (M = 1) QLoRA forward on gfx950:
//   Y[n] = sum_k X[k] dequant(Wt)[n][k] + sum_j bf16(s T[j]) L2[j][n],  T = X L1
// (QLoRA pages, diycv.top, section 关键公式; inference keeps the 4-bit base
// and the trained adapters, section 训练与推理流程 "推理").
//
// One token reads the whole packed weight once (0.52 B per weight) and does
// 2 flops per weight, so the call is a streaming read. Two launches:
//
//   t1_partial_kernel   T over K-slices of 256: one workgroup per slice, 8
//                       adapter columns per thread, a fixed-order LDS sum;
//                       writes part[slice][j] (fp32)
//   gemv1_kernel<NG>    one workgroup of 8 waves per CU, each owning a
//                       contiguous range of R <= 8 NG weight rows.
//
// A CU returns vector-load data in issue order, so the order of the loads
// decides when each operand arrives. gemv1 issues, in this order:
//   1. the small operands: X (copied straight into LDS), the E4M3 block
//      codes and group scales of its blocks, the slice partials and the L2
//      values it needs; then a barrier so that every wave's small loads are
//      queued before any code load;
//   2. the 4-bit codes of each wave's first chunks (12 x 16 bytes per lane:
//      for LLaMA-7B shapes the workgroup's whole weight share).
// While the codes stream in, the waves write the lookup table and the block
// constants a' into LDS and start the row sums from the LoRA term.
//
// The K loop: every wave owns the 256-k chunks c = wave, wave + 8, ... of all
// R rows; lane l holds 32 codes (16 bytes) of row 8 g + l/8, k in
// [256 c + 32 (l%8), +32), for each row group g.
//   * one LDS lookup per code byte: a 256-entry table maps a byte (two codes,
//     low nibble first) to the packed pair bf16(q[lo]) | bf16(q[hi]) << 16,
//     replicated 64 times (entry b, copy c at byte 256 b + 4 c, i.e. in bank
//     c; lane l reads copy l) so lookups never conflict, and the lookup
//     address (b << 8) | 4 l is one v_perm_b32 of the code word and the
//     lane's byte; v_dot2_f32_bf16 multiplies the pair with the matching X
//     pair (X in LDS) and accumulates in fp32;
//   * the 32 codes of a lane lie in one 64-block, so a' is applied once per
//     lane and chunk: acc += a' * sum. The effective weight is bf16(q) a'
//     rather than bf16(q a'); both round once at bf16 precision.
// The LoRA term is split over the waves by adapter column: lane (l/8, l%8)
// of wave w owns column j = 8 w + l%8, sums its partials of T[j] (slices
// l/8, l/8 + 8, ...; then the 8 lanes of the column by three exchanges),
// rounds st = bf16(s T[j]) and starts each of its row sums at
// st * L2[j][row]. The 8 lanes of a row are then added by DPP, the 8 waves'
// row sums through LDS in a fixed order, and Y is rounded to bf16 once.
// Every result is deterministic (fixed orders, no atomics).
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int kG1Waves = 8;
constexpr int kG1Threads = 64 * kG1Waves;
constexpr int kG1Chunk = 256;        // k per chunk: 8 lanes x 32 codes
constexpr int kG1Loads = 12;         // code loads per lane in flight
constexpr int kG1Copies = 64;       // one copy per lane: entry b, copy c at byte 256 b + 4 c (bank c)
constexpr uint32_t kG1TableBytes = 256u * kG1Copies * 4u;  // 64 KB
constexpr int kG1MaxRank = 64;
constexpr int kG1MaxSlices = 64;    // K / 256 <= 64
constexpr int kT1Rows = 256;         // k-rows of L1 per partial slice
constexpr int kRunsPerThread = 2;    // runs of 16 block codes per thread: R nblk <= 16 x 2 x 512 - 16

// LDS layout of gemv1_kernel (bytes).
struct G1Layout {
  uint32_t x_off, a_off, red_off, total;
};

__host__ __device__ inline G1Layout g1_layout(int K, int R, int nblk, int NG) {
  G1Layout L;
  uint32_t off = 0;                                            // the table is a static array before this
  L.x_off = off; off += ((uint32_t)K * 2u + 1023u) & ~1023u;   // whole 1 KB copy pieces
  L.a_off = off; off += (uint32_t)(R * (nblk + 1)) * 4u;      // rows padded by one (bank spread)
  L.red_off = off; off += (uint32_t)(kG1Waves * 8 * NG) * 4u;
  L.total = off;
  return L;
}

typedef __attribute__((address_space(3))) void g1_lds_t;

// part[p][j] = sum_{k in slice p} X[k] L1[k][j], slices of kT1Rows rows;
// thread t takes the 8 columns (t % 8) * 8 .. +8 of rows t / 8, t / 8 + 32, ...
__global__ __launch_bounds__(256) void t1_partial_kernel(const uint16_t* __restrict__ X, int K,
                                                        const uint16_t* __restrict__ L1, int r,
                                                        float* __restrict__ part) {
  __shared__ float red[32][kG1MaxRank];
  const int t = threadIdx.x, cc = t & 7, ph = t >> 3;
  const int k0 = blockIdx.x * kT1Rows;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bool col_in = cc * 8 < r;  // r % 8 == 0: a chunk of 8 columns is all in or all out
#pragma unroll
  for (int i = 0; i < kT1Rows / 32; ++i) {
    const int k = k0 + ph + 32 * i;
    const bool in = col_in && k < K;
    const int kc = in ? k : 0;
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(L1 + (int64_t)kc * r + (col_in ? cc * 8 : 0));
    const float x = in ? bf16_to_f32(X[kc]) : 0.0f;
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = __builtin_fmaf(x, bf16_to_f32(wv[e]), acc[2 * e]);
      acc[2 * e + 1] = __builtin_fmaf(x, bf16_to_f32(wv[e] >> 16), acc[2 * e + 1]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[ph][cc * 8 + e] = acc[e];
  __syncthreads();
  // column j = t / 4: lane t % 4 adds rows 8 (t % 4) .. +7 in order, then
  // the four lanes' sums are added pairwise by DPP, ((s0 + s1) + (s2 + s3)):
  // a fixed order (every lane of the four holds the same bits), with a
  // dependent chain of 10 additions instead of 32
  {
    const int j = t >> 2, p4 = t & 3;
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) v += red[8 * p4 + q][j];
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    if (p4 == 0 && j < r) part[(int64_t)blockIdx.x * r + j] = v;
  }
}

// Sum over each aligned group of 8 lanes, in lane 8i (DPP: swap neighbours,
// swap pairs, then the mirrored half-row of 8 adds the other quad).
__device__ __forceinline__ float sum8(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  return v;
}

template <int NG>
__global__ __launch_bounds__(kG1Threads, 1) void gemv1_kernel(NF4View Wt, NF4Table tab,
                                                              const uint16_t* __restrict__ X,
                                                              const float* __restrict__ part, int P, float s,
                                                              const uint16_t* __restrict__ L2, int r,
                                                              uint16_t* __restrict__ Y,
                                                              uint16_t* __restrict__ T_out) {
  constexpr int DC = NG >= kG1Loads ? 1 : kG1Loads / NG;  // chunks in flight per wave
  __shared__ __attribute__((aligned(256))) uint32_t g1_table[kG1TableBytes / 4];   // at LDS address 0
  extern __shared__ __attribute__((aligned(16))) unsigned char g1_smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = (int)Wt.cols, N = (int)Wt.rows;
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int n_lo = (int)((int64_t)b * N / G), n_hi = (int)((int64_t)(b + 1) * N / G);
  const int R = n_hi - n_lo;                       // 8 <= R <= 8 NG (the launcher checks)
  const int nblk = K / kBlock, NC = K / kG1Chunk;
  const G1Layout L = g1_layout(K, R, nblk, NG);
  const int sub = lane & 7, lrow = lane >> 3;
  const int myc = NC > wave ? (NC - wave + kG1Waves - 1) / kG1Waves : 0;
  auto ld16 = [](const void* base, uint32_t off) {
    return *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(base) + off);
  };

  // ==== 1. the small operands, issued before any code load (a CU returns
  // load data in issue order, so whatever is queued behind the weight
  // stream arrives with its end) ====
  // X straight into LDS in 1 KB pieces (wave w copies pieces w, w + 8, ...;
  // lanes past the end re-read X's last 16 bytes into the region's padding)
  {
    const uint32_t xbytes = 2u * (uint32_t)K;
    const int npieces = (int)((xbytes + 1023u) >> 10);
    const char* xb = reinterpret_cast<const char*>(X);
    for (int pc = wave; pc < npieces; pc += kG1Waves) {
      uint32_t off = ((uint32_t)pc << 10) + 16u * (uint32_t)lane;
      if (off > xbytes - 16u) off = xbytes - 16u;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(g1_lds_t*)(g1_smem + L.x_off + ((uint32_t)pc << 10)));
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(off), "s"(xb), "s"(m0) : "memory", "m0");
    }
  }
  // the E4M3 codes of the workgroup's blocks [gb_lo, gb_hi): thread t takes
  // the 16-aligned run of 16 blocks at gb_a + 16 t (and + 16 x 512), one
  // 16-byte load, with the run's group scale (a group of 256 blocks holds
  // the whole run; N nblk % 16 == 0 keeps the last run inside the array)
  const int gb_lo = n_lo * nblk, gb_hi = gb_lo + R * nblk;
  const int gb_a = gb_lo & ~15;
  const int nruns = (gb_hi - gb_a + 15) / 16;
  u32x4_t a16[kRunsPerThread];
  float sg[kRunsPerThread];
#pragma unroll
  for (int q = 0; q < kRunsPerThread; ++q) {
    int run = tid + q * kG1Threads;
    if (run > nruns - 1) run = nruns - 1;           // past the range: a valid run (not stored)
    const uint32_t gb = (uint32_t)(gb_a + 16 * run);
    a16[q] = ld16(Wt.absmax8, gb);
    sg[q] = Wt.scale2[gb >> 8];
  }
  const float mu = Wt.mean[0];
  // The LoRA term is split over the waves by adapter column: lane (lrow,
  // sub) of wave w owns column j = 8 w + sub. It loads the slice partials
  // part[p][j] for p = lrow, lrow + 8, ... and L2[j][row] of its row in
  // each row group (clamped addresses; the extras are masked below).
  const int jw = 8 * wave + sub, jc = jw < r ? jw : r - 1;
  float pt[kG1MaxSlices / 8];
  uint32_t l2g[NG];
#pragma unroll
  for (int m = 0; m < kG1MaxSlices / 8; ++m) {
    const int p = lrow + 8 * m;
    pt[m] = part[(uint32_t)(p < P ? p : P - 1) * (uint32_t)r + (uint32_t)jc];
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int row = 8 * g + lrow;
    l2g[g] = L2[(uint32_t)jc * (uint32_t)N + (uint32_t)(n_lo + (row < R ? row : R - 1))];
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();                     // every wave's small loads are queued
  __builtin_amdgcn_sched_barrier(0);

  // ==== 2. code loads of the wave's first DC chunks ====
  // byte offset of lane's 16 bytes in row group g, chunk c:
  //   row * K/2 + 128 c + 16 sub (rows clamped into the workgroup's range,
  //   chunks clamped into the row: those lanes and chunks are not used)
  uint32_t roff[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    int n = n_lo + 8 * g + lrow;
    if (n > n_hi - 1) n = n_hi - 1;
    roff[g] = __umul24((uint32_t)n, (uint32_t)(K >> 1)) + 16u * (uint32_t)sub;
  }
  auto chunk_of = [&](int ci) { const int c = wave + kG1Waves * ci; return c < NC ? c : (wave < NC ? wave : 0); };
  u32x4_t ring[DC][NG];
  auto load_chunk = [&](int ci, u32x4_t* slot) {
    const uint32_t cb = 128u * (uint32_t)chunk_of(ci);
#pragma unroll
    for (int g = 0; g < NG; ++g) slot[g] = ld16(Wt.codes, roff[g] + cb);
  };
#pragma unroll
  for (int d = 0; d < DC; ++d) load_chunk(d, ring[d]);
  __builtin_amdgcn_sched_barrier(0);

  // ==== 3. LDS operands and the LoRA term (the code loads in flight) ====
  // The lookup table: entry e (a code byte, low nibble first) holds the pair
  // bf16(q[e & 15]) | bf16(q[e >> 4]) << 16, copy c at byte 256 e + 4 c.
  // Store i writes bytes [1024 i, +1024), lane l the 16 bytes of entry
  // 4 i + l / 16 (copies 4 (l % 16) .. +4): consecutive lanes, consecutive
  // bytes. Wave w writes stores 8 w .. 8 w + 7; the entry's low nibble is
  // 4 (i % 4) + l / 16, its high nibble i / 4.
  {
    uint32_t qb[16];                                // bf16(q[j]), round to nearest even (finite q)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t u = __float_as_uint(tab.q[j]);
      qb[j] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    }
    const int lq = lane >> 4;
    uint32_t qlo[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      qlo[m] = lq == 0 ? qb[4 * m] : lq == 1 ? qb[4 * m + 1] : lq == 2 ? qb[4 * m + 2] : qb[4 * m + 3];
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(g1_table) + 64 * 8 * wave + lane;
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      const int i = 8 * wave + ii;                  // i % 4 = ii % 4
      const uint32_t hi = wave == 0 ? qb[ii >> 2] : wave == 1 ? qb[2 + (ii >> 2)] : wave == 2 ? qb[4 + (ii >> 2)]
                        : wave == 3 ? qb[6 + (ii >> 2)] : wave == 4 ? qb[8 + (ii >> 2)] : wave == 5 ? qb[10 + (ii >> 2)]
                        : wave == 6 ? qb[12 + (ii >> 2)] : qb[14 + (ii >> 2)];   // qb[i / 4], uniform
      (void)i;
      const uint32_t v = qlo[ii & 3] | (hi << 16);
      dst[64 * ii] = u32x4_t{v, v, v, v};
    }
  }
  // a' of the workgroup's blocks: row rr at rr (nblk + 1)
  float* aw = reinterpret_cast<float*>(g1_smem + L.a_off);
  const uint32_t mB = 0xFFFFFFFFu / (uint32_t)nblk + 1u;    // e / nblk by a multiply-high, exact for e < 2^16
#pragma unroll
  for (int q = 0; q < kRunsPerThread; ++q) {
    const int run = tid + q * kG1Threads;
    if (run < nruns) {
      const uint32_t bytes[4] = {a16[q].x, a16[q].y, a16[q].z, a16[q].w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rel = gb_a + 16 * run + e - gb_lo;   // block, relative to gb_lo
        if (rel >= 0 && rel < gb_hi - gb_lo) {
          const int rr = (int)__umulhi((uint32_t)rel, mB);
          aw[rel + rr] = block_scale((bytes[e >> 2] >> (8 * (e & 3))) & 0xFFu, sg[q], mu);
        }
      }
    }
  }
  // T[j] = the lane's partials in slice order, then the 8 lanes of column j
  // (stride 8) by three exchanges (every lane ends with the same sum);
  // st = bf16(s T). The row sums start from st[j] L2[j][row] (a product of
  // two bf16 values, exact in fp32), so the 8 lanes of a row and the 8 waves
  // together add every column once.
  float acc[NG];
  {
    float t = 0.0f;
#pragma unroll
    for (int m = 0; m < kG1MaxSlices / 8; ++m)
      if (lrow + 8 * m < P) t += pt[m];
    t += __shfl_xor(t, 8, 64);
    t += __shfl_xor(t, 16, 64);
    t += __shfl_xor(t, 32, 64);
    if (b == 0 && T_out && lrow == 0 && jw < r) T_out[jw] = f32_to_bf16(t);
    const float st = jw < r ? bf16_to_f32(f32_to_bf16(s * t)) : 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = st * bf16_to_f32(l2g[g]);
  }
  // the X copies (issued first) have landed once all but the code loads are done
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(DC * NG) : "memory");
  __syncthreads();

  // ==== 4. K loop: the wave's chunks, DC in flight ====
  // LDS byte address of code byte t of w in this lane's table copy:
  // (byte << 8) | 4 lane, one v_perm_b32 (byte 0 from lane4, byte 1 from w)
  const uint32_t lane4 = (uint32_t)lane << 2;
  auto lut = [&](uint32_t w, int t) -> uint32_t {
    const uint32_t addr = __builtin_amdgcn_perm(w, lane4, 0x0C0C0000u | ((4u + (uint32_t)t) << 8));
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const unsigned char*>(g1_table) + addr);
  };
  const unsigned char* xl = g1_smem + L.x_off;
  auto compute = [&](int ci, const u32x4_t* slot) {
    const int c = wave + kG1Waves * ci;
    const int koff = kG1Chunk * c + 32 * sub;        // first k of the lane's 32 codes
    const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xl + 2u * (uint32_t)koff);
    const u32x4_t x4[4] = {xp[0], xp[1], xp[2], xp[3]};
    const uint32_t xw[16] = {x4[0].x, x4[0].y, x4[0].z, x4[0].w, x4[1].x, x4[1].y, x4[1].z, x4[1].w,
                             x4[2].x, x4[2].y, x4[2].z, x4[2].w, x4[3].x, x4[3].y, x4[3].z, x4[3].w};
    const int blk = koff >> 6;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint32_t words[4] = {slot[g].x, slot[g].y, slot[g].z, slot[g].w};
      uint32_t lv[16];                               // all 16 lookups in flight, then the dot products
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) lv[4 * i + t] = lut(words[i], t);
      float sum = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lv[k]), __builtin_bit_cast(bf16x2_t, xw[k]),
                                              sum, false);
      int row = 8 * g + lrow;
      if (row > R - 1) row = R - 1;                  // lanes past the rows read a valid constant (unused)
      acc[g] = __builtin_fmaf(aw[row * (nblk + 1) + blk], sum, acc[g]);
    }
  };
  int base = 0;
  for (; base + DC < myc; base += DC) {
#pragma unroll
    for (int d = 0; d < DC; ++d) {
      compute(base + d, ring[d]);
      load_chunk(base + DC + d, ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < DC; ++d)
    if (base + d < myc) compute(base + d, ring[d]);

  // ==== 5. row sums: the 8 lanes of a row, then the 8 waves in order ====
  float* red = reinterpret_cast<float*>(g1_smem + L.red_off);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float v = sum8(acc[g]);
    if (sub == 0) red[wave * (8 * NG) + 8 * g + lrow] = v;
  }
  __syncthreads();
  if (tid < R) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kG1Waves; ++w) v += red[w * (8 * NG) + tid];
    Y[n_lo + tid] = f32_to_bf16(v);
  }
}

template <int NG>
hipError_t launch_g1(const NF4View& W, const NF4Table& tab, const uint16_t* X, const float* part, int P, float s,
                     const uint16_t* L2, int r, uint16_t* Y, uint16_t* T_out, int G, uint32_t lds,
                     hipStream_t stream) {
  static bool attr_set = false;  // raise the dynamic-LDS limit once per instantiation (idempotent)
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv1_kernel<NG>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - (int)kG1TableBytes);
    (void)hipGetLastError();  // a refusal shows up as a launch error below
    attr_set = true;
  }
  hipLaunchKernelGGL((gemv1_kernel<NG>), dim3((unsigned)G), dim3(kG1Threads), lds, stream, W, tab, X, part, P, s,
                     L2, r, Y, T_out);
  return hipGetLastError();
}

// Workgroups and row groups of the single-token kernel for N rows: one
// workgroup per CU (fewer when N is small), R <= 8 NG rows each.
struct G1Plan {
  int G, NG, P;
  uint32_t lds;
  bool ok;
};

G1Plan g1_plan(const NF4View& W, int r) {
  G1Plan p{0, 0, 0, 0u, false};
  const int64_t K = W.cols, N = W.rows;
  if (r > kG1MaxRank || K % kG1Chunk != 0 || K > 16384 || N < 8) return p;   // P = K / 256 <= 64
  if (W.absmax32 != nullptr || r % 8 != 0) return p;   // double-quantised weights only
  if (N * K / 2 >= ((int64_t)1 << 32) || N >= (1 << 24)) return p;   // 32-bit byte offsets, 24-bit products
  int G = device_cu_count();
  if (G > N / 8) G = (int)(N / 8);
  const int64_t R = (N + G - 1) / G;
  const int NG = (int)((R + 7) / 8);
  if (NG > 11) return p;
  const int nblk = (int)(K / kBlock);
  if (R * nblk > 16 * kRunsPerThread * kG1Threads - 16) return p;   // runs of block codes per thread
  if ((N * nblk) % 16 != 0) return p;                              // whole runs of 16 block codes
  const G1Layout L = g1_layout((int)K, (int)R, nblk, NG);
  if (L.total + kG1TableBytes > 160u * 1024u) return p;
  p.G = G;
  p.NG = NG;
  p.P = (int)((K + kT1Rows - 1) / kT1Rows);
  // more than half of a CU's LDS, so that exactly one workgroup lands on
  // each CU (with room for two, the dispatcher may stack them on some CUs)
  p.lds = L.total + kG1TableBytes > 84u * 1024u ? L.total : 84u * 1024u - kG1TableBytes;
  p.ok = true;
  return p;
}

}  // namespace

size_t gemv1_partial_bytes(int64_t K, int r) { return (size_t)((K + kT1Rows - 1) / kT1Rows) * (size_t)r * 4; }

bool gemv1_applies(const NF4View& W, int64_t M, int r) { return M == 1 && g1_plan(W, r).ok; }

hipError_t launch_gemv1(const NF4View& W, const NF4Table& tab, const uint16_t* X, const uint16_t* L1,
                        const uint16_t* L2, int r, float s, uint16_t* Y, uint16_t* T_out, float* part,
                        hipStream_t stream) {
  const G1Plan pl = g1_plan(W, r);
  if (!pl.ok) return hipErrorInvalidValue;
  hipLaunchKernelGGL(t1_partial_kernel, dim3((unsigned)pl.P), dim3(256), 0, stream, X, (int)W.cols, L1, r, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return timed(kTimeGemv, stream, [&]() -> hipError_t {
    switch (pl.NG) {
      case 1: return launch_g1<1>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 2: return launch_g1<2>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 3: return launch_g1<3>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 4: return launch_g1<4>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 5: return launch_g1<5>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 6: return launch_g1<6>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 7: return launch_g1<7>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 8: return launch_g1<8>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 9: return launch_g1<9>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      case 10: return launch_g1<10>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
      default: return launch_g1<11>(W, tab, X, part, pl.P, s, L2, r, Y, T_out, pl.G, pl.lds, stream);
    }
  });
}

}  // namespace qlora
