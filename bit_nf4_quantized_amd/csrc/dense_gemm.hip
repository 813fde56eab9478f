// bf16 MFMA GEMM core for the large-M QLoRA products on gfx950, and the
// streaming dequantisers that feed it.
//
//   C[M][N] = alpha * ( sum_k A[m][k] B[n][k]  +  sum_j A2[m][j] B2[n][j] )
//
// with A, B (and the LoRA slab A2, B2) bf16 row-major and the reduction
// contiguous ("NT"), fp32 accumulation and one RNE rounding to bf16. Used for
//   forward  Y  = X  . Wd^T + (s X L1) . L2          (B = Wd [N][K], B2 = L2^T)
//   backward dX = dY . Wd   + (s dY L2^T) . L1^T     (B = Wd^T [K][N], B2 = L1)
// where Wd is the doubleDequant of the NF4 weight (QLoRA pages, diycv.top,
// section 关键公式), written to a bf16 workspace by dequant_rows_kernel /
// dequant_cols_kernel just before the GEMM. Streaming the weight once more
// through HBM (2.5 B per weight, a few percent of the GEMM time at these
// shapes) keeps the MFMA loop free of per-weight VALU work.
//
// Tiling (one workgroup per 256 x 256 output tile, 512 threads = 8 waves,
// two waves per SIMD):
//   * each wave owns a 128 x 64 sub-tile = 4 x 2 v_mfma_f32_32x32x16_bf16
//     accumulators (128 fp32 registers per lane);
//   * K advances in stages of 64: the A and B stage tiles (2 x 32 KB) are
//     copied global -> LDS by global_load_lds_dwordx4 (no register staging);
//     A is double-buffered and B triple-buffered (all 160 KB of LDS);
//   * software pipeline: the fragments of k-step kk+1 are read from LDS into
//     a second register set while the 8 MFMAs of k-step kk run; the stage
//     barrier sits before the last k-step, so the first fragments of the
//     next stage are read while those MFMAs run;
//   * each stage copy is issued in two halves, each spread one instruction
//     per two MFMAs: the B tile of stage st+2 among the MFMAs of k-step 1 of
//     stage st (its third buffer held stage st-1), the A tile among those
//     right after the barrier of stage st. So the B copy has almost two
//     stages to land and the A copy one. Measured per launch against the
//     earlier schedule (both tiles double-buffered and issued as one burst
//     after the barrier): 3-8 % faster at K = 6656 and up to 13 % at
//     K = 17920, where the copies had waited for memory 23 % of the loop;
//   * the LDS copies are issued from inline assembly: with the compiler
//     builtin for them, the generated code waited for all fragment reads
//     (lgkmcnt(0)) and for the in-flight copy of the next stage (vmcnt(0))
//     before MFMA groups, which serialises the pipeline. The kernel places
//     the copy waits itself (vmcnt before each stage barrier);
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at
//     position c ^ ((r >> 1) & 7): two rows share one 256-byte line of the
//     64 LDS banks, so the 16-byte fragment reads of 16 consecutive rows hit
//     16 different bank groups (measured: fewer conflict cycles and faster
//     than the 8-row swizzle c ^ (r & 7));
//   * one workgroup runs per CU. When the tile count would leave at least
//     half of the CUs idle in the last round, the tile-columns holding that
//     remainder run as quarter-height (64 x 256) tiles if those fit in one
//     round, else as half-height (128 x 256) tiles, dispatched after the full
//     tiles so that they share the last round (8192 x 6656: 768 full tiles
//     and 256 quarter tiles instead of 832 full tiles in 3.25 rounds;
//     8192 x 11008: 1280 full tiles and 192 half tiles instead of 1376 full
//     tiles in 5.4 rounds);
//   * workgroups are numbered so that the 8 XCDs (each with its own L2) get
//     contiguous blocks of tiles, ordered in groups of 4 tile-rows so that
//     concurrently running tiles share A rows and B columns (measured: 4
//     and 6 tile-rows about 0.5 % faster per training step than 2, 8 or 16).
// Rows beyond M or N are read clamped (finite data) and never stored. Per-lane
// offsets are 32-bit: B (and B2) must be smaller than 2 GB, and the launcher
// runs the rows of A in chunks of at most 2 GB, one launch per chunk.
#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

constexpr int TM = 256, TN = 256, TK = 64;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int WGN = 4;           // waves along N (2 along M)
constexpr int WTM = 128;         // wave sub-tile: 128 rows x 64 columns
constexpr int WTN = 64;
constexpr int MI = WTM / 32;
constexpr int NJ = WTN / 32;
constexpr int RPI = 8;           // rows per wave load instruction (64 lanes x 16 B = 8 rows of 128 B)
constexpr int kStageElems = TM * TK;  // LDS elements per operand per stage (TM == TN)

// The tail of a launch whose tile count leaves the last round of workgroups
// mostly empty runs as half- or quarter-height tiles (TM / 2 or TM / 4
// rows, wave sub-tiles of 64 or 32 rows), so that the last round holds more,
// shorter tiles.
template <int TMX>
struct TileShape {
  static constexpr int kWtm = TMX / (kWaves / WGN);  // wave sub-tile rows
  static constexpr int kMi = kWtm / 32;
  static constexpr int kIpwA = TMX / RPI / kWaves;   // A load instructions per wave per stage
  static constexpr int kIpwB = TN / RPI / kWaves;    // B load instructions per wave per stage
};

struct DenseArgs {
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* A2;
  const uint16_t* B2;
  uint16_t* C;
  int64_t lda, ldb, ld2, ldc;
  int64_t M, N;
  int64_t K;        // main reduction, multiple of TK (operands readable up to K columns)
  int64_t K2;       // slab reduction, multiple of TK (0 = no slab)
  float alpha;
  int tiles_m, tiles_n;
  int full_n;       // tile-columns [0, full_n) run as TM x TN tiles, the rest as (TM/tail_split) x TN
  int tail_split;   // 2 or 4
  const float* E;   // ADD: fp32 addend [M][N] (row stride lde), C = bf16(alpha acc + E)
  int64_t lde;
};

// One stage of one operand: rows [row0, row0+256) x columns [k0, k0+64).
// Each wave moves 8 rows per instruction (64 lanes x 16 bytes), NI
// instructions per wave. Lane i of instruction j writes LDS bytes
// [16 i, 16 i + 16) of a 1 KB slice: row 8(NI w + j) + i/8, physical chunk
// i%8, which holds logical chunk (i%8) ^ swz(row). The address is a
// wave-uniform base (matrix + k0, advanced per stage) plus a per-lane 32-bit
// byte offset that is fixed for the whole K loop.
template <int NI>
struct StageOffsets {
  uint32_t off[NI];
};

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <int NI>
__device__ __forceinline__ StageOffsets<NI> stage_offsets(int64_t ld, int64_t row0, int64_t nrows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane >> 3;
  StageOffsets<NI> o;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int rloc = (wave * NI + j) * RPI + lr;
    const int chunk = (lane & 7) ^ swz(rloc);
    int64_t r = row0 + rloc;
    if (r > nrows - 1) r = nrows - 1;
    o.off[j] = (uint32_t)((r * ld + chunk * 8) * 2);
  }
  return o;
}

// Issues NI global_load_lds_dwordx4 (global address = uniform base in
// SGPRs + per-lane 32-bit offset; LDS address = M0 + 16 * lane). The copies
// are not visible to the compiler: the caller waits for them with an
// explicit vmcnt before the barrier that publishes the stage.
template <int NI>
__device__ __forceinline__ void stage_load_one(const uint16_t* __restrict__ P, const StageOffsets<NI>& o, uint16_t* lds,
                                               int j) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* base = reinterpret_cast<const char*>(P);
  const int slice = wave * NI + j;
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)(lds + slice * RPI * TK));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(o.off[j]), "s"(base), "s"(m0) : "memory", "m0");
}

template <int NI>
__device__ __forceinline__ void stage_load(const uint16_t* __restrict__ P, const StageOffsets<NI>& o, uint16_t* lds) {
#pragma unroll
  for (int j = 0; j < NI; ++j) stage_load_one(P, o, lds, j);
}

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * TK + ((chunk ^ swz(row)) << 3); }

// One TMX x TN output tile at (m0, n0). smem holds the stage tiles: two A
// buffers, then three B buffers, kStageElems elements each.
template <bool ADD, int TMX>
__device__ __forceinline__ void gemm_tile(const DenseArgs& p, int64_t m0, int64_t n0, uint16_t* smem) {
  using S = TileShape<TMX>;
  constexpr int WTM = S::kWtm, MI = S::kMi;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int nmain = (int)(p.K / TK), nslab = (int)(p.K2 / TK);
  const int nk = nmain + nslab;

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const StageOffsets<S::kIpwA> offA = stage_offsets<S::kIpwA>(p.lda, m0, p.M);
  const StageOffsets<S::kIpwB> offB = stage_offsets<S::kIpwB>(p.ldb, n0, p.N);
  const StageOffsets<S::kIpwA> offA2 = stage_offsets<S::kIpwA>(p.ld2, m0, p.M);
  const StageOffsets<S::kIpwB> offB2 = stage_offsets<S::kIpwB>(p.ld2, n0, p.N);
  // Stage st covers columns [64 st, 64 st + 64) of (A, B) for st < nmain,
  // then the slab (A2, B2). Operand selection is branch-free so that the
  // copy can be scheduled among the MFMAs of the same block.
  auto a_buf = [&](int st) { return smem + (st & 1) * kStageElems; };
  auto b_buf = [&](int st) { return smem + (2 + st % 3) * kStageElems; };
  auto issue = [&](int st) {
    const bool slab = st >= nmain;
    const int64_t k0 = (int64_t)(slab ? st - nmain : st) * TK;
    StageOffsets<S::kIpwA> oa;
    StageOffsets<S::kIpwB> ob;
#pragma unroll
    for (int j = 0; j < S::kIpwA; ++j) oa.off[j] = slab ? offA2.off[j] : offA.off[j];
#pragma unroll
    for (int j = 0; j < S::kIpwB; ++j) ob.off[j] = slab ? offB2.off[j] : offB.off[j];
    stage_load((slab ? p.A2 : p.A) + k0, oa, a_buf(st));
    stage_load((slab ? p.B2 : p.B) + k0, ob, b_buf(st));
  };
  // copy instruction q of stage st: q < kIpwA are the A tile's, the rest
  // the B tile's
  auto issue_one = [&](int st, int q) {
    const bool slab = st >= nmain;
    const int64_t k0 = (int64_t)(slab ? st - nmain : st) * TK;
    if (q < S::kIpwA) {
      StageOffsets<S::kIpwA> oa;
#pragma unroll
      for (int j = 0; j < S::kIpwA; ++j) oa.off[j] = slab ? offA2.off[j] : offA.off[j];
      stage_load_one((slab ? p.A2 : p.A) + k0, oa, a_buf(st), q);
    } else {
      StageOffsets<S::kIpwB> ob;
#pragma unroll
      for (int j = 0; j < S::kIpwB; ++j) ob.off[j] = slab ? offB2.off[j] : offB.off[j];
      stage_load_one((slab ? p.B2 : p.B) + k0, ob, b_buf(st), q - S::kIpwA);
    }
  };
  bf16x8_t fa[2][MI], fb[2][NJ];  // two register sets of k-step fragments
  auto frag = [&](int st, int kk, int set) {
    const uint16_t* As = a_buf(st);
    const uint16_t* Bs = b_buf(st);
    const int ch = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[set][i] = *reinterpret_cast<const bf16x8_t*>(As + lds_off(wm * WTM + i * 32 + (lane & 31), ch));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[set][j] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(wn * WTN + j * 32 + (lane & 31), ch));
  };
  auto mma = [&](int set) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
  };
  // scheduling hint: the reads of the next k-step interleaved with this
  // k-step's MFMAs (one read, then MFMAs) rather than issued as one burst
  // (measured 0.1-0.3 % faster)
  auto order = [&]() {
    constexpr int nr = MI + NJ, nm = MI * NJ;
    if constexpr (nm >= nr) {
      constexpr int per = nm / nr, left = nm - nr * per;
#pragma unroll
      for (int q = 0; q < nr; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one DS read
        __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMAs
      }
      if constexpr (left > 0) __builtin_amdgcn_sched_group_barrier(0x008, left, 0);
    } else {  // quarter tiles: fewer MFMAs than reads per k-step
#pragma unroll
      for (int q = 0; q < nm; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, nr - nm, 0);
    }
  };
  // The MFMAs of one k-step (register set `set`) with copy instructions
  // first .. first+cnt-1 of stage cst spread evenly among them (the order is
  // pinned: the scheduler would otherwise bunch them).
  auto mma_copies = [&](int set, int cst, int first, int cnt, bool on) {
    constexpr int nm = MI * NJ;
#pragma unroll
    for (int q = 0; q < nm; ++q) {
      acc[q / NJ][q % NJ] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][q / NJ], fb[set][q % NJ], acc[q / NJ][q % NJ], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < cnt; ++c)
        if (on && (c * nm) / cnt == q) issue_one(cst, first + c);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One stage. On entry the fragments of its k-step 0 are in set 0, and the
  // copies of stages st+1 (complete or in flight) and st+2 (the B tile, in
  // flight: the A tile goes out after this stage's barrier) were issued.
  // The prologue issued all of stages 0 and 1.
  auto stage = [&](int st, bool refill, bool next) {
#pragma unroll
    for (int kk = 0; kk < TK / 16 - 1; ++kk) {
      frag(st, kk + 1, (kk + 1) & 1);
      if (kk == 1) {
        mma_copies(1, st + 2, S::kIpwA, S::kIpwB, refill);  // B tile of stage st+2
      } else {
        mma(kk & 1);
        order();
      }
    }
    // every read of this stage's buffers by this wave has been issued; the
    // barrier's release fence completes them. The vmcnt completes this
    // wave's copies of stage st+1; the B copies of st+2, issued after them,
    // may stay in flight (copies complete in issue order)
    __builtin_amdgcn_sched_barrier(0);
    if (refill) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(S::kIpwB) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (next) frag(st + 1, 0, 0);
    mma_copies(1, st + 2, 0, S::kIpwA, refill);  // A tile of stage st+2
  };
  if (nk > 0) issue(0);
  if (nk > 1) issue(1);
  if (nk > 0) {
    if (nk > 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(S::kIpwA + S::kIpwB) : "memory");  // stage 0 landed
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    frag(0, 0, 0);
  }
  int st = 0;
  for (; st + 2 < nk; ++st) stage(st, true, true);
  if (st + 1 < nk) stage(st++, false, true);
  if (st < nk) stage(st, false, false);

  if constexpr (ADD) {
    // Epilogue with an fp32 addend: each wave stages a quarter of its 128 x 64
    // sub-tile (32 rows, one accumulator row-block) as fp32 in its own padded
    // LDS slice; then each lane takes 8 consecutive columns of a row, adds the
    // matching 32 bytes of E and stores 16 bytes of bf16.
    constexpr int kAddStride = WTN + 4;  // fp32 per padded row
    __syncthreads();
    float* ef = reinterpret_cast<float*>(smem) + wave * (32 * kAddStride);
    const int64_t row_base = m0 + wm * WTM, col_base = n0 + wn * WTN;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          ef[((v & 3) + 4 * (lane >> 5) + 8 * (v >> 2)) * kAddStride + j * 32 + (lane & 31)] = p.alpha * acc[i][j][v];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done (wave-private slice)
      constexpr int kLpr = WTN / 8;  // lanes per sub-tile row, 8 columns each
#pragma unroll
      for (int it = 0; it < 32 * kLpr / 64; ++it) {
        const int r = it * (64 / kLpr) + lane / kLpr;
        const int cc = (lane % kLpr) * 8;
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(ef + r * kAddStride + cc);
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(ef + r * kAddStride + cc + 4);
        const int64_t row = row_base + i * 32 + r, col = col_base + cc;
        const bool in = row < p.M && col < p.N;
        const float* ep = p.E + (in ? row * p.lde + col : 0);
        const f32x4_t e0 = *reinterpret_cast<const f32x4_t*>(ep);
        const f32x4_t e1 = *reinterpret_cast<const f32x4_t*>(ep + 4);
        const u32x4_t val = {pack_bf16x2(a0.x + e0.x, a0.y + e0.y), pack_bf16x2(a0.z + e0.z, a0.w + e0.w),
                             pack_bf16x2(a1.x + e1.x, a1.y + e1.y), pack_bf16x2(a1.z + e1.z, a1.w + e1.w)};
        if (in) *reinterpret_cast<u32x4_t*>(p.C + row * p.ldc + col) = val;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // reads of this quarter done before the next overwrites it
    }
    return;
  }

  // Epilogue through LDS (the stage buffers are free now): each wave writes
  // up to two 32-row blocks of its sub-tile (64 rows) as bf16 into its own
  // padded LDS slice, then stores them to C in 16-byte row chunks. In a
  // 32x32 accumulator, register v of lane l is row (v%4) + 4(l/32) +
  // 8(v/4), column l%32.
  constexpr int kEpiStride = WTN + 8;  // padded row (elements)
  constexpr int CPRO = WTN / 8;        // 16-byte chunks per sub-tile row
  constexpr int RPIT = 64 / CPRO;      // rows stored per iteration
  constexpr int RB = MI < 2 ? MI : 2;  // 32-row blocks staged per pass
  __syncthreads();
  uint16_t* ep = smem + wave * (64 * kEpiStride);
  const int64_t row_base = m0 + wm * WTM, col_base = n0 + wn * WTN;
#pragma unroll
  for (int h = 0; h < MI / RB; ++h) {
#pragma unroll
    for (int ii = 0; ii < RB; ++ii) {
      const int i = RB * h + ii;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = ii * 32 + (v & 3) + 4 * (lane >> 5) + 8 * (v >> 2);
          const int c = j * 32 + (lane & 31);
          ep[r * kEpiStride + c] = f32_to_bf16(p.alpha * acc[i][j][v]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done (wave-private slice)
#pragma unroll
    for (int it = 0; it < 32 * RB / RPIT; ++it) {
      const int r = it * RPIT + lane / CPRO;
      const int ch = lane % CPRO;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ep + r * kEpiStride + ch * 8);
      const int64_t row = row_base + h * 32 * RB + r;
      const int64_t col = col_base + ch * 8;
      if (row < p.M && col < p.N) *reinterpret_cast<u32x4_t*>(p.C + row * p.ldc + col) = val;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads of this half done before the next half overwrites it
  }
}

template <bool ADD>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(DenseArgs p) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[5 * kStageElems];  // A x 2, B x 3
  const int bid = blockIdx.x;
  const int nfull = p.tiles_m * p.full_n;
  if (bid < nfull) {
    // tile order: workgroup b runs on XCD b % 8; give each XCD a contiguous
    // range of tile ids (a bijection for any tile count), then walk the
    // tiles in groups of 4 tile-rows so that co-resident tiles share A and B.
    const int xcd = bid % 8, q = nfull / 8, rem = nfull % 8;
    const int t = xcd * q + (xcd < rem ? xcd : rem) + bid / 8;
    const int group = 4;
    const int g = t / (group * p.full_n);
    const int first_m = g * group;
    const int gm = (p.tiles_m - first_m) < group ? (p.tiles_m - first_m) : group;
    const int tl = t - g * group * p.full_n;
    const int tm = first_m + tl % gm;
    const int tn = tl / gm;
    gemm_tile<ADD, TM>(p, (int64_t)tm * TM, (int64_t)tn * TN, smem);
  } else {
    // the tail tile-columns, as half- or quarter-height tiles; dispatched
    // last, they fill the last round of workgroups
    const int h = bid - nfull;
    const int ncols = p.tiles_n - p.full_n;
    const int64_t m0 = (int64_t)(h / ncols) * (TM / p.tail_split);
    if (m0 >= p.M) return;  // a piece of a last tile-row beyond M (uniform per workgroup)
    const int64_t n0 = (int64_t)(p.full_n + h % ncols) * TN;
    if (p.tail_split == 4)
      gemm_tile<ADD, TM / 4>(p, m0, n0, smem);
    else
      gemm_tile<ADD, TM / 2>(p, m0, n0, smem);
  }
}

// Wd[n][k] for the forward product, the standalone dequant arithmetic
// (bf16(RN32(q[code] * a'))). A thread takes 4 units of 8 weights (one code
// dword, one 16-byte store) 256 units apart, so that every load and store
// instruction of a wave covers one contiguous range; the 4 code loads and
// block constants are issued before any store (measured 17.0 us against
// 19.5 us per launch for one unit of 16 weights per thread).
constexpr int kRowsUnits = 4;
__global__ __launch_bounds__(256) void dequant_rows_kernel(NF4View W, NF4Table tab, uint16_t* __restrict__ out) {
  __shared__ float s_q[16];
  if (threadIdx.x < 16) s_q[threadIdx.x] = tab.q[threadIdx.x];
  __syncthreads();
  const float mu = tensor_mean(W);
  const int64_t nunits = W.rows * W.cols / 8;  // cols % 64 == 0
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(W.codes);
  const int64_t stride = (int64_t)gridDim.x * 256 * kRowsUnits;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kRowsUnits + threadIdx.x; base < nunits; base += stride) {
    uint32_t c[kRowsUnits];
    float ap[kRowsUnits];
#pragma unroll
    for (int u = 0; u < kRowsUnits; ++u) {
      const int64_t un = base + (int64_t)u * 256;
      const int64_t uc = un < nunits ? un : nunits - 1;  // clamped: loads stay unconditional
      c[u] = codes[uc];
      ap[u] = block_const(W, uc >> 3, mu);  // 8 units per 64-block
    }
#pragma unroll
    for (int u = 0; u < kRowsUnits; ++u) {
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
}

// WdT[k][n] = Wd[n][k] for the dX product, rows padded to ldo >= N columns
// with zeros, without LDS: a thread dequantises two adjacent weight rows
// (n, n+1) over 32 k (16 code bytes each, inside one 64-block), so that each
// (row n, row n+1) pair at one k is one dword of output row k; the 64 lanes
// of a wave take 64 consecutive row pairs, so every store instruction
// writes 256 contiguous bytes. Workgroup: 128 rows n x 128 k (4 waves along k).
__global__ __launch_bounds__(256) void dequant_cols_kernel(NF4View W, NF4Table tab, uint16_t* __restrict__ out,
                                                           int64_t ldo) {
  __shared__ float s_q[16];
  if (threadIdx.x < 16) s_q[threadIdx.x] = tab.q[threadIdx.x];
  __syncthreads();
  const float mu = tensor_mean(W);
  const int64_t K = W.cols, N = W.rows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.y * 128 + 2 * lane;           // rows n, n + 1 (N % 8 == 0)
  const int64_t k0 = (int64_t)blockIdx.x * 128 + wave * 32;         // k0 .. k0 + 32
  if (k0 >= K) return;                                              // wave-uniform; no barrier follows
  const bool in = n < N;
  const int64_t na = in ? n : 0;
  const int64_t e0 = na * K + k0, e1 = e0 + K;
  const u32x4_t ca = *reinterpret_cast<const u32x4_t*>(W.codes + (e0 >> 1));
  const u32x4_t cb = *reinterpret_cast<const u32x4_t*>(W.codes + (e1 >> 1));
  const float aa = block_const(W, e0 / kBlock, mu), ab = block_const(W, e1 / kBlock, mu);
  const uint32_t wa[4] = {ca.x, ca.y, ca.z, ca.w}, wb[4] = {cb.x, cb.y, cb.z, cb.w};
  if (n >= ldo) return;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t qa = (wa[i >> 3] >> (4 * (i & 7))) & 15u;
    const uint32_t qb = (wb[i >> 3] >> (4 * (i & 7))) & 15u;
    const uint32_t v = in ? pack_bf16x2(s_q[qa] * aa, s_q[qb] * ab) : 0u;
    *reinterpret_cast<uint32_t*>(out + (k0 + i) * ldo + n) = v;
  }
}

}  // namespace

hipError_t launch_dequant_rows(const NF4View& W, const NF4Table& tab, uint16_t* out, hipStream_t stream) {
  const int64_t nunits = W.rows * W.cols / 8;
  const int64_t per_block = 256 * kRowsUnits;
  int64_t blocks = (nunits + per_block - 1) / per_block;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(dequant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, tab, out);
  return hipGetLastError();
}

hipError_t launch_dequant_cols(const NF4View& W, const NF4Table& tab, uint16_t* out, int64_t ldo,
                               hipStream_t stream) {
  const dim3 grid((unsigned)((W.cols + 127) / 128), (unsigned)((ldo + 127) / 128));
  hipLaunchKernelGGL(dequant_cols_kernel, grid, dim3(256), 0, stream, W, tab, out, ldo);
  return hipGetLastError();
}

namespace {

// One launch over all M rows (row offsets of A and A2 below 4 GB).
hipError_t launch_gemm_nt_rows(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N,
                               int64_t K, const uint16_t* A2, const uint16_t* B2, int64_t ld2, int64_t K2,
                               uint16_t* C, int64_t ldc, float alpha, hipStream_t stream, const float* E,
                               int64_t lde) {
  DenseArgs p;
  p.A = A; p.B = B; p.A2 = A2; p.B2 = B2; p.C = C;
  p.lda = lda; p.ldb = ldb; p.ld2 = ld2; p.ldc = ldc;
  p.M = M; p.N = N; p.K = K; p.K2 = K2; p.alpha = alpha;
  p.tiles_m = (int)((M + TM - 1) / TM);
  p.tiles_n = (int)((N + TN - 1) / TN);
  p.E = E; p.lde = lde;
  // One workgroup per CU at a time. When the last round of tiles would
  // leave at least half of the CUs idle, the last tile-columns that hold
  // those tiles run as quarter-height tiles if those fit in one round, else
  // as half-height tiles, all in that round.
  const int cus = device_cu_count();
  const int tiles = p.tiles_m * p.tiles_n;
  const int tail = tiles % cus;
  int tail_cols = 0;
  p.tail_split = 2;
  if (tail > 0) {
    const int tc = (tail + p.tiles_m - 1) / p.tiles_m;
    if (tc <= p.tiles_n && 4 * tc * p.tiles_m <= cus) {
      tail_cols = tc;
      p.tail_split = 4;
    } else if (tc <= p.tiles_n && 2 * tc * p.tiles_m <= cus) {
      tail_cols = tc;
    }
  }
  p.full_n = p.tiles_n - tail_cols;
  const int ntiles = p.tiles_m * p.full_n + p.tail_split * p.tiles_m * tail_cols;
  if (E)
    hipLaunchKernelGGL(gemm_nt_kernel<true>, dim3((unsigned)ntiles), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<false>, dim3((unsigned)ntiles), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                          int64_t M, int64_t N, int64_t K, const uint16_t* A2, const uint16_t* B2, int64_t ld2,
                          int64_t K2, uint16_t* C, int64_t ldc, float alpha, hipStream_t stream, const float* E,
                          int64_t lde) {
  // per-lane offsets are 32-bit: B and B2 must fit, and the rows of A (A2)
  // are taken in chunks of at most 2 GB, one launch each
  const int64_t two_gb = (int64_t)1 << 31;
  if (N * ldb * 2 >= two_gb || N * ld2 * 2 >= two_gb) return hipErrorInvalidValue;
  const int64_t widest = lda > ld2 ? lda : ld2;
  int64_t chunk = (two_gb - 1) / (widest * 2);
  chunk = chunk / TM * TM;
  if (chunk < TM) return hipErrorInvalidValue;
  for (int64_t r0 = 0; r0 < M; r0 += chunk) {
    const int64_t rows = M - r0 < chunk ? M - r0 : chunk;
    hipError_t e = launch_gemm_nt_rows(A + r0 * lda, lda, B, ldb, rows, N, K, A2 ? A2 + r0 * ld2 : nullptr, B2, ld2,
                                       K2, C + r0 * ldc, ldc, alpha, stream, E ? E + r0 * lde : nullptr, lde);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qlora
