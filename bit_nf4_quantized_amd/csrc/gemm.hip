// bf16 MFMA GEMM for the QLoRA linear layer on gfx950, with the NF4 double
// dequantisation fused into the staging of the weight tile.
//
// The layer (QLoRA pages, diycv.top, section 关键公式 and section 问题背景):
//   forward   Y  = X dequant(Wt)^T + s (X L1) L2
//   backward  dX = dY dequant(Wt) + s (dY L2^T) L1^T,
//             dL1 = s X^T (dY L2^T),  dL2 = s (X L1)^T dY   (no weight gradient)
//
// One kernel template computes C[M][N] = sum_k A[m][k] B[n][k] over a
// reduction range, optionally followed by a LoRA "slab" C += A2 B2^T of
// reduction length r, so that the adapter term of Y and dX is accumulated in
// the same fp32 registers as the base product and rounded to bf16 once.
//   A modes: A_ROW  A[m][k] stored row-major with k contiguous
//            A_COL  A stored as [k][m] (m contiguous), transposed while staging
//   B modes: B_ROW  B[n][k], k contiguous
//            B_COL  B stored as [k][n], transposed while staging
//            B_NF4T B[k][n] = dequant(Wt)[n][k] (the dX product reduces over
//                   the weight's rows): each thread dequantises an 8-row x
//                   4-column patch and writes it transposed
//
// Tiling: 256 threads (4 waves, 2 x 2), 128 x 128 output tile, K-step 64,
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, double-buffered LDS
// tiles [rows][64] with the 16-byte chunks XOR-swizzled by (row & 7) so that
// the fragment reads of 8 consecutive rows hit distinct banks. Global loads
// of step k+1 are issued before the MFMAs of step k; the weight tile is
// dequantised after them.
#include <initializer_list>

#include "common.h"
#include "launch.h"

namespace qlora {

namespace {

enum { A_ROW = 0, A_COL = 1 };
enum { B_ROW = 0, B_COL = 1, B_NF4T = 3 };
enum { EPI_BF16 = 0, EPI_F32 = 1 };

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NT = 256;

struct GemmArgs {
  int64_t M, N;      // output rows and columns
  int64_t K;         // main reduction length
  int64_t k_split;   // main reduction length handled per blockIdx.z (multiple of BK)
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  NF4View W;         // B_NF4T
  const uint16_t* A2;  // slab: A2[m][j], j < r, row stride r
  const uint16_t* B2;  // slab: B2[n][j], j < r, row stride r
  int r;
  void* C;
  int64_t ldc;
  float alpha;       // EPI_BF16 scale
  NF4Table tab;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

// ---- bf16 operand staging ---------------------------------------------------

struct RowRegs {
  u32x4_t v[4];
};

// rows [row0, row0+128) of a row-major matrix with the reduction contiguous.
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ P, int64_t ld, int64_t row0,
                                         int64_t nrows, int64_t k0, int64_t kend, RowRegs& R) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NT * i;
    const int row = c >> 3, ch = c & 7;
    const int64_t gr = row0 + row, gk = k0 + ch * 8;
    if (gr < nrows && gk < kend)
      R.v[i] = *reinterpret_cast<const u32x4_t*>(P + gr * ld + gk);
    else
      R.v[i] = u32x4_t{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void store_row(uint16_t* __restrict__ S, const RowRegs& R) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NT * i;
    const int row = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4_t*>(S + swz(row, ch)) = R.v[i];
  }
}

// tile columns [x0, x0+128) of a matrix stored [k][x] (x contiguous).
__device__ __forceinline__ void load_col(const uint16_t* __restrict__ P, int64_t ld, int64_t x0,
                                         int64_t nx, int64_t k0, int64_t kend, RowRegs& R) {
  const int tid = threadIdx.x;
  const int kq = tid >> 4, xq = tid & 15;
  const int64_t gx = x0 + xq * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gk = k0 + kq * 4 + i;
    if (gk < kend && gx < nx)
      R.v[i] = *reinterpret_cast<const u32x4_t*>(P + gk * ld + gx);
    else
      R.v[i] = u32x4_t{0, 0, 0, 0};
  }
}

__device__ __forceinline__ uint32_t half_of(const u32x4_t& v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

__device__ __forceinline__ void store_col(uint16_t* __restrict__ S, const RowRegs& R) {
  const int tid = threadIdx.x;
  const int kq = tid >> 4, xq = tid & 15;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = xq * 8 + e;
    const uint32_t p0 = half_of(R.v[0], e) | (half_of(R.v[1], e) << 16);
    const uint32_t p1 = half_of(R.v[2], e) | (half_of(R.v[3], e) << 16);
    *reinterpret_cast<u32x2_t*>(S + swz(row, kq >> 1) + (kq & 1) * 4) = u32x2_t{p0, p1};
  }
}

// ---- NF4 weight staging -------------------------------------------------------

struct NF4TRegs {
  uint32_t code16[8];  // 4 codes (2 bytes) of each of 8 weight rows
  float ap[8];
};

// B_NF4T: output columns = weight columns [c0, c0+128), reduction = weight
// rows [n0, n0+64). Thread: 4 consecutive columns x 8 consecutive rows.
__device__ __forceinline__ void load_nf4t(const NF4View& W, float mu, int64_t c0, int64_t n0, NF4TRegs& R) {
  const int tid = threadIdx.x;
  const int kq = tid & 31, ng8 = tid >> 5;
  const int64_t kw = W.cols;
  const int64_t gc = c0 + kq * 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t gn = n0 + ng8 * 8 + i;
    if (gn < W.rows && gc < kw) {
      R.code16[i] = *reinterpret_cast<const uint16_t*>(W.codes + gn * (kw >> 1) + (gc >> 1));
      const int64_t blk = gn * (kw / kBlock) + gc / kBlock;
      R.ap[i] = block_const(W, blk, mu);
    } else {
      R.code16[i] = 0x7777u;
      R.ap[i] = 0.0f;
    }
  }
}

__device__ __forceinline__ void store_nf4t(uint16_t* __restrict__ S, const float* __restrict__ sq,
                                           const NF4TRegs& R) {
  const int tid = threadIdx.x;
  const int kq = tid & 31, ng8 = tid >> 5;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float lo = sq[(R.code16[2 * p] >> (4 * kk)) & 15u] * R.ap[2 * p];
      const float hi = sq[(R.code16[2 * p + 1] >> (4 * kk)) & 15u] * R.ap[2 * p + 1];
      o[p] = pack_bf16x2(lo, hi);
    }
    const int row = kq * 4 + kk;
    *reinterpret_cast<u32x4_t*>(S + swz(row, ng8)) = u32x4_t{o[0], o[1], o[2], o[3]};
  }
}

// ---- the kernel ----------------------------------------------------------------

template <int AM, int BMODE, int EPI, bool SLAB>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
  __shared__ float sQ[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t kz0 = (int64_t)blockIdx.z * p.k_split;
  const int64_t kz1 = (kz0 + p.k_split < p.K) ? kz0 + p.k_split : p.K;
  const int nmain = kz0 < kz1 ? (int)((kz1 - kz0 + BK - 1) / BK) : 0;
  const int nslab = SLAB ? (p.r + BK - 1) / BK : 0;
  const int nsteps = nmain + nslab;

  float mu = 0.0f;
  if constexpr (BMODE == B_NF4T) {
    if (tid < 16) sQ[tid] = p.tab.q[tid];
    mu = tensor_mean(p.W);
  }

  RowRegs ra, rb;
  NF4TRegs rt;

  auto load_step = [&](int st) {
    if (st < nmain) {
      const int64_t k0 = kz0 + (int64_t)st * BK;
      if constexpr (AM == A_ROW) load_row(p.A, p.lda, m0, p.M, k0, kz1, ra);
      else load_col(p.A, p.lda, m0, p.M, k0, kz1, ra);
      if constexpr (BMODE == B_ROW) load_row(p.B, p.ldb, n0, p.N, k0, kz1, rb);
      else if constexpr (BMODE == B_COL) load_col(p.B, p.ldb, n0, p.N, k0, kz1, rb);
      else load_nf4t(p.W, mu, n0, k0, rt);
    } else {
      const int64_t j0 = (int64_t)(st - nmain) * BK;
      load_row(p.A2, p.r, m0, p.M, j0, p.r, ra);
      load_row(p.B2, p.r, n0, p.N, j0, p.r, rb);
    }
  };
  auto store_step = [&](int st, int buf) {
    if (st < nmain) {
      if constexpr (AM == A_ROW) store_row(sA[buf], ra);
      else store_col(sA[buf], ra);
      if constexpr (BMODE == B_ROW) store_row(sB[buf], rb);
      else if constexpr (BMODE == B_COL) store_col(sB[buf], rb);
      else store_nf4t(sB[buf], sQ, rt);
    } else {
      store_row(sA[buf], ra);
      store_row(sB[buf], rb);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  __syncthreads();  // sQ visible
  if (nsteps > 0) {
    load_step(0);
    store_step(0, 0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      const int buf = st & 1;
      if (st + 1 < nsteps) load_step(st + 1);
      const uint16_t* a_s = sA[buf];
      const uint16_t* b_s = sB[buf];
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        bf16x8_t af[2], bfr[2];
        const int ch = 2 * s + (lane >> 5);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int ra_row = wm * 64 + t * 32 + (lane & 31);
          const int rb_row = wn * 64 + t * 32 + (lane & 31);
          af[t] = *reinterpret_cast<const bf16x8_t*>(a_s + swz(ra_row, ch));
          bfr[t] = *reinterpret_cast<const bf16x8_t*>(b_s + swz(rb_row, ch));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (st + 1 < nsteps) store_step(st + 1, buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: lane l, register v of a 32x32 tile holds row (v%4) + 4(l/32) + 8(v/4), column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + (v & 3) + 4 * (lane >> 5) + 8 * (v >> 2);
        if (row < p.M && col < p.N) {
          if constexpr (EPI == EPI_BF16) {
            static_cast<uint16_t*>(p.C)[row * p.ldc + col] = f32_to_bf16(p.alpha * acc[i][j][v]);
          } else {
            float* Cz = static_cast<float*>(p.C) + (int64_t)blockIdx.z * p.M * p.ldc;
            Cz[row * p.ldc + col] = acc[i][j][v];
          }
        }
      }
    }
  }
}

// Fixed-order split-K reduction of partials P[z][rows][cols]:
//   out[m][j]  = alpha  * sum_z P[z][m][j]   (bf16 or fp32, row stride ldo;
//                columns [cols, ldo) of a bf16 out are zero-filled)
//   out2[m][j] = bf16(alpha2 * sum)          (optional, row stride cols)
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int Z, int64_t rows,
                                                            int64_t cols, float alpha, void* __restrict__ out,
                                                            int out_bf16, int64_t ldo, float alpha2,
                                                            uint16_t* __restrict__ out2) {
  const int64_t count = rows * cols;
  const int64_t total = rows * ldo;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / ldo, j = i - m * ldo;
    if (j >= cols) {  // padding columns of a bf16 slab operand
      static_cast<uint16_t*>(out)[i] = 0;
      continue;
    }
    const int64_t src = m * cols + j;
    float acc = 0.0f;
    for (int z = 0; z < Z; ++z) acc += P[(int64_t)z * count + src];
    const float v = alpha * acc;
    if (out_bf16) static_cast<uint16_t*>(out)[i] = f32_to_bf16(v);
    else static_cast<float*>(out)[i] = v;
    if (out2) out2[src] = f32_to_bf16(alpha2 * acc);
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// dst[c][r] = src[r][c] for a bf16 [R][C] matrix; dst rows have stride ldd
// >= R and columns [R, ldd) are zero.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int64_t R,
                                                             int64_t C, uint16_t* __restrict__ dst, int64_t ldd) {
  __shared__ uint16_t tile[32][33];
  const int64_t c0 = (int64_t)blockIdx.x * 32, r0 = (int64_t)blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int y = ty; y < 32; y += 8) {
    const int64_t r = r0 + y, c = c0 + tx;
    tile[y][tx] = (r < R && c < C) ? src[r * C + c] : 0;
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int64_t c = c0 + y, r = r0 + tx;
    if (r < ldd && c < C) dst[c * ldd + r] = tile[tx][y];
  }
}

// Two independent transposes of the kind above in one launch (the adapter
// matrices are small, so each alone is mostly launch latency): workgroups
// [0, a.tiles) take job a, the rest job b; tiles are 32 x 32, row-major
// over (src columns / 32) x (dst columns / 32).
struct TransposeJob {
  const uint16_t* src;
  int64_t R, C;
  uint16_t* dst;
  int64_t ldd;
  int gx, tiles;  // tiles along src columns; gx * (tiles along dst columns)
};

TransposeJob transpose_job(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst, int64_t ldd) {
  TransposeJob j{src, R, C, dst, ldd, (int)((C + 31) / 32), 0};
  j.tiles = j.gx * (int)((ldd + 31) / 32);
  return j;
}

__global__ __launch_bounds__(256) void transpose2_kernel(TransposeJob a, TransposeJob b) {
  __shared__ uint16_t tile[32][33];
  const bool first = (int)blockIdx.x < a.tiles;  // uniform per workgroup
  const TransposeJob& j = first ? a : b;
  const int id = first ? (int)blockIdx.x : (int)blockIdx.x - a.tiles;
  const int64_t c0 = (int64_t)(id % j.gx) * 32, r0 = (int64_t)(id / j.gx) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int y = ty; y < 32; y += 8) {
    const int64_t r = r0 + y, c = c0 + tx;
    tile[y][tx] = (r < j.R && c < j.C) ? j.src[r * j.C + c] : 0;
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int64_t c = c0 + y, r = r0 + tx;
    if (r < j.ldd && c < j.C) j.dst[c * j.ldd + r] = tile[tx][y];
  }
}

// dst[r][c] = src[r][c] for c < C, 0 for C <= c < ldd (bf16).
__global__ __launch_bounds__(256) void pad_cols_kernel(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                                       uint16_t* __restrict__ dst, int64_t ldd) {
  const int64_t total = R * ldd;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / ldd, c = i - r * ldd;
    dst[i] = c < C ? src[r * C + c] : 0;
  }
}

template <int AM, int BMODE, int EPI, bool SLAB>
hipError_t run_gemm(const GemmArgs& a, int Z, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM), (unsigned)Z);
  hipLaunchKernelGGL((gemm_kernel<AM, BMODE, EPI, SLAB>), grid, dim3(NT), 0, stream, a);
  return hipGetLastError();
}

// Split of a reduction of length klen over Z slices so that tiles * Z fills
// the chip; each slice is a multiple of BK.
struct Split {
  int Z;
  int64_t k_split;
};

Split choose_split(int64_t tiles, int64_t klen) {
  const int64_t steps = (klen + BK - 1) / BK;
  if (tiles < 1) tiles = 1;
  if (steps < 1) return Split{1, BK};
  int64_t z = (512 + tiles - 1) / tiles;
  if (z > 16) z = 16;
  const int64_t max_z = steps / 4 > 0 ? steps / 4 : 1;
  if (z > max_z) z = max_z;
  if (z < 1) z = 1;
  const int64_t per = (steps + z - 1) / z;
  Split s;
  s.k_split = per * BK;
  s.Z = (int)((steps + per - 1) / per);
  if (s.Z < 1) s.Z = 1;
  return s;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

hipError_t reduce(const float* P, int Z, int64_t rows, int64_t cols, float alpha, void* out, bool out_bf16,
                  int64_t ldo, float alpha2, uint16_t* out2, hipStream_t stream) {
  int64_t blocks = cdiv(rows * ldo, 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, P, Z, rows, cols, alpha,
                     out, out_bf16 ? 1 : 0, ldo, alpha2, out2);
  return hipGetLastError();
}

int64_t grid_for(int64_t total) {
  int64_t b = cdiv(total, 256);
  if (b > 4096) b = 4096;
  return b < 1 ? 1 : b;
}

GemmArgs base_args() {
  GemmArgs a = {};
  a.alpha = 1.0f;
  return a;
}

}  // namespace

size_t small_t_partial_bytes(int64_t M, int64_t K, int r);
hipError_t launch_small_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, float s,
                                  uint16_t* sT, int64_t ldst, uint16_t* T_out, float* part, hipStream_t stream);
hipError_t launch_gemv(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M,
                       const uint16_t* sT, const uint16_t* L2, int r, uint16_t* Y, hipStream_t stream);
int small_t_slices(int64_t K);
hipError_t launch_small_t_partial(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, float* part,
                                  hipStream_t stream);
bool gemv_fuses_t(const NF4View& W, int64_t M, int r);
hipError_t launch_gemv_fused_t(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M,
                               const float* part, int Z, float s, uint16_t* T_out, const uint16_t* L2, int r,
                               uint16_t* Y, hipStream_t stream);

LinearWorkspace linear_workspace_layout(int64_t M, int64_t K, int64_t N, int r, bool dropout) {
  LinearWorkspace L;
  const int64_t mtiles = cdiv(M, BM);
  const int64_t rp = cdiv(r, 64) * 64;  // LoRA slab width, zero-padded to the GEMM K-stage
  const int64_t np = cdiv(N, 64) * 64;
  const Split sT = choose_split(mtiles * cdiv(r, BN), K);
  const Split sU = choose_split(mtiles * cdiv(r, BN), N);
  const Split s1 = choose_split(cdiv(K, BM) * cdiv(r, BN), M);
  const Split s2 = choose_split(cdiv(r, BM) * cdiv(N, BN), M);
  size_t part = 0;
  auto upd = [&](size_t b) { part = b > part ? b : part; };
  upd((size_t)sT.Z * M * r * 4);
  upd((size_t)sU.Z * M * r * 4);
  upd((size_t)s1.Z * K * r * 4);
  upd((size_t)s2.Z * r * N * 4);
  size_t off = 0;
  L.l2t_off = off; off += align_up((size_t)N * rp * 2, 256);
  L.l1p_off = off; off += align_up((size_t)K * rp * 2, 256);
  L.st_off = off;  off += align_up((size_t)M * rp * 2, 256);
  L.t_off = off;   off += align_up((size_t)M * r * 2, 256);
  L.su_off = off;  off += align_up((size_t)M * rp * 2, 256);
  L.l1t_off = off; off += align_up((size_t)64 * K * 2, 256);
  L.l2p_off = off; off += align_up((size_t)64 * N * 2, 256);
  if (r <= 64) upd(skinny_partial_bytes(M, K, N));
  if (M <= kMidMaxM) upd(small_t_partial_bytes(M, K, r));
  if (M == 1) upd(gemv1_partial_bytes(K, r));
  upd(midm_partial_bytes(M, K, N));
  L.part_off = off; L.part_bytes = align_up(part, 256); off += L.part_bytes;
  // dense path: the dequantised weight (forward [N][K], backward [K][np])
  L.wd_off = off;
  L.wd_bytes = M > 16 ? align_up((size_t)K * (size_t)(np > N ? np : N) * 2, 256) : 0;
  off += L.wd_bytes;
  L.xd_off = L.dd_off = off;
  if (dropout) {
    L.xd_off = off; off += align_up((size_t)M * K * 2, 256);
    L.dd_off = off; off += align_up((size_t)M * K * 4, 256);
  }
  L.total = off > 0 ? off : 256;
  return L;
}

namespace {

// Dense (dequantise-then-GEMM) path limits: every operand of the NT GEMM is
// addressed with 32-bit per-lane offsets.
bool fits_dense(std::initializer_list<int64_t> bytes) {
  for (int64_t b : bytes)
    if (b >= ((int64_t)1 << 31)) return false;
  return true;
}

}  // namespace

// The skinny adapter kernels take rank <= 64 and address the streamed
// activation with 32-bit offsets.
static bool skinny_ok(int r, int64_t M, int64_t cols) { return r <= 64 && fits_dense({M * cols * 2}); }

// L1t[j][k] = L1[k][j] for j < r, zero rows for r <= j < 64 (the B operand of
// the skinny T product).
static hipError_t make_l1t(const uint16_t* L1, int64_t K, int r, uint16_t* l1t, hipStream_t stream) {
  if (r < 64) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)grid_for((64 - r) * K / 2)), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(l1t + (int64_t)r * K), (size_t)((64 - r) * K / 2));
  }
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)cdiv(r, 32), (unsigned)cdiv(K, 32)), dim3(256), 0, stream,
                     L1, K, (int64_t)r, l1t, K);
  return hipGetLastError();
}

// T = X L1 (fp32 split-K partials), then sT = bf16(s T) with row stride ldst
// (zero-padded columns) and optionally T_out = bf16(T) [M][r].
// dr (skinny path only): X is dropped in the skinny kernel's registers.
static hipError_t lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, float s,
                            uint16_t* sT, int64_t ldst, uint16_t* T_out, float* part, uint16_t* l1t,
                            hipStream_t stream, const DropoutParams* dr = nullptr, bool l1t_ready = false) {
  if (skinny_ok(r, M, K)) {
    hipError_t e = l1t_ready ? hipSuccess : make_l1t(L1, K, r, l1t, stream);
    if (e != hipSuccess) return e;
    return skinny_nt(X, K, l1t, K, M, K, r, part, s, sT, ldst, 1.0f, T_out, stream, dr);
  }
  if (dr) return hipErrorInvalidValue;
  GemmArgs a = base_args();
  a.M = M; a.N = r; a.K = K;
  a.A = X; a.lda = K;
  a.B = L1; a.ldb = r;
  const Split sp = choose_split(cdiv(M, BM) * cdiv(r, BN), K);
  a.k_split = sp.k_split;
  a.C = part; a.ldc = r;
  hipError_t e = run_gemm<A_ROW, B_COL, EPI_F32, false>(a, sp.Z, stream);
  if (e != hipSuccess) return e;
  return reduce(part, sp.Z, M, r, s, sT, true, ldst, 1.0f, T_out, stream);
}

SmallForwardScratch small_forward_scratch(int64_t M, int64_t K, int r) {
  SmallForwardScratch S;
  S.st_off = 0;
  S.part_off = align_up((size_t)M * r * 2, 256);
  const size_t pb = small_t_partial_bytes(M, K, r), p1 = gemv1_partial_bytes(K, r);
  S.total = S.part_off + align_up(pb > p1 ? pb : p1, 256);
  return S;
}

hipError_t linear_forward_small(const NF4View& W, const NF4Table& tab, const uint16_t* X, const uint16_t* Xa,
                                int64_t M, const uint16_t* L1, const uint16_t* L2, int r, float s, uint16_t* Y,
                                uint16_t* T_out, uint16_t* sT, float* part, hipStream_t stream) {
  if (Xa == X && gemv1_applies(W, M, r)) return launch_gemv1(W, tab, X, L1, L2, r, s, Y, T_out, part, stream);
  if (gemv_fuses_t(W, M, r)) {  // the slice partials of Xa L1 summed inside the GEMV (one launch fewer)
    hipError_t e = launch_small_t_partial(Xa, M, W.cols, L1, r, part, stream);
    if (e != hipSuccess) return e;
    return timed(kTimeGemv, stream, [&] {
      return launch_gemv_fused_t(W, tab, X, M, part, small_t_slices(W.cols), s, T_out, L2, r, Y, stream);
    });
  }
  hipError_t e = launch_small_lora_down(Xa, M, W.cols, L1, r, s, sT, r, T_out, part, stream);
  if (e != hipSuccess) return e;
  return timed(kTimeGemv, stream, [&] { return launch_gemv(W, tab, X, M, sT, L2, r, Y, stream); });
}

hipError_t linear_forward(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M,
                          const uint16_t* L1, const uint16_t* L2, int r, float s, uint16_t* Y,
                          uint16_t* T_out, void* ws, hipStream_t stream, const DropoutParams* dr) {
  const int64_t K = W.cols, N = W.rows;
  if (M == 0) return hipSuccess;
  const LinearWorkspace L = linear_workspace_layout(M, K, N, r, dr != nullptr);
  // the adapter branch's input: X, or its dropped copy. On the large-M path
  // with the skinny T kernel, that kernel drops X in registers and no copy
  // is written.
  const bool large_m = M > 16 && !(M <= kMidMaxM && midm_fits(M, K, N));
  const bool drop_in_t = dr && large_m && skinny_ok(r, M, K);
  const uint16_t* Xa = X;
  if (dr && !drop_in_t) {
    uint16_t* xd = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + L.xd_off);
    hipError_t e = launch_dropout_input(X, M * K, *dr, xd, stream);
    if (e != hipSuccess) return e;
    Xa = xd;
  }
  const int64_t rp = cdiv(r, 64) * 64;
  char* base = static_cast<char*>(ws);
  uint16_t* l2t = reinterpret_cast<uint16_t*>(base + L.l2t_off);
  uint16_t* sT = reinterpret_cast<uint16_t*>(base + L.st_off);
  float* part = reinterpret_cast<float*>(base + L.part_off);

  uint16_t* l1t = reinterpret_cast<uint16_t*>(base + L.l1t_off);
  if (M <= 16) return linear_forward_small(W, tab, X, Xa, M, L1, L2, r, s, Y, T_out, sT, part, stream);

  if (M <= kMidMaxM && midm_fits(M, K, N)) {   // batched decode: one pass over the 4-bit weight
    hipError_t e = launch_small_lora_down(Xa, M, K, L1, r, s, sT, rp, T_out, part, stream);
    if (e != hipSuccess) return e;
    return timed(kTimeMidGemm, stream, [&] { return launch_midm(W, tab, X, M, sT, L2, r, (int)rp, part, Y, stream); });
  }

  // the dequantised weight and L2^T are addressed with 32-bit offsets (the
  // token dimension is cut into chunks inside launch_gemm_nt); larger
  // weights are refused by the C ABI before anything is enqueued
  if (!fits_dense({N * K * 2, N * rp * 2})) return hipErrorInvalidValue;
  const int64_t ldst = rp;
  // L2^T for the GEMM's slab stage, and with the skinny T kernel also L1^T,
  // in one launch
  const bool skinny_t = skinny_ok(r, M, K);
  const TransposeJob jl2 = transpose_job(L2, (int64_t)r, N, l2t, ldst);
  if (skinny_t) {
    if (r < 64)  // rows r .. 63 of L1^T are zero
      hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)grid_for((64 - r) * K / 2)), dim3(256), 0, stream,
                         reinterpret_cast<uint32_t*>(l1t + (int64_t)r * K), (size_t)((64 - r) * K / 2));
    const TransposeJob jl1 = transpose_job(L1, K, (int64_t)r, l1t, K);
    hipLaunchKernelGGL(transpose2_kernel, dim3((unsigned)(jl1.tiles + jl2.tiles)), dim3(256), 0, stream, jl1, jl2);
  } else {
    hipLaunchKernelGGL(transpose2_kernel, dim3((unsigned)jl2.tiles), dim3(256), 0, stream, jl2, jl2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = lora_down(Xa, M, K, L1, r, s, sT, ldst, T_out, part, l1t, stream, drop_in_t ? dr : nullptr, skinny_t);
  if (e != hipSuccess) return e;

  uint16_t* wd = reinterpret_cast<uint16_t*>(base + L.wd_off);
  e = launch_dequant_rows(W, tab, wd, stream);
  if (e != hipSuccess) return e;
  return timed(kTimeFwdGemm, stream, [&] {
    return launch_gemm_nt(X, K, wd, K, M, N, K, sT, l2t, rp, rp, Y, N, 1.0f, stream);
  });
}

bool linear_forward_supported(int64_t M, int64_t K, int64_t N, int r) {
  if (M <= 16 || (M <= kMidMaxM && midm_fits(M, K, N))) return true;
  const int64_t rp = cdiv(r, 64) * 64;
  return fits_dense({N * K * 2, N * rp * 2});
}

hipError_t linear_backward(const NF4View& W, const NF4Table& tab, const uint16_t* X, const uint16_t* dY,
                           int64_t M, const uint16_t* L1, const uint16_t* L2, int r, float s,
                           const uint16_t* T, uint16_t* dX, void* dL1, void* dL2, bool grad_bf16,
                           void* ws, hipStream_t stream, const DropoutParams* dr) {
  const int64_t K = W.cols, N = W.rows;
  const LinearWorkspace L = linear_workspace_layout(M, K, N, r, dr != nullptr);
  const int64_t rp = cdiv(r, 64) * 64;
  char* base = static_cast<char*>(ws);
  uint16_t* tbuf = reinterpret_cast<uint16_t*>(base + L.t_off);
  uint16_t* sT = reinterpret_cast<uint16_t*>(base + L.st_off);
  uint16_t* sU = reinterpret_cast<uint16_t*>(base + L.su_off);
  uint16_t* l1p = reinterpret_cast<uint16_t*>(base + L.l1p_off);
  float* part = reinterpret_cast<float*>(base + L.part_off);
  hipError_t e;

  if (M == 0) {
    // empty batch: the adapter gradients are zero (a fill kernel, not a
    // memset node, so the call stays safe under stream capture)
    const size_t w1 = (size_t)K * r * (grad_bf16 ? 2 : 4) / 4, w2 = (size_t)r * N * (grad_bf16 ? 2 : 4) / 4;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint32_t*>(dL1), w1);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint32_t*>(dL2), w2);
    return hipGetLastError();
  }

  const bool dense = dX && M > 16 && (N % 64) == 0 && fits_dense({K * N * 2, K * rp * 2});
  const int64_t ldsu = dense ? rp : r;
  // the adapter branch's input: X, or its dropped copy (the same mask as the
  // forward). When T comes from the forward and both adapter gradients take
  // the skinny kernels, only dL1 reads the dropped input, and its kernel
  // drops X in registers: no copy is written.
  const bool skinny_grads = skinny_ok(r, M, K) && skinny_ok(r, M, N);
  const bool drop_in_dl1 = dr && T && skinny_grads;
  const uint16_t* Xa = X;
  float* dd = reinterpret_cast<float*>(base + L.dd_off);
  if (dr && !drop_in_dl1) {
    uint16_t* xd = reinterpret_cast<uint16_t*>(base + L.xd_off);
    e = launch_dropout_input(X, M * K, *dr, xd, stream);
    if (e != hipSuccess) return e;
    Xa = xd;
  }

  uint16_t* l1t = reinterpret_cast<uint16_t*>(base + L.l1t_off);
  uint16_t* l2p = reinterpret_cast<uint16_t*>(base + L.l2p_off);
  // U = dY L2^T -> sU = bf16(s U)
  if (skinny_ok(r, M, N) && (N % 64) == 0) {
    const uint16_t* b = L2;
    if (r < 64) {  // B operand with 64 rows: L2 then zero rows
      hipLaunchKernelGGL(pad_cols_kernel, dim3((unsigned)grid_for(64 * N)), dim3(256), 0, stream, L2, (int64_t)1,
                         (int64_t)r * N, l2p, (int64_t)64 * N);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      b = l2p;
    }
    e = skinny_nt(dY, N, b, N, M, N, r, part, s, sU, ldsu, 0.0f, nullptr, stream);
    if (e != hipSuccess) return e;
  } else {
    GemmArgs a = base_args();
    a.M = M; a.N = r; a.K = N;
    a.A = dY; a.lda = N;
    a.B = L2; a.ldb = N;
    const Split sp = choose_split(cdiv(M, BM) * cdiv(r, BN), N);
    a.k_split = sp.k_split;
    a.C = part; a.ldc = r;
    e = run_gemm<A_ROW, B_ROW, EPI_F32, false>(a, sp.Z, stream);
    if (e != hipSuccess) return e;
    e = reduce(part, sp.Z, M, r, s, sU, true, ldsu, 0.0f, nullptr, stream);
    if (e != hipSuccess) return e;
  }
  // dX = dY dequant(Wt) + sU L1^T
  if (dX && dense) {
    const uint16_t* l1s = L1;
    if (rp != r) {
      hipLaunchKernelGGL(pad_cols_kernel, dim3((unsigned)grid_for(K * rp)), dim3(256), 0, stream, L1, K,
                         (int64_t)r, l1p, rp);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      l1s = l1p;
    }
    uint16_t* wdt = reinterpret_cast<uint16_t*>(base + L.wd_off);
    e = launch_dequant_cols(W, tab, wdt, N, stream);
    if (e != hipSuccess) return e;
    if (dr) {
      // dropout: the masked LoRA term D in fp32, added in the GEMM's epilogue
      e = launch_masked_lora(sU, ldsu, L1, r, M, K, *dr, nullptr, dd, nullptr, stream);
      if (e != hipSuccess) return e;
      e = timed(kTimeDxGemm, stream, [&] {
        return launch_gemm_nt(dY, N, wdt, N, M, K, N, sU, l1s, rp, 0, dX, K, 1.0f, stream, dd, K);
      });
    } else {
      e = timed(kTimeDxGemm, stream, [&] {
        return launch_gemm_nt(dY, N, wdt, N, M, K, N, sU, l1s, rp, rp, dX, K, 1.0f, stream);
      });
    }
    if (e != hipSuccess) return e;
  } else if (dX && dr) {
    // dropout, small M or ragged N: the main product in fp32, then dX = bf16(main + D)
    GemmArgs a = base_args();
    a.M = M; a.N = K; a.K = N; a.k_split = N;
    a.A = dY; a.lda = N;
    a.W = W; a.tab = tab;
    a.C = dd; a.ldc = K;
    e = timed(kTimeDxGemm, stream, [&] { return run_gemm<A_ROW, B_NF4T, EPI_F32, false>(a, 1, stream); });
    if (e != hipSuccess) return e;
    e = launch_masked_lora(sU, ldsu, L1, r, M, K, *dr, dd, nullptr, dX, stream);
    if (e != hipSuccess) return e;
  } else if (dX) {
    GemmArgs a = base_args();
    a.M = M; a.N = K; a.K = N; a.k_split = N;
    a.A = dY; a.lda = N;
    a.W = W; a.tab = tab;
    a.A2 = sU; a.B2 = L1; a.r = r;
    a.C = dX; a.ldc = K;
    e = timed(kTimeDxGemm, stream, [&] { return run_gemm<A_ROW, B_NF4T, EPI_BF16, true>(a, 1, stream); });
    if (e != hipSuccess) return e;
  }
  // T = bf16(X L1) unless the caller kept it from the forward pass
  if (!T) {
    e = lora_down(Xa, M, K, L1, r, 1.0f, tbuf, r, nullptr, part, l1t, stream);
    if (e != hipSuccess) return e;
    T = tbuf;
  }
  if (skinny_grads) {
    // dL1 = X^T sU  ([K][r]);  dL2 = s (dY^T T)^T  ([r][N])
    e = skinny_tn(Xa, K, K, sU, ldsu, M, r, part, 1.0f, false, grad_bf16, dL1, stream,
                  drop_in_dl1 ? dr : nullptr);
    if (e != hipSuccess) return e;
    return skinny_tn(dY, N, N, T, r, M, r, part, s, true, grad_bf16, dL2, stream);
  }
  // dL1 = X^T sU
  {
    GemmArgs a = base_args();
    a.M = K; a.N = r; a.K = M;
    a.A = Xa; a.lda = K;
    a.B = sU; a.ldb = ldsu;
    const Split sp = choose_split(cdiv(K, BM) * cdiv(r, BN), M);
    a.k_split = sp.k_split;
    a.C = part; a.ldc = r;
    e = run_gemm<A_COL, B_COL, EPI_F32, false>(a, sp.Z, stream);
    if (e != hipSuccess) return e;
    e = reduce(part, sp.Z, K, r, 1.0f, dL1, grad_bf16, r, 0.0f, nullptr, stream);
    if (e != hipSuccess) return e;
  }
  // dL2 = s T^T dY
  {
    GemmArgs a = base_args();
    a.M = r; a.N = N; a.K = M;
    a.A = T; a.lda = r;
    a.B = dY; a.ldb = N;
    const Split sp = choose_split(cdiv(r, BM) * cdiv(N, BN), M);
    a.k_split = sp.k_split;
    a.C = part; a.ldc = N;
    e = run_gemm<A_COL, B_COL, EPI_F32, false>(a, sp.Z, stream);
    if (e != hipSuccess) return e;
    e = reduce(part, sp.Z, r, N, s, dL2, grad_bf16, N, 0.0f, nullptr, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qlora
