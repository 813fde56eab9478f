// Internal (C++) interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace qlora {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Optional per-thread event brackets around one kernel class (measurement
// only; see qlora_set_timing). Classes match the QLORA_TIMING_* constants.
enum TimingClass { kTimeFwdGemm = 0, kTimeDxGemm = 1, kTimeGemv = 2, kTimeQuant = 3, kTimeDequant = 4,
                   kTimeMidGemm = 5, kTimeClasses = 6 };

struct TimingSlot {
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
  int n = 0;
  int* count = nullptr;
};

TimingSlot* timing_slots();  // thread-local array of kTimeClasses slots

// Records start before and stop after `launch()` when the class is being timed.
template <typename F>
hipError_t timed(int cls, hipStream_t stream, F&& launch) {
  TimingSlot& t = timing_slots()[cls];
  const bool on = t.n > 0 && t.count && *t.count < t.n;
  if (on) {
    hipError_t e = hipEventRecord(t.start[*t.count], stream);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (on) {
    e = hipEventRecord(t.stop[*t.count], stream);
    if (e != hipSuccess) return e;
    ++*t.count;
  }
  return hipSuccess;
}

// Scratch of qlora_quantize: fp32 block absmax values and two float64 arrays
// for the per-group tree sums and their fold.
struct QuantWorkspace {
  size_t absmax_off, sum_a_off, sum_b_off, total;
};

inline QuantWorkspace quant_workspace_layout(int64_t numel) {
  const size_t nb = (size_t)((numel + kBlock - 1) / kBlock);
  const size_t ng = (nb + kDqBlock - 1) / kDqBlock;
  QuantWorkspace L;
  L.absmax_off = 0;
  L.sum_a_off = align_up(nb * sizeof(float), 256);
  L.sum_b_off = L.sum_a_off + align_up(ng * sizeof(double), 256);
  L.total = L.sum_b_off + align_up(ng * sizeof(double), 256);
  if (L.total == 0) L.total = 256;
  return L;
}

// absmax32 != nullptr: no double quantisation, the block absmax goes there
// (absmax8, scale2 and mean are not touched)
hipError_t launch_quantize(const void* w, bool bf16_in, int64_t numel, const NF4Thresholds& th,
                           uint8_t* codes, uint8_t* absmax8, float* scale2, float* mean, float* absmax32,
                           void* ws, hipStream_t stream);

// Several tensors in one pass: one launch of the block kernel over all their
// DQ groups, one fold launch (a workgroup per tensor), one E4M3 launch.
// Every tensor's arithmetic is that of launch_quantize on it alone.
// absmax32 != null: that tensor keeps fp32 block constants (no DQ passes).
// ws: the tensor's own scratch, quant_workspace_layout(numel).total bytes.
constexpr int kQuantBatchMax = 16;
struct QuantItem {
  const void* w;
  int64_t numel;
  uint8_t* codes;
  uint8_t* absmax8;
  float* scale2;
  float* mean;
  float* absmax32;
  void* ws;
};
hipError_t launch_quantize_batch(const QuantItem* items, int n, bool bf16_in, const NF4Thresholds& th,
                                 hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* absmax8, const float* scale2,
                             const float* mean, const float* absmax32, const NF4Table& tab, int64_t numel,
                             uint16_t* out, hipStream_t stream);

// Blockwise Int8 absmax codec (int8.hip); blocks of 2^block_log2 elements,
// block_log2 in [6, 12].
hipError_t launch_int8_quantize(const void* x, bool bf16_in, int64_t numel, int block_log2, int8_t* codes,
                                float* absmax, hipStream_t stream);
hipError_t launch_int8_dequantize(const int8_t* codes, const float* absmax, int64_t numel, int block_log2,
                                  void* out, bool bf16_out, hipStream_t stream);

// Views of a quantised weight for the GEMM kernels.
struct NF4View {
  const uint8_t* codes;
  const uint8_t* absmax8;
  const float* scale2;
  const float* mean;
  int64_t rows, cols;       // stored [rows][cols]
  const float* absmax32;    // without double quantisation: the fp32 block absmax (else nullptr)
};

// First-level constant a' of block blk: the fp32 absmax itself without
// double quantisation, else the doubleDequant of its 8-bit code.
__device__ __forceinline__ float block_const(const NF4View& W, int64_t blk, float mu) {
  return W.absmax32 ? W.absmax32[blk] : block_scale(W.absmax8[blk], W.scale2[blk / kDqBlock], mu);
}

// The DQ mean (unused, 0, without double quantisation).
__device__ __forceinline__ float tensor_mean(const NF4View& W) { return W.absmax32 ? 0.0f : W.mean[0]; }

// Compute units of the current device, queried once (every device this
// library runs on is the same part); 256 if the query fails.
inline int device_cu_count() {
  static int cus = 0;
  if (cus <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cus = n;
    (void)hipGetLastError();
    if (cus <= 0) cus = 256;
  }
  return cus;
}

// Forward for 16 < M <= kMidMaxM (midm.hip): fused dequant-GEMM over K-slices
// plus a fixed-order reduction; sT = bf16(s X L1) [M][rp] (columns < r
// used), L2 [r][N]; part holds midm_partial_bytes.
constexpr int kMidMaxM = 128;
size_t midm_partial_bytes(int64_t M, int64_t K, int64_t N);
bool midm_fits(int64_t M, int64_t K, int64_t N);   // sizes the kernel's 32-bit offsets cover
hipError_t launch_midm(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M, const uint16_t* sT,
                       const uint16_t* L2, int r, int rp, float* part, uint16_t* Y, hipStream_t stream);

// Optimiser step (optim.hip). part: 1024 doubles of workspace.
struct AdamHyper {
  float lr, beta1, beta2, eps, wd;
  int64_t step;
};
hipError_t launch_clip_norm(const float* g, int64_t n, double max_norm, float* coef, double* norm, double* part,
                            hipStream_t stream);
hipError_t launch_adam(float* theta, const float* g, float* m, float* v, int64_t n, const AdamHyper& h,
                       const float* coef, uint16_t* theta_bf16, hipStream_t stream);

// Adapter merge into the bf16 dequantised base (merge.hip).
hipError_t launch_merge(const NF4View& W, const NF4Table& tab, const uint16_t* L1, const uint16_t* L2, int r,
                        float s, uint16_t* out, hipStream_t stream);

// LoRA dropout (dropout.hip): keep iff the element's Philox word >= thr,
// kept values scaled by c.
struct DropoutParams {
  uint32_t thr;    // floor(p 2^32)
  float c;         // RN32(1 / (1 - p))
  uint64_t seed;
};

// Skinny adapter products (rank <= 64), skinny_gemm.hip.
struct SkinnySplit {
  int Z;        // reduction slices
  int64_t len;  // reduction length per slice (multiple of 64)
};
SkinnySplit skinny_split(int64_t tiles, int64_t klen, int64_t fit = 0);
size_t skinny_partial_bytes(int64_t M, int64_t K, int64_t N);
// dr: A is the adapter input X ([M][K], lda == K), dropped in registers.
hipError_t skinny_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t K, int r,
                     float* part, float alpha, uint16_t* out, int64_t ldo, float alpha2, uint16_t* out2,
                     hipStream_t stream, const DropoutParams* dr = nullptr);
// dr: L is the adapter input X ([M][W], ldl == W), dropped in registers.
hipError_t skinny_tn(const uint16_t* L, int64_t ldl, int64_t W, const uint16_t* S, int64_t lds, int64_t M, int r,
                     float* part, float alpha, bool transpose, bool out_bf16, void* out, hipStream_t stream,
                     const DropoutParams* dr = nullptr);

// Workspace of the linear layer (shared by forward and backward).
struct LinearWorkspace {
  size_t l2t_off;    // bf16 [N][rp]  L2 transposed (rp = r rounded up to 64, zero-padded)
  size_t l1p_off;    // bf16 [K][rp]  L1 zero-padded to rp columns
  size_t st_off;     // bf16 [M][rp]  s * (X L1)
  size_t t_off;      // bf16 [M][r]   X L1 (when the caller gives no T)
  size_t su_off;     // bf16 [M][rp]  s * (dY L2^T)
  size_t l1t_off;    // bf16 [64][K]  L1 transposed, rows >= r zero (skinny path)
  size_t l2p_off;    // bf16 [64][N]  L2 with rows >= r zero (skinny path, r < 64)
  size_t part_off;   // fp32 split-K partials
  size_t part_bytes;
  size_t wd_off;     // bf16 dequantised weight for the dense GEMM path
  size_t wd_bytes;
  size_t xd_off;     // dropout: bf16 [M][K] dropped adapter input
  size_t dd_off;     // dropout: fp32 [M][K] masked LoRA term of dX (or the main product)
  size_t total;
};

LinearWorkspace linear_workspace_layout(int64_t M, int64_t K, int64_t N, int r, bool dropout = false);

hipError_t launch_dequant_rows(const NF4View& W, const NF4Table& tab, uint16_t* out, hipStream_t stream);
hipError_t launch_dequant_cols(const NF4View& W, const NF4Table& tab, uint16_t* out, int64_t ldo,
                               hipStream_t stream);
// E (optional): fp32 addend [M][N] with row stride lde; C = bf16(alpha acc + E).
hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t M, int64_t N,
                          int64_t K, const uint16_t* A2, const uint16_t* B2, int64_t ld2, int64_t K2, uint16_t* C,
                          int64_t ldc, float alpha, hipStream_t stream, const float* E = nullptr,
                          int64_t lde = 0);

DropoutParams dropout_params(float p, uint64_t seed);
hipError_t launch_dropout_input(const uint16_t* X, int64_t numel, const DropoutParams& d, uint16_t* Xd,
                                hipStream_t stream);
// D[m][k] = keep c sum_j sU[m][j] L1[k][j] (fp32); with F, dX = bf16(F + D) instead.
hipError_t launch_masked_lora(const uint16_t* sU, int64_t ldsu, const uint16_t* L1, int r, int64_t M, int64_t K,
                              const DropoutParams& d, const float* F, float* D, uint16_t* dX, hipStream_t stream);

// Single-token forward (gemv1.hip): one launch for the LoRA partials over
// K-slices (fp32 [K/256][r] in part), then the streaming dequant-GEMV that
// reduces them and adds the LoRA term. gemv1_applies says whether the shape
// takes this path (M == 1, r <= 64, K a multiple of 256 up to 16384).
bool gemv1_applies(const NF4View& W, int64_t M, int r);
size_t gemv1_partial_bytes(int64_t K, int r);
hipError_t launch_gemv1(const NF4View& W, const NF4Table& tab, const uint16_t* X, const uint16_t* L1,
                        const uint16_t* L2, int r, float s, uint16_t* Y, uint16_t* T_out, float* part,
                        hipStream_t stream);

// The device conversions applied to fp32 bit patterns first .. first +
// count - 1 (convcheck.hip); any output may be null.
hipError_t launch_convcheck(uint32_t first, int64_t count, uint16_t* bf, uint8_t* e8, float* table,
                            hipStream_t stream);

// Measurement aids (probe.hip): a register-only MFMA loop (clocks[0] =
// shader clocks, clocks[1] = 100 MHz ticks of workgroup 0's loop) and a
// streaming read of `bytes` (a multiple of read_probe_granule()).
hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, unsigned long long* clocks, hipStream_t stream);
size_t read_probe_granule();
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t never, uint32_t* sink, hipStream_t stream);

// Decode-path forward (M <= 16): the K-slice partials of Xa L1 into part,
// then the dequant-GEMV with the LoRA term; bf16(s Xa L1) goes through sT
// ([M][r]) from a separate reduction unless the GEMV sums the partials
// itself. Xa is the adapter branch's input (X, or its dropped copy).
hipError_t linear_forward_small(const NF4View& W, const NF4Table& tab, const uint16_t* X, const uint16_t* Xa,
                                int64_t M, const uint16_t* L1, const uint16_t* L2, int r, float s, uint16_t* Y,
                                uint16_t* T_out, uint16_t* sT, float* part, hipStream_t stream);

// Scratch of linear_forward_small packed back to back: sT, then the partials.
struct SmallForwardScratch {
  size_t st_off, part_off, total;
};
SmallForwardScratch small_forward_scratch(int64_t M, int64_t K, int r);

// With dr, the adapter branch reads the dropped input (regenerated from
// dr's seed in both passes) and the workspace is linear_workspace_layout(...,
// true).
// Whether linear_forward takes these sizes: the large-M path needs the bf16
// dequantised weight (and L2^T) below 2 GB.
bool linear_forward_supported(int64_t M, int64_t K, int64_t N, int r);

hipError_t linear_forward(const NF4View& W, const NF4Table& tab, const uint16_t* X, int64_t M,
                          const uint16_t* L1, const uint16_t* L2, int r, float s, uint16_t* Y,
                          uint16_t* T_out, void* ws, hipStream_t stream, const DropoutParams* dr = nullptr);

hipError_t linear_backward(const NF4View& W, const NF4Table& tab, const uint16_t* X, const uint16_t* dY,
                           int64_t M, const uint16_t* L1, const uint16_t* L2, int r, float s,
                           const uint16_t* T, uint16_t* dX, void* dL1, void* dL2, bool grad_bf16,
                           void* ws, hipStream_t stream, const DropoutParams* dr = nullptr);

}  // namespace qlora
