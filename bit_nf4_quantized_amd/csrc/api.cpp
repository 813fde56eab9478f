// C ABI of the QLoRA NF4 library: host-side validation, sizes, the NF4
// codebook, and stream-ordered kernel launches. See include/qlora_nf4.h.
#include "qlora_nf4.h"

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "launch.h"

using qlora::LinearWorkspace;
using qlora::NF4Table;
using qlora::NF4Thresholds;
using qlora::NF4View;

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return QLORA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// N(0,1) quantile by bisection on the CDF 1/2 erfc(-x / sqrt 2), to full
// double precision.
double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 400; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (0.5 * erfc(-mid / sqrt(2.0)) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

// S_c = { 1/2 [Q(i/(c+2)) + Q((i+1)/(c+2))] : i = 1..c } for odd c (QLoRA
// pages, diycv.top, section 方法总览 item 2, with c = 15 giving the
// denominator 2^4 + 1); its middle element is exactly 0.
void quantile_set(int c, double* out) {
  const double d = (double)(c + 2);
  for (int i = 1; i <= c; ++i) out[i - 1] = 0.5 * (normal_quantile(i / d) + normal_quantile((i + 1) / d));
  out[c / 2] = 0.0;
}

struct Tables {
  NF4Table tab;
  NF4Thresholds th;
};

// The 16 ascending table values of a 4-bit data type, in float64 before the
// one fp32 rounding.
//   NF4: 7 negative members of S_15 over |min S_15|, an exact 0, and 8
//     positive members of S_17 over max S_17 (diycv.top, section 方法总览
//     item 2).
//   Int4: the Int8 absmax formula of the same section (item 1) with 4-bit
//     signed integers, levels k/7; entry k + 8 holds k/7 for k = -8..7
//     (k = -8 is never produced: |x| <= 1).
//   FP4 E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit: 0, 0.5,
//     1, 1.5, 2, 3, 4, 6) and FP4 E3M0 (exponent field 0 = zero, else a
//     power of two: 0, 2^-6 .. 1 after scaling) scaled so that the largest
//     magnitude is 1; +-0 are one value, so entry 0 holds an unused -2.
//   (The pages name Int4, FP4 E2M1 and FP4 E3M0 in section 实验设置与主要结果
//   item 1 without defining them; these are the plainest readings.)
void type_values(int qtype, double* v) {
  if (qtype == QLORA_QTYPE_NF4) {
    double s15[15], s17[17];
    quantile_set(15, s15);
    quantile_set(17, s17);
    int n = 0;
    for (int i = 0; i < 7; ++i) v[n++] = s15[i] / (-s15[0]);
    v[n++] = 0.0;
    for (int i = 9; i < 17; ++i) v[n++] = s17[i] / s17[16];
    v[0] = -1.0;
    v[15] = 1.0;
  } else if (qtype == QLORA_QTYPE_INT4) {
    for (int k = -8; k < 8; ++k) v[k + 8] = (double)k / 7.0;
  } else {
    const double e2m1[7] = {0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double mag[7];
    for (int i = 0; i < 7; ++i) mag[i] = qtype == QLORA_QTYPE_FP4_E2M1 ? e2m1[i] / 6.0 : ldexp(1.0, i - 6);
    v[0] = -2.0;
    for (int i = 0; i < 7; ++i) v[1 + i] = -mag[6 - i];
    v[8] = 0.0;
    for (int i = 0; i < 7; ++i) v[9 + i] = mag[i];
  }
}

// The table of a data type (one fp32 rounding per value), plus the decision
// thresholds between neighbouring codes.
Tables build_tables(int qtype) {
  double v[16];
  type_values(qtype, v);
  Tables T;
  for (int i = 0; i < 16; ++i) T.tab.q[i] = (float)v[i];
  for (int j = 0; j < 15; ++j) {
    // exact midpoint of two fp32 values, then the smallest fp32 strictly above it
    const double m = 0.5 * ((double)T.tab.q[j] + (double)T.tab.q[j + 1]);
    float f = (float)m;
    if (!((double)f > m)) f = nextafterf(f, INFINITY);
    T.th.t[j] = f;
  }
  return T;
}

constexpr int kQTypes = 4;

const Tables& tables(int qtype) {
  static const Tables T[kQTypes] = {build_tables(0), build_tables(1), build_tables(2), build_tables(3)};  // one-time init
  return T[qtype];
}

bool valid_qtype(int qtype) { return qtype >= 0 && qtype < kQTypes; }

bool valid_nf4(const qlora_nf4* q) {
  if (!q || !q->codes || !valid_qtype(q->qtype) || (q->no_dq != 0 && q->no_dq != 1)) return false;
  return q->no_dq ? q->absmax32 != nullptr : (q->absmax8 && q->scale2 && q->mean);
}

NF4View view_of(const qlora_nf4* q) {
  NF4View v;
  v.codes = q->codes;
  v.absmax8 = q->absmax8;
  v.scale2 = q->scale2;
  v.mean = q->mean;
  v.rows = q->rows;
  v.cols = q->cols;
  v.absmax32 = q->no_dq ? q->absmax32 : nullptr;
  return v;
}

// Shape rules shared by the linear entry points.
int check_linear(const qlora_nf4* W, int64_t M, int r, float scale) {
  if (!valid_nf4(W)) return QLORA_ERR_ARG;
  if (!isfinite(scale)) return QLORA_ERR_ARG;
  if (r < 8 || r > QLORA_MAX_RANK || (r % 8) != 0) return QLORA_ERR_ARG;
  if (M < 0 || W->rows <= 0 || W->cols <= 0) return QLORA_ERR_SHAPE;
  if ((W->cols % QLORA_BLOCK) != 0 || (W->rows % 8) != 0) return QLORA_ERR_SHAPE;
  if (M > (int64_t)1 << 31 || W->rows > (int64_t)1 << 31 || W->cols > (int64_t)1 << 31) return QLORA_ERR_SHAPE;
  if (!aligned16(W->codes)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// log2 of an Int8 codec block size (a power of two in [64, 4096]), or -1.
int int8_block_log2(int block) {
  for (int lg = 6; lg <= 12; ++lg)
    if (block == (1 << lg)) return lg;
  return -1;
}

}  // namespace

extern "C" {

const char* qlora_status_str(int status) {
  switch (status) {
    case QLORA_OK: return "QLORA_OK";
    case QLORA_ERR_ARG: return "QLORA_ERR_ARG: invalid argument";
    case QLORA_ERR_SHAPE: return "QLORA_ERR_SHAPE: unsupported or inconsistent shape";
    case QLORA_ERR_ALIGN: return "QLORA_ERR_ALIGN: device pointer not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "QLORA_ERR_WORKSPACE: workspace missing or too small";
    case QLORA_ERR_HIP: return "QLORA_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown qlora status";
  }
}

const char* qlora_last_error(void) { return g_last_error; }

int qlora_nf4_codebook(float* out16) {
  if (!out16) return QLORA_ERR_ARG;
  memcpy(out16, tables(QLORA_QTYPE_NF4).tab.q, sizeof(float) * 16);
  return QLORA_OK;
}

int qlora_codebook(int qtype, float* out16) {
  if (!out16 || !valid_qtype(qtype)) return QLORA_ERR_ARG;
  memcpy(out16, tables(qtype).tab.q, sizeof(float) * 16);
  return QLORA_OK;
}

int qlora_quant_sizes(int64_t rows, int64_t cols, size_t* codes_bytes, size_t* absmax8_bytes,
                      size_t* scale2_bytes, size_t* workspace_bytes) {
  if (rows < 0 || cols < 0) return QLORA_ERR_SHAPE;
  if (cols > 0 && rows > INT64_MAX / 2 / cols) return QLORA_ERR_SHAPE;
  const int64_t numel = rows * cols;
  const int64_t nb = (numel + QLORA_BLOCK - 1) / QLORA_BLOCK;
  const int64_t ng = (nb + QLORA_DQ_BLOCK - 1) / QLORA_DQ_BLOCK;
  if (codes_bytes) *codes_bytes = (size_t)((numel + 1) / 2);
  if (absmax8_bytes) *absmax8_bytes = (size_t)nb;
  if (scale2_bytes) *scale2_bytes = (size_t)ng * sizeof(float);
  if (workspace_bytes) *workspace_bytes = qlora::quant_workspace_layout(numel).total;
  return QLORA_OK;
}

int qlora_quantize(const void* W, qlora_dtype in_dtype, const qlora_nf4* q, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  if (!q) return QLORA_ERR_ARG;
  if (in_dtype != QLORA_F32 && in_dtype != QLORA_BF16) return QLORA_ERR_ARG;
  if (q->rows < 0 || q->cols < 0) return QLORA_ERR_SHAPE;
  if (q->cols > 0 && q->rows > INT64_MAX / 2 / q->cols) return QLORA_ERR_SHAPE;
  const int64_t numel = q->rows * q->cols;
  if (numel == 0) return QLORA_OK;
  if ((numel + QLORA_BLOCK * QLORA_DQ_BLOCK - 1) / (QLORA_BLOCK * QLORA_DQ_BLOCK) > 0x7FFFFFFF)
    return QLORA_ERR_SHAPE;
  if (!W || !valid_nf4(q) || !ws) return QLORA_ERR_ARG;
  if (!aligned16(W) || !aligned16(q->codes) || !aligned16(ws)) return QLORA_ERR_ALIGN;
  if (ws_bytes < qlora::quant_workspace_layout(numel).total) return QLORA_ERR_WORKSPACE;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_quantize(W, in_dtype == QLORA_BF16, numel, tables(q->qtype).th, q->codes,
                                              q->absmax8, q->scale2, q->mean, q->no_dq ? q->absmax32 : nullptr,
                                              ws, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

// Byte offset of tensor k's scratch in a batch workspace (each part rounded
// up to 256); k = n gives the total.
static size_t batch_ws_offset(int k, const int64_t* numel) {
  size_t off = 0;
  for (int j = 0; j < k; ++j) off += qlora::align_up(qlora::quant_workspace_layout(numel[j]).total, 256);
  return off;
}

// rows/cols -> numel with the single-tensor shape rules; QLORA_OK or an error.
static int batch_numel(int64_t rows, int64_t cols, int64_t* numel) {
  if (rows < 0 || cols < 0) return QLORA_ERR_SHAPE;
  if (cols > 0 && rows > INT64_MAX / 2 / cols) return QLORA_ERR_SHAPE;
  *numel = rows * cols;
  if ((*numel + QLORA_BLOCK * QLORA_DQ_BLOCK - 1) / (QLORA_BLOCK * QLORA_DQ_BLOCK) > 0x7FFFFFFF)
    return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

int qlora_quant_batch_workspace(int n, const int64_t* rows, const int64_t* cols, size_t* bytes) {
  if (n < 1 || n > QLORA_QUANT_BATCH_MAX || !rows || !cols || !bytes) return QLORA_ERR_ARG;
  int64_t numel[QLORA_QUANT_BATCH_MAX];
  for (int k = 0; k < n; ++k) {
    const int st = batch_numel(rows[k], cols[k], &numel[k]);
    if (st != QLORA_OK) return st;
  }
  *bytes = batch_ws_offset(n, numel);
  return QLORA_OK;
}

int qlora_quantize_batch(int n, const void* const* W, qlora_dtype in_dtype, const qlora_nf4* const* q, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (n < 1 || n > QLORA_QUANT_BATCH_MAX || !W || !q) return QLORA_ERR_ARG;
  if (in_dtype != QLORA_F32 && in_dtype != QLORA_BF16) return QLORA_ERR_ARG;
  int64_t numel[QLORA_QUANT_BATCH_MAX];
  int first = -1;                                // the first non-empty tensor
  for (int k = 0; k < n; ++k) {
    if (!q[k]) return QLORA_ERR_ARG;
    const int st = batch_numel(q[k]->rows, q[k]->cols, &numel[k]);
    if (st != QLORA_OK) return st;
    if (numel[k] == 0) continue;
    if (!W[k] || !valid_nf4(q[k])) return QLORA_ERR_ARG;
    if (first < 0) first = k;
    if (q[k]->qtype != q[first]->qtype) return QLORA_ERR_ARG;     // one threshold table per launch
    if (!aligned16(W[k]) || !aligned16(q[k]->codes)) return QLORA_ERR_ALIGN;
  }
  if (first < 0) return QLORA_OK;                // nothing to quantise
  int64_t groups = 0;                            // one workgroup per DQ group of the whole batch
  for (int k = 0; k < n; ++k) groups += (numel[k] + QLORA_BLOCK * QLORA_DQ_BLOCK - 1) / (QLORA_BLOCK * QLORA_DQ_BLOCK);
  if (groups > 0x7FFFFFFF) return QLORA_ERR_SHAPE;
  if (!ws) return QLORA_ERR_ARG;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (ws_bytes < batch_ws_offset(n, numel)) return QLORA_ERR_WORKSPACE;
  qlora::QuantItem items[QLORA_QUANT_BATCH_MAX];
  for (int k = 0; k < n; ++k) {
    const qlora_nf4* t = q[k];
    items[k] = qlora::QuantItem{W[k], numel[k], t->codes, t->absmax8, t->scale2, t->mean,
                                t->no_dq ? t->absmax32 : nullptr, static_cast<char*>(ws) + batch_ws_offset(k, numel)};
  }
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e =
      qlora::launch_quantize_batch(items, n, in_dtype == QLORA_BF16, tables(q[first]->qtype).th, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_dequantize(const qlora_nf4* q, uint16_t* out, hipStream_t stream) {
  if (!q) return QLORA_ERR_ARG;
  if (q->rows < 0 || q->cols < 0) return QLORA_ERR_SHAPE;
  if (q->cols > 0 && q->rows > INT64_MAX / 2 / q->cols) return QLORA_ERR_SHAPE;
  const int64_t numel = q->rows * q->cols;
  if (numel == 0) return QLORA_OK;
  if (!valid_nf4(q) || !out) return QLORA_ERR_ARG;
  if (!aligned16(q->codes) || !aligned16(out)) return QLORA_ERR_ALIGN;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e =
      qlora::launch_dequantize(q->codes, q->absmax8, q->scale2, q->mean, q->no_dq ? q->absmax32 : nullptr,
                               tables(q->qtype).tab, numel, out, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_int8_quantize(const void* X, qlora_dtype in_dtype, int64_t numel, int block, int8_t* codes,
                        float* absmax, hipStream_t stream) {
  const int lg = int8_block_log2(block);
  if (lg < 0 || (in_dtype != QLORA_F32 && in_dtype != QLORA_BF16)) return QLORA_ERR_ARG;
  if (numel < 0 || numel > QLORA_INT8_MAX_NUMEL) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!X || !codes || !absmax) return QLORA_ERR_ARG;
  if (!aligned16(X) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(absmax) & 3u)) return QLORA_ERR_ALIGN;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_int8_quantize(X, in_dtype == QLORA_BF16, numel, lg, codes, absmax, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_int8_dequantize(const int8_t* codes, const float* absmax, int64_t numel, int block, void* out,
                          qlora_dtype out_dtype, hipStream_t stream) {
  const int lg = int8_block_log2(block);
  if (lg < 0 || (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16)) return QLORA_ERR_ARG;
  if (numel < 0 || numel > QLORA_INT8_MAX_NUMEL) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!codes || !absmax || !out) return QLORA_ERR_ARG;
  if (!aligned16(codes) || !aligned16(out) || (reinterpret_cast<uintptr_t>(absmax) & 3u)) return QLORA_ERR_ALIGN;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e =
      qlora::launch_int8_dequantize(codes, absmax, numel, lg, out, out_dtype == QLORA_BF16, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_merge_adapters(const qlora_nf4* W, const uint16_t* L1, const uint16_t* L2, int r, float scale,
                         uint16_t* out, hipStream_t stream) {
  const int st = check_linear(W, 0, r, scale);
  if (st != QLORA_OK) return st;
  if (!L1 || !L2 || !out) return QLORA_ERR_ARG;
  if (!aligned16(L1) || !aligned16(L2) || !aligned16(out)) return QLORA_ERR_ALIGN;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_merge(view_of(W), tables(W->qtype).tab, L1, L2, r, scale, out, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_linear_workspace(int64_t M, int64_t K, int64_t N, int r, size_t* bytes) {
  if (!bytes) return QLORA_ERR_ARG;
  if (r < 8 || r > QLORA_MAX_RANK || (r % 8) != 0) return QLORA_ERR_ARG;
  if (M < 0 || K <= 0 || N <= 0 || (K % QLORA_BLOCK) != 0 || (N % 8) != 0) return QLORA_ERR_SHAPE;
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31 || K > (int64_t)1 << 31) return QLORA_ERR_SHAPE;
  *bytes = qlora::linear_workspace_layout(M, K, N, r).total;
  return QLORA_OK;
}

int qlora_linear_workspace_dropout(int64_t M, int64_t K, int64_t N, int r, size_t* bytes) {
  const int st = qlora_linear_workspace(M, K, N, r, bytes);
  if (st != QLORA_OK) return st;
  *bytes = qlora::linear_workspace_layout(M, K, N, r, true).total;
  return QLORA_OK;
}

}  // extern "C"

namespace {

int linear_fwd_impl(const qlora_nf4* W, const uint16_t* X, int64_t M, const uint16_t* L1, const uint16_t* L2, int r,
                    float scale, uint16_t* Y, uint16_t* T_out, void* ws, size_t ws_bytes, hipStream_t stream,
                    const qlora::DropoutParams* dr) {
  int st = check_linear(W, M, r, scale);
  if (st != QLORA_OK) return st;
  if (!L1 || !L2) return QLORA_ERR_ARG;
  if (M > 0 && (!X || !Y)) return QLORA_ERR_ARG;
  if (!ws) return QLORA_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(L1) || !aligned16(L2) || !aligned16(Y) || !aligned16(T_out) || !aligned16(ws))
    return QLORA_ERR_ALIGN;
  if (!qlora::linear_forward_supported(M, W->cols, W->rows, r)) return QLORA_ERR_SHAPE;
  if (ws_bytes < qlora::linear_workspace_layout(M, W->cols, W->rows, r, dr != nullptr).total)
    return QLORA_ERR_WORKSPACE;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::linear_forward(view_of(W), tables(W->qtype).tab, X, M, L1, L2, r, scale, Y, T_out, ws,
                                             stream, dr);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int linear_bwd_impl(const qlora_nf4* W, const uint16_t* X, const uint16_t* dY, int64_t M, const uint16_t* L1,
                    const uint16_t* L2, int r, float scale, const uint16_t* T, uint16_t* dX, void* dL1, void* dL2,
                    qlora_dtype grad_dtype, void* ws, size_t ws_bytes, hipStream_t stream,
                    const qlora::DropoutParams* dr) {
  int st = check_linear(W, M, r, scale);
  if (st != QLORA_OK) return st;
  if (grad_dtype != QLORA_F32 && grad_dtype != QLORA_BF16) return QLORA_ERR_ARG;
  if (!L1 || !L2 || !dL1 || !dL2) return QLORA_ERR_ARG;
  if (M > 0 && (!X || !dY)) return QLORA_ERR_ARG;
  if (!ws) return QLORA_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(L1) || !aligned16(L2) || !aligned16(T) || !aligned16(dX) ||
      !aligned16(dL1) || !aligned16(dL2) || !aligned16(ws))
    return QLORA_ERR_ALIGN;
  if (ws_bytes < qlora::linear_workspace_layout(M, W->cols, W->rows, r, dr != nullptr).total)
    return QLORA_ERR_WORKSPACE;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::linear_backward(view_of(W), tables(W->qtype).tab, X, dY, M, L1, L2, r, scale, T, dX, dL1,
                                              dL2, grad_dtype == QLORA_BF16, ws, stream, dr);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

bool valid_dropout(float p) { return isfinite(p) && p >= 0.0f && p < 1.0f; }

// The device-side address of p: device memory as it is, pinned host memory
// through its device mapping; nullptr for anything else (pageable host
// memory, managed memory, or an address HIP does not know).
void* device_view(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice && !a.isManaged) return const_cast<void*>(p);
  if (a.type == hipMemoryTypeHost && a.devicePointer && a.hostPointer && !a.isManaged)
    return static_cast<char*>(a.devicePointer) + (static_cast<const char*>(p) - static_cast<const char*>(a.hostPointer));
  return nullptr;
}

// ---- the allocation-free decode forward ----------------------------------------
//
// Scratch of qlora_linear_fwd_noalloc: one array per device, in the module's
// device memory (zero-initialised when the code object loads; held until the
// process ends). Host code never passes the array's name to a kernel: the
// name is a host-side stand-in. The device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// that address is what the kernels receive. Calls that overlap on one device
// share the array and race.
__device__ __align__(256) unsigned char scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on the first call on
// that device).
int device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return QLORA_ERR_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" {

int qlora_linear_fwd_noalloc(const qlora_nf4* W, const uint16_t* X, int64_t M, const uint16_t* L1,
                             const uint16_t* L2, int r, float scale, uint16_t* Y, uint16_t* T_out,
                             hipStream_t stream) {
  int st = check_linear(W, M, r, scale);
  if (st != QLORA_OK) return st;
  if (M > 16) return QLORA_ERR_SHAPE;
  if (!L1 || !L2) return QLORA_ERR_ARG;
  if (M > 0 && (!X || !Y)) return QLORA_ERR_ARG;
  if (!aligned16(X) || !aligned16(L1) || !aligned16(L2) || !aligned16(Y) || !aligned16(T_out))
    return QLORA_ERR_ALIGN;
  const qlora::SmallForwardScratch S = qlora::small_forward_scratch(M, W->cols, r);
  if (S.total > QLORA_NOALLOC_SCRATCH_BYTES) return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;
  void* base = nullptr;
  st = device_scratch(&base);
  if (st != QLORA_OK) return st;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  char* p = static_cast<char*>(base);
  const hipError_t e = qlora::linear_forward_small(
      view_of(W), tables(W->qtype).tab, X, X, M, L1, L2, r, scale, Y, T_out, reinterpret_cast<uint16_t*>(p + S.st_off),
      reinterpret_cast<float*>(p + S.part_off), stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_linear_fwd(const qlora_nf4* W, const uint16_t* X, int64_t M, const uint16_t* L1, const uint16_t* L2,
                     int r, float scale, uint16_t* Y, uint16_t* T_out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  return linear_fwd_impl(W, X, M, L1, L2, r, scale, Y, T_out, ws, ws_bytes, stream, nullptr);
}

int qlora_linear_bwd(const qlora_nf4* W, const uint16_t* X, const uint16_t* dY, int64_t M, const uint16_t* L1,
                     const uint16_t* L2, int r, float scale, const uint16_t* T, uint16_t* dX, void* dL1,
                     void* dL2, qlora_dtype grad_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  return linear_bwd_impl(W, X, dY, M, L1, L2, r, scale, T, dX, dL1, dL2, grad_dtype, ws, ws_bytes, stream, nullptr);
}

int qlora_linear_fwd_dropout(const qlora_nf4* W, const uint16_t* X, int64_t M, const uint16_t* L1,
                             const uint16_t* L2, int r, float scale, float p, uint64_t seed, uint16_t* Y,
                             uint16_t* T_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dropout(p)) return QLORA_ERR_ARG;
  const qlora::DropoutParams d = qlora::dropout_params(p, seed);
  return linear_fwd_impl(W, X, M, L1, L2, r, scale, Y, T_out, ws, ws_bytes, stream, &d);
}

int qlora_linear_bwd_dropout(const qlora_nf4* W, const uint16_t* X, const uint16_t* dY, int64_t M,
                             const uint16_t* L1, const uint16_t* L2, int r, float scale, float p, uint64_t seed,
                             const uint16_t* T, uint16_t* dX, void* dL1, void* dL2, qlora_dtype grad_dtype,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dropout(p)) return QLORA_ERR_ARG;
  const qlora::DropoutParams d = qlora::dropout_params(p, seed);
  return linear_bwd_impl(W, X, dY, M, L1, L2, r, scale, T, dX, dL1, dL2, grad_dtype, ws, ws_bytes, stream, &d);
}

int qlora_clip_grad_norm(const float* g, int64_t n, float max_norm, float* coef, double* norm, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (n < 0) return QLORA_ERR_SHAPE;
  if (!(max_norm > 0.0f) || isnan(max_norm)) return QLORA_ERR_ARG;
  if ((n > 0 && !g) || (!coef && !norm)) return QLORA_ERR_ARG;
  if (!ws || ws_bytes < QLORA_CLIP_WORKSPACE_BYTES) return QLORA_ERR_WORKSPACE;
  if (!aligned16(g) || !aligned16(ws) || (reinterpret_cast<uintptr_t>(coef) & 3u) ||
      (reinterpret_cast<uintptr_t>(norm) & 7u))
    return QLORA_ERR_ALIGN;
  const float* gd = n > 0 ? static_cast<const float*>(device_view(g)) : g;
  float* cd = coef ? static_cast<float*>(device_view(coef)) : nullptr;
  double* nd = norm ? static_cast<double*>(device_view(norm)) : nullptr;
  double* wd = static_cast<double*>(device_view(ws));
  if ((n > 0 && !gd) || (coef && !cd) || (norm && !nd) || !wd) return QLORA_ERR_ARG;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_clip_norm(gd, n, (double)max_norm, cd, nd, wd, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_adam_step(float* theta, const float* g, float* m, float* v, int64_t n, const qlora_adam_params* hp,
                    const float* coef, uint16_t* theta_bf16, hipStream_t stream) {
  if (!hp) return QLORA_ERR_ARG;
  if (n < 0) return QLORA_ERR_SHAPE;
  if (hp->step < 1 || !(hp->lr >= 0.0f) || !isfinite(hp->lr) || !(hp->eps >= 0.0f) || !isfinite(hp->eps) ||
      !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) ||
      !isfinite(hp->weight_decay))
    return QLORA_ERR_ARG;
  if (n == 0) return QLORA_OK;
  if (!theta || !g || !m || !v) return QLORA_ERR_ARG;
  if (!aligned16(theta) || !aligned16(g) || !aligned16(m) || !aligned16(v) || !aligned16(theta_bf16) ||
      (reinterpret_cast<uintptr_t>(coef) & 3u))
    return QLORA_ERR_ALIGN;
  float* td = static_cast<float*>(device_view(theta));
  const float* gd = static_cast<const float*>(device_view(g));
  float* md = static_cast<float*>(device_view(m));
  float* vd = static_cast<float*>(device_view(v));
  const float* cd = coef ? static_cast<const float*>(device_view(coef)) : nullptr;
  uint16_t* bd = theta_bf16 ? static_cast<uint16_t*>(device_view(theta_bf16)) : nullptr;
  if (!td || !gd || !md || !vd || (coef && !cd) || (theta_bf16 && !bd)) return QLORA_ERR_ARG;
  qlora::AdamHyper h;
  h.lr = hp->lr; h.beta1 = hp->beta1; h.beta2 = hp->beta2; h.eps = hp->eps; h.wd = hp->weight_decay;
  h.step = hp->step;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_adam(td, gd, md, vd, n, h, cd, bd, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_lora_dropout(const uint16_t* X, int64_t numel, float p, uint64_t seed, uint16_t* Xd, hipStream_t stream) {
  if (!valid_dropout(p)) return QLORA_ERR_ARG;
  if (numel < 0 || (numel % 8) != 0 || numel > ((int64_t)1 << 40)) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!X || !Xd) return QLORA_ERR_ARG;
  if (!aligned16(X) || !aligned16(Xd)) return QLORA_ERR_ALIGN;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_dropout_input(X, numel, qlora::dropout_params(p, seed), Xd, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_check_conversions(uint32_t first, int64_t count, uint16_t* bf16_out, uint8_t* e4m3_out,
                            float* e4m3_table, hipStream_t stream) {
  if (count < 0 || count > ((int64_t)1 << 32)) return QLORA_ERR_SHAPE;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_convcheck(first, count, bf16_out, e4m3_out, e4m3_table, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_probe_mfma(int workgroups, int iters, float* sink, uint64_t* clocks, hipStream_t stream) {
  if (!sink || !clocks || workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20))
    return QLORA_ERR_ARG;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_mfma_probe(workgroups, iters, sink,
                                                reinterpret_cast<unsigned long long*>(clocks), stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_probe_read(const void* src, size_t bytes, uint32_t never, uint32_t* sink, hipStream_t stream) {
  static_assert(QLORA_PROBE_READ_GRANULE == 65536, "granule");
  if (bytes == 0 || bytes % qlora::read_probe_granule() != 0 || bytes >= ((size_t)1 << 40)) return QLORA_ERR_SHAPE;
  if (!src || !sink) return QLORA_ERR_ARG;
  if (!aligned16(src)) return QLORA_ERR_ALIGN;
  (void)hipGetLastError();  // drop an error left by an earlier, unrelated runtime call
  const hipError_t e = qlora::launch_read_probe(src, bytes, never, sink, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

int qlora_set_timing(int kernel, hipEvent_t* start, hipEvent_t* stop, int n, int* count) {
  if (kernel < 0 || kernel >= QLORA_TIMING_CLASSES || n < 0) return QLORA_ERR_ARG;
  qlora::TimingSlot& t = qlora::timing_slots()[kernel];
  if (n == 0 || !start || !stop || !count) {
    t = qlora::TimingSlot();
    return QLORA_OK;
  }
  t.start = start;
  t.stop = stop;
  t.n = n;
  t.count = count;
  return QLORA_OK;
}

}  // extern "C"

namespace qlora {
TimingSlot* timing_slots() {
  static thread_local TimingSlot slots[kTimeClasses];
  return slots;
}
}  // namespace qlora
