/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) QLoRA NF4 library.
 *
 * The library implements the data-parallel hot path of QLoRA as described
 * on the QLoRA pages (page diycv.top "QLoRA 论文解读"; neura.market
 * "QLoRA" analysis):
 *
 *   - NF4 blockwise quantisation of a frozen weight with block size 64,
 *     and double quantisation (DQ) of the per-block absmax constants:
 *     mean-subtracted, stored as 8-bit floats in groups of 256 blocks with
 *     one fp32 scale per group (section 方法总览 items 1-3);
 *   - doubleDequant(c1, c2, W) = dequant(dequant(c1, c2), W) to bf16
 *     (section 关键公式);
 *   - the QLoRA linear layer Y = X dequant(W) + s X L1 L2 (section
 *     问题背景, LoRA equation; section 关键公式) and its backward pass,
 *     which returns dX and the adapter gradients dL1, dL2 but no weight
 *     gradient (section 关键公式, text after the dtype table).
 *
 * Conventions for every entry point
 *   - Device pointers are HIP device addresses on the current device; host
 *     pointers are marked "host". Matrices are dense row-major.
 *   - The frozen weight is stored as Wt[N][K]: N = out_features (rows),
 *     K = in_features (cols). Blocks of 64 run along the row-major
 *     flattening; block b covers elements [64b, 64b+64), DQ group g covers
 *     blocks [256g, 256g+256). The last block and group may be short.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Ownership: the caller allocates and frees every buffer, including
 *     workspaces sized by the query functions. The library allocates no
 *     memory and keeps no mutable state, and calls are reentrant, with one
 *     exception: qlora_linear_fwd_noalloc uses a library-held device array
 *     per device (see there).
 *   - Asynchrony: work is enqueued on `stream` and the call returns without
 *     synchronising. Errors found on the host (arguments, shapes,
 *     alignment, workspace size) are returned before anything is enqueued.
 *     A failed launch returns QLORA_ERR_HIP. Device faults surface at the
 *     caller's next synchronisation.
 *   - Outputs are overwritten, never accumulated into.
 *   - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 *   - Alignment: every device pointer must be 16-byte aligned unless noted.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_ARG = -1,        /* null pointer, bad enum or scalar, r out of range */
  QLORA_ERR_SHAPE = -2,      /* unsupported or inconsistent sizes */
  QLORA_ERR_ALIGN = -3,      /* a device pointer is not 16-byte aligned */
  QLORA_ERR_WORKSPACE = -4,  /* workspace missing or smaller than required */
  QLORA_ERR_HIP = -5         /* a HIP launch or runtime call failed */
} qlora_status;

/* Element types of the float operands. C callers may pass any int here; the
 * C++ view gives the enum an int underlying type so that the library can
 * read and reject values outside the list (QLORA_ERR_ARG) without undefined
 * behaviour. */
#ifdef __cplusplus
enum qlora_dtype_values : int { QLORA_F32 = 0, QLORA_BF16 = 1 };
typedef qlora_dtype_values qlora_dtype;
#else
typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;
#endif

enum {
  QLORA_BLOCK = 64,      /* weights per first-level absmax constant */
  QLORA_DQ_BLOCK = 256,  /* first-level constants per second-level scale */
  QLORA_MAX_RANK = 256   /* largest LoRA rank r accepted */
};

/*
 * 4-bit data types of the codes. NF4 is the pages' type; the others are the
 * 4-bit types the pages compare it with (diycv.top, section 实验设置与主要结果
 * item 1: Int4, FP4 E2M1, FP4 E3M0), which the pages name but do not define.
 * Every type is a table of 16 ascending fp32 values in [-1, 1] (the FP4
 * types have 15 distinct values and an unused entry 0 = -2; Int4 has the
 * unused level -8/7 at entry 0), used with the same blockwise absmax scaling,
 * nearest-code rounding and double quantisation (qlora_codebook returns the
 * table):
 *   QLORA_QTYPE_INT4      entry k + 8 = k/7, k = -8..7 (the Int8 absmax
 *                         formula of section 方法总览 item 1 at 4 bits)
 *   QLORA_QTYPE_FP4_E2M1  {0, 0.5, 1, 1.5, 2, 3, 4, 6} / 6 with signs
 *   QLORA_QTYPE_FP4_E3M0  {0, 2^-6, ..., 2^-1, 1} with signs
 */
typedef enum {
  QLORA_QTYPE_NF4 = 0,
  QLORA_QTYPE_INT4 = 1,
  QLORA_QTYPE_FP4_E2M1 = 2,
  QLORA_QTYPE_FP4_E3M0 = 3
} qlora_qtype;

/*
 * One quantised tensor: the pages' (c1, c2, W^NF4) triple plus the DQ mean
 * and the 4-bit data type of the codes. Double quantisation is on by
 * default (no_dq = 0); with no_dq = 1 the first-level constants stay fp32
 * (the blockwise quantisation of section 方法总览 item 1 without item 3). The struct itself lives in host
 * memory; its buffer pointers are device pointers owned by the caller.
 * Sizes (nb = ceil(rows*cols/64), ng = ceil(nb/256)):
 *   codes   [ceil(rows*cols/2)] u8   4-bit codes; element 2j is the low
 *                                    nibble of byte j, element 2j+1 the high
 *                                    nibble; an unused last high nibble is 0.
 *   absmax8 [nb] u8                  E4M3 (OCP "E4M3FN") codes of
 *                                    (absmax_b - mean) / scale2_g.
 *   scale2  [ng] f32                 per-group second-level scale.
 *   mean    [1]  f32                 per-tensor mean of the block absmax.
 * `codes` must be 16-byte aligned; absmax8, scale2 and mean need only their
 * natural alignment.
 */
typedef struct {
  int64_t rows;
  int64_t cols;
  uint8_t *codes;
  uint8_t *absmax8;
  float *scale2;
  float *mean;
  int32_t qtype;  /* qlora_qtype of the codes (QLORA_QTYPE_NF4 = 0); others return QLORA_ERR_ARG */
  int32_t no_dq;  /* 0: double quantisation (absmax8, scale2, mean); 1: none, absmax32 holds the
                     fp32 block absmax and absmax8, scale2, mean are not used (may be NULL) */
  float *absmax32; /* [nb] f32 (no_dq = 1 only; 4 * absmax8_bytes of qlora_quant_sizes) */
} qlora_nf4;

/* Human-readable name of a status code (static string, never NULL). */
const char *qlora_status_str(int status);

/* Message of the last HIP failure on the calling thread ("" if none). */
const char *qlora_last_error(void);

/*
 * qlora_nf4_codebook: the library's 16 NF4 values (host, ascending).
 * Built once on the host from N(0,1) quantile midpoints
 * q_i = 1/2 [Q(i/(c+2)) + Q((i+1)/(c+2))], i = 1..c (diycv.top, section
 * 方法总览 item 2, with c = 2^4 - 1 = 15 for the pages' denominator 17):
 * the 7 negative members of the 15-value set divided by its largest
 * magnitude, an exact 0, and the 8 positive members of the 17-value set
 * divided by its maximum; rounded once to fp32. Index 0 = -1, 7 = 0,
 * 15 = +1. out16: host array of 16 floats. Returns QLORA_ERR_ARG if NULL.
 */
int qlora_nf4_codebook(float *out16);

/*
 * qlora_codebook: the 16 ascending fp32 values of a 4-bit data type (host).
 * qtype = QLORA_QTYPE_NF4 gives the same table as qlora_nf4_codebook.
 * out16: host array of 16 floats. Returns QLORA_ERR_ARG if NULL or if qtype
 * is not a qlora_qtype.
 */
int qlora_codebook(int qtype, float *out16);

/*
 * qlora_quant_sizes: buffer sizes in bytes for a rows x cols tensor (host
 * only, no device work). Any output pointer may be NULL. workspace_bytes is
 * the scratch that qlora_quantize needs. rows, cols >= 0.
 */
int qlora_quant_sizes(int64_t rows, int64_t cols, size_t *codes_bytes, size_t *absmax8_bytes,
                      size_t *scale2_bytes, size_t *workspace_bytes);

/*
 * qlora_quantize: NF4 + DQ quantisation of the weight W (diycv.top, section
 * 方法总览 items 1-3; training step 1-2 of section 训练与推理流程), or
 * quantisation to the 4-bit type q->qtype with the same steps.
 *   W         device, rows*cols elements of in_dtype (QLORA_F32 or
 *             QLORA_BF16), row-major [rows][cols].
 *   q         host struct; q->rows, q->cols give the shape; its buffers
 *             receive codes, absmax8, scale2 and mean (codes and absmax32
 *             when q->no_dq = 1: the block absmax a, no DQ steps).
 *   ws        device scratch of at least qlora_quant_sizes(...).workspace
 *             bytes, 16-byte aligned.
 * Per block: a = max|w| (a below 2^-126 makes a zero block: every code is
 * the table's zero, 7 for NF4); x = RN32(w * RN32(1/a)); code = nearest
 * table value, ties to the lower code. DQ: mean = RN32(S/nb) with S the float64 adjacent-pair tree sum of
 * the block absmax values; per group sigma = RN32(max|a - mean| / 448);
 * absmax8 = E4M3 round-to-nearest-even of RN32((a - mean)/sigma),
 * saturating at +-448 (0 where sigma is 0). Results are bit-for-bit
 * deterministic. Empty tensors enqueue nothing.
 */
int qlora_quantize(const void *W, qlora_dtype in_dtype, const qlora_nf4 *q, void *ws,
                   size_t ws_bytes, hipStream_t stream);

/*
 * qlora_quantize_batch: qlora_quantize applied to n tensors (1 <= n <=
 * QLORA_QUANT_BATCH_MAX) in one pass, e.g. the seven linears of a
 * transformer layer (gptget.net abstract and diycv.top, section 方法总览
 * items 1-3: every frozen linear of the model is stored in NF4 + DQ). Each
 * tensor is quantised exactly as by qlora_quantize on it alone (the same
 * codes and constants, bit for bit); the tensors share the launches: one
 * over all their 64-blocks, one fold of the per-tensor means, one 8-bit
 * float pass.
 *   W       host array of n device pointers, all fp32 or all bf16 (in_dtype).
 *   q       host array of n structs, as for qlora_quantize (each with its
 *           own rows, cols, output buffers and no_dq flag); all non-empty
 *           ones with the same qtype. Empty tensors are skipped.
 *   ws      device scratch of at least qlora_quant_batch_workspace bytes.
 * Errors: QLORA_ERR_ARG (n out of range, null pointers, mixed qtypes, bad
 * dtype), QLORA_ERR_SHAPE (a tensor as for qlora_quantize, or more than
 * 2^31 - 1 groups of 16384 weights in the batch), QLORA_ERR_ALIGN,
 * QLORA_ERR_WORKSPACE, all before anything is enqueued; QLORA_ERR_HIP.
 */
#define QLORA_QUANT_BATCH_MAX 16
int qlora_quantize_batch(int n, const void *const *W, qlora_dtype in_dtype, const qlora_nf4 *const *q,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * qlora_quant_batch_workspace: scratch bytes of qlora_quantize_batch for n
 * tensors of rows[k] x cols[k] (host only; the sum of the single-tensor
 * scratch sizes, each rounded up to 256 bytes).
 */
int qlora_quant_batch_workspace(int n, const int64_t *rows, const int64_t *cols, size_t *bytes);

/*
 * qlora_dequantize: doubleDequant to bf16 (diycv.top, section 关键公式):
 *   a'_b = RN32(RN32(e4m3(absmax8_b) * scale2_g) + mean)   (absmax32_b when no_dq)
 *   out_e = bf16_RNE(RN32(q[code_e] * a'_b)), q = the table of q->qtype
 *   out  device uint16_t[rows*cols] (bf16 bits), 16-byte aligned.
 */
int qlora_dequantize(const qlora_nf4 *q, uint16_t *out, hipStream_t stream);

/*
 * qlora_int8_quantize: blockwise Int8 absmax quantisation (diycv.top,
 * section 方法总览 item 1: X_int8 = round(127 / absmax(X) * X), one constant
 * per block of the flattened tensor).
 *   X       device, numel elements of in_dtype (QLORA_F32 or QLORA_BF16),
 *           16-byte aligned.
 *   numel   0 .. QLORA_INT8_MAX_NUMEL (0 enqueues nothing).
 *   block   elements per block: 64, 128, 256, 512, 1024, 2048 or 4096.
 *   codes   device int8[numel], 16-byte aligned.
 *   absmax  device f32[ceil(numel / block)] receiving each block's absmax a.
 * Per block: c = RN32(127 / a) (IEEE division); code = round(RN32(x * c)),
 * to nearest with ties to even, clamped to [-127, 127]. A block with a below
 * 2^-120 (zeros, or too small for the factor to be finite) gets code 0
 * everywhere. The last block may be short. Deterministic.
 * Returns QLORA_ERR_ARG for a bad block, dtype or NULL pointer,
 * QLORA_ERR_SHAPE for numel out of range, QLORA_ERR_ALIGN for misaligned
 * pointers.
 */
enum { QLORA_INT8_MAX_NUMEL_LOG2 = 40 };
#define QLORA_INT8_MAX_NUMEL (((int64_t)1) << QLORA_INT8_MAX_NUMEL_LOG2)
int qlora_int8_quantize(const void *X, qlora_dtype in_dtype, int64_t numel, int block, int8_t *codes,
                        float *absmax, hipStream_t stream);

/*
 * qlora_int8_dequantize: out_e = RN32(code_e * RN32(a_b / 127)) for every
 * element e of block b, written as fp32 (out_dtype QLORA_F32) or rounded to
 * bf16 with round-to-nearest-even (QLORA_BF16, uint16_t bits).
 *   codes, absmax, numel, block   as written by qlora_int8_quantize.
 *   out     device [numel] of out_dtype, 16-byte aligned.
 * Errors as for qlora_int8_quantize.
 */
int qlora_int8_dequantize(const int8_t *codes, const float *absmax, int64_t numel, int block, void *out,
                          qlora_dtype out_dtype, hipStream_t stream);

/*
 * qlora_linear_workspace: bytes of device workspace that qlora_linear_fwd
 * and qlora_linear_bwd need for M tokens, in_features K, out_features N and
 * rank r (host only). One workspace of this size serves both calls.
 */
int qlora_linear_workspace(int64_t M, int64_t K, int64_t N, int r, size_t *bytes);

/*
 * qlora_linear_fwd: Y = X dequant(Wt)^T + s (X L1) L2, computed with bf16
 * operands and fp32 accumulation, rounded once to bf16 (diycv.top, section
 * 关键公式 and section 问题背景; dequant as in qlora_dequantize, done on
 * the fly inside the kernels). The LoRA branch rounds s*(X L1) to bf16
 * before its second product.
 *   W      host struct of the NF4+DQ weight [N][K] (rows = N, cols = K).
 *   X      device bf16 [M][K];  L1 device bf16 [K][r];  L2 device bf16 [r][N].
 *   scale  the LoRA scale s (finite).
 *   Y      device bf16 [M][N].
 *   T_out  optional device bf16 [M][r] receiving bf16(X L1) for the
 *          backward pass (NULL to skip).
 *   ws     device workspace of qlora_linear_workspace(M, K, N, r) bytes.
 * Shapes: M >= 0; K a positive multiple of 64; N a positive multiple of 8;
 * r a multiple of 8 in [8, 256]. M <= 16 takes the bandwidth-bound GEMV
 * kernel, 16 < M <= 128 a one-pass fused dequant-GEMM over K-slices with a
 * fixed-order reduction, larger M the MFMA GEMM on the dequantised weight
 * (written to the workspace); all return the same layer. The MFMA path
 * needs that bf16 weight below 2 GB (N K < 2^30), else QLORA_ERR_SHAPE; it
 * takes any M (the token rows run in chunks of at most 2 GB).
 */
int qlora_linear_fwd(const qlora_nf4 *W, const uint16_t *X, int64_t M, const uint16_t *L1,
                     const uint16_t *L2, int r, float scale, uint16_t *Y, uint16_t *T_out,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * qlora_linear_fwd_noalloc: qlora_linear_fwd for M <= 16 (the decode path)
 * without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. It allocates nothing; its scratch (bf16(s X L1) and the
 * fp32 K-slice partials of X L1) lives in a library-held device array of
 * QLORA_NOALLOC_SCRATCH_BYTES per device, held until the process ends. The
 * caller passes inputs and outputs as for qlora_linear_fwd and gets the same
 * bits: the same kernels run.
 *   Errors as for qlora_linear_fwd, plus QLORA_ERR_SHAPE for M > 16 and
 *   QLORA_ERR_WORKSPACE when the scratch the shape needs,
 *   2 M r + 4 M r ceil(K / 512) bytes (each part rounded up to 256), exceeds
 *   the array (with M = 16 and r = 256 that allows K up to 67072).
 *   Calls on one device share the array: calls that overlap on one device
 *   (other streams, other threads) race and must be serialised by the caller.
 */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)(2u << 20) + (size_t)(64u << 10))
int qlora_linear_fwd_noalloc(const qlora_nf4 *W, const uint16_t *X, int64_t M, const uint16_t *L1,
                             const uint16_t *L2, int r, float scale, uint16_t *Y, uint16_t *T_out,
                             hipStream_t stream);

/*
 * qlora_linear_bwd: gradients of the layer for the upstream gradient dY
 * (diycv.top, section 关键公式, text after the dtype table: gradients pass
 * through the dequantised bf16 base to the input; only the adapters get
 * parameter gradients):
 *   dX  = dY dequant(Wt) + s (dY L2^T) L1^T      bf16 [M][K]
 *   dL1 = s X^T (dY L2^T)                        [K][r] in grad_dtype
 *   dL2 = s (X L1)^T dY                          [r][N] in grad_dtype
 * No gradient of the frozen weight is formed.
 *   T      optional device bf16 [M][r] = bf16(X L1) from qlora_linear_fwd's
 *          T_out; NULL recomputes it.
 *   dX     device bf16 [M][K], or NULL to skip the input gradient.
 *   dL1, dL2  device buffers of grad_dtype (QLORA_F32 or QLORA_BF16).
 * Other arguments and shape rules as for qlora_linear_fwd. dL1 and dL2 are
 * reduced over M in a fixed order, so repeated calls are bit-identical.
 */
int qlora_linear_bwd(const qlora_nf4 *W, const uint16_t *X, const uint16_t *dY, int64_t M,
                     const uint16_t *L1, const uint16_t *L2, int r, float scale,
                     const uint16_t *T, uint16_t *dX, void *dL1, void *dL2,
                     qlora_dtype grad_dtype, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * LoRA dropout on the adapter branch (diycv.top, section 训练与推理流程: the
 * Guanaco runs use LoRA dropout 0.1 for 7B/13B and 0.05 for 33B/65B). The
 * adapter branch reads Xd instead of X:
 *   Xd[m][k] = keep(m, k) ? bf16_RNE(RN32(X[m][k] * c)) : +0,  c = RN32(1 / (1 - p)),
 *   keep(m, k) = u >= floor(p 2^32), u = word e % 4 of Philox4x32-10 (Salmon
 *   et al., SC 2011) with counter (lo(e/4), hi(e/4), 0, 0) and key
 *   (lo(seed), hi(seed)), e = m K + k.
 * The forward is Y = X Wd^T + s (Xd L1) L2 (T_out = bf16(Xd L1)); the
 * backward, given the same (p, seed), is
 *   dX  = dY Wd + keep * c * (bf16(s dY L2^T) L1^T)   (fp32, one bf16 rounding)
 *   dL1 = s Xd^T (dY L2^T),  dL2 = s (Xd L1)^T dY.
 * Nothing is stored between the passes: the mask is regenerated from
 * (p, seed). p must be finite, 0 <= p < 1 (else QLORA_ERR_ARG); other
 * arguments, shapes and errors as for qlora_linear_fwd / qlora_linear_bwd,
 * except that the workspace is qlora_linear_workspace_dropout bytes (it adds
 * 6 M K bytes for Xd and the fp32 masked LoRA term of dX).
 */
int qlora_linear_workspace_dropout(int64_t M, int64_t K, int64_t N, int r, size_t *bytes);
int qlora_linear_fwd_dropout(const qlora_nf4 *W, const uint16_t *X, int64_t M, const uint16_t *L1,
                             const uint16_t *L2, int r, float scale, float p, uint64_t seed, uint16_t *Y,
                             uint16_t *T_out, void *ws, size_t ws_bytes, hipStream_t stream);
int qlora_linear_bwd_dropout(const qlora_nf4 *W, const uint16_t *X, const uint16_t *dY, int64_t M,
                             const uint16_t *L1, const uint16_t *L2, int r, float scale, float p, uint64_t seed,
                             const uint16_t *T, uint16_t *dX, void *dL1, void *dL2, qlora_dtype grad_dtype,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * qlora_lora_dropout: the dropped adapter input Xd alone (as above, element
 * e of a row-major tensor of numel bf16 values; numel a multiple of 8, at
 * most 2^40). X, Xd: device, 16-byte aligned. Errors: QLORA_ERR_ARG (p, NULL),
 * QLORA_ERR_SHAPE (numel), QLORA_ERR_ALIGN.
 */
int qlora_lora_dropout(const uint16_t *X, int64_t numel, float p, uint64_t seed, uint16_t *Xd, hipStream_t stream);

/*
 * The adapters' optimiser step (diycv.top, section 训练与推理流程: Adam with
 * beta2 = 0.999, max grad norm 0.3, constant learning rate; section 方法总览
 * item 4: the optimiser state is paged between GPU and CPU memory). The
 * adapter parameters, gradients and state are flat fp32 vectors of n
 * elements (the caller lays all adapters out in one buffer). Every pointer
 * may be device memory or pinned host memory (hipHostMalloc / a pinned torch
 * tensor): pinned host memory is read and written in place by the kernels
 * over the host link, which keeps that state out of HBM ("paged out");
 * anything else (pageable or managed memory) is rejected with QLORA_ERR_ARG.
 * Both calls are deterministic and enqueue on `stream`.
 *
 * qlora_clip_grad_norm: norm = sqrt(sum g^2) (float64, fixed order) and
 * coef = min(1, max_norm / (norm + 1e-6)) (float64, stored as fp32).
 *   g       [n] fp32, 16-byte aligned.   max_norm > 0 (may be +inf: coef = 1).
 *   coef    device/pinned fp32 [1] or NULL;  norm: fp64 [1] or NULL (not both NULL).
 *   ws      QLORA_CLIP_WORKSPACE_BYTES of device memory, 16-byte aligned.
 */
enum { QLORA_CLIP_WORKSPACE_BYTES = 8192 };
int qlora_clip_grad_norm(const float *g, int64_t n, float max_norm, float *coef, double *norm, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * qlora_adam_step: one Adam step (Kingma and Ba, ICLR 2015) on the clipped
 * gradient, in fp32, element by element:
 *   g' = coef g;  m = b1 m + (1-b1) g';  v = b2 v + (1-b2) g'^2;
 *   theta -= lr ( (m / bc1) / (sqrt(v / bc2) + eps) + weight_decay theta ),
 *   bc1 = 1 - b1^step, bc2 = 1 - b2^step (float64, rounded to fp32);
 *   theta_bf16 (optional) receives bf16_RNE(theta), the adapters the layer reads.
 *   theta, m, v updated in place; g read; all [n] and 16-byte aligned.
 *   coef    fp32 [1] from qlora_clip_grad_norm, or NULL for 1.
 *   hp      step >= 1; 0 <= beta1, beta2 < 1; lr, eps >= 0; finite values.
 */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
  int64_t step;
} qlora_adam_params;
int qlora_adam_step(float *theta, const float *g, float *m, float *v, int64_t n, const qlora_adam_params *hp,
                    const float *coef, uint16_t *theta_bf16, hipStream_t stream);

/*
 * qlora_merge_adapters: the trained adapters merged into the bf16
 * dequantised base, for inference without the adapter branch (robocikowo.com
 * "QLoRA", the list of common mistakes, entry on merging: merge into the
 * 16-bit dequantised base, never back into the 4-bit one; diycv.top, section 关键公式 for the dequant):
 *   out[n][k] = bf16_RNE(RN32(Wd[n][k] + RN32(s * D[k][n]))),
 *   Wd = bf16(RN32(q[code] * a')) as in qlora_dequantize,
 *   D  = L1 L2 with bf16 operands and fp32 accumulation,
 * so that X out^T is the layer of qlora_linear_fwd up to rounding.
 *   W      host struct of the quantised weight [N][K].
 *   L1     device bf16 [K][r];  L2 device bf16 [r][N].
 *   scale  the LoRA scale s (finite).
 *   out    device bf16 [N][K] (uint16_t bits), 16-byte aligned.
 * Shape rules as for qlora_linear_fwd (K a multiple of 64, N of 8, r a
 * multiple of 8 in [8, 256]). The 4-bit weight is left unchanged.
 */
int qlora_merge_adapters(const qlora_nf4 *W, const uint16_t *L1, const uint16_t *L2, int r, float scale,
                         uint16_t *out, hipStream_t stream);

/*
 * qlora_set_timing: measurement hook; it changes no result. While set on the
 * calling thread for a kernel class, each launch of that class by the
 * entry points above is bracketed by hipEventRecord(start[i]) and
 * hipEventRecord(stop[i]) on the call's stream, for i = 0 .. n-1 in launch
 * order; *count (host) receives the number of brackets recorded so far.
 * Launches beyond n are not recorded. n = 0 (or NULL arrays) clears the
 * hook for that class. The event arrays and count are host memory owned by
 * the caller and must stay valid while the hook is set; the events must
 * have been created by the caller (hipEventCreate).
 *   kernel  QLORA_TIMING_FWD_GEMM  fused dequant-GEMM producing Y (M > 128)
 *           QLORA_TIMING_DX_GEMM   fused transposed-dequant GEMM producing dX
 *           QLORA_TIMING_GEMV      small-M dequant-GEMV producing Y (M <= 16)
 *           QLORA_TIMING_QUANT     first quantisation pass (codes + absmax)
 *           QLORA_TIMING_DEQUANT   standalone dequant kernel
 *           QLORA_TIMING_MID_GEMM  forward for 16 < M <= 128: the fused
 *                                  dequant-GEMM and its K-slice reduction
 * Returns QLORA_ERR_ARG for an unknown class or negative n.
 */
enum {
  QLORA_TIMING_FWD_GEMM = 0,
  QLORA_TIMING_DX_GEMM = 1,
  QLORA_TIMING_GEMV = 2,
  QLORA_TIMING_QUANT = 3,
  QLORA_TIMING_DEQUANT = 4,
  QLORA_TIMING_MID_GEMM = 5,
  QLORA_TIMING_CLASSES = 6
};
int qlora_set_timing(int kernel, hipEvent_t *start, hipEvent_t *stop, int n, int *count);

/*
 * qlora_check_conversions: verification entry point (it computes nothing of
 * the method). Runs the device number conversions that every kernel uses
 * on the fp32 bit patterns first, first + 1, ..., first + count - 1 (mod
 * 2^32), so that the formats the pages fix (first-level constants in an
 * 8-bit float, products in bf16: diycv.top, section 关键公式, the dtype
 * table) can be checked against their definitions over every pattern:
 *   bf16_out[i]  bf16 bits of the pattern rounded to nearest, ties to even,
 *                by the packed-pair conversion the kernels use (both halves
 *                of the pair must agree; 0xFFFF marks a pair that did not)
 *   e4m3_out[i]  E4M3 (E4M3FN) code: nearest value, ties to the even code,
 *                saturating at +-448, sign bit = the input's sign bit
 *   e4m3_table   optional device f32[256]: the decoded value of each code
 *                (the NaN codes 0x7F and 0xFF give unspecified values).
 * bf16_out (device uint16_t[count]) and e4m3_out (device uint8_t[count])
 * may each be NULL. Non-finite patterns, and finite ones that round beyond
 * the largest bf16, give unspecified results (the library never converts
 * them). count in [0, 2^32]. Returns QLORA_ERR_SHAPE for count out of range.
 */
int qlora_check_conversions(uint32_t first, int64_t count, uint16_t *bf16_out, uint8_t *e4m3_out,
                            float *e4m3_table, hipStream_t stream);

/*
 * Measurement aids for the benchmark's roofline figures; they compute
 * nothing of the method and change no state of the library.
 *
 * qlora_probe_mfma: `workgroups` workgroups of 8 waves; each wave runs
 * `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on register
 * operands (2^18 flops per wave per round, no memory traffic in the loop).
 *   sink    device f32[workgroups * 512], overwritten (keeps the work).
 *   clocks  device uint64[2]: shader clocks (s_memtime) and 100 MHz ticks
 *           (s_memrealtime) spent in workgroup 0's loop, for the clock rate.
 * Returns QLORA_ERR_ARG for NULL pointers or workgroups, iters outside
 * [1, 2^20].
 *
 * qlora_probe_read: reads `bytes` of src once with 16-byte loads (every
 * thread's loads issued before any use) and stores nothing unless the XOR
 * of a thread's words equals `never` (choose a value the data cannot give).
 *   src     device, 16-byte aligned; bytes a positive multiple of
 *           QLORA_PROBE_READ_GRANULE and below 2^40.
 *   sink    device uint32[1].
 * Returns QLORA_ERR_SHAPE for a bad size, QLORA_ERR_ARG for NULL pointers,
 * QLORA_ERR_ALIGN for a misaligned src.
 */
#define QLORA_PROBE_READ_GRANULE 65536
int qlora_probe_mfma(int workgroups, int iters, float *sink, uint64_t *clocks, hipStream_t stream);
int qlora_probe_read(const void *src, size_t bytes, uint32_t never, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
