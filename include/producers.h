/*
 * producers.h -- C ABI of GPTQ and AWQ in the same library (libw4a16.so):
 * calibration-driven producers of the packed group-wise weights that
 * q4_quantize_pack / q8_quantize_pack write and q4_gemv / q4_gemm consume.
 *
 * Sources (cited by page title and section):
 *   [Guide] "27届大模型面试准备十九 模型量化全攻略 -- INT8/INT4、GPTQ、AWQ、
 *           SmoothQuant 与 KV Cache 量化" (dksg.cn):
 *           §4.3 GPTQ: minimize ||X W^T - X W_hat^T||; H = 2 X^T X from
 *           calibration tokens, damped by 0.01 * mean(diag H); the upper
 *           Cholesky factor of H^-1; column by column, group parameters from
 *           the current weights, the code, and the error (w - w') / U[i][i]
 *           pushed onto the later columns as w_j -= err * U[i][j]; lazy
 *           updates in blocks of 128 columns.
 *           §4.4 AWQ: s_j = (mean |X_j|)^alpha per input channel, W diag(s)
 *           quantized and the activation divided by s; alpha searched on a
 *           grid over [0, 1] for the smallest reconstruction error.
 *
 * Conventions (status codes, streams, ownership: as in w4a16.h)
 * -------------------------------------------------------------
 *  - Caller-owned device pointers; the library allocates nothing: scratch
 *    memory is a caller-provided device `workspace` of at least the size the
 *    matching *_workspace_size() returns (a smaller size is Q4_ERR_SHAPE).
 *    Calls sharing a workspace must not overlap.
 *  - W fp32 [n_out][n]; calibration tokens X fp16 [tokens][n]; outputs in the
 *    packed format of q4_quantize_pack (bits 4) or q8_quantize_pack (bits 8),
 *    with the same group sizes (32, 64, 128, 256 or n) and symmetric mode.
 *  - Precision: H, the damping and the factor in binary64, the column loop
 *    and the AWQ scaling in binary32, AWQ's errors in binary64, each value
 *    from the same sequence of IEEE operations as a plain sequential
 *    implementation of the pages' loops (correctly rounded division and
 *    square root, no contraction), so results are reproducible bit for bit.
 *    Codes use the fp32 scale, errors the stored fp16 scale.
 *  - Sizes: n a multiple of 32 in [32, 32768]; n_out and tokens in [1, 2^24].
 *    H must be positive definite after damping (otherwise the outputs are
 *    unspecified, but memory-safe).
 *  - Alignment: w, qweight and workspace 16 bytes (workspace 256), x, scales,
 *    zeros 2 bytes, u, s and losses 4 bytes.
 */
#ifndef PRODUCERS_H
#define PRODUCERS_H

#include <stdint.h>

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes of gptq_hinv_factor (n x n binary64 twice). */
int64_t gptq_factor_workspace_size(int64_t n);

/*
 * U fp32 [n][n] (upper triangular, zeros below) with U^T U = H^-1, H = 2 X^T X
 * + damp * mean(diag(2 X^T X)) * I from the tokens x (damp = 0.01 on the page,
 * passed as a binary64 value).
 */
int gptq_hinv_factor(const uint16_t *x, int64_t tokens, int64_t n, double damp, void *workspace,
                     int64_t workspace_bytes, float *u, void *stream);

/* Workspace bytes of gptq_quantize (a working copy of W and one block of errors). */
int64_t gptq_quantize_workspace_size(int64_t n_out, int64_t n);

/*
 * The GPTQ column loop on w with the factor u: qweight, scales, zeros in the
 * packed format.  w itself is not modified.
 */
int gptq_quantize(const float *w, const float *u, int64_t n_out, int64_t n, int32_t group_size,
                  int32_t bits, int32_t symmetric, void *workspace, int64_t workspace_bytes,
                  uint32_t *qweight, uint16_t *scales, uint16_t *zeros, void *stream);

/*
 * gptq_quantize without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid allocation).  Same arguments and
 * results as gptq_quantize (bit for bit); the working copy of W and the
 * block errors live in a scratch array of gptq_quantize_noalloc_max_bytes()
 * bytes (72 MiB) that the library holds on every GPU it runs on until the
 * process ends.  A problem with gptq_quantize_workspace_size(n_out, n) above
 * that size returns Q4_ERR_CAPACITY before any HIP call (n_out x n = 4096 x
 * 4096 fits).  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * serialized by the caller.  The scratch needs no clearing: each call writes
 * every part of it before reading it.
 */
int gptq_quantize_noalloc(const float *w, const float *u, int64_t n_out, int64_t n, int32_t group_size,
                          int32_t bits, int32_t symmetric, uint32_t *qweight, uint16_t *scales,
                          uint16_t *zeros, void *stream);

/* Size in bytes of gptq_quantize_noalloc's scratch on each GPU. */
int64_t gptq_quantize_noalloc_max_bytes(void);

/* Workspace bytes of awq_quantize. */
int64_t awq_workspace_size(int64_t n_out, int64_t n, int64_t tokens, int32_t n_grid, int32_t group_size);

/*
 * AWQ: the grid alpha = i / n_grid, i = 0..n_grid (n_grid in [1, 100]); for
 * each, s = max(float((mean_t |x_tj|)^alpha), 1e-5), W diag(s) quantized and
 * dequantized, and the error sum_t sum_n (sum_k x_tk (w_nk - w'_nk / s_k))^2;
 * the first smallest error wins.  Writes the winner's packed weights, s fp32
 * [n] (divide the activations by it, or fold it into the previous layer),
 * optionally the winning index (int32, device) and every error (fp32 [n_grid
 * + 1], device); pass NULL to skip those.
 */
int awq_quantize(const float *w, const uint16_t *x, int64_t tokens, int64_t n_out, int64_t n,
                 int32_t group_size, int32_t bits, int32_t symmetric, int32_t n_grid, void *workspace,
                 int64_t workspace_bytes, uint32_t *qweight, uint16_t *scales, uint16_t *zeros, float *s,
                 int32_t *best, float *losses, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PRODUCERS_H */
