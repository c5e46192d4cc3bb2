/*
 * w8a8.h -- C ABI of the W8A8 linear layer with SmoothQuant in the same
 * library (libw4a16.so): calibration maxima, smoothing factors, per-channel
 * INT8 weights, per-token INT8 activations and the int8 matrix-core product.
 *
 * Sources (cited by page title and section):
 *   [Guide] "27届大模型面试准备十九 模型量化全攻略 -- INT8/INT4、GPTQ、AWQ、
 *           SmoothQuant 与 KV Cache 量化" (dksg.cn):
 *           §4.2 SmoothQuant: Y = (X diag(s)^-1)(diag(s) W), s_j =
 *           max|X_j|^alpha / max|W_j|^(1 - alpha), alpha = 0.5 the practical
 *           optimum, max|W_j| over every linear sharing the input, both
 *           clamped at 1e-5, diag(s)^-1 foldable into the preceding LayerNorm;
 *           W8A8 runs on INT8 matrix units at twice the FP16 rate;
 *           §2.2 INT8 weights per output channel; §6 the per-token symmetric
 *           map (qmax = 127, scale = max|v| / 127 floored at 1e-8, q =
 *           clamp(round(v / scale), -128, 127)).
 *
 * Conventions (status codes, streams, ownership: as in w4a16.h)
 * -------------------------------------------------------------
 *  - Caller-owned device pointers; no allocation or synchronization; work is
 *    enqueued on `stream`.
 *  - Activations fp16 bit patterns [m][k]; weights fp32 [n_out][k] (W is
 *    [out, in]); codes int8 row-major; scales and factors fp32.
 *  - Every step is one IEEE binary32 operation with RNE (correctly rounded
 *    division and square root), so maxima, factors (alpha = 0.5), codes,
 *    scales and y are bit-exact and independent of the launch configuration;
 *    with alpha != 0.5 the factors use powf and may differ from another libm
 *    by an ulp.
 *  - Sizes: k (= n_in = cols) a multiple of 32 with k <= 32768 for the
 *    quantizers and the product (the int32 sums then cannot overflow), cols a
 *    multiple of 8 for the maxima; m, n_out, rows in [1, 2^24].
 *  - Alignment: x, w, qx, qw and the factor array s 16 bytes; amax, sx, sw 4
 *    bytes; y 2 bytes.  Q4_ERR_NULL / Q4_ERR_SHAPE / Q4_ERR_ALIGN as in
 *    w4a16.h, all before any HIP call.
 *  - Inputs containing NaN or Inf give unspecified (memory-safe) results.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stdint.h>

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Calibration: amax[j] = max(amax[j], max_r |x[r][j]|) for fp16 x [rows][cols]
 * (activations) or fp32 w [rows][cols] (weights).  amax must hold
 * non-negative values (zeros before the first batch); repeated calls fold in
 * more batches, or every linear that shares the input, exactly and in any
 * order.
 */
int sq_absmax_update_f16(const uint16_t *x, int64_t rows, int32_t cols, float *amax, void *stream);
int sq_absmax_update_f32(const float *w, int64_t rows, int32_t cols, float *amax, void *stream);

/*
 * Smoothing factors s[j] = max(act_max[j]^alpha / max(w_max[j], 1e-5)^(1 -
 * alpha), 1e-5) for n channels, 0 <= alpha <= 1 ([Guide] §4.2).  With
 * alpha = 0.5 both powers are correctly rounded square roots.
 */
int sq_smooth_factors(const float *act_max, const float *w_max, int32_t n, float alpha, float *s,
                      void *stream);

/*
 * Per-channel INT8 weights of W diag(s) (s NULL: W itself): qw int8
 * [n_out][k], sw fp32 [n_out], row n quantized symmetrically over its k
 * values ([Guide] §2.2, §4.2).
 */
int w8a8_quantize_weight(const float *w, const float *s, int64_t n_out, int64_t k, int8_t *qw,
                         float *sw, void *stream);

/*
 * Per-token INT8 activations of X diag(s)^-1 (s NULL: X itself, e.g. when
 * the divisor is already folded into the LayerNorm): qx int8 [m][k], sx fp32
 * [m], one symmetric scale per token row, computed at run time.
 */
int w8a8_quantize_act(const uint16_t *x, const float *s, int64_t m, int64_t k, int8_t *qx,
                      float *sx, void *stream);

/*
 * y fp16 [m][n_out] = fp16((float(acc) * sx[m]) * sw[n]) with acc = sum_k
 * qx[m][k] qw[n][k] exact in int32, on the int8 matrix cores
 * (v_mfma_i32_32x32x32_i8).  Bit-exact.
 */
int w8a8_gemm(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw, int64_t m,
              int64_t n_out, int64_t k, uint16_t *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
