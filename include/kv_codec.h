/*
 * kv_codec.h -- C ABI of the KV-cache codec in the same library (libw4a16.so):
 * symmetric INT8 / INT4 quantization of attention keys per channel and of
 * values per token, their dequantization, and the flush of FP16 window blocks
 * into a pool of quantized blocks.
 *
 * Sources (cited by page title and section):
 *   [Guide] "27届大模型面试准备十九 模型量化全攻略 -- INT8/INT4、GPTQ、AWQ、
 *           SmoothQuant 与 KV Cache 量化" (dksg.cn), §6 KV Cache 量化:
 *           K quantized per channel (its outliers sit in fixed channels), V per
 *           token; the most recent tokens (about 128) kept in FP16; the
 *           per-token listing: qmax = 2^(b-1) - 1, scale = max|v| / qmax
 *           floored at 1e-8, q = clamp(round(v / scale), -qmax - 1, qmax) as
 *           int8.
 *   [Intro] "大模型量化技术入门：为什么我们需要量化？" (devpress.csdn.net),
 *           §3.2: separate scale factors for K and V.
 *
 * Conventions (shared with w4a16.h: status codes, streams, ownership)
 * -------------------------------------------------------------------
 *  - Pointers are caller-owned device pointers; the library never allocates,
 *    frees or synchronizes; work is enqueued on `stream` (a hipStream_t).
 *  - Cached values are fp16 bit patterns; codes are int8 (two's complement)
 *    for both widths; scales are fp32.
 *  - Every step is one IEEE binary32 operation with round-to-nearest-even on
 *    the exactly widened fp16 inputs (correctly rounded division), so codes
 *    and scales are bit-exact and independent of the launch configuration.
 *    Dequantized values are fp16(q * scale), the binary32 product rounded
 *    once more to fp16.
 *  - Head dimension d: a multiple of 8 in [8, 512].  bits: 4 or 8 (INT4
 *    codes lie in [-8, 7], one per byte).  Per-channel blocks hold t tokens
 *    with 1 <= t <= 32 * (2048 / d) (t <= 512 at d = 128).
 *  - Alignment: fp16 and int8 arrays 16 bytes; scale arrays 4 bytes (16 for
 *    kv_dequant_channels).  Violations return Q4_ERR_ALIGN; bad sizes or bits
 *    Q4_ERR_SHAPE; NULL pointers Q4_ERR_NULL; all before any HIP call.
 *  - Inputs containing NaN or Inf give unspecified (memory-safe) results.
 */
#ifndef KV_CODEC_H
#define KV_CODEC_H

#include <stdint.h>

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Per-token quantization (the V side): x fp16 [rows][d] -> q int8 [rows][d],
 * scale fp32 [rows], one symmetric scale per row over its d values
 * ([Guide] §6, quant_kv_per_token).  A [B][H][S][D] cache is rows = B*H*S.
 */
int kv_quant_tokens(const uint16_t *x, int64_t rows, int32_t d, int32_t bits,
                    int8_t *q, float *scale, void *stream);

/*
 * Per-channel quantization (the K side): x fp16 [blocks][t][d] -> q int8
 * [blocks][t][d], scale fp32 [blocks][d]; channel j of a block gets one
 * symmetric scale over the block's t tokens ([Guide] §6: K per channel).  A
 * block is t consecutive tokens of one head, e.g. the 128 tokens that leave
 * the FP16 window together.
 */
int kv_quant_channels(const uint16_t *x, int64_t blocks, int32_t t, int32_t d,
                      int32_t bits, int8_t *q, float *scale, void *stream);

/* out fp16 [rows][d] = fp16(q * scale[row]). */
int kv_dequant_tokens(const int8_t *q, const float *scale, int64_t rows, int32_t d,
                      uint16_t *out, void *stream);

/* out fp16 [blocks][t][d] = fp16(q * scale[block][channel]). */
int kv_dequant_channels(const int8_t *q, const float *scale, int64_t blocks, int32_t t,
                        int32_t d, uint16_t *out, void *stream);

/*
 * Flush of FP16 window blocks into a block pool in one launch: block p of k
 * and v (fp16 [blocks][t][d] each) is quantized -- K per channel, V per token
 * -- into pool slot dst[p] (int32 device array [blocks]): k_pool / v_pool
 * int8 [pool_blocks][t][d], k_scale fp32 [pool_blocks][d], v_scale fp32
 * [pool_blocks][t].  Entries of dst outside [0, pool_blocks) are skipped
 * (their slots are not written); two entries naming the same slot race.
 * Slots not named by dst are left unchanged.
 */
int kv_flush_blocks(const uint16_t *k, const uint16_t *v, int64_t blocks, int32_t t,
                    int32_t d, int32_t bits, const int32_t *dst, int64_t pool_blocks,
                    int8_t *k_pool, float *k_scale, int8_t *v_pool, float *v_scale,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KV_CODEC_H */
