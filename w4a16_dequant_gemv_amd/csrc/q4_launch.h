// q4_launch.h -- internal launchers (validated arguments only; see q4_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// bits is 4 or 8; group_size is 32..256 or n_in (per-channel).
hipError_t q4_launch_quantize_pack(const float *w, int64_t n_out, int64_t n_in, int group_size,
                                   int bits, bool symmetric, uint32_t *qweight, uint16_t *scales,
                                   uint16_t *zeros, hipStream_t stream);

hipError_t q4_launch_dequant(const uint32_t *qweight, const uint16_t *scales,
                             const uint16_t *zeros, int64_t n_out, int64_t n_in,
                             int group_size, int bits, float *out, hipStream_t stream);

hipError_t q4_launch_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, int bits, uint16_t *y, hipStream_t stream);

hipError_t q4_launch_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, int bits, uint16_t *y, hipStream_t stream);

// KV-cache codec (kv_codec.hip); 8 <= d <= 512, d % 8 == 0, bits 4 or 8,
// per-channel blocks of t tokens with ceil(t / (2048 / d)) <= 32.
hipError_t kv_launch_quant_tokens(const uint16_t *x, int64_t rows, int d, int bits, int8_t *q, float *scale,
                                  hipStream_t stream);
hipError_t kv_launch_quant_channels(const uint16_t *x, int64_t blocks, int t, int d, int bits, int8_t *q,
                                    float *scale, hipStream_t stream);
hipError_t kv_launch_flush(const uint16_t *k, const uint16_t *v, int64_t blocks, int t, int d, int bits,
                           const int32_t *dst, int64_t pool_blocks, int8_t *k_pool, float *k_scale, int8_t *v_pool,
                           float *v_scale, hipStream_t stream);
hipError_t kv_launch_dequant_tokens(const int8_t *q, const float *scale, int64_t rows, int d, uint16_t *out,
                                    hipStream_t stream);
hipError_t kv_launch_dequant_channels(const int8_t *q, const float *scale, int64_t blocks, int t, int d,
                                      uint16_t *out, hipStream_t stream);
