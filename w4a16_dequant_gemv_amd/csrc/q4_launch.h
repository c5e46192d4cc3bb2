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
