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

// With `query` non-null the linear-layer launchers launch nothing and make
// no HIP call: *query is set to the name of the kernel instantiation the
// dispatch rules select for these arguments (x and y are not read; only the
// addresses of scales and zeros are inspected, for their alignment).
hipError_t q4_launch_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, int bits, uint16_t *y, hipStream_t stream,
                          const char **query = nullptr);

hipError_t q4_launch_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, int bits, uint16_t *y, hipStream_t stream,
                          const char **query = nullptr);

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

// W8A8 with SmoothQuant (w8a8.hip); cols % 8 == 0, k % 32 == 0, k <= 32768.
hipError_t w8a8_launch_col_absmax(const void *src, bool f32, int64_t rows, int cols, float *out,
                                  hipStream_t stream);
hipError_t w8a8_launch_smooth_factors(const float *act_max, const float *w_max, int n, float alpha, float *s,
                                      hipStream_t stream);
hipError_t w8a8_launch_quant_weight(const float *w, const float *s, int64_t n_out, int n_in, int8_t *q, float *sw,
                                    hipStream_t stream);
hipError_t w8a8_launch_quant_act(const uint16_t *x, const float *s, int64_t m, int k, int8_t *q, float *sx,
                                 hipStream_t stream);
hipError_t w8a8_launch_gemm(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw, int64_t m,
                            int64_t n_out, int64_t k, uint16_t *y, hipStream_t stream);

// GPTQ and AWQ (producers.hip).  Workspace sizes in bytes.
int64_t gptq_factor_workspace(int64_t n);
int64_t gptq_loop_workspace(int64_t n_out, int64_t n);
int64_t awq_workspace(int64_t n_out, int64_t n, int64_t t, int n_grid, int group_size);
hipError_t gptq_launch_factor(const uint16_t *x, int64_t t, int n, double damp, void *workspace, float *u,
                              hipStream_t stream);
hipError_t gptq_launch_loop(const float *w, const float *u, int64_t n_out, int n, int group_size, int bits,
                            bool symmetric, void *workspace, uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                            hipStream_t stream);
// The no-allocation GPTQ column loop's scratch: its size, and this
// stream's device copy of it (looked up once per device).
constexpr int64_t kGptqNoAllocScratchBytes = int64_t(72) << 20;
hipError_t gptq_noalloc_scratch(hipStream_t stream, void **ptr);
hipError_t awq_launch(const float *w, const uint16_t *x, int64_t t, int64_t n_out, int n, int group_size, int bits,
                      bool symmetric, int n_grid, void *workspace, uint32_t *qweight, uint16_t *scales,
                      uint16_t *zeros, float *s_out, int32_t *best_out, float *losses_out, hipStream_t stream);
