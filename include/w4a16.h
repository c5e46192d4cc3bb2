/*
 * w4a16.h -- C ABI of the W4A16 library for AMD Instinct MI355X (gfx950):
 * group-wise (or per-channel) INT4 weight quantization with packing,
 * dequantization, and the linear layer y = x W'^T that unpacks and
 * dequantizes the weights on the fly (decode GEMV for 1..16 rows of x,
 * prefill GEMM for any number of rows); the same for INT8 weights (W8A16,
 * the q8_* entry points).
 *
 * Sources (cited by page title and section):
 *   [Guide] "27届大模型面试准备十九 模型量化全攻略 -- INT8/INT4、GPTQ、AWQ、
 *           SmoothQuant 与 KV Cache 量化" (dksg.cn)
 *   [Path]  "从 FP32 到 INT4：大模型推理加速中的量化优化实战路径" (adg.csdn.net)
 *   [Zero]  "从0到1：大模型量化" (pinyinjj.github.io)
 *   [Kern]  "大模型量化技术定义与主流方案解析" (cloud.baidu.com)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are device pointers (memory from hipMalloc or a torch CUDA
 *    tensor), owned by the caller.  The library never allocates, frees or
 *    synchronizes.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) and is complete only when the caller synchronizes it.
 *  - Layouts are dense row-major.  W and W' are [n_out][n_in] ([Guide] §2.2
 *    takes W as [out_features, in_features]); groups run along n_in.
 *  - fp16 values travel as uint16_t bit patterns (IEEE binary16).
 *  - Packed weights, q4_*: uint32_t [n_out][n_in / 8]; element k of a row is
 *    the 4-bit code in bits 4*(k % 8) .. 4*(k % 8) + 3 of word k / 8.
 *    q8_*: uint32_t [n_out][n_in / 4]; element k is the byte in bits
 *    8*(k % 4) .. 8*(k % 4) + 7 of word k / 4.
 *  - Scales and zero-points: fp16 [n_out][n_in / group_size].  Symmetric
 *    quantization stores its signed b-bit codes q in [-2^(b-1), 2^(b-1) - 1]
 *    as q + 2^(b-1) with a stored zero-point of 2^(b-1) (8 for INT4, 128 for
 *    INT8), so every consumer computes w' = s * (code - z).
 *  - Outputs are fully overwritten; inputs must not overlap outputs.
 *  - Return value: Q4_OK, or one of the Q4_ERR_* codes below.  Argument
 *    errors are detected before any HIP call is made.  A fault inside a
 *    kernel surfaces at the caller's next synchronization, not here.
 *  - Supported group sizes are 32, 64, 128 and 256 ([Zero] §3.1 names
 *    blocks of 32 and 256, [Path] §2.2 groups of 128 and 64), and
 *    group_size == n_in: one scale and zero-point per output channel
 *    ([Guide] §2.2, the usual granularity for INT8 weights), for any n_in
 *    that is a multiple of 32.  Any other size is rejected with
 *    Q4_ERR_GROUP rather than served by a slow generic path.
 *  - Inputs containing NaN or Inf give unspecified (but memory-safe) results.
 *  - Calls are thread-safe; the library keeps no mutable global state.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_ABI_VERSION 4

enum {
    Q4_OK = 0,
    Q4_ERR_NULL = 1,   /* a required pointer is NULL */
    Q4_ERR_SHAPE = 2,  /* a size <= 0 or too large, n_in % group_size != 0,
                          or m outside the entry point's range */
    Q4_ERR_GROUP = 3,  /* group_size not in {32, 64, 128, 256} and not
                          n_in (per-channel with n_in a multiple of 32) */
    Q4_ERR_ALIGN = 4,  /* w, w_out, qweight or x not 16-byte aligned, or an
                          fp16 array not 2-byte aligned */
    Q4_ERR_HIP = 5,    /* the HIP runtime refused the launch; see
                          q4_last_hip_error() */
    Q4_ERR_CAPACITY = 6 /* a no-allocation entry point was given a problem
                           larger than its fixed scratch memory */
};

/* Largest sizes accepted: n_in <= 2^20, n_out <= 2^24, m <= 2^24, and
 * n_out * n_in, m * n_in and m * n_out each <= 2^34 elements. */

/* Q4_ABI_VERSION of the loaded library. */
int q4_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *q4_strerror(int status);

/* hipError_t of the last launch failure on the calling thread (0 if none). */
int q4_last_hip_error(void);

/*
 * Group-wise INT4 quantization and packing of W (fp32 [n_out][n_in]).
 * For every group of `group_size` consecutive elements of a row, all in
 * binary32 with round-to-nearest-even ([Guide] §2.1 gives the affine map
 * q = clamp(round(x/s) + z) with min-max calibration; [Path] §2.1 clips z
 * and the codes):
 *   asymmetric: s = max((max - min) / 15, 1e-8), z = clamp(rint(-min/s), 0, 15),
 *               code = clamp(rint(w/s) + z, 0, 15);
 *   symmetric:  s = max(max|w| / 7, 1e-8), q = clamp(rint(w/s), -8, 7),
 *               code = q + 8, stored zero-point 8.
 * Writes qweight (u32 [n_out][n_in/8]), scales = fp16(s) and zeros = fp16(z)
 * (fp16 [n_out][n_in/group_size]).  Results are bit-exact: every step is a
 * single IEEE operation, independent of launch configuration.
 * w and qweight must be 16-byte aligned.
 */
int q4_quantize_pack(const float *w, int64_t n_out, int64_t n_in,
                     int32_t group_size, int32_t symmetric,
                     uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                     void *stream);

/*
 * Dequantization w' = s * (code - z) into fp32 w_out [n_out][n_in]
 * ([Guide] §2.1, dequantize_tensor; [Zero] §2, f' = S (q - Z)).  The product
 * of an fp16 scale and an integer in [-15, 15] is exact in binary32, so the
 * result is bit-exact.  qweight and w_out must be 16-byte aligned.
 */
int q4_dequant(const uint32_t *qweight, const uint16_t *scales, const uint16_t *zeros,
               int64_t n_out, int64_t n_in, int32_t group_size, float *w_out,
               void *stream);

/*
 * Decode-shaped W4A16 linear layer: y = x W'^T for 1 <= m <= 16, with
 * x fp16 [m][n_in] and y fp16 [m][n_out].  The packed weights are unpacked
 * and dequantized in registers and never written back ([Kern] §4: fused
 * dequantization inside the matrix product; [Guide] §2.3: INT4 weights, FP16
 * activations).  Products accumulate in fp32; y is rounded to fp16 once.
 * Error bound per element: |y - x w'| <= 2e-3 * sum_k |x_k w'_k| + 1e-5.
 * Results are deterministic for a given shape.  qweight and x must be
 * 16-byte aligned.  m > 16 returns Q4_ERR_SHAPE (use q4_gemm).
 */
int q4_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
            const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
            int32_t group_size, uint16_t *y, void *stream);

/*
 * Prefill-shaped W4A16 linear layer: the same contract as q4_gemv for any
 * m >= 1, organised for large m: packed weight tiles are dequantized into
 * LDS as fp16 and fed to the fp16 matrix cores with fp32 accumulation
 * ([Guide] §2.3: W4A16 dequantizes to FP16 before the product, so prefill is
 * compute-bound).  Same error bound and alignment rules as q4_gemv.
 */
int q4_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
            const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
            int32_t group_size, uint16_t *y, void *stream);

/*
 * INT8 weights (W8A16, [Guide] §2.3: INT8 weights, FP16 activations).
 * Group-wise or per-channel INT8 quantization and packing of W (fp32
 * [n_out][n_in]), the 8-bit case of the same affine map ([Guide] §2.1:
 * asymmetric s = (max - min)/(2^b - 1), symmetric s = max|x|/(2^(b-1) - 1);
 * [Path] §2.1 clips z and the codes), all in binary32 with RNE:
 *   asymmetric: s = max((max - min) / 255, 1e-8), z = clamp(rint(-min/s), 0, 255),
 *               code = clamp(rint(w/s) + z, 0, 255);
 *   symmetric:  s = max(max|w| / 127, 1e-8), q = clamp(rint(w/s), -128, 127),
 *               code = q + 128, stored zero-point 128.
 * Writes qweight (u32 [n_out][n_in/4]), scales and zeros (fp16
 * [n_out][n_in/group_size]), bit-exact.  group_size == n_in gives one scale
 * per output channel.  Same alignment rules as q4_quantize_pack.
 */
int q8_quantize_pack(const float *w, int64_t n_out, int64_t n_in,
                     int32_t group_size, int32_t symmetric,
                     uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                     void *stream);

/*
 * INT8 dequantization w' = s * (code - z) into fp32 w_out [n_out][n_in];
 * the product of an fp16 scale and an integer in [-255, 255] is exact in
 * binary32, so the result is bit-exact.  Same alignment rules as q4_dequant.
 */
int q8_dequant(const uint32_t *qweight, const uint16_t *scales, const uint16_t *zeros,
               int64_t n_out, int64_t n_in, int32_t group_size, float *w_out,
               void *stream);

/*
 * Decode-shaped W8A16 linear layer: y = x W'^T for 1 <= m <= 16 with INT8
 * weights packed as q8_quantize_pack writes them; the codes are dequantized
 * in registers as (1024 + c) - (1024 + z), exact in fp16, times s.  Same
 * error bound, alignment rules and m range as q4_gemv.
 */
int q8_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
            const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
            int32_t group_size, uint16_t *y, void *stream);

/*
 * Prefill-shaped W8A16 linear layer for any m >= 1: INT8 weight tiles are
 * dequantized into LDS as fp16 and fed to the fp16 matrix cores, as in
 * q4_gemm.  Same error bound and alignment rules as q4_gemv.
 */
int q8_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
            const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
            int32_t group_size, uint16_t *y, void *stream);

/*
 * Kernel selection report, for tests and profiling.  Writes to `name` the
 * kernel instantiation that q4_gemv (op 0) or q4_gemm (op 1) -- q8_gemv and
 * q8_gemm for bits 8 -- launches for these sizes, in the form profilers
 * print kernel names (e.g. "gemv_resident_kernel<8, 1, 1, 2, true, 4,
 * false>"), NUL-terminated and truncated to name_len bytes.  Nothing is
 * launched and no HIP call is made, so it also works on a host without a
 * GPU.  The selection can depend on the alignment of the scale and
 * zero-point arrays, so their addresses are passed: they are inspected,
 * never dereferenced (any value with the alignment of the real arrays will
 * do).  Returns the status the linear-layer entry point would return for
 * these sizes (Q4_ERR_SHAPE also for op or bits outside {0, 1} / {4, 8} or
 * name_len < 1; Q4_ERR_NULL for a NULL scales, zeros or name).
 */
int q4_linear_config(int32_t op, int32_t bits, int64_t m, int64_t n_out, int64_t n_in,
                     int32_t group_size, const void *scales, const void *zeros,
                     char *name, int64_t name_len);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
