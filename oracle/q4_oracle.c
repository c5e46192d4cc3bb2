/*
 * q4_oracle.c -- CPU oracle for group-wise INT4 / INT8 weight quantization
 * (per group or per output channel), the W4A16 / W8A16 linear layer, the
 * KV-cache codec (V per token, K per channel, symmetric INT8 / INT4), the
 * W8A8 linear layer with SmoothQuant, and GPTQ / AWQ as producers of the
 * packed weight format.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg load it.  It shares no
 * code, header, table or constant generator with the HIP library, and the
 * HIP library never loads it.
 *
 * Sources (cited by page title and section):
 *   [Guide]  "27届大模型面试准备十九 模型量化全攻略 -- INT8/INT4、GPTQ、AWQ、
 *            SmoothQuant 与 KV Cache 量化" (dksg.cn)
 *   [Path]   "从 FP32 到 INT4：大模型推理加速中的量化优化实战路径" (adg.csdn.net)
 *   [Zero]   "从0到1：大模型量化" (pinyinjj.github.io)
 *   [Intro]  "大模型量化技术入门：为什么我们需要量化？" (devpress.csdn.net)
 *
 * Precision.  The pages state the quantizer on float32 tensors ([Guide] §2.1,
 * the quantize_tensor snippet; [Path] §2.1, the NumPy quantizers), so every
 * quantizer step here is one IEEE binary32 operation with round-to-nearest-
 * even.  Build with -ffp-contract=off and without fast-math so that no step
 * is fused or reassociated.  The reference product is accumulated in binary64.
 *
 * Readings where the pages are silent or disagree (all listed in the design
 * notes of the repository):
 *   - the 1e-8 floor on s is applied before z and the codes are computed;
 *   - z is clipped to [0, 2^b - 1] as in [Path] §2.1;
 *   - codes are computed from the fp32 s; fp16 is the storage type of s, z;
 *   - rounding is round-half-to-even (torch.round / np.round semantics);
 *   - symmetric b-bit codes q in [-2^(b-1), 2^(b-1) - 1] are stored
 *     offset-binary as q + 2^(b-1) with a stored zero-point of 2^(b-1), so
 *     dequantization is mode-agnostic;
 *   - packing (not on the pages): element (32/b) j + t of a row sits in bits
 *     b t .. b t + b - 1 of 32-bit word j of that row, rows are
 *     [n_out][n_in * b / 32];
 *   - per-channel quantization is the group size n_in (one group per row).
 *
 * Parity status of each function is stated beside it.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Thread count of the parallel loops below (timing of the CPU baseline on
 * one core and on all of them; results do not depend on it). */
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* binary32 <-> binary16, written from the IEEE 754 definitions.             */
/* Pinned against numpy.float16 over every binary32 bit pattern.             */
/* ------------------------------------------------------------------------ */

static uint32_t bits_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
static float float_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

/* Round-to-nearest-even conversion.  Subnormal halves are produced, values
 * whose magnitude rounds past the largest half (65504) become infinity, and
 * NaN stays NaN (payload not specified). */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t b = bits_of(f);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t e8 = (b >> 23) & 0xFFu;
    uint32_t frac = b & 0x7FFFFFu;

    if (e8 == 0xFFu)                       /* inf or NaN */
        return (uint16_t)(sign | (frac ? 0x7E00u : 0x7C00u));
    if (e8 == 0)                           /* binary32 zero/subnormal: < 2^-126 */
        return sign;

    /* |f| = sig * 2^(e - 23) with a 24-bit significand. */
    int e = (int)e8 - 127;
    uint32_t sig = frac | 0x800000u;

    /* The half result is q * 2^(E - 10) for normal halves (E = max(e, -14))
     * and q * 2^-24 for subnormal ones; both cases drop `shift` low bits. */
    int shift = (e >= -14) ? 13 : (-1 - e);
    if (shift > 24)                        /* below half of the least subnormal */
        return sign;
    uint32_t q = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;                           /* round to nearest, ties to even */

    uint32_t h;
    if (e >= -14) {
        if (e > 15)
            return (uint16_t)(sign | 0x7C00u);
        /* q holds the implicit bit (0x400); a carry out of the significand
         * moves into the exponent field, which is exactly the right result,
         * including the step from 65504 up to infinity. */
        h = ((uint32_t)(e + 14) << 10) + q;
        if (h >= 0x7C00u)
            h = 0x7C00u;
    } else {
        h = q;                              /* 0x400 here is the least normal */
    }
    return (uint16_t)(sign | h);
}

/* Exact widening. */
float orc_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e5 = ((uint32_t)h >> 10) & 0x1Fu;
    uint32_t frac = (uint32_t)h & 0x3FFu;
    if (e5 == 0) {
        float mag = (float)frac * 0x1p-24f;           /* exact */
        return float_of(bits_of(mag) | sign);
    }
    if (e5 == 0x1Fu)
        return float_of(sign | 0x7F800000u | (frac << 13));
    return float_of(sign | ((e5 - 15u + 127u) << 23) | (frac << 13));
}

void orc_f32_to_f16_array(const float *src, uint16_t *dst, int64_t n)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        dst[i] = orc_f32_to_f16(src[i]);
}

/* Converts the binary32 values whose bit patterns are first, first+1, ...,
 * first+count-1 (used by the exhaustive converter test). */
void orc_f32_bits_range_to_f16(uint32_t first, int64_t count, uint16_t *dst)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++)
        dst[i] = orc_f32_to_f16(float_of(first + (uint32_t)i));
}

void orc_f16_to_f32_array(const uint16_t *src, float *dst, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        dst[i] = orc_f16_to_f32(src[i]);
}

/* ------------------------------------------------------------------------ */
/* Uniform affine quantization of one group.                                 */
/* [Guide] §2.1 (q = clamp(round(x/s) + z, qmin, qmax); min-max calibration: */
/* symmetric s = max|x| / (2^(b-1) - 1), asymmetric s = (max - min)/(2^b-1), */
/* z = round(-min/s); s floored at 1e-8); [Path] §2.1 (z clipped to         */
/* [0, 2^b - 1], symmetric codes clipped to [-2^(b-1), 2^(b-1) - 1]);       */
/* [Intro] §2.2 and [Zero] §2 (Q = round(X/scale) + zero_point).             */
/* Pinned by brute force over all codes, the worked per-tensor example of    */
/* [Guide] §3, the s/2 bound, idempotence, grid-exact and constant groups.   */
/* ------------------------------------------------------------------------ */

static float clampf(float v, float lo, float hi)
{
    if (v < lo) v = lo;
    if (v > hi) v = hi;
    return v;
}

/* v[0..n) -> fp32 scale *s, integer zero-point *z and integer codes q[].
 * Asymmetric codes lie in [0, 2^b - 1]; symmetric codes in
 * [-2^(b-1), 2^(b-1) - 1] with z = 0. */
void orc_quantize_group(const float *v, int64_t n, int bits, int symmetric,
                        float *s_out, int32_t *z_out, int32_t *q)
{
    if (symmetric) {
        const float qmax = (float)((1 << (bits - 1)) - 1);
        const float qmin = -(float)(1 << (bits - 1));
        float amax = 0.0f;
        for (int64_t i = 0; i < n; i++)
            if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
        float s = amax / qmax;
        if (s < 1e-8f) s = 1e-8f;
        for (int64_t i = 0; i < n; i++)
            q[i] = (int32_t)clampf(rintf(v[i] / s), qmin, qmax);
        *s_out = s;
        *z_out = 0;
    } else {
        const float qmax = (float)((1 << bits) - 1);
        float mn = v[0], mx = v[0];
        for (int64_t i = 1; i < n; i++) {
            if (v[i] < mn) mn = v[i];
            if (v[i] > mx) mx = v[i];
        }
        float s = (mx - mn) / qmax;
        if (s < 1e-8f) s = 1e-8f;
        int32_t z = (int32_t)clampf(rintf(-mn / s), 0.0f, qmax);
        for (int64_t i = 0; i < n; i++)
            q[i] = (int32_t)clampf(rintf(v[i] / s) + (float)z, 0.0f, qmax);
        *s_out = s;
        *z_out = z;
    }
}

/* ------------------------------------------------------------------------ */
/* Per-group b-bit quantization (b = 4 or 8) of W[n_out][n_in] along the     */
/* input dimension, fp16 storage of s and z, and packing of 32/b codes per   */
/* 32-bit word.                                                              */
/* [Guide] §2.2 (W[out_features, in_features]; one scale per group of 128    */
/* input elements per output channel for INT4, one scale per output channel */
/* -- per-channel -- for INT8 weights; fp16 scale); [Guide] §2.3 (W8A16:     */
/* INT8 weights, FP16 activations); [Guide] §2.1 and [Path] §2.1 (the b-bit  */
/* code ranges); [Zero] §3.1 (each block keeps its own S and Z); [Path] §2.2 */
/* (group_size 128 / 64).  group_size may be any divisor of n_in;           */
/* group_size == n_in is the per-channel case.  Symmetric codes q are        */
/* stored offset-binary as q + 2^(b-1) with a stored zero-point of 2^(b-1).  */
/* The packing order is this library's convention (element k of a row in    */
/* bits b*(k % (32/b)) .. of word k / (32/b)); it is pinned only by the      */
/* brute-force unpack (parity unpinned against the pages, which give none).  */
/* Returns 0, 1 for an unsupported shape, 2 if scratch memory ran out.       */
/* ------------------------------------------------------------------------ */
int orc_quantize_pack_bits(const float *w, int64_t n_out, int64_t n_in,
                           int32_t group_size, int32_t bits, int32_t symmetric,
                           uint32_t *packed, uint16_t *scales, uint16_t *zeros,
                           float *s_fp32 /* may be NULL */)
{
    if ((bits != 4 && bits != 8) || group_size <= 0 || n_in % group_size != 0 ||
        n_in % (32 / bits) != 0)
        return 1;
    const int per_word = 32 / bits;
    const int64_t words = n_in / per_word;
    const int64_t groups = n_in / group_size;
    const int32_t offset = 1 << (bits - 1);
    int failed = 0;

    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_out; n++) {
        int32_t *codes = (int32_t *)malloc((size_t)group_size * sizeof(int32_t));
        if (!codes) {
            #pragma omp atomic write
            failed = 1;
            continue;
        }
        uint32_t *row = packed + n * words;
        memset(row, 0, (size_t)words * sizeof(uint32_t));
        for (int64_t j = 0; j < groups; j++) {
            const float *v = w + n * n_in + j * group_size;
            float s;
            int32_t z;
            orc_quantize_group(v, group_size, bits, symmetric, &s, &z, codes);
            int32_t z_store = symmetric ? offset : z;
            for (int64_t t = 0; t < group_size; t++) {
                uint32_t u = (uint32_t)(symmetric ? codes[t] + offset : codes[t]);
                int64_t k = j * group_size + t;
                row[k / per_word] |= u << (bits * (k % per_word));
            }
            scales[n * groups + j] = orc_f32_to_f16(s);
            zeros[n * groups + j] = orc_f32_to_f16((float)z_store);
            if (s_fp32)
                s_fp32[n * groups + j] = s;
        }
        free(codes);
    }
    return failed ? 2 : 0;
}

/* The INT4 case: 8 codes per word, [n_out][n_in/8]. */
int orc_quantize_pack(const float *w, int64_t n_out, int64_t n_in,
                      int32_t group_size, int32_t symmetric,
                      uint32_t *packed, uint16_t *scales, uint16_t *zeros,
                      float *s_fp32 /* may be NULL */)
{
    return orc_quantize_pack_bits(w, n_out, n_in, group_size, 4, symmetric, packed,
                                  scales, zeros, s_fp32);
}

/* ------------------------------------------------------------------------ */
/* Dequantization w' = s * (q - z) in float32.                               */
/* [Guide] §2.1 (x_hat = s * (q - z); dequantize_tensor returns float32);    */
/* [Zero] §2 (f' = S * (q - Z)).  The product of an fp16 scale and an        */
/* integer in [-255, 255] is exact in binary32.                              */
/* ------------------------------------------------------------------------ */
void orc_dequant_bits(const uint32_t *packed, const uint16_t *scales,
                      const uint16_t *zeros, int64_t n_out, int64_t n_in,
                      int32_t group_size, int32_t bits, float *out)
{
    const int per_word = 32 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t groups = n_in / group_size;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_out; n++) {
        for (int64_t k = 0; k < n_in; k++) {
            uint32_t word = packed[n * (n_in / per_word) + k / per_word];
            int32_t u = (int32_t)((word >> (bits * (k % per_word))) & mask);
            float s = orc_f16_to_f32(scales[n * groups + k / group_size]);
            int32_t z = (int32_t)orc_f16_to_f32(zeros[n * groups + k / group_size]);
            out[n * n_in + k] = s * (float)(u - z);
        }
    }
}

void orc_dequant(const uint32_t *packed, const uint16_t *scales,
                 const uint16_t *zeros, int64_t n_out, int64_t n_in,
                 int32_t group_size, float *out)
{
    orc_dequant_bits(packed, scales, zeros, n_out, n_in, group_size, 4, out);
}

/* ------------------------------------------------------------------------ */
/* Reference product of the linear layer on the dequantized weights:         */
/* y[m][n] = sum_k x[m][k] * w'[n][k] and a[m][n] = sum_k |x[m][k] w'[n][k]| */
/* in binary64 (each product is exact there).  [Guide] §2.2 (W is           */
/* [out_features, in_features]) and §2.3 (W4A16: INT4 weights, FP16          */
/* activations, weights dequantized before the product).                    */
/* Pinned against numpy float64 matmul and one-hot inputs.                   */
/* ------------------------------------------------------------------------ */
void orc_linear_ref(const uint16_t *x_f16, const float *w_deq,
                    int64_t m, int64_t n_out, int64_t n_in,
                    double *y, double *a)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_out; n++) {
        for (int64_t i = 0; i < m; i++) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t k = 0; k < n_in; k++) {
                double p = (double)orc_f16_to_f32(x_f16[i * n_in + k])
                         * (double)w_deq[n * n_in + k];
                acc += p;
                acc_abs += fabs(p);
            }
            y[i * n_out + n] = acc;
            a[i * n_out + n] = acc_abs;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* KV-cache codec.                                                           */
/* [Guide] §6 (KV Cache 量化): K and V are quantized differently -- K per    */
/* channel (its outliers sit in fixed channels), V per token -- and the      */
/* most recent tokens (about 128) stay in FP16.  Its quant_kv_per_token      */
/* listing is the symmetric map with one scale per token over the head       */
/* dimension: qmax = 2^(b-1) - 1, scale = max|v| / qmax floored at 1e-8,     */
/* q = clamp(round(v / scale), -qmax - 1, qmax) stored as int8.  [Intro]     */
/* §3.2 asks for separate scale factors for K and V.                         */
/* Readings: the cache holds fp16 values, widened exactly to binary32; every */
/* step is one binary32 operation (the weight quantizer's precision); the    */
/* scale is kept in binary32; K is quantized per channel over a block of t   */
/* consecutive tokens of one head (the block that leaves the FP16 window);   */
/* dequantization is the binary32 product q * scale, rounded once more to    */
/* fp16 for the cache consumer.  Both quantizers are the symmetric case of   */
/* orc_quantize_group (pinned above) applied to a token row or to a channel  */
/* column; pinned by brute force, the [Guide] §3 worked example, the s/2     */
/* bound, the K/V transposition identity and the [Guide] §6 cache sizes.     */
/* ------------------------------------------------------------------------ */
int orc_kv_quant_tokens(const uint16_t *x, int64_t rows, int32_t d, int32_t bits,
                        int8_t *q, float *scale)
{
    if (bits < 2 || bits > 8 || d <= 0)
        return 1;
    int failed = 0;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float *v = (float *)malloc((size_t)d * sizeof(float));
        int32_t *c = (int32_t *)malloc((size_t)d * sizeof(int32_t));
        if (!v || !c) {
            #pragma omp atomic write
            failed = 1;
            free(v);
            free(c);
            continue;
        }
        for (int32_t i = 0; i < d; i++)
            v[i] = orc_f16_to_f32(x[r * d + i]);
        float s;
        int32_t z;
        orc_quantize_group(v, d, bits, 1, &s, &z, c);
        for (int32_t i = 0; i < d; i++)
            q[r * d + i] = (int8_t)c[i];
        scale[r] = s;
        free(v);
        free(c);
    }
    return failed ? 2 : 0;
}

/* x [blocks][t][d] -> q [blocks][t][d], scale [blocks][d]: channel j of a
 * block is quantized over its t tokens. */
int orc_kv_quant_channels(const uint16_t *x, int64_t blocks, int32_t t, int32_t d,
                          int32_t bits, int8_t *q, float *scale)
{
    if (bits < 2 || bits > 8 || d <= 0 || t <= 0)
        return 1;
    int failed = 0;
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < blocks; b++) {
        float *v = (float *)malloc((size_t)t * sizeof(float));
        int32_t *c = (int32_t *)malloc((size_t)t * sizeof(int32_t));
        if (!v || !c) {
            #pragma omp atomic write
            failed = 1;
            free(v);
            free(c);
            continue;
        }
        const uint16_t *xb = x + b * (int64_t)t * d;
        for (int32_t j = 0; j < d; j++) {
            for (int32_t i = 0; i < t; i++)
                v[i] = orc_f16_to_f32(xb[(int64_t)i * d + j]);
            float s;
            int32_t z;
            orc_quantize_group(v, t, bits, 1, &s, &z, c);
            for (int32_t i = 0; i < t; i++)
                q[b * (int64_t)t * d + (int64_t)i * d + j] = (int8_t)c[i];
            scale[b * d + j] = s;
        }
        free(v);
        free(c);
    }
    return failed ? 2 : 0;
}

/* Dequantization of per-token rows: out = fp16(q * scale[row]). */
void orc_kv_dequant_tokens(const int8_t *q, const float *scale, int64_t rows, int32_t d,
                           uint16_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int32_t i = 0; i < d; i++)
            out[r * d + i] = orc_f32_to_f16((float)q[r * d + i] * scale[r]);
}

/* Dequantization of per-channel blocks: out = fp16(q * scale[block][channel]). */
void orc_kv_dequant_channels(const int8_t *q, const float *scale, int64_t blocks, int32_t t,
                             int32_t d, uint16_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < blocks; b++)
        for (int32_t i = 0; i < t; i++)
            for (int32_t j = 0; j < d; j++) {
                const int64_t e = b * (int64_t)t * d + (int64_t)i * d + j;
                out[e] = orc_f32_to_f16((float)q[e] * scale[b * d + j]);
            }
}

/* [Guide] §6: KV cache bytes = 2 (K and V) x layers x kv_heads x head_dim x
 * seq x batch x bytes per element (codes only, scales not counted). */
double orc_kv_cache_bytes(int64_t layers, int64_t kv_heads, int64_t head_dim, int64_t seq,
                          int64_t batch, int32_t bits)
{
    return 2.0 * (double)layers * (double)kv_heads * (double)head_dim * (double)seq *
           (double)batch * (double)bits / 8.0;
}

/* ------------------------------------------------------------------------ */
/* W8A8 with SmoothQuant.                                                    */
/* [Guide] §4.2 (SmoothQuant): Y = (X diag(s)^-1)(diag(s) W) with per input  */
/* channel s_j = max|X_j|^alpha / max|W_j|^(1 - alpha), alpha = 0.5 the      */
/* practical optimum; its smooth_ln_linear listing takes max|W_j| over all   */
/* linears sharing the input, clamps it and s at 1e-5, multiplies the       */
/* weights by s and divides the activations (folded into the LayerNorm).     */
/* W8A8 = INT8 weights and activations on INT8 matrix units ([Guide] §2.3,   */
/* §4.2); INT8 weights per output channel ([Guide] §2.2); activations        */
/* quantized per token at run time, the per-token symmetric map of the      */
/* [Guide] §6 listing.                                                       */
/* Readings: everything in binary32 with RNE; alpha = 0.5 takes both powers  */
/* as square roots (correctly rounded, so bit-exact); other alphas use powf; */
/* the smoothed weight is the binary32 product w * s; the smoothed          */
/* activation is the binary32 quotient x / s; the integer product is exact   */
/* (int64 here); y = fp16((float(acc) * sx[m]) * sw[n]), evaluated left to   */
/* right.  Pinned by the SmoothQuant identity, the alpha = 0.5 balance and   */
/* the alpha = 0 / 1 limits, brute force of the row quantizers, numpy's      */
/* int64 matmul and an error bound of the whole product.                     */
/* ------------------------------------------------------------------------ */
void orc_col_absmax_f16(const uint16_t *x, int64_t rows, int64_t cols, float *out)
{
    for (int64_t j = 0; j < cols; j++)
        out[j] = 0.0f;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t j = 0; j < cols; j++) {
            const float a = fabsf(orc_f16_to_f32(x[r * cols + j]));
            if (a > out[j]) out[j] = a;
        }
}

void orc_col_absmax_f32(const float *w, int64_t rows, int64_t cols, float *out)
{
    for (int64_t j = 0; j < cols; j++)
        out[j] = 0.0f;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t j = 0; j < cols; j++) {
            const float a = fabsf(w[r * cols + j]);
            if (a > out[j]) out[j] = a;
        }
}

void orc_smooth_factors(const float *act_max, const float *w_max, int64_t cols, float alpha, float *s)
{
    for (int64_t j = 0; j < cols; j++) {
        const float w = w_max[j] < 1e-5f ? 1e-5f : w_max[j];
        float num, den;
        if (alpha == 0.5f) {
            num = sqrtf(act_max[j]);
            den = sqrtf(w);
        } else {
            num = powf(act_max[j], alpha);
            den = powf(w, 1.0f - alpha);
        }
        float v = num / den;
        s[j] = v < 1e-5f ? 1e-5f : v;
    }
}

/* W [n_out][n_in] fp32, s [n_in] (NULL: no smoothing) -> q int8 [n_out][n_in],
 * sw [n_out]: row n of W * diag(s) quantized symmetrically to INT8. */
int orc_w8a8_quant_weight(const float *w, const float *s, int64_t n_out, int64_t n_in,
                          int8_t *q, float *sw)
{
    int failed = 0;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_out; n++) {
        float *v = (float *)malloc((size_t)n_in * sizeof(float));
        int32_t *c = (int32_t *)malloc((size_t)n_in * sizeof(int32_t));
        if (!v || !c) {
            #pragma omp atomic write
            failed = 1;
            free(v);
            free(c);
            continue;
        }
        for (int64_t k = 0; k < n_in; k++)
            v[k] = s ? w[n * n_in + k] * s[k] : w[n * n_in + k];
        float sc;
        int32_t z;
        orc_quantize_group(v, n_in, 8, 1, &sc, &z, c);
        for (int64_t k = 0; k < n_in; k++)
            q[n * n_in + k] = (int8_t)c[k];
        sw[n] = sc;
        free(v);
        free(c);
    }
    return failed ? 2 : 0;
}

/* x fp16 [m][k], s [k] (NULL: no smoothing) -> q int8 [m][k], sx [m]: token
 * row m of x * diag(s)^-1 quantized symmetrically to INT8. */
int orc_w8a8_quant_act(const uint16_t *x, const float *s, int64_t m, int64_t k, int8_t *q, float *sx)
{
    int failed = 0;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; r++) {
        float *v = (float *)malloc((size_t)k * sizeof(float));
        int32_t *c = (int32_t *)malloc((size_t)k * sizeof(int32_t));
        if (!v || !c) {
            #pragma omp atomic write
            failed = 1;
            free(v);
            free(c);
            continue;
        }
        for (int64_t j = 0; j < k; j++) {
            const float xv = orc_f16_to_f32(x[r * k + j]);
            v[j] = s ? xv / s[j] : xv;
        }
        float sc;
        int32_t z;
        orc_quantize_group(v, k, 8, 1, &sc, &z, c);
        for (int64_t j = 0; j < k; j++)
            q[r * k + j] = (int8_t)c[j];
        sx[r] = sc;
        free(v);
        free(c);
    }
    return failed ? 2 : 0;
}

/* acc[m][n] = sum_k qx[m][k] qw[n][k] exactly; y = fp16((float(acc) sx[m]) sw[n]). */
void orc_w8a8_gemm(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                   int64_t m, int64_t n_out, int64_t k, int64_t *acc, uint16_t *y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_out; n++)
        for (int64_t i = 0; i < m; i++) {
            int64_t a = 0;
            for (int64_t j = 0; j < k; j++)
                a += (int64_t)qx[i * k + j] * (int64_t)qw[n * k + j];
            if (acc)
                acc[i * n_out + n] = a;
            const float v = ((float)a * sx[i]) * sw[n];
            y[i * n_out + n] = orc_f32_to_f16(v);
        }
}

/* ------------------------------------------------------------------------ */
/* GPTQ ([Guide] §4.3).                                                      */
/* Minimize ||X W^T - X W_hat^T|| per layer: H = 2 X^T X from calibration    */
/* tokens, damped by lambda * mean(diag H) (lambda = 0.01); the upper        */
/* Cholesky factor U of H^-1 (U^T U = H^-1); then column by column: at each  */
/* group start the group's scale and zero-point come from the current        */
/* (already compensated) weights, the column is quantized, and its error     */
/* (w - w') / U[i][i] is pushed onto every later column j as                 */
/* w_j -= err * U[i][j].  The pages' block-128 lazy update changes only when */
/* a column receives its corrections, not their order.                       */
/* Readings: H, the damping and U in binary64 (H's sums run over the tokens  */
/* in order; the diagonal mean sums in index order); U is formed without an  */
/* explicit H^-1 -- with J the index reversal, J H J = L L^T (lower          */
/* Cholesky) gives H = R R^T, R = J L J upper, and U = R^-1 = J L^-1 J is     */
/* the unique upper factor with U^T U = H^-1 (pinned against that           */
/* definition); both factorizations are right-looking, every element's       */
/* updates applied in pivot order, one multiply and one subtract each; the   */
/* column loop runs in binary32 with U rounded to binary32; codes use the    */
/* fp32 scale and the error uses the stored fp16 scale (the value the        */
/* kernels dequantize), natural column order (no activation reordering).     */
/* ------------------------------------------------------------------------ */
void orc_gptq_hessian(const uint16_t *x, int64_t t, int64_t n, double *h)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        for (int64_t j = 0; j <= i; j++) {
            double acc = 0.0;
            for (int64_t r = 0; r < t; r++)
                acc += (double)orc_f16_to_f32(x[r * n + i]) * (double)orc_f16_to_f32(x[r * n + j]);
            h[i * n + j] = 2.0 * acc;
            h[j * n + i] = 2.0 * acc;
        }
}

void orc_gptq_damp(double *h, int64_t n, double lambda)
{
    double sum = 0.0;
    for (int64_t i = 0; i < n; i++)
        sum += h[i * n + i];
    const double add = lambda * (sum / (double)n);
    for (int64_t i = 0; i < n; i++)
        h[i * n + i] += add;
}

/* Right-looking lower Cholesky of a [n][n] (lower triangle used) in place:
 * for each pivot j the column is scaled and the trailing lower triangle
 * updated, a[i][k] -= l[i][j] * l[k][j].  Returns 1 if a pivot is not
 * positive. */
static int chol_lower_right_looking(double *a, int64_t n)
{
    for (int64_t j = 0; j < n; j++) {
        if (!(a[j * n + j] > 0.0))
            return 1;
        const double d = sqrt(a[j * n + j]);
        a[j * n + j] = d;
        for (int64_t i = j + 1; i < n; i++)
            a[i * n + j] = a[i * n + j] / d;
        for (int64_t i = j + 1; i < n; i++)
            for (int64_t k = j + 1; k <= i; k++)
                a[i * n + k] = a[i * n + k] - a[i * n + j] * a[k * n + j];
    }
    for (int64_t i = 0; i < n; i++)
        for (int64_t k = i + 1; k < n; k++)
            a[i * n + k] = 0.0;
    return 0;
}

/* M = L^-1 for lower triangular L, right-looking: B = I; for each pivot j,
 * row j of M is B[j][.] / l[j][j] and every later row i loses
 * l[i][j] * M[j][.]. */
static void tri_inverse_lower_right_looking(const double *l, int64_t n, double *m)
{
    for (int64_t i = 0; i < n * n; i++)
        m[i] = 0.0;
    for (int64_t i = 0; i < n; i++)
        m[i * n + i] = 1.0;
    for (int64_t j = 0; j < n; j++) {
        const double d = l[j * n + j];
        for (int64_t c = 0; c <= j; c++)
            m[j * n + c] = m[j * n + c] / d;
        for (int64_t i = j + 1; i < n; i++)
            for (int64_t c = 0; c <= j; c++)
                m[i * n + c] = m[i * n + c] - l[i * n + j] * m[j * n + c];
    }
}

/* U (upper, [n][n]) with U^T U = H^-1, from the damped H.  Returns 0, 1 if
 * H is not positive definite, 2 if memory ran out. */
int orc_gptq_hinv_chol(const double *h, int64_t n, double *u)
{
    double *a = (double *)malloc((size_t)(n * n) * sizeof(double));
    double *m = (double *)malloc((size_t)(n * n) * sizeof(double));
    if (!a || !m) {
        free(a);
        free(m);
        return 2;
    }
    for (int64_t i = 0; i < n; i++)            /* J H J */
        for (int64_t k = 0; k < n; k++)
            a[i * n + k] = h[(n - 1 - i) * n + (n - 1 - k)];
    if (chol_lower_right_looking(a, n)) {
        free(a);
        free(m);
        return 1;
    }
    tri_inverse_lower_right_looking(a, n, m);
    for (int64_t i = 0; i < n; i++)            /* U = J L^-1 J */
        for (int64_t k = 0; k < n; k++)
            u[i * n + k] = m[(n - 1 - i) * n + (n - 1 - k)];
    free(a);
    free(m);
    return 0;
}

/* The column loop on w [n_out][n] (fp32, updated in place) with u [n][n]
 * (fp32 upper factor): packed codes, fp16 scales and zeros in the library's
 * format (as orc_quantize_pack_bits).  Returns 0, 1 for an unsupported
 * shape, 2 if memory ran out. */
int orc_gptq_quantize(float *w, const float *u, int64_t n_out, int64_t n, int32_t group_size,
                      int32_t bits, int32_t symmetric, uint32_t *packed, uint16_t *scales,
                      uint16_t *zeros)
{
    if ((bits != 4 && bits != 8) || group_size <= 0 || n % group_size != 0 || n % (32 / bits) != 0)
        return 1;
    const int per_word = 32 / bits;
    const int64_t words = n / per_word, groups = n / group_size;
    const int32_t offset = 1 << (bits - 1);
    const float top = symmetric ? (float)(offset - 1) : (float)((1 << bits) - 1);
    const float bottom = symmetric ? -(float)offset : 0.0f;
    int failed = 0;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_out; r++) {
        int32_t *codes = (int32_t *)malloc((size_t)group_size * sizeof(int32_t));
        if (!codes) {
            #pragma omp atomic write
            failed = 1;
            continue;
        }
        float *row = w + r * n;
        uint32_t *prow = packed + r * words;
        memset(prow, 0, (size_t)words * sizeof(uint32_t));
        float s = 1.0f, s16 = 1.0f;
        int32_t z = 0;
        for (int64_t i = 0; i < n; i++) {
            if (i % group_size == 0) {
                orc_quantize_group(row + i, group_size, bits, symmetric, &s, &z, codes);
                const uint16_t sh = orc_f32_to_f16(s);
                s16 = orc_f16_to_f32(sh);
                scales[r * groups + i / group_size] = sh;
                zeros[r * groups + i / group_size] = orc_f32_to_f16((float)(symmetric ? offset : z));
            }
            const float q = clampf(rintf(row[i] / s) + (float)z, bottom, top);
            const float deq = s16 * (q - (float)z);
            const float err = (row[i] - deq) / u[i * n + i];
            const uint32_t code = (uint32_t)(int32_t)(symmetric ? q + (float)offset : q);
            prow[i / per_word] |= code << (bits * (i % per_word));
            for (int64_t j = i + 1; j < n; j++)
                row[j] = row[j] - err * u[i * n + j];
        }
        free(codes);
    }
    return failed ? 2 : 0;
}

/* ------------------------------------------------------------------------ */
/* AWQ ([Guide] §4.4).                                                       */
/* Per input channel s_j = (mean_t |X_tj|)^alpha; the weights are scaled by  */
/* s, quantized group-wise, and the activation is divided by s at run time   */
/* (so the effective weight is dequant(Q(W diag(s))) / s); alpha is searched */
/* on a grid over [0, 1] for the smallest reconstruction error of the        */
/* layer output on the calibration tokens.                                   */
/* Readings: the mean of |x| sums the tokens in order in binary64; s =       */
/* float(pow(mean, alpha)) floored at 1e-5 (the SmoothQuant listing's       */
/* floor); W * s and dequant / s in binary32; the error is                   */
/* sum_t sum_n (sum_k x_tk (w_nk - w_eff_nk))^2 in binary64, each inner sum   */
/* over k in order, the outer sums over t then n in order; the grid is       */
/* alpha = i / n_grid, i = 0..n_grid, and the first smallest error wins.     */
/* ------------------------------------------------------------------------ */
void orc_awq_act_mean(const uint16_t *x, int64_t t, int64_t n, double *mean)
{
    for (int64_t j = 0; j < n; j++) {
        double acc = 0.0;
        for (int64_t r = 0; r < t; r++)
            acc += fabs((double)orc_f16_to_f32(x[r * n + j]));
        mean[j] = acc / (double)t;
    }
}

void orc_awq_scales(const double *mean, int64_t n, double alpha, float *s)
{
    for (int64_t j = 0; j < n; j++) {
        const float v = (float)pow(mean[j], alpha);
        s[j] = v < 1e-5f ? 1e-5f : v;
    }
}

/* Effective weights of one alpha: w_eff = dequant(Q(W diag(s))) / s, with
 * the packed result of Q written out. */
int orc_awq_apply(const float *w, const float *s, int64_t n_out, int64_t n, int32_t group_size,
                  int32_t bits, int32_t symmetric, uint32_t *packed, uint16_t *scales,
                  uint16_t *zeros, float *w_eff)
{
    float *ws = (float *)calloc((size_t)(n_out * n), sizeof(float));
    if (!ws)
        return 2;
    for (int64_t r = 0; r < n_out; r++)
        for (int64_t k = 0; k < n; k++)
            ws[r * n + k] = w[r * n + k] * s[k];
    int rc = orc_quantize_pack_bits(ws, n_out, n, group_size, bits, symmetric, packed, scales, zeros, NULL);
    if (rc == 0) {
        orc_dequant_bits(packed, scales, zeros, n_out, n, group_size, bits, ws);
        for (int64_t r = 0; r < n_out; r++)
            for (int64_t k = 0; k < n; k++)
                w_eff[r * n + k] = ws[r * n + k] / s[k];
    }
    free(ws);
    return rc;
}

double orc_awq_loss(const uint16_t *x, int64_t t, const float *w, const float *w_eff, int64_t n_out, int64_t n)
{
    double *part = (double *)malloc((size_t)n_out * sizeof(double));
    if (!part)
        return -1.0;
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n_out; c++) {
        double acc = 0.0;
        for (int64_t r = 0; r < t; r++) {
            double y = 0.0;
            for (int64_t k = 0; k < n; k++)
                y += (double)orc_f16_to_f32(x[r * n + k]) *
                     ((double)w[c * n + k] - (double)w_eff[c * n + k]);
            acc += y * y;
        }
        part[c] = acc;
    }
    double total = 0.0;
    for (int64_t c = 0; c < n_out; c++)
        total += part[c];
    free(part);
    return total;
}
