// q4_api.hip -- the C ABI declared in include/w4a16.h: argument validation
// (before any HIP call), then one launch on the caller's stream.
#include "w4a16.h"
#include "kv_codec.h"
#include "w8a8.h"
#include "producers.h"

#include "q4_launch.h"

namespace {

constexpr int64_t kMaxIn = int64_t(1) << 20;
constexpr int64_t kMaxOut = int64_t(1) << 24;
constexpr int64_t kMaxRows = int64_t(1) << 24;
constexpr int64_t kMaxElems = int64_t(1) << 34;

thread_local int g_last_hip_error = 0;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Groups of 32, 64, 128 or 256 elements, or one group per row (per-channel)
// when the row is a whole number of 32-element slices.
int check_group(int32_t group_size, int64_t n_in)
{
    switch (group_size) {
    case 32: case 64: case 128: case 256: return Q4_OK;
    default: return (group_size == n_in && n_in % 32 == 0) ? Q4_OK : Q4_ERR_GROUP;
    }
}

// Shape rules common to every entry point: positive sizes within limits and
// whole groups per row (the n_in % 8 and % 4 packing rules follow from
// n_in % 32 == 0).
int check_weight_shape(int64_t n_out, int64_t n_in, int32_t group_size)
{
    if (n_out <= 0 || n_in <= 0 || n_out > kMaxOut || n_in > kMaxIn) return Q4_ERR_SHAPE;
    if (n_out * n_in > kMaxElems) return Q4_ERR_SHAPE;
    if (int rc = check_group(group_size, n_in)) return rc;
    if (n_in % group_size != 0) return Q4_ERR_SHAPE;
    return Q4_OK;
}

int finish(hipError_t e)
{
    if (e == hipSuccess) return Q4_OK;
    g_last_hip_error = (int)e;
    return Q4_ERR_HIP;
}

int check_linear(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                 const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                 int32_t group_size, const uint16_t *y, int64_t max_m)
{
    if (!x || !qweight || !scales || !zeros || !y) return Q4_ERR_NULL;
    if (int rc = check_weight_shape(n_out, n_in, group_size)) return rc;
    if (m <= 0 || m > max_m || m * n_in > kMaxElems || m * n_out > kMaxElems) return Q4_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(qweight, 16) || !aligned(scales, 2) || !aligned(zeros, 2) ||
        !aligned(y, 2))
        return Q4_ERR_ALIGN;
    return Q4_OK;
}

// W8A8 shapes: k a multiple of 32 in [32, 32768]; rows and outputs in [1, 2^24].
int check_w8a8_k(int64_t k) { return (k >= 32 && k <= 32768 && k % 32 == 0) ? Q4_OK : Q4_ERR_SHAPE; }

int check_rows(int64_t r) { return (r >= 1 && r <= kMaxRows) ? Q4_OK : Q4_ERR_SHAPE; }

// GPTQ / AWQ shapes: n a multiple of 32 in [32, 32768], the weight group rules.
int check_producer(int64_t n_out, int64_t n, int32_t group_size, int32_t bits)
{
    if (n < 32 || n > 32768 || n % 32 != 0 || check_rows(n_out) || n_out * n > kMaxElems) return Q4_ERR_SHAPE;
    if (bits != 4 && bits != 8) return Q4_ERR_SHAPE;
    if (int rc = check_group(group_size, n)) return rc;
    return n % group_size == 0 ? Q4_OK : Q4_ERR_SHAPE;
}

// KV codec shapes: head dimension d a multiple of 8 in [8, 512]; per-channel
// blocks of t tokens fit 32 rows per thread (t <= 32 * (2048 / d)).
int check_kv_bits(int32_t bits) { return (bits == 4 || bits == 8) ? Q4_OK : Q4_ERR_SHAPE; }

int check_kv_d(int32_t d) { return (d >= 8 && d <= 512 && d % 8 == 0) ? Q4_OK : Q4_ERR_SHAPE; }

int check_kv_block(int64_t blocks, int32_t t, int32_t d)
{
    if (int rc = check_kv_d(d)) return rc;
    if (blocks <= 0 || blocks > kMaxRows || t <= 0 || t > 32 * (2048 / d)) return Q4_ERR_SHAPE;
    if (blocks * t * d > kMaxElems) return Q4_ERR_SHAPE;
    return Q4_OK;
}

int check_kv_rows(int64_t rows, int32_t d)
{
    if (int rc = check_kv_d(d)) return rc;
    if (rows <= 0 || rows * d > kMaxElems) return Q4_ERR_SHAPE;
    return Q4_OK;
}

}  // namespace

extern "C" {

int q4_abi_version(void) { return Q4_ABI_VERSION; }

const char *q4_strerror(int status)
{
    switch (status) {
    case Q4_OK: return "success";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "invalid shape: a size is <= 0 or too large, n_in is not a multiple "
                              "of group_size, or m is outside the entry point's range";
    case Q4_ERR_GROUP: return "unsupported group_size (supported: 32, 64, 128, 256, and n_in "
                              "itself for one group per output channel when n_in % 32 == 0)";
    case Q4_ERR_ALIGN: return "misaligned pointer: w, w_out, qweight and x need 16 bytes, fp16 "
                              "arrays 2 bytes";
    case Q4_ERR_HIP: return "the HIP runtime refused the launch (see q4_last_hip_error)";
    case Q4_ERR_CAPACITY: return "the problem needs more scratch memory than the no-allocation entry point "
                                 "holds (see gptq_quantize_noalloc_max_bytes)";
    default: return "unknown status";
    }
}

int q4_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

namespace {

int quantize_pack(int bits, const float *w, int64_t n_out, int64_t n_in, int32_t group_size,
                  int32_t symmetric, uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                  void *stream)
{
    if (!w || !qweight || !scales || !zeros) return Q4_ERR_NULL;
    if (int rc = check_weight_shape(n_out, n_in, group_size)) return rc;
    if (!aligned(w, 16) || !aligned(qweight, 16) || !aligned(scales, 2) || !aligned(zeros, 2))
        return Q4_ERR_ALIGN;
    return finish(q4_launch_quantize_pack(w, n_out, n_in, group_size, bits, symmetric != 0, qweight,
                                          scales, zeros, (hipStream_t)stream));
}

int dequant(int bits, const uint32_t *qweight, const uint16_t *scales, const uint16_t *zeros,
            int64_t n_out, int64_t n_in, int32_t group_size, float *w_out, void *stream)
{
    if (!qweight || !scales || !zeros || !w_out) return Q4_ERR_NULL;
    if (int rc = check_weight_shape(n_out, n_in, group_size)) return rc;
    if (!aligned(qweight, 16) || !aligned(w_out, 16) || !aligned(scales, 2) || !aligned(zeros, 2))
        return Q4_ERR_ALIGN;
    return finish(q4_launch_dequant(qweight, scales, zeros, n_out, n_in, group_size, bits, w_out,
                                    (hipStream_t)stream));
}

}  // namespace

extern "C" {

int q4_quantize_pack(const float *w, int64_t n_out, int64_t n_in, int32_t group_size,
                     int32_t symmetric, uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                     void *stream)
{
    return quantize_pack(4, w, n_out, n_in, group_size, symmetric, qweight, scales, zeros, stream);
}

int q8_quantize_pack(const float *w, int64_t n_out, int64_t n_in, int32_t group_size,
                     int32_t symmetric, uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                     void *stream)
{
    return quantize_pack(8, w, n_out, n_in, group_size, symmetric, qweight, scales, zeros, stream);
}

int q4_dequant(const uint32_t *qweight, const uint16_t *scales, const uint16_t *zeros,
               int64_t n_out, int64_t n_in, int32_t group_size, float *w_out, void *stream)
{
    return dequant(4, qweight, scales, zeros, n_out, n_in, group_size, w_out, stream);
}

int q8_dequant(const uint32_t *qweight, const uint16_t *scales, const uint16_t *zeros,
               int64_t n_out, int64_t n_in, int32_t group_size, float *w_out, void *stream)
{
    return dequant(8, qweight, scales, zeros, n_out, n_in, group_size, w_out, stream);
}

int q4_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
            const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in, int32_t group_size,
            uint16_t *y, void *stream)
{
    if (int rc = check_linear(x, qweight, scales, zeros, m, n_out, n_in, group_size, y, 16))
        return rc;
    return finish(q4_launch_gemv(x, qweight, scales, zeros, m, n_out, n_in, group_size, 4, y,
                                 (hipStream_t)stream));
}

int q8_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
            const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in, int32_t group_size,
            uint16_t *y, void *stream)
{
    if (int rc = check_linear(x, qweight, scales, zeros, m, n_out, n_in, group_size, y, 16))
        return rc;
    return finish(q4_launch_gemv(x, qweight, scales, zeros, m, n_out, n_in, group_size, 8, y,
                                 (hipStream_t)stream));
}

int q4_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
            const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in, int32_t group_size,
            uint16_t *y, void *stream)
{
    if (int rc = check_linear(x, qweight, scales, zeros, m, n_out, n_in, group_size, y, kMaxRows))
        return rc;
    return finish(q4_launch_gemm(x, qweight, scales, zeros, m, n_out, n_in, group_size, 4, y,
                                 (hipStream_t)stream));
}

int q8_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
            const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in, int32_t group_size,
            uint16_t *y, void *stream)
{
    if (int rc = check_linear(x, qweight, scales, zeros, m, n_out, n_in, group_size, y, kMaxRows))
        return rc;
    return finish(q4_launch_gemm(x, qweight, scales, zeros, m, n_out, n_in, group_size, 8, y,
                                 (hipStream_t)stream));
}

int q4_linear_config(int32_t op, int32_t bits, int64_t m, int64_t n_out, int64_t n_in, int32_t group_size,
                     const void *scales, const void *zeros, char *name, int64_t name_len)
{
    if (!scales || !zeros || !name) return Q4_ERR_NULL;
    if ((op != 0 && op != 1) || (bits != 4 && bits != 8) || name_len < 1) return Q4_ERR_SHAPE;
    if (int rc = check_weight_shape(n_out, n_in, group_size)) return rc;
    const int64_t max_m = op == 0 ? 16 : kMaxRows;
    if (m <= 0 || m > max_m || m * n_in > kMaxElems || m * n_out > kMaxElems) return Q4_ERR_SHAPE;
    if (!aligned(scales, 2) || !aligned(zeros, 2)) return Q4_ERR_ALIGN;
    // only the two addresses are inspected (for their alignment); nothing is
    // dereferenced and no HIP call is made
    const uint16_t *s = static_cast<const uint16_t *>(scales), *z = static_cast<const uint16_t *>(zeros);
    const char *cfg = nullptr;
    const hipError_t e = op == 0 ? q4_launch_gemv(nullptr, nullptr, s, z, m, n_out, n_in, group_size, bits, nullptr,
                                                  nullptr, &cfg)
                                 : q4_launch_gemm(nullptr, nullptr, s, z, m, n_out, n_in, group_size, bits, nullptr,
                                                  nullptr, &cfg);
    if (e != hipSuccess || !cfg) return finish(e == hipSuccess ? hipErrorInvalidValue : e);
    int64_t i = 0;
    for (; i + 1 < name_len && cfg[i]; ++i) name[i] = cfg[i];
    name[i] = '\0';
    return Q4_OK;
}

int kv_quant_tokens(const uint16_t *x, int64_t rows, int32_t d, int32_t bits, int8_t *q, float *scale,
                    void *stream)
{
    if (!x || !q || !scale) return Q4_ERR_NULL;
    if (int rc = check_kv_rows(rows, d)) return rc;
    if (int rc = check_kv_bits(bits)) return rc;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return Q4_ERR_ALIGN;
    return finish(kv_launch_quant_tokens(x, rows, d, bits, q, scale, (hipStream_t)stream));
}

int kv_quant_channels(const uint16_t *x, int64_t blocks, int32_t t, int32_t d, int32_t bits, int8_t *q,
                      float *scale, void *stream)
{
    if (!x || !q || !scale) return Q4_ERR_NULL;
    if (int rc = check_kv_block(blocks, t, d)) return rc;
    if (int rc = check_kv_bits(bits)) return rc;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return Q4_ERR_ALIGN;
    return finish(kv_launch_quant_channels(x, blocks, t, d, bits, q, scale, (hipStream_t)stream));
}

int kv_dequant_tokens(const int8_t *q, const float *scale, int64_t rows, int32_t d, uint16_t *out,
                      void *stream)
{
    if (!q || !scale || !out) return Q4_ERR_NULL;
    if (int rc = check_kv_rows(rows, d)) return rc;
    if (!aligned(q, 16) || !aligned(scale, 4) || !aligned(out, 16)) return Q4_ERR_ALIGN;
    return finish(kv_launch_dequant_tokens(q, scale, rows, d, out, (hipStream_t)stream));
}

int kv_dequant_channels(const int8_t *q, const float *scale, int64_t blocks, int32_t t, int32_t d,
                        uint16_t *out, void *stream)
{
    if (!q || !scale || !out) return Q4_ERR_NULL;
    if (int rc = check_kv_block(blocks, t, d)) return rc;
    if (!aligned(q, 16) || !aligned(scale, 16) || !aligned(out, 16)) return Q4_ERR_ALIGN;
    return finish(kv_launch_dequant_channels(q, scale, blocks, t, d, out, (hipStream_t)stream));
}

int kv_flush_blocks(const uint16_t *k, const uint16_t *v, int64_t blocks, int32_t t, int32_t d,
                    int32_t bits, const int32_t *dst, int64_t pool_blocks, int8_t *k_pool,
                    float *k_scale, int8_t *v_pool, float *v_scale, void *stream)
{
    if (!k || !v || !dst || !k_pool || !k_scale || !v_pool || !v_scale) return Q4_ERR_NULL;
    if (int rc = check_kv_block(blocks, t, d)) return rc;
    if (int rc = check_kv_bits(bits)) return rc;
    if (pool_blocks <= 0 || pool_blocks > kMaxRows || pool_blocks * t * d > kMaxElems) return Q4_ERR_SHAPE;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(dst, 4) || !aligned(k_pool, 16) ||
        !aligned(k_scale, 4) || !aligned(v_pool, 16) || !aligned(v_scale, 4))
        return Q4_ERR_ALIGN;
    return finish(kv_launch_flush(k, v, blocks, t, d, bits, dst, pool_blocks, k_pool, k_scale, v_pool,
                                  v_scale, (hipStream_t)stream));
}

int sq_absmax_update_f16(const uint16_t *x, int64_t rows, int32_t cols, float *amax, void *stream)
{
    if (!x || !amax) return Q4_ERR_NULL;
    if (check_rows(rows) || cols < 8 || cols > kMaxIn || cols % 8 != 0 || rows * cols > kMaxElems)
        return Q4_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(amax, 4)) return Q4_ERR_ALIGN;
    return finish(w8a8_launch_col_absmax(x, false, rows, cols, amax, (hipStream_t)stream));
}

int sq_absmax_update_f32(const float *w, int64_t rows, int32_t cols, float *amax, void *stream)
{
    if (!w || !amax) return Q4_ERR_NULL;
    if (check_rows(rows) || cols < 8 || cols > kMaxIn || cols % 8 != 0 || rows * cols > kMaxElems)
        return Q4_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(amax, 4)) return Q4_ERR_ALIGN;
    return finish(w8a8_launch_col_absmax(w, true, rows, cols, amax, (hipStream_t)stream));
}

int sq_smooth_factors(const float *act_max, const float *w_max, int32_t n, float alpha, float *s,
                      void *stream)
{
    if (!act_max || !w_max || !s) return Q4_ERR_NULL;
    if (n <= 0 || n > kMaxIn || !(alpha >= 0.0f && alpha <= 1.0f)) return Q4_ERR_SHAPE;
    if (!aligned(act_max, 4) || !aligned(w_max, 4) || !aligned(s, 4)) return Q4_ERR_ALIGN;
    return finish(w8a8_launch_smooth_factors(act_max, w_max, n, alpha, s, (hipStream_t)stream));
}

int w8a8_quantize_weight(const float *w, const float *s, int64_t n_out, int64_t k, int8_t *qw,
                         float *sw, void *stream)
{
    if (!w || !qw || !sw) return Q4_ERR_NULL;
    if (check_rows(n_out) || check_w8a8_k(k) || n_out * k > kMaxElems) return Q4_ERR_SHAPE;
    if (!aligned(w, 16) || (s && !aligned(s, 16)) || !aligned(qw, 16) || !aligned(sw, 4)) return Q4_ERR_ALIGN;
    return finish(w8a8_launch_quant_weight(w, s, n_out, (int)k, qw, sw, (hipStream_t)stream));
}

int w8a8_quantize_act(const uint16_t *x, const float *s, int64_t m, int64_t k, int8_t *qx,
                      float *sx, void *stream)
{
    if (!x || !qx || !sx) return Q4_ERR_NULL;
    if (check_rows(m) || check_w8a8_k(k) || m * k > kMaxElems) return Q4_ERR_SHAPE;
    if (!aligned(x, 16) || (s && !aligned(s, 16)) || !aligned(qx, 16) || !aligned(sx, 4)) return Q4_ERR_ALIGN;
    return finish(w8a8_launch_quant_act(x, s, m, (int)k, qx, sx, (hipStream_t)stream));
}

int w8a8_gemm(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw, int64_t m,
              int64_t n_out, int64_t k, uint16_t *y, void *stream)
{
    if (!qx || !sx || !qw || !sw || !y) return Q4_ERR_NULL;
    if (check_rows(m) || check_rows(n_out) || check_w8a8_k(k)) return Q4_ERR_SHAPE;
    if (m * k > kMaxElems || n_out * k > kMaxElems || m * n_out > kMaxElems) return Q4_ERR_SHAPE;
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(sx, 4) || !aligned(sw, 4) || !aligned(y, 2))
        return Q4_ERR_ALIGN;
    return finish(w8a8_launch_gemm(qx, sx, qw, sw, m, n_out, k, y, (hipStream_t)stream));
}

int64_t gptq_factor_workspace_size(int64_t n) { return n > 0 ? gptq_factor_workspace(n) : 0; }

int64_t gptq_quantize_workspace_size(int64_t n_out, int64_t n)
{
    return (n_out > 0 && n > 0) ? gptq_loop_workspace(n_out, n) : 0;
}

int gptq_quantize_noalloc(const float *w, const float *u, int64_t n_out, int64_t n, int32_t group_size,
                          int32_t bits, int32_t symmetric, uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                          void *stream)
{
    if (!w || !u || !qweight || !scales || !zeros) return Q4_ERR_NULL;
    if (int rc = check_producer(n_out, n, group_size, bits)) return rc;
    if (gptq_loop_workspace(n_out, n) > kGptqNoAllocScratchBytes) return Q4_ERR_CAPACITY;
    if (!aligned(w, 16) || !aligned(u, 4) || !aligned(qweight, 16) || !aligned(scales, 2) || !aligned(zeros, 2))
        return Q4_ERR_ALIGN;
    void *ws = nullptr;
    if (hipError_t e = gptq_noalloc_scratch((hipStream_t)stream, &ws)) return finish(e);
    return finish(gptq_launch_loop(w, u, n_out, (int)n, group_size, bits, symmetric != 0, ws, qweight, scales, zeros,
                                   (hipStream_t)stream));
}

int64_t gptq_quantize_noalloc_max_bytes(void) { return kGptqNoAllocScratchBytes; }

int64_t awq_workspace_size(int64_t n_out, int64_t n, int64_t tokens, int32_t n_grid, int32_t group_size)
{
    if (n_out <= 0 || n <= 0 || tokens <= 0 || n_grid <= 0 || group_size <= 0) return 0;
    return awq_workspace(n_out, n, tokens, n_grid, group_size);
}

int gptq_hinv_factor(const uint16_t *x, int64_t tokens, int64_t n, double damp, void *workspace,
                     int64_t workspace_bytes, float *u, void *stream)
{
    if (!x || !workspace || !u) return Q4_ERR_NULL;
    if (n < 32 || n > 32768 || n % 32 != 0 || check_rows(tokens) || tokens * n > kMaxElems) return Q4_ERR_SHAPE;
    if (!(damp >= 0.0 && damp < 1e6)) return Q4_ERR_SHAPE;
    if (workspace_bytes < gptq_factor_workspace(n)) return Q4_ERR_SHAPE;
    if (!aligned(x, 2) || !aligned(workspace, 256) || !aligned(u, 4)) return Q4_ERR_ALIGN;
    return finish(gptq_launch_factor(x, tokens, (int)n, damp, workspace, u, (hipStream_t)stream));
}

int gptq_quantize(const float *w, const float *u, int64_t n_out, int64_t n, int32_t group_size,
                  int32_t bits, int32_t symmetric, void *workspace, int64_t workspace_bytes,
                  uint32_t *qweight, uint16_t *scales, uint16_t *zeros, void *stream)
{
    if (!w || !u || !workspace || !qweight || !scales || !zeros) return Q4_ERR_NULL;
    if (int rc = check_producer(n_out, n, group_size, bits)) return rc;
    if (workspace_bytes < gptq_loop_workspace(n_out, n)) return Q4_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(u, 4) || !aligned(workspace, 256) || !aligned(qweight, 16) ||
        !aligned(scales, 2) || !aligned(zeros, 2))
        return Q4_ERR_ALIGN;
    return finish(gptq_launch_loop(w, u, n_out, (int)n, group_size, bits, symmetric != 0, workspace, qweight,
                                   scales, zeros, (hipStream_t)stream));
}

int awq_quantize(const float *w, const uint16_t *x, int64_t tokens, int64_t n_out, int64_t n,
                 int32_t group_size, int32_t bits, int32_t symmetric, int32_t n_grid, void *workspace,
                 int64_t workspace_bytes, uint32_t *qweight, uint16_t *scales, uint16_t *zeros, float *s,
                 int32_t *best, float *losses, void *stream)
{
    if (!w || !x || !workspace || !qweight || !scales || !zeros || !s) return Q4_ERR_NULL;
    if (int rc = check_producer(n_out, n, group_size, bits)) return rc;
    if (check_rows(tokens) || tokens * n > kMaxElems || tokens * n_out > kMaxElems) return Q4_ERR_SHAPE;
    if (n_grid < 1 || n_grid > 100) return Q4_ERR_SHAPE;
    if (workspace_bytes < awq_workspace(n_out, n, tokens, n_grid, group_size)) return Q4_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(x, 2) || !aligned(workspace, 256) || !aligned(qweight, 16) ||
        !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(s, 4) || (best && !aligned(best, 4)) ||
        (losses && !aligned(losses, 4)))
        return Q4_ERR_ALIGN;
    return finish(awq_launch(w, x, tokens, n_out, (int)n, group_size, bits, symmetric != 0, n_grid, workspace,
                             qweight, scales, zeros, s, best, losses, (hipStream_t)stream));
}

}  // extern "C"
