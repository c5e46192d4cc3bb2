// kv_codec.hip -- KV-cache codec: symmetric b-bit quantization of V per token
// and of K per channel, dequantization, and the flush of window blocks into a
// block pool.
//
// [Guide] §6 (KV Cache 量化): K and V are treated differently -- K has fixed
// outlier channels, so it gets one scale per channel; V is flatter and gets
// one scale per token -- and the most recent tokens (about 128) stay in FP16.
// Its per-token listing fixes the map: qmax = 2^(b-1) - 1, scale = max|v| /
// qmax floored at 1e-8, q = clamp(round(v / scale), -qmax - 1, qmax), stored
// as int8.  [Intro] §3.2: separate scale factors for K and V.
//
// Every step is one binary32 operation on the exactly widened fp16 inputs
// (this unit is built without FMA contraction and with correctly rounded
// division), so codes and scales are bit-exact and independent of the launch
// shape.  Dequantization is the binary32 product q * scale rounded to fp16.
//
// Per token: d/8 lanes share a token row (8 halves per lane, one 16-byte
// load), reduce max|v| with a butterfly of lane shuffles, and store 8 codes
// as one 8-byte word.  Per channel: one workgroup per block of t tokens; each
// thread keeps its rows' 16-byte chunks in registers, partial maxima go
// through LDS, and the codes are written from the registers, so the block is
// read from HBM once.  The flush does both for one window block per
// workgroup and writes to the pool slot the block table names.
#include "q4_device.h"
#include "q4_launch.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float kv_scale(float amax, float qmax)
{
    float s = amax / qmax;
    return s < 1e-8f ? 1e-8f : s;
}

// round(v / s) clamped to [-qmax - 1, qmax], as the byte of an int8.  The
// product with r, the hardware reciprocal of s (within 1 ulp), is within
// 2^-21.5 * |v / s| of the correctly rounded quotient; for |v / s| < 2^7 that
// is below 2^-14, so both round to the same integer unless the product lies
// within 2^-14 of a half-integer.  There, and for larger quotients, the
// correctly rounded division decides: the code is the one round(v / s)
// gives, bit for bit.
__device__ __forceinline__ uint32_t kv_code(float v, float s, float r, float qmax)
{
    const float a = v * r;
    float c = __builtin_rintf(a);
    if (fabsf(a - c) > 0.5f - 0x1p-14f || fabsf(a) >= 128.0f) c = __builtin_rintf(v / s);
    c = fminf(fmaxf(c, -qmax - 1.0f), qmax);
    return (uint32_t)(int32_t)c & 0xFFu;
}

__device__ __forceinline__ void widen8(const u32x4 &raw, float v[8])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = half_bits_to_float((uint16_t)(raw[e >> 1] >> (16 * (e & 1))));
}

// Eight codes of one token row against the row's scale s (reciprocal r).
__device__ __forceinline__ u32x2 codes8(const float v[8], float s, float r, float qmax)
{
    u32x2 w = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e >> 2] |= kv_code(v[e], s, r, qmax) << (8 * (e & 3));
    return w;
}

// Eight codes of one chunk against eight channel scales.
__device__ __forceinline__ u32x2 codes8(const float v[8], const float s[8], const float r[8], float qmax)
{
    u32x2 w = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e >> 2] |= kv_code(v[e], s[e], r[e], qmax) << (8 * (e & 3));
    return w;
}

// Per-token quantization of rows r_first + k * r_step < r_end: LPR lanes per
// row, lanes past d/8 hold zeros.  Each pass handles U rows per lane, their
// loads issued together so that U * 16 bytes per lane are in flight.
template <int LPR, int U>
__device__ __forceinline__ void quant_rows(const uint16_t *__restrict__ x, int64_t r_first, int64_t r_end,
                                           int64_t r_step, int d, float qmax, int8_t *__restrict__ q,
                                           float *__restrict__ scale)
{
    const int li = threadIdx.x % LPR;
    const bool active = li < d / 8;
    for (int64_t r = r_first + threadIdx.x / LPR; r < r_end; r += U * r_step) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t ru = r + u * r_step;
            raw[u] = u32x4{0u, 0u, 0u, 0u};
            if (active && ru < r_end) raw[u] = *reinterpret_cast<const u32x4 *>(x + ru * d + li * 8);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t ru = r + u * r_step;
            float v[8];
            widen8(raw[u], v);
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
            const float s = kv_scale(a, qmax);
            const float rc = __builtin_amdgcn_rcpf(s);
            if (ru < r_end) {
                if (active) *reinterpret_cast<u32x2 *>(q + ru * d + li * 8) = codes8(v, s, rc, qmax);
                if (li == 0) scale[ru] = s;
            }
        }
    }
}

// Per-channel quantization of one block x[t][d] into q[t][d], scale[d].
// Thread tid owns chunk tid % CH (CH = d / 8) of rows tid / CH + i * RS
// (RS = 256 / CH rows per pass); threads past CH * RS idle.
template <int RPT>
__device__ __forceinline__ void quant_block_channels(const uint16_t *__restrict__ x, int t, int d, float qmax,
                                                     int8_t *__restrict__ q, float *__restrict__ scale,
                                                     float *part, float *chan_scale)
{
    const int ch = d / 8, rs = kThreads / ch;
    const int tid = threadIdx.x, c = tid % ch, r0 = tid / ch;
    const bool act = r0 < rs;
    u32x4 reg[RPT];
    float amax[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) amax[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = r0 + i * rs;
        reg[i] = u32x4{0u, 0u, 0u, 0u};
        if (act && r < t) reg[i] = *reinterpret_cast<const u32x4 *>(x + (int64_t)r * d + c * 8);
        float v[8];
        widen8(reg[i], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax[e] = fmaxf(amax[e], fabsf(v[e]));
    }
    if (act) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[r0 * d + c * 8 + e] = amax[e];
    }
    __syncthreads();
    for (int j = tid; j < d; j += kThreads) {
        float a = 0.0f;
        for (int rr = 0; rr < rs; ++rr) a = fmaxf(a, part[rr * d + j]);
        const float s = kv_scale(a, qmax);
        chan_scale[j] = s;
        scale[j] = s;
    }
    __syncthreads();
    float s8[8], r8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s8[e] = chan_scale[c * 8 + e];
        r8[e] = __builtin_amdgcn_rcpf(s8[e]);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = r0 + i * rs;
        if (act && r < t) {
            float v[8];
            widen8(reg[i], v);
            *reinterpret_cast<u32x2 *>(q + (int64_t)r * d + c * 8) = codes8(v, s8, r8, qmax);
        }
    }
}

template <int LPR>
__global__ __launch_bounds__(kThreads) void kv_quant_tokens_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                                  int d, float qmax, int8_t *__restrict__ q,
                                                                  float *__restrict__ scale)
{
    constexpr int RPW = kThreads / LPR;
    quant_rows<LPR, 4>(x, (int64_t)blockIdx.x * RPW, rows, (int64_t)gridDim.x * RPW, d, qmax, q, scale);
}

// LDS of the per-channel reduction: partial maxima [rows per pass][d] and the
// channel scales [d] (d <= 512); rows per pass * d = 8 * 256 floats whatever d is.
struct ChannelLds {
    float part[kThreads * 8];
    float chan_scale[512];
};

template <int RPT>
__global__ __launch_bounds__(kThreads) void kv_quant_channels_kernel(const uint16_t *__restrict__ x, int t, int d,
                                                                    float qmax, int8_t *__restrict__ q,
                                                                    float *__restrict__ scale)
{
    __shared__ ChannelLds lds;
    const int64_t b = blockIdx.x;
    quant_block_channels<RPT>(x + b * t * d, t, d, qmax, q + b * t * d, scale + b * d, lds.part, lds.chan_scale);
}

// Block p of the window (K and V, [t][d] each) into pool slot dst[p]; slots
// outside [0, pool_blocks) are skipped.
template <int RPT, int LPR>
__global__ __launch_bounds__(kThreads) void kv_flush_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                                           int t, int d, float qmax, const int32_t *__restrict__ dst,
                                                           int64_t pool_blocks, int8_t *__restrict__ k_pool,
                                                           float *__restrict__ k_scale, int8_t *__restrict__ v_pool,
                                                           float *__restrict__ v_scale)
{
    __shared__ ChannelLds lds;
    const int64_t p = blockIdx.x;
    const int64_t slot = dst[p];
    if (slot < 0 || slot >= pool_blocks) return;           // uniform across the workgroup
    const int64_t e0 = p * t * d, o0 = slot * t * d;
    quant_block_channels<RPT>(k + e0, t, d, qmax, k_pool + o0, k_scale + slot * d, lds.part, lds.chan_scale);
    quant_rows<LPR, 2>(v + e0, 0, t, kThreads / LPR, d, qmax, v_pool + o0, v_scale + slot * t);
}

// Dequantization, eight elements per thread: out = fp16(q * scale).
__device__ __forceinline__ u32x4 dequant8(u32x2 w, const float s[8])
{
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const float a = (float)(int8_t)(w[e >> 2] >> (8 * (e & 3))) * s[e];
        const float b = (float)(int8_t)(w[(e + 1) >> 2] >> (8 * ((e + 1) & 3))) * s[e + 1];
        const f16x2 h = {(_Float16)a, (_Float16)b};
        out[e >> 1] = bitcast<uint32_t>(h);
    }
    return out;
}

__global__ __launch_bounds__(kThreads) void kv_dequant_tokens_kernel(const int8_t *__restrict__ q,
                                                                    const float *__restrict__ scale, int64_t chunks,
                                                                    int d, uint16_t *__restrict__ out)
{
    const int cpr = d / 8;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i0 < chunks; i0 += 4 * stride) {
        u32x2 w[4];
        float s[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * stride;
            w[u] = u32x2{0u, 0u};
            s[u] = 0.0f;
            if (i < chunks) {
                w[u] = *reinterpret_cast<const u32x2 *>(q + i * 8);
                s[u] = scale[i / cpr];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * stride;
            float s8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) s8[e] = s[u];
            if (i < chunks) *reinterpret_cast<u32x4 *>(out + i * 8) = dequant8(w[u], s8);
        }
    }
}

__global__ __launch_bounds__(kThreads) void kv_dequant_channels_kernel(const int8_t *__restrict__ q,
                                                                      const float *__restrict__ scale, int64_t chunks,
                                                                      int t, int d, uint16_t *__restrict__ out)
{
    const int cpr = d / 8;
    const int64_t cpb = (int64_t)t * cpr;                  // chunks per block
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i0 < chunks; i0 += 4 * stride) {
        u32x2 w[4];
        f32x4 lo[4], hi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * stride;
            w[u] = u32x2{0u, 0u};
            lo[u] = hi[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < chunks) {
                const float *sp = scale + (i / cpb) * d + (int)(i % cpr) * 8;
                w[u] = *reinterpret_cast<const u32x2 *>(q + i * 8);
                lo[u] = *reinterpret_cast<const f32x4 *>(sp);
                hi[u] = *reinterpret_cast<const f32x4 *>(sp + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * stride;
            const float s8[8] = {lo[u][0], lo[u][1], lo[u][2], lo[u][3], hi[u][0], hi[u][1], hi[u][2], hi[u][3]};
            if (i < chunks) *reinterpret_cast<u32x4 *>(out + i * 8) = dequant8(w[u], s8);
        }
    }
}

// Lanes per token row: the power of two at or above d / 8.
int lanes_per_row(int d)
{
    int l = 1;
    while (l < d / 8) l <<= 1;
    return l;
}

// Rows per thread of the per-channel layout, rounded up to a power of two.
int rows_per_thread(int t, int d)
{
    const int rs = kThreads / (d / 8);
    const int need = (t + rs - 1) / rs;
    int r = 1;
    while (r < need) r <<= 1;
    return r;
}

unsigned grid_for(int64_t work, int64_t per_block)
{
    const int64_t g = (work + per_block - 1) / per_block;
    return (unsigned)(g < 65536 ? g : 65536);
}

template <int LPR>
hipError_t launch_tokens(const uint16_t *x, int64_t rows, int d, float qmax, int8_t *q, float *scale,
                         hipStream_t stream)
{
    // four rows per lane per pass (quant_rows<LPR, 4>)
    kv_quant_tokens_kernel<LPR><<<grid_for(rows, 4 * (kThreads / LPR)), kThreads, 0, stream>>>(x, rows, d, qmax, q,
                                                                                                scale);
    return hipGetLastError();
}

template <int RPT>
hipError_t launch_channels(const uint16_t *x, int64_t blocks, int t, int d, float qmax, int8_t *q, float *scale,
                           hipStream_t stream)
{
    kv_quant_channels_kernel<RPT><<<(unsigned)blocks, kThreads, 0, stream>>>(x, t, d, qmax, q, scale);
    return hipGetLastError();
}

template <int RPT, int LPR>
hipError_t launch_flush(const uint16_t *k, const uint16_t *v, int64_t blocks, int t, int d, float qmax,
                        const int32_t *dst, int64_t pool_blocks, int8_t *k_pool, float *k_scale, int8_t *v_pool,
                        float *v_scale, hipStream_t stream)
{
    kv_flush_kernel<RPT, LPR><<<(unsigned)blocks, kThreads, 0, stream>>>(k, v, t, d, qmax, dst, pool_blocks, k_pool,
                                                                         k_scale, v_pool, v_scale);
    return hipGetLastError();
}

template <int LPR>
hipError_t flush_by_rpt(int rpt, const uint16_t *k, const uint16_t *v, int64_t blocks, int t, int d, float qmax,
                        const int32_t *dst, int64_t pool_blocks, int8_t *k_pool, float *k_scale, int8_t *v_pool,
                        float *v_scale, hipStream_t stream)
{
    switch (rpt) {
    case 1: return launch_flush<1, LPR>(k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 2: return launch_flush<2, LPR>(k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 4: return launch_flush<4, LPR>(k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 8: return launch_flush<8, LPR>(k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 16: return launch_flush<16, LPR>(k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 32: return launch_flush<32, LPR>(k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t kv_launch_quant_tokens(const uint16_t *x, int64_t rows, int d, int bits, int8_t *q, float *scale,
                                  hipStream_t stream)
{
    const float qmax = (float)((1 << (bits - 1)) - 1);
    switch (lanes_per_row(d)) {
    case 1: return launch_tokens<1>(x, rows, d, qmax, q, scale, stream);
    case 2: return launch_tokens<2>(x, rows, d, qmax, q, scale, stream);
    case 4: return launch_tokens<4>(x, rows, d, qmax, q, scale, stream);
    case 8: return launch_tokens<8>(x, rows, d, qmax, q, scale, stream);
    case 16: return launch_tokens<16>(x, rows, d, qmax, q, scale, stream);
    case 32: return launch_tokens<32>(x, rows, d, qmax, q, scale, stream);
    case 64: return launch_tokens<64>(x, rows, d, qmax, q, scale, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t kv_launch_quant_channels(const uint16_t *x, int64_t blocks, int t, int d, int bits, int8_t *q,
                                    float *scale, hipStream_t stream)
{
    const float qmax = (float)((1 << (bits - 1)) - 1);
    switch (rows_per_thread(t, d)) {
    case 1: return launch_channels<1>(x, blocks, t, d, qmax, q, scale, stream);
    case 2: return launch_channels<2>(x, blocks, t, d, qmax, q, scale, stream);
    case 4: return launch_channels<4>(x, blocks, t, d, qmax, q, scale, stream);
    case 8: return launch_channels<8>(x, blocks, t, d, qmax, q, scale, stream);
    case 16: return launch_channels<16>(x, blocks, t, d, qmax, q, scale, stream);
    case 32: return launch_channels<32>(x, blocks, t, d, qmax, q, scale, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t kv_launch_flush(const uint16_t *k, const uint16_t *v, int64_t blocks, int t, int d, int bits,
                           const int32_t *dst, int64_t pool_blocks, int8_t *k_pool, float *k_scale, int8_t *v_pool,
                           float *v_scale, hipStream_t stream)
{
    const float qmax = (float)((1 << (bits - 1)) - 1);
    const int rpt = rows_per_thread(t, d);
    switch (lanes_per_row(d)) {
    case 1: return flush_by_rpt<1>(rpt, k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 2: return flush_by_rpt<2>(rpt, k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 4: return flush_by_rpt<4>(rpt, k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 8: return flush_by_rpt<8>(rpt, k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 16: return flush_by_rpt<16>(rpt, k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 32: return flush_by_rpt<32>(rpt, k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    case 64: return flush_by_rpt<64>(rpt, k, v, blocks, t, d, qmax, dst, pool_blocks, k_pool, k_scale, v_pool, v_scale, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t kv_launch_dequant_tokens(const int8_t *q, const float *scale, int64_t rows, int d, uint16_t *out,
                                    hipStream_t stream)
{
    const int64_t chunks = rows * (d / 8);
    kv_dequant_tokens_kernel<<<grid_for(chunks, 4 * kThreads), kThreads, 0, stream>>>(q, scale, chunks, d, out);
    return hipGetLastError();
}

hipError_t kv_launch_dequant_channels(const int8_t *q, const float *scale, int64_t blocks, int t, int d,
                                      uint16_t *out, hipStream_t stream)
{
    const int64_t chunks = blocks * t * (d / 8);
    kv_dequant_channels_kernel<<<grid_for(chunks, 4 * kThreads), kThreads, 0, stream>>>(q, scale, chunks, t, d,
                                                                                          out);
    return hipGetLastError();
}
