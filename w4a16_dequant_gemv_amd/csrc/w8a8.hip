// w8a8.hip -- W8A8 linear layer with SmoothQuant on the gfx950 int8 matrix
// cores: calibration maxima, smoothing factors, per-channel INT8 weights,
// per-token INT8 activations and the int8 x int8 -> int32 product.
//
// [Guide] §4.2 (SmoothQuant): activations are hard to quantize because of
// outlier channels, weights are easy, so Y = (X diag(s)^-1)(diag(s) W) moves
// difficulty from X to W with s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)
// (alpha = 0.5 in practice; max|W_j| taken over every linear sharing the
// input; both clamped at 1e-5), and diag(s)^-1 can be folded into the
// preceding LayerNorm.  W8A8 runs the product on INT8 matrix units at twice
// the fp16 rate ([Guide] §4.2, §2.3); INT8 weights carry one scale per
// output channel ([Guide] §2.2); activations are quantized per token at run
// time with the symmetric map of [Guide] §6's per-token listing.
//
// Arithmetic (this unit is built without FMA contraction and with correctly
// rounded division and square root): the smoothed weight is w * s and the
// smoothed activation x / s in binary32; scale = max|.| / 127 floored at
// 1e-8; code = clamp(round(v / scale), -128, 127), where the product with the
// hardware reciprocal decides unless it lies within 2^-14 of a half-integer
// (then the correctly rounded division does), so codes are bit-exact; the
// integer product is exact in int32 (|code| <= 128, K <= 32768); and
// y = fp16((float(acc) * sx[m]) * sw[n]).  Every output is therefore
// bit-exact; only alpha != 0.5 (powf) may differ from another libm by an ulp.
//
// GEMM tiling follows the W4A16 kernel (q4_gemm.hip) without the
// dequantization: 256 x 128 output tiles, k in steps of 128 bytes = two
// v_mfma_i32_16x16x64_i8 substeps, three LDS stages of (x tile | weight tile)
// with one barrier per step, warp specialization (four consumer waves stacked
// along m, 64 x 128 each, and four producer waves that move both tiles by
// direct global->LDS loads), the XCD-aware tile order and the conflict-free
// chunk swizzle of gemm_tile.h.  The MFMAs take the weight fragment first, so
// each lane holds runs of 4 consecutive output channels and the epilogue
// stores whole rows through LDS.  With the consumers' instruction streams
// holding only fragment reads and MFMAs, the 16x16x64 form measured 3-8 %
// faster than v_mfma_i32_32x32x32_i8 (same operand bytes per op); in the
// earlier kernel, where every wave also loaded and stored, it was slower.
#include <type_traits>

#include "gemm_tile.h"
#include "q4_device.h"
#include "q4_launch.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr float kQmax = 127.0f;

// ---------------------------------------------------------------------------
// Calibration: column maxima of |x| folded into out[] with an atomic maximum
// on the float bits (non-negative floats order like their bit patterns), so
// several batches (or several linears sharing an input) accumulate exactly.
// ---------------------------------------------------------------------------
template <bool F32>
__global__ __launch_bounds__(kThreads) void col_absmax_kernel(const void *__restrict__ src, int64_t rows, int cols,
                                                              int rows_per_block, float *__restrict__ out)
{
    const int cpr = cols / 8;
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= cpr) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
    float mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mx[e] = 0.0f;
#pragma unroll 4
    for (int64_t r = r0; r < r1; ++r) {
        float v[8];
        if constexpr (F32) {
            const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(src) + r * cols + c * 8);
            const f32x4 a = p[0], b = p[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = a[e];
                v[e + 4] = b[e];
            }
        } else {
            const u32x4 raw =
                *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(src) + r * cols + c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = half_bits_to_float((uint16_t)(raw[e >> 1] >> (16 * (e & 1))));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], fabsf(v[e]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        atomicMax(reinterpret_cast<unsigned int *>(out) + c * 8 + e, __float_as_uint(mx[e]));
}

__global__ __launch_bounds__(kThreads) void smooth_factors_kernel(const float *__restrict__ act_max,
                                                                  const float *__restrict__ w_max, int n,
                                                                  float alpha, float *__restrict__ s)
{
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const float w = w_max[i] < 1e-5f ? 1e-5f : w_max[i];
    float num, den;
    if (alpha == 0.5f) {
        num = __builtin_sqrtf(act_max[i]);
        den = __builtin_sqrtf(w);
    } else {
        num = powf(act_max[i], alpha);
        den = powf(w, 1.0f - alpha);
    }
    const float v = num / den;
    s[i] = v < 1e-5f ? 1e-5f : v;
}

// ---------------------------------------------------------------------------
// Row quantizers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sym_scale(float amax)
{
    const float s = amax / kQmax;
    return s < 1e-8f ? 1e-8f : s;
}

// round(v / s) clamped to int8 (see the file comment for the reciprocal test)
__device__ __forceinline__ uint32_t sym_code(float v, float s, float r)
{
    const float a = v * r;
    float c = __builtin_rintf(a);
    if (fabsf(a - c) > 0.5f - 0x1p-14f || fabsf(a) >= 128.0f) c = __builtin_rintf(v / s);
    c = fminf(fmaxf(c, -kQmax - 1.0f), kQmax);
    return (uint32_t)(int32_t)c & 0xFFu;
}

__device__ __forceinline__ u32x2 sym_codes8(const float v[8], float s, float r)
{
    u32x2 w = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e >> 2] |= sym_code(v[e], s, r) << (8 * (e & 3));
    return w;
}

// Maximum over the workgroup (every thread gets it).
__device__ __forceinline__ float block_max(float a, float *red)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return a;
}

// One workgroup per weight row: w * s, its maximum, then the codes (the row
// is read twice; the second read is served by the caches).
__global__ __launch_bounds__(kThreads) void quant_weight_kernel(const float *__restrict__ w,
                                                                const float *__restrict__ s, int n_in,
                                                                int8_t *__restrict__ q, float *__restrict__ sw)
{
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float *wr = w + row * n_in;
    const int cpr = n_in / 8;
    auto load8 = [&](int c, float v[8]) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(wr + c * 8);
        const f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[e + 4] = b[e];
        }
        if (s) {
            const f32x4 *sp = reinterpret_cast<const f32x4 *>(s + c * 8);
            const f32x4 sa = sp[0], sb = sp[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = v[e] * sa[e];
                v[e + 4] = v[e + 4] * sb[e];
            }
        }
    };
    float a = 0.0f;
    for (int c = threadIdx.x; c < cpr; c += kThreads) {
        float v[8];
        load8(c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
    }
    const float sc = sym_scale(block_max(a, red));
    const float rc = __builtin_amdgcn_rcpf(sc);
    for (int c = threadIdx.x; c < cpr; c += kThreads) {
        float v[8];
        load8(c, v);
        *reinterpret_cast<u32x2 *>(q + row * n_in + c * 8) = sym_codes8(v, sc, rc);
    }
    if (threadIdx.x == 0) sw[row] = sc;
}

// One workgroup per token row, the row's x / s kept in registers (CPT chunks
// of 8 per thread, k <= CPT * 2048).
template <int CPT>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(const uint16_t *__restrict__ x,
                                                             const float *__restrict__ s, int k,
                                                             int8_t *__restrict__ q, float *__restrict__ sx)
{
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const int cpr = k / 8;
    float v[CPT][8];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + i * kThreads;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
        if (c < cpr) {
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(x + row * k + c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = half_bits_to_float((uint16_t)(raw[e >> 1] >> (16 * (e & 1))));
            if (s) {
                const f32x4 *sp = reinterpret_cast<const f32x4 *>(s + c * 8);
                const f32x4 sa = sp[0], sb = sp[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[i][e] = v[i][e] / sa[e];
                    v[i][e + 4] = v[i][e + 4] / sb[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[i][e]));
        }
    }
    const float sc = sym_scale(block_max(a, red));
    const float rc = __builtin_amdgcn_rcpf(sc);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + i * kThreads;
        if (c < cpr) *reinterpret_cast<u32x2 *>(q + row * k + c * 8) = sym_codes8(v[i], sc, rc);
    }
    if (threadIdx.x == 0) sx[row] = sc;
}

// ---------------------------------------------------------------------------
// int8 GEMM.
// ---------------------------------------------------------------------------
// Warp-specialized form: four consumer waves (fragment reads and MFMAs
// only) and four producer waves per workgroup, two waves per SIMD.  With no
// dequantization the producers only issue direct global->LDS loads
// (buffer_load ... lds: no registers, no LDS store instructions) of step
// k+2's x and weight tiles into stage (k+2) % 3 and wait for them before the
// step's barrier; lane i of a load lands at row i / 8, physical chunk i % 8
// and fetches the logical chunk that the row's swizzle places there.
template <int BM, int BN>
__global__ __launch_bounds__(512) void w8a8_gemm_ws_kernel(
    const int8_t *__restrict__ qx, const float *__restrict__ sx, const int8_t *__restrict__ qw,
    const float *__restrict__ sw, uint16_t *__restrict__ y, int m, int n_out, int k, int tiles_m, int tiles_n)
{
    constexpr int BK = 128, NC = 4, THREADS = 512;     // BK: two 64-wide substeps
    constexpr int WT_M = BM / NC, WT_N = BN;
    constexpr int TM = WT_M / 16, TN = WT_N / 16;
    constexpr int XL = BM / NC / 8, WL = BN / NC / 8;    // direct loads per producer wave per step
    static_assert(TM * 16 == WT_M && TN * 16 == WT_N, "wave tile not a multiple of 16");
    static_assert(XL * 8 * NC == BM && WL * 8 * NC == BN, "tile rows do not split over the producers");
    constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
    constexpr int A_CHUNKS = BM * 8 / THREADS, B_CHUNKS = BN * 8 / THREADS;   // tail step, all threads
    static_assert(kStages == 3, "the loop is unrolled for three stages");
    static_assert(kStages * STAGE <= 160 * 1024, "stages exceed LDS");
    extern __shared__ __attribute__((aligned(16))) char smem[];

    int tile_m, tile_n;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ksteps = k / BK, krem = k % BK;

    // Per-tile buffer resources; rows past m or n_out read the last row (never stored).
    const int rows_m = min(BM, m - m0), rows_n = min(BN, n_out - n0);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(qx + (int64_t)m0 * k), (short)0, rows_m * k, kBufferFlags);
    const __amdgpu_buffer_rsrc_t wr_ = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(qw + (int64_t)n0 * k), (short)0, rows_n * k, kBufferFlags);

    struct Frag {
        i32x4 a[TM], b[TN];
    };
    const int frow = lane & 15, fkg = lane >> 4, fswz = swz(frow);
    const uint32_t fa = (wave * WT_M + frow) * 128, fb = A_BYTES + frow * 128;
    // Fragments of substep ks (64 k): lane (row l % 16, k group l / 16) reads chunk 4 ks + l / 16.
    auto read_frag = [&](Frag &f, uint32_t buf, int ks) {
        const uint32_t cofs = ((4 * ks + fkg) ^ fswz) * 16;
#pragma unroll
        for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const i32x4 *>(smem + buf + fa + cofs + i * 16 * 128);
#pragma unroll
        for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const i32x4 *>(smem + buf + fb + cofs + j * 16 * 128);
    };
    i32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0;
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
    };

    if (wave < NC) {
        // ---------------- consumer ----------------
        if (ksteps > 0) {
            __syncthreads();                            // stages 0 and 1 written
            Frag f0, f1;
            read_frag(f0, 0, 0);
            // Step k (k % 3 == J): substep 1 from stage J, then step k+1's
            // first fragments from stage (J+1) % 3; one barrier.
            auto step = [&](auto J_) {
                constexpr int J = decltype(J_)::value;
                constexpr uint32_t cur = J * STAGE, nxt = ((J + 1) % 3) * STAGE;
                read_frag(f1, cur, 1);
                mma(f0);
                read_frag(f0, nxt, 0);
                mma(f1);
                __syncthreads();
            };
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            int kk = 0;
            for (; kk + 3 <= ksteps; kk += 3) {
                step(I0{});
                step(I1{});
                step(I2{});
            }
            if (kk < ksteps) step(I0{});
            if (kk + 1 < ksteps) step(I1{});
        }
    } else {
        // ---------------- producer ----------------
        typedef __attribute__((address_space(3))) char lds_char;
        const int pw = wave - NC;
        uint32_t xdoff[XL], wdoff[WL];
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const int r = pw * XL * 8 + 8 * j + (lane >> 3);
            xdoff[j] = (uint32_t)min(r, rows_m - 1) * (uint32_t)k + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
        }
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            const int r = pw * WL * 8 + 8 * j + (lane >> 3);
            wdoff[j] = (uint32_t)min(r, rows_n - 1) * (uint32_t)k + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
        }
        // (the offsets are passed as int explicitly: with an implicit
        // conversion this toolchain's host pass dropped the kernel's launch stub)
        auto load = [&](uint32_t buf, int kt) {
            lds_char *dx = (lds_char *)smem + buf + pw * XL * 8 * 128;
            lds_char *dw = (lds_char *)smem + buf + A_BYTES + pw * WL * 8 * 128;
#pragma unroll
            for (int j = 0; j < XL; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void *)(dx + j * 8 * 128),
                                                         16, (int)xdoff[j], kt * BK, 0, 0);
#pragma unroll
            for (int j = 0; j < WL; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr_, (__attribute__((address_space(3))) void *)(dw + j * 8 * 128),
                                                         16, (int)wdoff[j], kt * BK, 0, 0);
        };
        if (ksteps > 0) {
            const int kmax = ksteps - 1;
            load(0, 0);
            load(STAGE, min(1, kmax));
            __syncthreads();                            // (waits for every load, direct ones included)
            // Step k (k % 3 == J): step k+2 into stage (J+2) % 3, which the
            // consumers finished reading before the previous barrier; steps
            // past the last one rewrite the last step.
            auto step = [&](auto J_, int kk) {
                constexpr int J = decltype(J_)::value;
                load(((J + 2) % 3) * STAGE, min(kk + 2, kmax));
                __syncthreads();
            };
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            int kk = 0;
            for (; kk + 3 <= ksteps; kk += 3) {
                step(I0{}, kk);
                step(I1{}, kk + 1);
                step(I2{}, kk + 2);
            }
            if (kk < ksteps) step(I0{}, kk);
            if (kk + 1 < ksteps) step(I1{}, kk + 1);
        }
    }

    if (krem) {
        // Final partial step of krem = 32, 64 or 96 bytes, loaded by every
        // thread: the chunks past krem are zero in LDS, so the substeps that
        // hold data run (one for krem <= 64, two for 96).  Every wave passed the last barrier after its last
        // LDS access, so stage 0 is free.
        const int kt = ksteps;
        const int st_row = tid >> 3;
        const uint32_t a_st = st_row * 128 + (((tid & 7) ^ swz(st_row)) * 16);
        const bool valid = (tid & 7) * 16 < krem;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + i * THREADS;
            const uint32_t off = (uint32_t)min(c >> 3, rows_m - 1) * (uint32_t)k + (uint32_t)(c & 7) * 16u;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (valid) v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, kt * BK, 0);
            *reinterpret_cast<u32x4 *>(smem + a_st + i * THREADS * 16) = v;
        }
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            const int c = tid + i * THREADS;
            const uint32_t off = (uint32_t)min(c >> 3, rows_n - 1) * (uint32_t)k + (uint32_t)(c & 7) * 16u;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (valid) v = __builtin_amdgcn_raw_buffer_load_b128(wr_, off, kt * BK, 0);
            *reinterpret_cast<u32x4 *>(smem + A_BYTES + a_st + i * THREADS * 16) = v;
        }
        __syncthreads();
        if (wave < NC) {
            for (int ks = 0; ks < (krem + 63) / 64; ++ks) {
                Frag f;
                read_frag(f, 0, ks);
                mma(f);
            }
        }
    }

    // Epilogue: tile (i, j) holds y^T -- lane l, register r is output channel
    // 4 (l / 16) + r of the tile's 16, for x row l % 16.
    // y = fp16((float(acc) * sx[row]) * sw[channel]) goes through LDS (rows
    // padded to YS bytes) and leaves as 16-byte pieces of whole rows, stored
    // by all eight waves.
    constexpr int YS = BN * 2 + 16;
    static_assert(BM * YS <= kStages * STAGE, "output tile exceeds LDS");
    __syncthreads();
    if (wave < NC) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wave * WT_M + i * 16 + (lane & 15);
            const float sxv = sx[m0 + min(r, rows_m - 1)];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int c = j * 16 + 4 * (lane >> 4);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float swv = sw[n0 + min(c + e, rows_n - 1)];
                    v[e] = ((float)acc[i][j][e] * sxv) * swv;
                }
                const f16x2 lo = {(_Float16)v[0], (_Float16)v[1]};
                const f16x2 hi = {(_Float16)v[2], (_Float16)v[3]};
                *reinterpret_cast<u32x2 *>(smem + r * YS + c * 2) =
                    u32x2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
            }
        }
    }
    __syncthreads();
    constexpr int CPR = BN / 8;
    constexpr int RPP = THREADS / CPR;
    static_assert(CPR * RPP == THREADS && BM % RPP == 0, "output tile does not split evenly");
    const bool vec16 = ((reinterpret_cast<uintptr_t>(y) & 15) == 0) && ((n_out & 7) == 0);
    const int pc = tid % CPR, col = n0 + pc * 8;
#pragma unroll 4
    for (int r = tid / CPR; r < BM; r += RPP) {
        const int row = m0 + r;
        if (row >= m) break;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + r * YS + pc * 16);
        uint16_t *yp = y + (int64_t)row * n_out + col;
        if (vec16 && col + 8 <= n_out) {
            *reinterpret_cast<u32x4 *>(yp) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (col + e < n_out) yp[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
    }
}

template <typename K>
hipError_t allow_full_lds(K kernel)
{
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return e;
}

template <int CPT>
hipError_t launch_act(const uint16_t *x, const float *s, int64_t m, int k, int8_t *q, float *sx,
                      hipStream_t stream)
{
    quant_act_kernel<CPT><<<(unsigned)m, kThreads, 0, stream>>>(x, s, k, q, sx);
    return hipGetLastError();
}

}  // namespace

hipError_t w8a8_launch_col_absmax(const void *src, bool f32, int64_t rows, int cols, float *out,
                                  hipStream_t stream)
{
    const int cpr = cols / 8;
    const int rows_per_block = 64;
    const int64_t slices = (rows + rows_per_block - 1) / rows_per_block;
    const dim3 grid((unsigned)((cpr + kThreads - 1) / kThreads), (unsigned)slices);
    if (f32)
        col_absmax_kernel<true><<<grid, kThreads, 0, stream>>>(src, rows, cols, rows_per_block, out);
    else
        col_absmax_kernel<false><<<grid, kThreads, 0, stream>>>(src, rows, cols, rows_per_block, out);
    return hipGetLastError();
}

hipError_t w8a8_launch_smooth_factors(const float *act_max, const float *w_max, int n, float alpha, float *s,
                                      hipStream_t stream)
{
    smooth_factors_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, stream>>>(act_max, w_max, n,
                                                                                             alpha, s);
    return hipGetLastError();
}

hipError_t w8a8_launch_quant_weight(const float *w, const float *s, int64_t n_out, int n_in, int8_t *q, float *sw,
                                    hipStream_t stream)
{
    quant_weight_kernel<<<(unsigned)n_out, kThreads, 0, stream>>>(w, s, n_in, q, sw);
    return hipGetLastError();
}

hipError_t w8a8_launch_quant_act(const uint16_t *x, const float *s, int64_t m, int k, int8_t *q, float *sx,
                                 hipStream_t stream)
{
    const int chunks = (k / 8 + kThreads - 1) / kThreads;      // per thread
    if (chunks <= 1) return launch_act<1>(x, s, m, k, q, sx, stream);
    if (chunks <= 2) return launch_act<2>(x, s, m, k, q, sx, stream);
    if (chunks <= 4) return launch_act<4>(x, s, m, k, q, sx, stream);
    if (chunks <= 8) return launch_act<8>(x, s, m, k, q, sx, stream);
    if (chunks <= 16) return launch_act<16>(x, s, m, k, q, sx, stream);
    return hipErrorInvalidValue;
}

hipError_t w8a8_launch_gemm(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw, int64_t m,
                            int64_t n_out, int64_t k, uint16_t *y, hipStream_t stream)
{
    constexpr int BM = 256, BN = 128;
    const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n_out + BN - 1) / BN);
    auto kernel = w8a8_gemm_ws_kernel<BM, BN>;
    const hipError_t e = allow_full_lds(kernel);
    if (e != hipSuccess) return e;
    const size_t lds = kStages * (size_t)(BM + BN) * 128;
    kernel<<<(unsigned)(tiles_m * tiles_n), 512, lds, stream>>>(qx, sx, qw, sw, y, (int)m, (int)n_out, (int)k,
                                                               tiles_m, tiles_n);
    return hipGetLastError();
}
