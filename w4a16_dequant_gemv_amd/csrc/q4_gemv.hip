// q4_gemv.hip -- decode-shaped W4A16 linear layer, y[m][n] = sum_k x[m][k] w'[n][k]
// for 1 <= m <= 16, with w' = s (code - z) formed on the fly.
//
// [Kern] §4: the dequantization is fused into the product, the fp16 weights
// are never materialized in memory.  [Guide] §1.2: at decode sizes every
// weight byte is read once per call and the arithmetic intensity is a few
// FLOP per byte, so the kernel is bound by HBM bandwidth.
//
// What limits it on gfx950 is the number of vector-memory instructions, not
// arithmetic: every global load, however small, occupies the CU's address
// and data path for several cycles, so per-lane gathers of x, scales and
// zero-points cost as much as the 1-KiB weight loads themselves.  The kernel
// therefore issues exactly one global load per 1 KiB of packed weights per
// wave; x (pre-permuted into MFMA fragment order) and the scale|zero pairs
// of the workgroup's rows are staged cooperatively in LDS, one k window at a
// time, and read back with ds_read.
//
// Matrix-core mapping.  v_mfma_f32_16x16x32_f16 multiplies a 16x32 A block
// (rows = the m rows of x, padded to 16 with copies of row m-1 whose results
// are discarded) by a 32x16 B block (columns = 16 output channels).  Lane l
// supplies row/column l % 16 and eight k values selected by l / 16 (the same
// eight for A and B).  In one 128-wide k block, lane (column c, quarter q)
// loads the 16 bytes (four packed words, 32 codes) of channel c at
// k = kb + 32q .. kb + 32q + 31.  MFMA number t (t = 0..3) takes from each of
// the lane's words j the codes at nibble positions t and t + 4, i.e.
// k = kb + 32q + 8j + {t, t+4}; x is stored in LDS in the same order, which
// leaves every dot product unchanged.
//
// Two ways of forming B:
//  * group_size >= 128 (every 128-wide k block lies in one group):
//    masking a packed word with 0x000F000F leaves codes (c_t, c_{t+4}) as the
//    fp16 bit patterns of the subnormals c * 2^-24 -- exact values, two
//    codes per AND.  Masking with 0x00F000F0 gives c * 2^-20.  So B costs
//    five VALU instructions per word (mask, mask, shift, mask, mask) and the
//    scale and zero-point are applied once per block to the fp32 MFMA
//    results:  y += s * 2^24 * (P24 + P20 / 16 - z X),  where P24 sums
//    x c 2^-24 over the codes masked in place, P20 sums x c 2^-20 over the
//    codes masked four bits up, and X = 2^-24 sum_k x_k comes from one more
//    MFMA chain against B = 2^-24.  Nothing is rounded before the fp32
//    accumulation; the subtraction is between terms of similar size (codes
//    and z are both in 0..15), so it loses no accuracy to speak of.
//  * group_size 32 or 64 (a block spans several groups): the classic form,
//    OR-ing codes into the half 1024 (0x6400), subtracting 1024 + z (exact)
//    and multiplying by s in fp16 (the only rounding, 2^-11 relative).
//
// Work split.  A workgroup of SPLIT waves owns CT tiles of 16 output
// channels.  k is cut into windows of WB = SPLIT * UNROLL blocks; in each
// window wave w handles blocks w*UNROLL .. w*UNROLL + UNROLL - 1, so the
// workgroup reads WB * 64 contiguous bytes of each of its rows per window.
// The next window's weights (registers) and x / scale|zero (registers, then
// LDS) are fetched while the current window is computed; one barrier per
// window hands the LDS buffers over.  Partial results of the SPLIT waves are
// summed in LDS in a fixed order, so results are deterministic.
#include "q4_device.h"
#include "q4_launch.h"

namespace {

// Per-lane weight registers for one window: UNROLL blocks x CT tiles.
template <int CT, int UNROLL>
struct Stage {
    u32x4 w[UNROLL][CT];
};

// Cooperative copy of one window's x and scale|zero pairs: each thread owns
// at most XC chunks of 32 x values and SC (row, group) items.
template <int XC, int SC>
struct Coop {
    u32x4 x[XC][4];
    uint16_t s[SC], z[SC];
};

// Eight consecutive x values (four dwords) -> the dwords (x[t], x[t+4]) of
// MFMA t, for the j-th word of a lane's 32 codes.
__device__ __forceinline__ uint32_t pick_pair(const u32x4 &v, int t)
{
    const uint32_t lo = v[t >> 1], hi = v[(t >> 1) + 2];
    return __builtin_amdgcn_perm(hi, lo, (t & 1) ? 0x07060302u : 0x05040100u);
}

struct Geometry {
    int m, n_out, n_in, group_shift;
    int words_per_row, groups_per_row, kblocks;
    int last_full_quarter;  // quarters beyond it in the last block are padding
    int sz_stride;          // u32 per LDS row of scale|zero pairs (odd)
    int x_row_bytes;        // LDS bytes per x row per window (padded)
};

template <int SPLIT, int CT, int UNROLL, bool FOLD>
__global__ __launch_bounds__(64 * SPLIT) void gemv_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, Geometry geo)
{
    constexpr int THREADS = 64 * SPLIT;
    constexpr int WB = SPLIT * UNROLL;          // k blocks per window
    constexpr int ROWS = 16 * CT;               // output channels per workgroup
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int m = geo.m, n_out = geo.n_out, n_in = geo.n_in, gshift = geo.group_shift;
    const int kblocks = geo.kblocks;
    const int groups_win = (WB * 128) >> gshift;        // groups per row per window
    const int x_buf_bytes = m * geo.x_row_bytes;
    const int sz_buf_bytes = ROWS * geo.sz_stride * 4;
    char *x_lds = lds;                                   // [2][m][x_row_bytes]
    char *sz_lds = lds + 2 * x_buf_bytes;                // [2][ROWS][sz_stride] u32

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int quarter = lane >> 4;
    const int row0 = blockIdx.x * ROWS;
    const int nwin = (kblocks + WB - 1) / WB;

    // ---- per-lane weight addressing (wave-uniform base + fixed offset) ----
    const char *qbase = reinterpret_cast<const char *>(qweight + (int64_t)row0 * geo.words_per_row);
    uint32_t woff[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
        const int r = min(t * 16 + col, n_out - 1 - row0);
        woff[t] = (uint32_t)(r * geo.words_per_row + quarter * 4) * 4u;
    }
    auto qshift_of = [&](int kb) {
        return (kb == kblocks - 1 && quarter > geo.last_full_quarter) ? geo.last_full_quarter - quarter : 0;
    };
    auto load_weights = [&](Stage<CT, UNROLL> &st, int win) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = min(win * WB + wave * UNROLL + u, kblocks - 1);
            // a masked quarter is moved back onto the last whole slice; the
            // offset is summed as a 32-bit value before it meets the base
            const uint32_t kw = (uint32_t)(kb * 16 + qshift_of(kb) * 4) * 4u;
#pragma unroll
            for (int t = 0; t < CT; ++t) {
                const uint32_t wo = woff[t] + kw;
                st.w[u][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(qbase + wo));
            }
        }
    };

    // ---- cooperative staging of x and scale|zero pairs for one window ----
    constexpr int MAX_XCHUNKS = 16 * WB * 4;               // m <= 16 rows
    constexpr int XC = (MAX_XCHUNKS + THREADS - 1) / THREADS;
    constexpr int MAX_SITEMS = ROWS * WB * 4;              // group_size >= 32
    constexpr int SC = (MAX_SITEMS + THREADS - 1) / THREADS;
    const int n_xchunks = m * WB * 4;
    const int n_sitems = ROWS * groups_win;
    auto coop_load = [&](Coop<XC, SC> &c, int win) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int ch = tid + i * THREADS;
            const int cc = min(ch, n_xchunks - 1);          // idle threads repeat a valid chunk
            const int r = cc / (WB * 4), rem = cc % (WB * 4);
            const int kb = min(win * WB + rem / 4, kblocks - 1);
            const int k = min((kb << 7) + ((rem & 3) << 5), n_in - 32);
            const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (int64_t)r * n_in + k);
#pragma unroll
            for (int j = 0; j < 4; ++j) c.x[i][j] = src[j];
        }
#pragma unroll
        for (int i = 0; i < SC; ++i) {
            const int it = min(tid + i * THREADS, n_sitems - 1);
            const int r = min(row0 + it / groups_win, n_out - 1);
            const int gidx = min(win * groups_win + it % groups_win, geo.groups_per_row - 1);
            const int64_t off = (int64_t)r * geo.groups_per_row + gidx;
            c.s[i] = scales[off];
            c.z[i] = zeros[off];
        }
    };
    auto coop_store = [&](const Coop<XC, SC> &c, int buf) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int ch = tid + i * THREADS;
            if (ch < n_xchunks) {
                const int r = ch / (WB * 4), rem = ch % (WB * 4);     // rem = block * 4 + quarter
                char *dst = x_lds + buf * x_buf_bytes + r * geo.x_row_bytes + rem * 64;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    u32x4 d;
#pragma unroll
                    for (int j = 0; j < 4; ++j) d[j] = pick_pair(c.x[i][j], t);
                    *reinterpret_cast<u32x4 *>(dst + 16 * t) = d;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < SC; ++i) {
            const int it = tid + i * THREADS;
            if (it < n_sitems) {
                const int r = it / groups_win, gw = it % groups_win;
                reinterpret_cast<uint32_t *>(sz_lds + buf * sz_buf_bytes)[r * geo.sz_stride + gw] =
                    (uint32_t)c.s[i] | ((uint32_t)c.z[i] << 16);
            }
        }
    };

    f32x4 acc[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int xrow = min(col, m - 1);
    auto compute = [&](const Stage<CT, UNROLL> &st, int win, int buf) {
        const char *xb = x_lds + buf * x_buf_bytes + xrow * geo.x_row_bytes;
        const uint32_t *szb = reinterpret_cast<const uint32_t *>(sz_lds + buf * sz_buf_bytes);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kbl = wave * UNROLL + u;             // block within the window
            const int kb = win * WB + kbl;
            // blocks past the end and padding quarters contribute nothing:
            // their scale is taken as zero
            const bool valid = kb < kblocks && !(kb == kblocks - 1 && quarter > geo.last_full_quarter);
            f16x8 a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                a[t] = *reinterpret_cast<const f16x8 *>(xb + (kbl * 4 + quarter) * 64 + 16 * t);
            const int gw = ((kbl << 7) + (quarter << 5)) >> gshift;
            if (FOLD) {
                // X = 2^-24 * sum of this lane-row's x over the block.
                const f16x8 tiny = bitcast<f16x8>(u32x4{0x00010001u, 0x00010001u, 0x00010001u, 0x00010001u});
                f32x4 xs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], tiny, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int t = 1; t < 4; ++t) xs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], tiny, xs, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < CT; ++t) {
                    u32x4 b0, b1, b2, b3;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t w = st.w[u][t][j];
                        const uint32_t w8 = w >> 8;
                        b0[j] = w & 0x000F000Fu;     // codes 0,4 as c * 2^-24
                        b1[j] = w & 0x00F000F0u;     // codes 1,5 as c * 2^-20
                        b2[j] = w8 & 0x000F000Fu;    // codes 2,6 as c * 2^-24
                        b3[j] = w8 & 0x00F000F0u;    // codes 3,7 as c * 2^-20
                    }
                    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
                    f32x4 p24 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], bitcast<f16x8>(b0), zero4, 0, 0, 0);
                    f32x4 p20 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], bitcast<f16x8>(b1), zero4, 0, 0, 0);
                    p24 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2], bitcast<f16x8>(b2), p24, 0, 0, 0);
                    p20 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[3], bitcast<f16x8>(b3), p20, 0, 0, 0);
                    const uint32_t sz = szb[(t * 16 + col) * geo.sz_stride + gw];
                    const float s = valid ? half_bits_to_float((uint16_t)sz) * 16777216.0f : 0.0f;  // s * 2^24, exact
                    const float nz = -half_bits_to_float((uint16_t)(sz >> 16));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = __builtin_fmaf(p20[r], 0.0625f, p24[r]);
                        acc[t][r] = __builtin_fmaf(s, __builtin_fmaf(nz, xs[r], v), acc[t][r]);
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < CT; ++t) {
                    const uint32_t sz = szb[(t * 16 + col) * geo.sz_stride + gw];
                    const _Float16 s = valid ? bitcast<_Float16>((uint16_t)sz) : (_Float16)0.0f;
                    const _Float16 zb = bitcast<_Float16>((uint16_t)(sz >> 16)) + (_Float16)1024.0f;
                    const f16x2 scale = {s, s}, bias = {zb, zb};
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        u32x4 b;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t h = ((st.w[u][t][j] >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
                            b[j] = bitcast<uint32_t>((bitcast<f16x2>(h) - bias) * scale);
                        }
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[p], bitcast<f16x8>(b), acc[t], 0, 0, 0);
                    }
                }
            }
        }
    };

    // ---- main loop: two register stages, two LDS buffers ----
    // The body is unrolled by two and free of data-dependent branches, so
    // the compiler can keep the next window's loads in flight while the
    // current one is computed (it waits only for the older stage).  The last
    // prefetch of an even window count re-reads the final window, which is
    // still cache-resident, instead of branching around the loads.
    Stage<CT, UNROLL> s0, s1;
    Coop<XC, SC> cp;
    coop_load(cp, 0);
    load_weights(s0, 0);
    coop_store(cp, 0);
    __syncthreads();
    int win = 0;
    for (; win + 1 < nwin; win += 2) {
        coop_load(cp, win + 1);
        load_weights(s1, win + 1);
        compute(s0, win, 0);
        coop_store(cp, 1);
        __syncthreads();
        const int next = min(win + 2, nwin - 1);
        coop_load(cp, next);
        load_weights(s0, next);
        compute(s1, win + 1, 1);
        coop_store(cp, 0);
        __syncthreads();
    }
    if (win < nwin) compute(s0, win, 0);      // odd count: the last window sits in s0 / buffer 0
    if (SPLIT > 1) __syncthreads();           // the partial sums below reuse the x buffers

    // Lane l holds rows 4*(l/16) + r (r = 0..3) of column l % 16 of each tile.
    if (SPLIT > 1) {
        f32x4 *partial = reinterpret_cast<f32x4 *>(lds);       // [SPLIT][CT][64], reuses the x buffers
#pragma unroll
        for (int t = 0; t < CT; ++t) partial[(wave * CT + t) * 64 + lane] = acc[t];
        __syncthreads();
        if (wave >= CT) return;
        // wave t finishes tile t, summing the waves in a fixed order
        const int t = wave;
        f32x4 sum = partial[t * 64 + lane];
#pragma unroll
        for (int w = 1; w < SPLIT; ++w) sum += partial[(w * CT + t) * 64 + lane];
        const int n = row0 + t * 16 + col;
        if (n >= n_out) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * quarter + r;
            if (row < m) y[(int64_t)row * n_out + n] = bitcast<uint16_t>((_Float16)sum[r]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            const int n = row0 + t * 16 + col;
            if (n >= n_out) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * quarter + r;
                if (row < m) y[(int64_t)row * n_out + n] = bitcast<uint16_t>((_Float16)acc[t][r]);
            }
        }
    }
}

template <int SPLIT, int CT, int UNROLL, bool FOLD>
size_t lds_bytes(const Geometry &g)
{
    const size_t x_region = 2 * (size_t)g.m * g.x_row_bytes;
    const size_t partial = SPLIT > 1 ? (size_t)SPLIT * CT * 64 * 16 : 0;
    return (x_region > partial ? x_region : partial) + 2 * (size_t)16 * CT * g.sz_stride * 4;
}

constexpr size_t kMaxLds = 64 * 1024;

template <int SPLIT, int CT, int UNROLL, bool FOLD>
bool plan(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
          const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
          uint16_t *y, hipStream_t stream, hipError_t *err)
{
    static_assert(SPLIT >= CT || SPLIT == 1, "the LDS reduction assigns one wave per tile");
    static_assert(SPLIT * UNROLL % 2 == 0, "a window must hold whole groups of 256");
    constexpr int WB = SPLIT * UNROLL;
    Geometry g;
    g.m = m;
    g.n_out = n_out;
    g.n_in = n_in;
    g.group_shift = group_shift;
    g.words_per_row = n_in >> 3;
    g.groups_per_row = n_in >> group_shift;
    g.kblocks = (n_in + 127) >> 7;
    g.last_full_quarter = ((n_in - ((g.kblocks - 1) << 7)) >> 5) - 1;
    g.sz_stride = ((WB * 128) >> group_shift) | 1;
    g.x_row_bytes = WB * 256 + 16;
    const size_t lds = lds_bytes<SPLIT, CT, UNROLL, FOLD>(g);
    if (lds > kMaxLds) return false;           // x window too large for this m
    const int tiles = (n_out + 15) / 16;
    const dim3 grid((unsigned)((tiles + CT - 1) / CT)), block(64 * SPLIT);
    gemv_kernel<SPLIT, CT, UNROLL, FOLD><<<grid, block, lds, stream>>>(x, qweight, scales, zeros, y, g);
    *err = hipGetLastError();
    return true;
}

// Deep windows for long rows, shallower ones when m makes the x window
// large or the rows are short.
template <bool FOLD>
hipError_t dispatch(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                    const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                    uint16_t *y, hipStream_t stream)
{
    hipError_t e = hipSuccess;
    const int kblocks = (n_in + 127) >> 7;
#define Q4_TRY(S, C, U) \
    if (plan<S, C, U, FOLD>(x, qweight, scales, zeros, m, n_out, n_in, group_shift, y, stream, &e)) return e
    if (kblocks >= 32) {
        Q4_TRY(8, 2, 2);
        Q4_TRY(8, 2, 1);
        Q4_TRY(4, 2, 1);
    }
    if (kblocks >= 8) {
        Q4_TRY(4, 2, 2);
        Q4_TRY(4, 2, 1);
    }
    Q4_TRY(1, 1, 2);
#undef Q4_TRY
    return hipErrorInvalidValue;                // unreachable for m <= 16
}

}  // namespace

hipError_t q4_launch_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, uint16_t *y, hipStream_t stream)
{
    int shift = 0;
    while ((1 << shift) < group_size) ++shift;
    return group_size >= 128
               ? dispatch<true>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream)
               : dispatch<false>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream);
}
