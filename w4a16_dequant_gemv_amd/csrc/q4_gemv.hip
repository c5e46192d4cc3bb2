// q4_gemv.hip -- decode-shaped W4A16 linear layer, y[m][n] = sum_k x[m][k] w'[n][k]
// for 1 <= m <= 16, with w' = s (code - z) formed on the fly.
//
// [Kern] §4: the dequantization is fused into the product, the fp16 weights
// are never materialized in memory.  [Guide] §1.2: at decode sizes every
// weight byte is read once per call and the arithmetic intensity is a few
// FLOP per byte, so the kernel is bound by HBM bandwidth.
//
// What limits it on gfx950 is how many weight bytes each CU keeps in flight
// and how many instructions each KiB of weights costs a wave, not FLOPs.
// Per-lane gathers of x, scales and zero-points cost as many vector-memory
// issue slots as the 1-KiB weight loads themselves, so x (pre-permuted) and
// the scale|zero pairs of the workgroup's rows are staged cooperatively in
// LDS and read back with ds_read, and each wave issues one global load per
// 1 KiB of weights.  For one row of x (m = 1) the row-streaming kernel below
// drops the matrix cores altogether: it spends fewer instructions per KiB
// than any MFMA mapping, whose 16-wide tiles are mostly padding there.
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
// leaves every dot product unchanged.  (On rows of 8192 codes and more the
// weights of two blocks are read as whole 128-byte lines of 8 rows and
// rearranged into this layout in registers; see PairAddr.)
//
// Two ways of forming B:
//  * group_size 128 or 256 (every 128-wide k block lies in one group):
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
//  * group_size 32 or 64 (a block spans several groups), or one group per
//    row (per-channel, where most codes equal z and the fold would cancel
//    large terms): the classic form,
//    OR-ing codes into the half 1024 (0x6400), subtracting 1024 + z (exact)
//    and multiplying by s in fp16 (the only rounding, 2^-11 relative).
//
// INT8 weights (BITS = 8, W8A16).  A lane's 32 codes of a block are 32
// bytes, two 16-byte loads (eight words).  MFMA t takes words 2t and 2t+1:
// masking with 0x00FF00FF before and after a shift by 8 leaves the byte
// pairs (k, k+2) and (k+1, k+3), OR-ed into the half 1024, so x is staged
// with the middle two of every four values swapped; z is subtracted exactly
// and s multiplied in fp16, as in the second form above (8-bit weights never
// take the fold).
//
// Work split.  A workgroup of SPLIT waves owns CT tiles of 16 output
// channels.  Its k blocks are dealt out in stages of SPLIT * UNROLL: in stage
// i wave w takes blocks (i * SPLIT + w) * UNROLL + u, so at any moment the
// workgroup reads a contiguous run of each of its rows.  Two kernels:
//  * resident: all of x and all scale|zero pairs of the workgroup's rows fit
//    in LDS (gfx950 gives a workgroup up to 160 KiB).  They are staged once,
//    behind a single barrier, and every wave then streams its weights through
//    a ring of DEPTH register stages with no further synchronization.
//  * windowed: for larger m * n_in, x and scale|zero pairs are staged one
//    window (one stage of blocks) ahead in double-buffered LDS, with one
//    barrier per window.
// and, for m = 1 with rows of up to 16384 codes, the row-streaming kernels
// (one wave per row, VALU dot products; INT4 and INT8), described where
// they are defined.
// Loads past the last block are redirected to x (hot in L2) rather than
// re-reading weights, so no load is conditional and the compiler keeps the
// ring in flight.  Partial results of the SPLIT waves are summed in LDS in a
// fixed order, so results are deterministic.
#include <atomic>
#include <string>

#include "gemm_tile.h"
#include "q4_device.h"
#include "q4_launch.h"

namespace {

struct Geometry {
    int m, n_out, n_in, group_shift;
    int words_per_row, groups_per_row, kblocks;
    int last_full_quarter;  // quarters beyond it in the last block are padding
    int sz_stride;          // u32 per LDS row of scale|zero pairs (odd)
    int x_row_bytes;        // LDS bytes per row of x (padded)
    int sz_vector;          // scale/zero arrays allow 16-byte loads
    int groups;             // tile groups (persistent kernel)
};

// Per-lane weight registers of one stage: UNROLL blocks x CT tiles x the
// 16-byte loads of one block (BITS / 4: one for INT4, two for INT8).
template <int CT, int UNROLL, int BITS = 4>
struct Stage {
    u32x4 w[UNROLL][CT * (BITS / 4)];
};

// Eight consecutive x values (four dwords) -> the dword (x[t], x[t+4]) used
// by MFMA t.
__device__ __forceinline__ uint32_t pick_pair(const u32x4 &v, int t)
{
    const uint32_t lo = v[t >> 1], hi = v[(t >> 1) + 2];
    return __builtin_amdgcn_perm(hi, lo, (t & 1) ? 0x07060302u : 0x05040100u);
}

// LDS layout of x: per row, per block of 128 k: [t][quarter] x 16 bytes, i.e.
// the A fragment of MFMA t for lane quarter q sits at kb*256 + t*64 + q*16.
// Four consecutive 16-byte x chunks (32 values at k = 32q ..) -> their four
// fragment dwords-quads, written at t*64 + q*16 (conflict-free: consecutive
// chunks land in consecutive 16-byte slots).
template <int BITS = 4>
__device__ __forceinline__ void store_x_chunk(char *row_block, int quarter, const u32x4 c[4])
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        u32x4 d;
        if (BITS == 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) d[j] = pick_pair(c[j], t);
        } else {
            // INT8: MFMA t takes x[8t .. 8t+7] as (0,2) (1,3) (4,6) (5,7)
            d[0] = __builtin_amdgcn_perm(c[t][1], c[t][0], 0x05040100u);
            d[1] = __builtin_amdgcn_perm(c[t][1], c[t][0], 0x07060302u);
            d[2] = __builtin_amdgcn_perm(c[t][3], c[t][2], 0x05040100u);
            d[3] = __builtin_amdgcn_perm(c[t][3], c[t][2], 0x07060302u);
        }
        *reinterpret_cast<u32x4 *>(row_block + t * 64 + quarter * 16) = d;
    }
}

// One 128-wide k block of CT tiles: B from the packed words, A from LDS,
// scale|zero from LDS; `valid` false contributes nothing.
template <int CT, bool FOLD, int BITS = 4>
__device__ __forceinline__ void process_block(f32x4 acc[CT], const f16x8 a[4], const u32x4 *w,
                                              const uint32_t sz[CT], bool valid)
{
    if (BITS == 8) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const _Float16 s = valid ? bitcast<_Float16>((uint16_t)sz[c]) : (_Float16)0.0f;
            const _Float16 zb = bitcast<_Float16>((uint16_t)(sz[c] >> 16)) + (_Float16)1024.0f;
            const f16x2 scale = {s, s}, bias = {zb, zb};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 &l = w[c * 2 + (t >> 1)];
                const uint32_t w0 = l[(2 * t) & 3], w1 = l[(2 * t + 1) & 3];
                u32x4 b;
                b[0] = (w0 & 0x00FF00FFu) | 0x64006400u;           // k = 8t + 0, 8t + 2
                b[1] = ((w0 >> 8) & 0x00FF00FFu) | 0x64006400u;    // 8t + 1, 8t + 3
                b[2] = (w1 & 0x00FF00FFu) | 0x64006400u;           // 8t + 4, 8t + 6
                b[3] = ((w1 >> 8) & 0x00FF00FFu) | 0x64006400u;    // 8t + 5, 8t + 7
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = bitcast<uint32_t>((bitcast<f16x2>(b[j]) - bias) * scale);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], bitcast<f16x8>(b), acc[c], 0, 0, 0);
            }
        }
    } else if (FOLD) {
        // X = 2^-24 * sum of this lane-row's x over the block.
        const f16x8 tiny = bitcast<f16x8>(u32x4{0x00010001u, 0x00010001u, 0x00010001u, 0x00010001u});
        f32x4 xs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], tiny, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int t = 1; t < 4; ++t) xs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], tiny, xs, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            u32x4 b0, b1, b2, b3;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t v = w[c][j];
                const uint32_t v8 = v >> 8;
                b0[j] = v & 0x000F000Fu;     // codes 0,4 as c * 2^-24
                b1[j] = v & 0x00F000F0u;     // codes 1,5 as c * 2^-20
                b2[j] = v8 & 0x000F000Fu;    // codes 2,6 as c * 2^-24
                b3[j] = v8 & 0x00F000F0u;    // codes 3,7 as c * 2^-20
            }
            const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
            f32x4 p24 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], bitcast<f16x8>(b0), zero4, 0, 0, 0);
            f32x4 p20 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], bitcast<f16x8>(b1), zero4, 0, 0, 0);
            p24 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2], bitcast<f16x8>(b2), p24, 0, 0, 0);
            p20 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[3], bitcast<f16x8>(b3), p20, 0, 0, 0);
            const float s = valid ? half_bits_to_float((uint16_t)sz[c]) * 16777216.0f : 0.0f;  // s * 2^24, exact
            const float nz = -half_bits_to_float((uint16_t)(sz[c] >> 16));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = __builtin_fmaf(p20[r], 0.0625f, p24[r]);
                acc[c][r] = __builtin_fmaf(s, __builtin_fmaf(nz, xs[r], v), acc[c][r]);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const _Float16 s = valid ? bitcast<_Float16>((uint16_t)sz[c]) : (_Float16)0.0f;
            const _Float16 zb = bitcast<_Float16>((uint16_t)(sz[c] >> 16)) + (_Float16)1024.0f;
            const f16x2 scale = {s, s}, bias = {zb, zb};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                u32x4 b;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t h = ((w[c][j] >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
                    b[j] = bitcast<uint32_t>((bitcast<f16x2>(h) - bias) * scale);
                }
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[p], bitcast<f16x8>(b), acc[c], 0, 0, 0);
            }
        }
    }
}

// Sum of the SPLIT waves' partial tiles (fixed order) and the fp16 store.
// Lane l holds rows 4*(l/16) + r (r = 0..3) of column l % 16 of each tile.
template <int SPLIT, int CT>
__device__ __forceinline__ void finish(f32x4 acc[CT], char *lds, uint16_t *y, int m, int n_out,
                                       int row0, int wave, int lane)
{
    const int col = lane & 15, quarter = lane >> 4;
    if (SPLIT > 1) {
        f32x4 *partial = reinterpret_cast<f32x4 *>(lds);       // [SPLIT][CT][64]
#pragma unroll
        for (int t = 0; t < CT; ++t) partial[(wave * CT + t) * 64 + lane] = acc[t];
        __syncthreads();
        if (wave >= CT) return;
        const int t = wave;                                     // wave t finishes tile t
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

// Per-lane weight addressing shared by both kernels: a wave-uniform base
// plus fixed 32-bit lane offsets.  Rows past n_out are clamped to a valid
// row (their outputs are never stored).
template <int CT, int BITS = 4>
struct WeightAddr {
    static constexpr int WPQ = BITS;          // packed words per lane per block (one quarter's 32 codes)
    const char *qbase;
    const char *xsafe;      // 16-byte-aligned, L2-hot target for loads past the end
    uint32_t woff[CT];
    int quarter, kblocks, last_full_quarter;

    __device__ __forceinline__ void init(const uint32_t *qweight, const uint16_t *x,
                                         const Geometry &geo, int row0, int col, int q)
    {
        qbase = reinterpret_cast<const char *>(qweight + (int64_t)row0 * geo.words_per_row);
        xsafe = reinterpret_cast<const char *>(x);
        quarter = q;
        kblocks = geo.kblocks;
        last_full_quarter = geo.last_full_quarter;
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            const int r = min(t * 16 + col, geo.n_out - 1 - row0);
            woff[t] = (uint32_t)(r * geo.words_per_row + q * WPQ) * 4u;
        }
    }
    // A block past the end, or a padding quarter of a partial last block.
    __device__ __forceinline__ bool valid(int kb) const
    {
        return kb < kblocks && !(kb == kblocks - 1 && quarter > last_full_quarter);
    }
    // Load l (0 .. BITS/4 - 1) of block kb of tile t.
    __device__ __forceinline__ u32x4 load(int kb, int t, int l = 0) const
    {
        // a padding quarter is moved back onto the last whole slice; the
        // offsets are summed as 32-bit values before meeting the base, so the
        // wrapped negative part cancels
        const int qs = (kb == kblocks - 1 && quarter > last_full_quarter) ? last_full_quarter - quarter : 0;
        const bool inside = kb < kblocks;
        const uint32_t off = inside ? woff[t] + (uint32_t)(kb * 4 * WPQ + qs * WPQ + l * 4) * 4u : 0u;
        const char *base = inside ? qbase : xsafe;
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + off));
    }
};

// Paired weight loads.  HBM serves a load shaped 16 rows x 64 bytes (the
// fragment layout above) well below its streaming rate, whole 128-byte lines
// far better.  So two loads cover a 16-row tile over 128 bytes per row (two
// INT4 blocks, or one INT8 block): load 0 reads rows 0-7, load 1 rows 8-15,
// each row as one whole 128-byte line, and a select plus a rotation by 8
// lanes within each 16-lane row (DPP row_ror:8) turn them into the
// fragments.  INT4: lane (column c, quarter q) of load 0 reads row c % 8 at
// byte 16q (c < 8) or 64 + 16q (c >= 8), load 1 row 8 + c % 8 the other way
// round, so the select gives each lane its row's bytes 16q (first block) and
// the rotated other select its bytes 64 + 16q (second block).  INT8: the
// same with bytes 32q and 32q + 16, the two 16-byte halves of one block.
template <int CT, int BITS>
struct PairAddr {
    const char *qbase;
    const char *xsafe;            // 16-byte-aligned, L2-hot target for loads past the end
    uint32_t rowoff[CT][2];       // byte offset of this lane's row, loads 0 and 1
    uint32_t laneoff[2];          // byte offset within the 128-byte run
    uint32_t last;                // last 16-byte slot of a row
    int kblocks;

    __device__ __forceinline__ void init(const uint32_t *qweight, const uint16_t *x, const Geometry &geo,
                                         int row0, int col, int q)
    {
        const uint32_t row_bytes = (uint32_t)geo.words_per_row * 4u;
        qbase = reinterpret_cast<const char *>(qweight) + (int64_t)row0 * row_bytes;
        xsafe = reinterpret_cast<const char *>(x);
        kblocks = geo.kblocks;
        last = row_bytes - 16u;
        const bool low = col < 8;
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            const int ra = min(t * 16 + (col & 7), geo.n_out - 1 - row0);
            const int rb = min(t * 16 + 8 + (col & 7), geo.n_out - 1 - row0);
            rowoff[t][0] = (uint32_t)ra * row_bytes;
            rowoff[t][1] = (uint32_t)rb * row_bytes;
        }
        const uint32_t first = BITS == 4 ? 16u * (uint32_t)q : 32u * (uint32_t)q;
        const uint32_t second = BITS == 4 ? 64u + 16u * (uint32_t)q : 32u * (uint32_t)q + 16u;
        laneoff[0] = low ? first : second;
        laneoff[1] = low ? second : first;
    }
    // Load h (0, 1) of run p (128 bytes per row: INT4 blocks 2p and 2p+1,
    // INT8 block p) of tile t.  Bytes past the end of a row repeat its last
    // 16 (they belong to padding quarters).
    __device__ __forceinline__ u32x4 load(int p, int t, int h) const
    {
        const bool inside = (BITS == 4 ? 2 * p : p) < kblocks;
        const uint32_t off = inside ? rowoff[t][h] + min((uint32_t)p * 128u + laneoff[h], last) : 0u;
        const char *base = inside ? qbase : xsafe;
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + off));
    }
};

// The fragments (INT4: of blocks 2p and 2p+1; INT8: the two halves of block
// p) from the two loads of a pair.
__device__ __forceinline__ void unpair(const u32x4 &l0, const u32x4 &l1, bool low, u32x4 &b0, u32x4 &b1)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        b0[j] = low ? l0[j] : l1[j];
        const uint32_t other = low ? l1[j] : l0[j];
        b1[j] = (uint32_t)__builtin_amdgcn_mov_dpp((int)other, 0x128, 0xF, 0xF, false);   // row_ror:8
    }
}

// ---------------------------------------------------------------------------
// Resident kernel: x and all scale|zero pairs staged once in LDS.
// ---------------------------------------------------------------------------
template <int SPLIT, int CT, int UNROLL, int DEPTH, bool FOLD, int BITS = 4, bool PAIRED = false>
__global__ __launch_bounds__(64 * SPLIT) void gemv_resident_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, Geometry geo)
{
    constexpr int THREADS = 64 * SPLIT;
    constexpr int ROWS = 16 * CT;
    constexpr int SB = SPLIT * UNROLL;             // blocks per stage
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int m = geo.m, n_out = geo.n_out, n_in = geo.n_in, gshift = geo.group_shift;
    const int kblocks = geo.kblocks, G = geo.groups_per_row;
    const int x_bytes = m * geo.x_row_bytes;
    const int part_bytes = SPLIT > 1 ? SPLIT * CT * 1024 : 0;
    char *x_lds = lds;
    uint32_t *sz_lds = reinterpret_cast<uint32_t *>(lds + max(x_bytes, part_bytes));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int quarter = lane >> 4;
    const int row0 = blockIdx.x * ROWS;

    constexpr int LPB = BITS / 4;                  // 16-byte weight loads per block per tile
    static_assert(!PAIRED || BITS == 8 || UNROLL % 2 == 0, "paired INT4 loads cover two blocks");
    WeightAddr<CT, BITS> wa;
    wa.init(qweight, x, geo, row0, col, quarter);
    PairAddr<CT, BITS> pa;
    if constexpr (PAIRED) pa.init(qweight, x, geo, row0, col, quarter);
    auto load_stage = [&](Stage<CT, UNROLL, BITS> &st, int i) {
        if constexpr (PAIRED && BITS == 4) {
            // slots 2v, 2v+1 hold the two loads of pair (i * SPLIT + wave) * UNROLL / 2 + v
#pragma unroll
            for (int v = 0; v < UNROLL / 2; ++v)
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        st.w[2 * v + h][t] = pa.load((i * SPLIT + wave) * (UNROLL / 2) + v, t, h);
        } else if constexpr (PAIRED) {
            // INT8: the two loads of a block sit where its two halves go
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int h = 0; h < 2; ++h) st.w[u][t * 2 + h] = pa.load((i * SPLIT + wave) * UNROLL + u, t, h);
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int l = 0; l < LPB; ++l)
                        st.w[u][t * LPB + l] = wa.load((i * SPLIT + wave) * UNROLL + u, t, l);
        }
    };

    // ---- staging of x (chunk c = (row, block, quarter) holds 32 values) and
    // of the scale|zero pairs of rows row0 .. row0 + ROWS.  The first batch
    // of staging loads is issued before the first DEPTH weight stages (the
    // whole ring), so the LDS stores below wait only for the staging data
    // while every ring stage stays in flight across the barrier; a wave with
    // at most DEPTH stages has all its weights requested before it.
    const int nstages = (kblocks + SB - 1) / SB;
    const int n_chunks = m * kblocks * 4;
    const int n_items = ROWS * G;
    const bool sz_vec = geo.sz_vector && row0 + ROWS <= n_out;
    const u32x4 *sv = reinterpret_cast<const u32x4 *>(scales + (int64_t)row0 * G);
    const u32x4 *zv = reinterpret_cast<const u32x4 *>(zeros + (int64_t)row0 * G);

    auto x_load = [&](int c, u32x4 v[4]) {
        c = min(c, n_chunks - 1);
        const int r = c / (kblocks * 4), rem = c % (kblocks * 4);
        const int k = min(rem * 32, n_in - 32);          // padding quarters repeat a valid slice
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (int64_t)r * n_in + k);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = src[j];
    };
    auto x_store = [&](int c, const u32x4 v[4]) {
        if (c < n_chunks) {
            const int r = c / (kblocks * 4), rem = c % (kblocks * 4);
            store_x_chunk<BITS>(x_lds + r * geo.x_row_bytes + (rem >> 2) * 256, rem & 3, v);
        }
    };
    // vector path: the rows are one contiguous, 16-byte-aligned run of both
    // arrays, 8 pairs per chunk; otherwise one pair per item
    auto sz_load = [&](int c, u32x4 &s8, u32x4 &z8) {
        if (sz_vec) {
            c = min(c, n_items / 8 - 1);
            s8 = sv[c];
            z8 = zv[c];
        } else {
            c = min(c, n_items - 1);
            const int r = c / G, g = c - r * G;
            const int64_t off = (int64_t)min(row0 + r, n_out - 1) * G + g;
            s8 = u32x4{(uint32_t)scales[off], 0u, 0u, 0u};
            z8 = u32x4{(uint32_t)zeros[off], 0u, 0u, 0u};
        }
    };
    auto sz_store = [&](int c, const u32x4 &s8, const u32x4 &z8) {
        if (sz_vec) {
            if (c < n_items / 8) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = c * 8 + i, r = e / G, g = e - r * G;
                    const uint32_t sh = (s8[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                    const uint32_t zh = (z8[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                    sz_lds[r * geo.sz_stride + g] = sh | (zh << 16);
                }
            }
        } else if (c < n_items) {
            const int r = c / G, g = c - r * G;
            sz_lds[r * geo.sz_stride + g] = s8[0] | (z8[0] << 16);
        }
    };
    const int sz_units = sz_vec ? n_items / 8 : n_items;

    u32x4 xv[4], s8, z8;
    x_load(tid, xv);
    sz_load(tid, s8, z8);
    Stage<CT, UNROLL, BITS> ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_stage(ring[d], d);
    x_store(tid, xv);
    sz_store(tid, s8, z8);
    for (int c = tid + THREADS; c < n_chunks; c += THREADS) {
        x_load(c, xv);
        x_store(c, xv);
    }
    for (int c = tid + THREADS; c < sz_units; c += THREADS) {
        sz_load(c, s8, z8);
        sz_store(c, s8, z8);
    }
    __syncthreads();

    f32x4 acc[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const char *xrow = x_lds + min(col, m - 1) * geo.x_row_bytes;
    const uint32_t *szrow = sz_lds + col * geo.sz_stride;
    auto compute = [&](const Stage<CT, UNROLL, BITS> &st, int i) {
        Stage<CT, UNROLL, BITS> up;                // PAIRED: the loads turned into block fragments
        if constexpr (PAIRED && BITS == 4) {
#pragma unroll
            for (int v = 0; v < UNROLL / 2; ++v)
#pragma unroll
                for (int t = 0; t < CT; ++t)
                    unpair(st.w[2 * v][t], st.w[2 * v + 1][t], col < 8, up.w[2 * v][t], up.w[2 * v + 1][t]);
        } else if constexpr (PAIRED) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int t = 0; t < CT; ++t)
                    unpair(st.w[u][t * 2], st.w[u][t * 2 + 1], col < 8, up.w[u][t * 2], up.w[u][t * 2 + 1]);
        }
        const Stage<CT, UNROLL, BITS> &frag = PAIRED ? up : st;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = (i * SPLIT + wave) * UNROLL + u;
            const int kbc = min(kb, kblocks - 1);
            f16x8 a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                a[t] = *reinterpret_cast<const f16x8 *>(xrow + kbc * 256 + t * 64 + quarter * 16);
            // a padding quarter of a partial last block reads the last real
            // group (its contribution is masked), never past the row
            const int qe = (kbc == kblocks - 1) ? min(quarter, geo.last_full_quarter) : quarter;
            const int g = ((kbc << 7) + (qe << 5)) >> gshift;
            uint32_t sz[CT];
#pragma unroll
            for (int t = 0; t < CT; ++t) sz[t] = szrow[t * 16 * geo.sz_stride + g];
            process_block<CT, FOLD, BITS>(acc, a, frag.w[u], sz, wa.valid(kb));
        }
    };

    // ---- stream the weights through the register ring: each slot is
    // refilled with the stage DEPTH ahead as soon as it has been consumed ----
    for (int i0 = 0; i0 < nstages; i0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int i = i0 + d;
            if (i < nstages) compute(ring[d], i);
            load_stage(ring[d], i + DEPTH);
        }
    }
    if (SPLIT > 1) __syncthreads();           // the partial sums reuse the x buffer
    finish<SPLIT, CT>(acc, lds, y, m, n_out, row0, wave, lane);
}

// ---------------------------------------------------------------------------
// Row-streaming kernel (m = 1, INT4, groups of at least 32 codes or one per
// row, n_in <= 16384).
//
// Every load instruction of a wave reads one contiguous KiB of one row (2048
// codes; lane l holds codes 32l .. 32l + 31 of the chunk), the access pattern
// HBM serves fastest, and a wave streams RW whole rows.  With one row of x
// the matrix cores would waste fifteen sixteenths of their work, so the
// products run on the VALU as v_dot2_f32_f16: masking a packed word with
// 0x000F000F leaves the codes (c_t, c_{t+4}) as the fp16 subnormals c 2^-24
// (with 0x00F000F0, four bits up: c 2^-20), exact, and the lane's x slice is
// permuted once into the matching pairs (x_t, x_{t+4}).  A lane's 32 codes
// lie in one group (groups have at least 32 codes), so its scale and
// zero-point are applied once, in fp32:
//   y += s 2^24 (A + B / 16 - z X24),
// A and B the dot products of the c 2^-24 and c 2^-20 codes, X24 = 2^-24
// times the sum of the lane's 32 x.  x, pre-permuted, and the sums X24 are
// staged once per workgroup in LDS, 80 bytes per 64-byte lane slot (the
// padding keeps the 16-byte reads of neighbouring lanes on distinct banks),
// with the workgroup's scale and zero-point rows beside them.  A row's
// partial sums are added across the wave with DPP row rotations and the
// gfx950 permlane swaps, all on the VALU.
// ---------------------------------------------------------------------------
constexpr int kRsSlot = 80;          // LDS bytes per lane slot of x (64 + padding)

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return bitcast<float>(__builtin_amdgcn_mov_dpp(bitcast<int>(v), CTRL, 0xF, 0xF, false));
}

// The sum of v over the 64 lanes, in every lane.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f32<0x128>(v);          // row_ror:8
    v += dpp_f32<0x124>(v);          // row_ror:4
    v += dpp_f32<0x4E>(v);           // quad_perm [2,3,0,1]
    v += dpp_f32<0xB1>(v);           // quad_perm [1,0,3,2]
    const auto a = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(v), bitcast<uint32_t>(v), false, false);
    v = bitcast<float>(a[0]) + bitcast<float>(a[1]);          // rows 0+1, 2+3
    const auto b = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(v), bitcast<uint32_t>(v), false, false);
    return bitcast<float>(b[0]) + bitcast<float>(b[1]);       // halves
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(bitcast<f16x2>(a), bitcast<f16x2>(b), c, false);
}

// 16 bytes at offset o of a scale or zero-point run of `bytes` bytes (even).
// A vector that straddles the end is read as halves, each wholly inside or
// wholly past the run; past it a buffer load reads 0.
__device__ __forceinline__ u32x4 meta_vec(__amdgpu_buffer_rsrc_t r, int o, int bytes)
{
    if (o + 16 <= bytes || o >= bytes) return __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, o + 4 * i, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, o + 4 * i + 2, 0, 0);
        v[i] = lo | (hi << 16);
    }
    return v;
}

template <int NC, int RW, int W>
__global__ __launch_bounds__(64 * W) void gemv_rowstream_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, Geometry geo)
{
    constexpr int R = W * RW;             // rows per workgroup
    constexpr int L = RW * NC;            // loads per wave
    constexpr int THREADS = 64 * W;
    constexpr int XP = NC * 256;          // 16-byte pieces of x (past n_in they read as 0)
    constexpr int XI = (XP + THREADS - 1) / THREADS;
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int n_out = geo.n_out, n_in = geo.n_in, G = geo.groups_per_row, gshift = geo.group_shift;
    char *x_lds = lds;                                                    // [NC * 64][kRsSlot]
    float *xs_lds = reinterpret_cast<float *>(lds + NC * 64 * kRsSlot);   // [NC * 64]
    uint16_t *s_lds = reinterpret_cast<uint16_t *>(xs_lds + NC * 64);     // [R][G]
    uint16_t *z_lds = s_lds + ((R * G + 7) & ~7);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wg_row0 = blockIdx.x * R, row0 = wg_row0 + wave * RW;
    const int row_bytes = n_in / 2;

    // staging loads: this workgroup's scale and zero-point rows (bytes past
    // the last row read as 0) and x, issued before the weights
    const int meta = min(R, n_out - wg_row0) * G * 2;
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(scales + (int64_t)wg_row0 * G), (short)0, meta, kBufferFlags);
    const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(zeros + (int64_t)wg_row0 * G), (short)0, meta, kBufferFlags);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x), (short)0, n_in * 2, kBufferFlags);
    const int n_vec = (R * G * 2 + 15) >> 4;
    const u32x4 sv = meta_vec(sr, tid * 16, meta);
    const u32x4 zv = meta_vec(zr, tid * 16, meta);
    u32x4 xv[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, (tid + i * THREADS) * 16, 0, 0);

    // the weights: load i is chunk i % NC of row row0 + i / NC.  Rows past
    // n_out read the last row, and lanes past the end of a row its last 16
    // bytes (their x is 0); neither is ever stored.
    const char *wbase = reinterpret_cast<const char *>(qweight);
    u32x4 ring[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int r = min(row0 + i / NC, n_out - 1);
        const uint32_t off = min((uint32_t)(1024 * (i % NC) + 16 * lane), (uint32_t)row_bytes - 16u);
        ring[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wbase + (int64_t)r * row_bytes + off));
    }

    if (tid < n_vec) {
        reinterpret_cast<u32x4 *>(s_lds)[tid] = sv;
        reinterpret_cast<u32x4 *>(z_lds)[tid] = zv;
    }
    for (int v = tid + THREADS; v < n_vec; v += THREADS) {
        reinterpret_cast<u32x4 *>(s_lds)[v] = meta_vec(sr, v * 16, meta);
        reinterpret_cast<u32x4 *>(z_lds)[v] = meta_vec(zr, v * 16, meta);
    }
    // piece p holds x[8p .. 8p + 7]; slot p / 4 is (chunk, lane); the four
    // threads of a slot are neighbouring lanes, so a quad sum gives X24
    const uint32_t ones = 0x3C003C00u;
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int p = tid + i * THREADS;
        const u32x4 pp = bitcast<u32x4>(pair_order(xv[i]));
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) t = dot2_f16(pp[e], ones, t);
        t += dpp_f32<0xB1>(t);
        t += dpp_f32<0x4E>(t);
        if (p < XP) {
            *reinterpret_cast<u32x4 *>(x_lds + (p >> 2) * kRsSlot + (p & 3) * 16) = pp;
            if ((p & 3) == 0) xs_lds[p >> 2] = t * 5.9604644775390625e-08f;     // 2^-24
        }
    }
    barrier_keep_vmem();

    u32x4 xp[NC][4];
    float x24[NC];
#pragma unroll
    for (int h = 0; h < NC; ++h) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xp[h][j] = *reinterpret_cast<const u32x4 *>(x_lds + (h * 64 + lane) * kRsSlot + 16 * j);
        x24[h] = xs_lds[h * 64 + lane];
    }
    float acc[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int r = i / NC, h = i % NC;
        const u32x4 w = ring[i];
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t v = w[j], v8 = v >> 8;
            a = dot2_f16(v & 0x000F000Fu, xp[h][j][0], a);      // codes 8j, 8j+4 as c 2^-24
            b = dot2_f16(v & 0x00F000F0u, xp[h][j][1], b);      // codes 8j+1, 8j+5 as c 2^-20
            a = dot2_f16(v8 & 0x000F000Fu, xp[h][j][2], a);     // 8j+2, 8j+6
            b = dot2_f16(v8 & 0x00F000F0u, xp[h][j][3], b);     // 8j+3, 8j+7
        }
        const int e = (wave * RW + r) * G + min((2048 * h + 32 * lane) >> gshift, G - 1);
        const float s = half_bits_to_float(s_lds[e]) * 16777216.0f;     // s 2^24, exact
        const float z = half_bits_to_float(z_lds[e]);
        acc[r] = __builtin_fmaf(s, __builtin_fmaf(-z, x24[h], __builtin_fmaf(b, 0.0625f, a)), acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const float t = wave_sum(acc[r]);
        if (lane == r && row0 + r < n_out) y[row0 + r] = bitcast<uint16_t>((_Float16)t);
    }
}

// Row streaming for INT8 weights (m = 1, any group: 32..256 or one per
// row): a load instruction of a wave reads one contiguous KiB of its row
// (lane l: codes 16l .. 16l + 15 of a 1024-code chunk); masking a word with
// 0x00FF00FF leaves the byte codes (c0, c2) as the fp16 subnormals c 2^-24,
// the word shifted by 8 gives (c1, c3), and x is pre-permuted into the
// matching pairs.  A lane's 16 codes lie in one group (groups have at least
// 32 codes), so its scale and zero-point are applied once per chunk:
// y += s 2^24 (A - z X24), the cancellation between A and z X24 confined to
// 16 terms.  Each chunk's x is read from LDS where it is used (48-byte lane
// slots: 32 of x, padding against bank conflicts).
constexpr int kRs8Slot = 48;

template <int NC, int W>
__global__ __launch_bounds__(64 * W) void gemv_rowstream8_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, Geometry geo)
{
    constexpr int THREADS = 64 * W;
    constexpr int XP = NC * 128;          // 16-byte pieces of x (past n_in they read as 0)
    constexpr int XI = (XP + THREADS - 1) / THREADS;
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int n_out = geo.n_out, n_in = geo.n_in, G = geo.groups_per_row, gshift = geo.group_shift;
    char *x_lds = lds;                                                    // [NC * 64][kRs8Slot]
    float *xs_lds = reinterpret_cast<float *>(lds + NC * 64 * kRs8Slot);  // [NC * 64]
    uint16_t *s_lds = reinterpret_cast<uint16_t *>(xs_lds + NC * 64);     // [W][G]
    uint16_t *z_lds = s_lds + ((W * G + 7) & ~7);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wg_row0 = blockIdx.x * W, row = wg_row0 + wave;
    const int row_bytes = n_in;

    const int meta = min(W, n_out - wg_row0) * G * 2;
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(scales + (int64_t)wg_row0 * G), (short)0, meta, kBufferFlags);
    const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(zeros + (int64_t)wg_row0 * G), (short)0, meta, kBufferFlags);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x), (short)0, n_in * 2, kBufferFlags);
    const int n_vec = (W * G * 2 + 15) >> 4;
    const u32x4 sv = meta_vec(sr, tid * 16, meta);
    const u32x4 zv = meta_vec(zr, tid * 16, meta);
    u32x4 xv[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, (tid + i * THREADS) * 16, 0, 0);

    // the row's chunks: rows past n_out read the last row, lanes past the end
    // of a row its last 16 bytes (their x is 0); neither is stored
    const char *wrow = reinterpret_cast<const char *>(qweight) + (int64_t)min(row, n_out - 1) * row_bytes;
    u32x4 ring[NC];
#pragma unroll
    for (int h = 0; h < NC; ++h) {
        const uint32_t off = min((uint32_t)(1024 * h + 16 * lane), (uint32_t)row_bytes - 16u);
        ring[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrow + off));
    }

    if (tid < n_vec) {
        reinterpret_cast<u32x4 *>(s_lds)[tid] = sv;
        reinterpret_cast<u32x4 *>(z_lds)[tid] = zv;
    }
    for (int v = tid + THREADS; v < n_vec; v += THREADS) {
        reinterpret_cast<u32x4 *>(s_lds)[v] = meta_vec(sr, v * 16, meta);
        reinterpret_cast<u32x4 *>(z_lds)[v] = meta_vec(zr, v * 16, meta);
    }
    // piece p holds x[8p .. 8p + 7]; slot p / 2 is (chunk, lane), its two
    // pieces in neighbouring lanes, whose pair sum gives X24
    const uint32_t ones = 0x3C003C00u;
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int p = tid + i * THREADS;
        u32x4 pp;
        pp[0] = __builtin_amdgcn_perm(xv[i][1], xv[i][0], 0x05040100u);      // (x0, x2)
        pp[1] = __builtin_amdgcn_perm(xv[i][1], xv[i][0], 0x07060302u);      // (x1, x3)
        pp[2] = __builtin_amdgcn_perm(xv[i][3], xv[i][2], 0x05040100u);      // (x4, x6)
        pp[3] = __builtin_amdgcn_perm(xv[i][3], xv[i][2], 0x07060302u);      // (x5, x7)
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) t = dot2_f16(pp[e], ones, t);
        t += dpp_f32<0xB1>(t);
        if (p < XP) {
            *reinterpret_cast<u32x4 *>(x_lds + (p >> 1) * kRs8Slot + (p & 1) * 16) = pp;
            if ((p & 1) == 0) xs_lds[p >> 1] = t * 5.9604644775390625e-08f;   // 2^-24
        }
    }
    barrier_keep_vmem();

    float acc = 0.f;
#pragma unroll
    for (int h = 0; h < NC; ++h) {
        const u32x4 w = ring[h];
        const u32x4 xa = *reinterpret_cast<const u32x4 *>(x_lds + (h * 64 + lane) * kRs8Slot);
        const u32x4 xb = *reinterpret_cast<const u32x4 *>(x_lds + (h * 64 + lane) * kRs8Slot + 16);
        const float x24 = xs_lds[h * 64 + lane];
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 &xp = j < 2 ? xa : xb;
            const uint32_t v = w[j];
            a = dot2_f16(v & 0x00FF00FFu, xp[(j & 1) * 2], a);             // codes 4j, 4j+2
            a = dot2_f16((v >> 8) & 0x00FF00FFu, xp[(j & 1) * 2 + 1], a);  // 4j+1, 4j+3
        }
        const int e = wave * G + min((1024 * h + 16 * lane) >> gshift, G - 1);
        const float s = half_bits_to_float(s_lds[e]) * 16777216.0f;      // s 2^24, exact
        const float z = half_bits_to_float(z_lds[e]);
        acc = __builtin_fmaf(s, __builtin_fmaf(-z, x24, a), acc);
    }
    const float t = wave_sum(acc);
    if (lane == 0 && row < n_out) y[row] = bitcast<uint16_t>((_Float16)t);
}

// ---------------------------------------------------------------------------
// Persistent kernel (INT4, 2 <= m <= 8): a workgroup stages x once and then
// walks the tile groups blockIdx.x, blockIdx.x + gridDim.x, ...  The weight
// ring runs on across group boundaries (the last stages of a group load the
// first stages of the next), so HBM stays busy while a group's partial sums
// are reduced and stored and the next group's scale|zero pairs are staged.
// The pairs and the partial sums share one LDS region; only quarters 0 and 1
// of the MFMA output (rows 0..7) are kept, since m <= 8.
// ---------------------------------------------------------------------------
template <int CT, bool PAIRED>
struct GroupLoads {
    struct Group {
        const char *base;            // the group's first row
        uint32_t off[CT][2];         // byte offset of this lane's rows (clamped to the matrix)
        bool live;                   // false: past the last group, loads go to x
    };
    const char *qweight, *xsafe;
    uint32_t row_bytes, last;        // last: final 16-byte slot of a row
    uint32_t lanepart[2];            // this lane's bytes within a block (paired: a 128-byte run)
    int lrow[CT][2];                 // this lane's rows within a group, unclamped
    int kblocks, last_full_quarter, quarter;

    __device__ __forceinline__ void init(const uint32_t *qw, const uint16_t *x, const Geometry &geo, int col, int q)
    {
        qweight = reinterpret_cast<const char *>(qw);
        xsafe = reinterpret_cast<const char *>(x);
        row_bytes = (uint32_t)geo.words_per_row * 4u;
        last = row_bytes - 16u;
        kblocks = geo.kblocks;
        last_full_quarter = geo.last_full_quarter;
        quarter = q;
        const bool low = col < 8;
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            lrow[t][0] = t * 16 + (PAIRED ? (col & 7) : col);
            lrow[t][1] = t * 16 + 8 + (col & 7);
        }
        if (PAIRED) {
            lanepart[0] = low ? 16u * (uint32_t)q : 64u + 16u * (uint32_t)q;
            lanepart[1] = low ? 64u + 16u * (uint32_t)q : 16u * (uint32_t)q;
        } else {
            lanepart[0] = lanepart[1] = 16u * (uint32_t)q;
        }
    }
    __device__ __forceinline__ void set(Group &g, int row0, int n_out, bool live) const
    {
        g.live = live;
        g.base = qweight + (int64_t)(live ? row0 : 0) * row_bytes;
        const int lim = live ? n_out - 1 - row0 : 0;
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) g.off[t][h] = (uint32_t)min(lrow[t][h], lim) * row_bytes;
    }
    // Load h of unit u of tile t: paired, u is a 128-byte run (blocks 2u and
    // 2u+1); otherwise u is a 128-code block and h is 0.  Past the end (or a
    // dead group) the load reads x instead.
    __device__ __forceinline__ u32x4 load(const char *base, const uint32_t (&off)[CT][2], bool live, int u, int t,
                                          int h) const
    {
        uint32_t o;
        bool inside;
        if (PAIRED) {
            inside = live && 2 * u < kblocks;
            o = off[t][h] + min((uint32_t)u * 128u + lanepart[h], last);
        } else {
            // a padding quarter of a partial last block reads the last whole slice
            const int qs = (u == kblocks - 1 && quarter > last_full_quarter) ? last_full_quarter - quarter : 0;
            inside = live && u < kblocks;
            o = off[t][0] + lanepart[0] + (uint32_t)(u * 64 + qs * 16);
        }
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>((inside ? base : xsafe) + (inside ? o : 0u)));
    }
};

template <int SPLIT, int CT, int UNROLL, int DEPTH, bool FOLD, bool PAIRED>
__global__ __launch_bounds__(64 * SPLIT) void gemv_persistent_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, Geometry geo)
{
    constexpr int THREADS = 64 * SPLIT;
    constexpr int ROWS = 16 * CT;
    constexpr int SB = SPLIT * UNROLL;
    static_assert(!PAIRED || UNROLL % 2 == 0, "paired loads cover two blocks");
    static_assert(SPLIT >= CT || SPLIT == 1, "the LDS reduction assigns one wave per tile");
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int m = geo.m, n_out = geo.n_out, n_in = geo.n_in, gshift = geo.group_shift;
    const int kblocks = geo.kblocks, G = geo.groups_per_row, ngroups = geo.groups;
    const int x_bytes = m * geo.x_row_bytes;
    char *x_lds = lds;
    uint32_t *sz_lds = reinterpret_cast<uint32_t *>(lds + x_bytes);
    f32x4 *part = reinterpret_cast<f32x4 *>(lds + x_bytes);     // [SPLIT][CT][32], after the pairs are read

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int quarter = lane >> 4;
    const int nstages = (kblocks + SB - 1) / SB;

    using GL = GroupLoads<CT, PAIRED>;
    GL gl;
    gl.init(qweight, x, geo, col, quarter);
    typename GL::Group cur, nxt;
    int tg = blockIdx.x;
    int ntg = tg + (int)gridDim.x;
    gl.set(cur, tg * ROWS, n_out, true);
    gl.set(nxt, ntg * ROWS, n_out, ntg < ngroups);

    // Stage i of the current group; i >= nstages is stage i - nstages of the next.
    auto load_stage = [&](Stage<CT, UNROLL, 4> &st, int i) {
        const bool in_cur = i < nstages;
        const int ii = in_cur ? i : i - nstages;
        const char *base = in_cur ? cur.base : nxt.base;
        const bool live = in_cur ? cur.live : nxt.live;
        uint32_t off[CT][2];
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) off[t][h] = in_cur ? cur.off[t][h] : nxt.off[t][h];
        if constexpr (PAIRED) {
#pragma unroll
            for (int v = 0; v < UNROLL / 2; ++v)
#pragma unroll
                for (int t = 0; t < CT; ++t)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        st.w[2 * v + h][t] = gl.load(base, off, live, (ii * SPLIT + wave) * (UNROLL / 2) + v, t, h);
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int t = 0; t < CT; ++t) st.w[u][t] = gl.load(base, off, live, (ii * SPLIT + wave) * UNROLL + u, t, 0);
        }
    };

    // ---- x, staged once (chunk c = (row, block, quarter) holds 32 values)
    const int n_chunks = m * kblocks * 4;
    auto x_load = [&](int c, u32x4 v[4]) {
        c = min(c, n_chunks - 1);
        const int r = c / (kblocks * 4), rem = c % (kblocks * 4);
        const int k = min(rem * 32, n_in - 32);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (int64_t)r * n_in + k);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = src[j];
    };
    auto x_store = [&](int c, const u32x4 v[4]) {
        if (c < n_chunks) {
            const int r = c / (kblocks * 4), rem = c % (kblocks * 4);
            store_x_chunk<4>(x_lds + r * geo.x_row_bytes + (rem >> 2) * 256, rem & 3, v);
        }
    };
    // ---- scale|zero pairs of the group starting at row `row0`
    const int n_items = ROWS * G;
    auto sz_vec = [&](int row0) { return geo.sz_vector && row0 + ROWS <= n_out; };
    auto sz_units = [&](int row0) { return sz_vec(row0) ? n_items / 8 : n_items; };
    auto sz_load = [&](int row0, int c, u32x4 &s8, u32x4 &z8) {
        if (sz_vec(row0)) {
            c = min(c, n_items / 8 - 1);
            s8 = reinterpret_cast<const u32x4 *>(scales + (int64_t)row0 * G)[c];
            z8 = reinterpret_cast<const u32x4 *>(zeros + (int64_t)row0 * G)[c];
        } else {
            c = min(c, n_items - 1);
            const int r = c / G, g = c - r * G;
            const int64_t off = (int64_t)min(row0 + r, n_out - 1) * G + g;
            s8 = u32x4{(uint32_t)scales[off], 0u, 0u, 0u};
            z8 = u32x4{(uint32_t)zeros[off], 0u, 0u, 0u};
        }
    };
    auto sz_store = [&](int row0, int c, const u32x4 &s8, const u32x4 &z8) {
        if (sz_vec(row0)) {
            if (c < n_items / 8) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = c * 8 + i, r = e / G, g = e - r * G;
                    const uint32_t sh = (s8[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                    const uint32_t zh = (z8[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                    sz_lds[r * geo.sz_stride + g] = sh | (zh << 16);
                }
            }
        } else if (c < n_items) {
            const int r = c / G, g = c - r * G;
            sz_lds[r * geo.sz_stride + g] = s8[0] | (z8[0] << 16);
        }
    };

    int row0 = tg * ROWS;
    u32x4 xv[4], s8, z8;
    x_load(tid, xv);
    sz_load(row0, tid, s8, z8);
    Stage<CT, UNROLL, 4> ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_stage(ring[d], d);
    x_store(tid, xv);
    sz_store(row0, tid, s8, z8);
    for (int c = tid + THREADS; c < n_chunks; c += THREADS) {
        x_load(c, xv);
        x_store(c, xv);
    }
    for (int c = tid + THREADS; c < sz_units(row0); c += THREADS) {
        sz_load(row0, c, s8, z8);
        sz_store(row0, c, s8, z8);
    }
    __syncthreads();

    const char *xrow = x_lds + min(col, m - 1) * geo.x_row_bytes;
    const uint32_t *szrow = sz_lds + col * geo.sz_stride;
    for (;;) {
        // the next group's first batch of scale|zero pairs is requested
        // before this group's weights, so waiting for it at the group
        // boundary leaves the ring's prefetched stages in flight
        const bool has_next = ntg < ngroups;
        const int nrow0 = ntg * ROWS;
        if (has_next) sz_load(nrow0, tid, s8, z8);
        f32x4 acc[CT];
#pragma unroll
        for (int t = 0; t < CT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](const Stage<CT, UNROLL, 4> &st, int i) {
            Stage<CT, UNROLL, 4> up;
            if constexpr (PAIRED) {
#pragma unroll
                for (int v = 0; v < UNROLL / 2; ++v)
#pragma unroll
                    for (int t = 0; t < CT; ++t)
                        unpair(st.w[2 * v][t], st.w[2 * v + 1][t], col < 8, up.w[2 * v][t], up.w[2 * v + 1][t]);
            }
            const Stage<CT, UNROLL, 4> &frag = PAIRED ? up : st;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int kb = (i * SPLIT + wave) * UNROLL + u;
                const int kbc = min(kb, kblocks - 1);
                f16x8 a[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    a[t] = *reinterpret_cast<const f16x8 *>(xrow + kbc * 256 + t * 64 + quarter * 16);
                const int qe = (kbc == kblocks - 1) ? min(quarter, geo.last_full_quarter) : quarter;
                const int g = ((kbc << 7) + (qe << 5)) >> gshift;
                uint32_t sz[CT];
#pragma unroll
                for (int t = 0; t < CT; ++t) sz[t] = szrow[t * 16 * geo.sz_stride + g];
                const bool valid = kb < kblocks && !(kb == kblocks - 1 && quarter > geo.last_full_quarter);
                process_block<CT, FOLD, 4>(acc, a, frag.w[u], sz, valid);
            }
        };
        for (int i0 = 0; i0 < nstages; i0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int i = i0 + d;
                if (i < nstages) compute(ring[d], i);
                load_stage(ring[d], i + DEPTH);
            }
        }
        // nstages is a multiple of DEPTH (the planner checks it), so slot d
        // now holds stage d of the next group
        barrier_keep_vmem();                              // every wave is done with the pairs
        const int col_n = row0 + col;
        if (SPLIT > 1) {
            if (lane < 32) {
#pragma unroll
                for (int t = 0; t < CT; ++t) part[(wave * CT + t) * 32 + lane] = acc[t];
            }
            barrier_keep_vmem();
            if (wave < CT && lane < 32) {
                const int t = wave;
                f32x4 sum = part[t * 32 + lane];
#pragma unroll
                for (int w = 1; w < SPLIT; ++w) sum += part[(w * CT + t) * 32 + lane];
                const int n = col_n + t * 16;
                if (n < n_out) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 4 * quarter + r;
                        if (row < m) y[(int64_t)row * n_out + n] = bitcast<uint16_t>((_Float16)sum[r]);
                    }
                }
            }
        } else if (lane < 32) {
#pragma unroll
            for (int t = 0; t < CT; ++t) {
                const int n = col_n + t * 16;
                if (n >= n_out) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * quarter + r;
                    if (row < m) y[(int64_t)row * n_out + n] = bitcast<uint16_t>((_Float16)acc[t][r]);
                }
            }
        }
        if (!has_next) break;
        barrier_keep_vmem();                              // the partial sums have been read
        sz_store(nrow0, tid, s8, z8);
        for (int c = tid + THREADS; c < sz_units(nrow0); c += THREADS) {
            sz_load(nrow0, c, s8, z8);
            sz_store(nrow0, c, s8, z8);
        }
        barrier_keep_vmem();
        tg = ntg;
        row0 = nrow0;
        ntg = tg + (int)gridDim.x;
        cur = nxt;
        gl.set(nxt, ntg * ROWS, n_out, ntg < ngroups);
    }
}

// ---------------------------------------------------------------------------
// Windowed kernel: x and scale|zero pairs staged one window ahead.
// ---------------------------------------------------------------------------
template <int XC, int SC>
struct Coop {
    u32x4 x[XC][4];
    uint16_t s[SC], z[SC];
};

template <int SPLIT, int CT, int UNROLL, bool FOLD, int MMAX, int BITS = 4>
__global__ __launch_bounds__(64 * SPLIT) void gemv_window_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, Geometry geo)
{
    constexpr int THREADS = 64 * SPLIT;
    constexpr int WB = SPLIT * UNROLL;          // k blocks per window
    constexpr int ROWS = 16 * CT;
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int m = geo.m, n_out = geo.n_out, n_in = geo.n_in, gshift = geo.group_shift;
    const int kblocks = geo.kblocks;
    const int groups_win = max(1, (WB * 128) >> gshift);
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

    constexpr int LPB = BITS / 4;
    WeightAddr<CT, BITS> wa;
    wa.init(qweight, x, geo, row0, col, quarter);
    auto load_weights = [&](Stage<CT, UNROLL, BITS> &st, int win) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int t = 0; t < CT; ++t)
#pragma unroll
                for (int l = 0; l < LPB; ++l) st.w[u][t * LPB + l] = wa.load(win * WB + wave * UNROLL + u, t, l);
    };

    constexpr int MAX_XCHUNKS = MMAX * WB * 4;             // m <= MMAX rows
    constexpr int XC = (MAX_XCHUNKS + THREADS - 1) / THREADS;
    constexpr int MAX_SITEMS = ROWS * WB * 4;              // group_size >= 32
    constexpr int SC = (MAX_SITEMS + THREADS - 1) / THREADS;
    const int n_xchunks = m * WB * 4;
    const int n_sitems = ROWS * groups_win;
    auto coop_load = [&](Coop<XC, SC> &c, int win) {
        // windows past the end re-read the last one (small, cache-resident)
        const int wv = min(win, nwin - 1);
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int cc = min(tid + i * THREADS, n_xchunks - 1);
            const int r = cc / (WB * 4), rem = cc % (WB * 4);
            const int kb = min(wv * WB + rem / 4, kblocks - 1);
            const int k = min((kb << 7) + ((rem & 3) << 5), n_in - 32);
            const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (int64_t)r * n_in + k);
#pragma unroll
            for (int j = 0; j < 4; ++j) c.x[i][j] = src[j];
        }
#pragma unroll
        for (int i = 0; i < SC; ++i) {
            const int it = min(tid + i * THREADS, n_sitems - 1);
            const int r = min(row0 + it / groups_win, n_out - 1);
            const int gidx = min(wv * groups_win + it % groups_win, geo.groups_per_row - 1);
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
                store_x_chunk<BITS>(x_lds + buf * x_buf_bytes + r * geo.x_row_bytes + (rem >> 2) * 256, rem & 3,
                                    c.x[i]);
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
    const int xr = min(col, m - 1);
    auto compute = [&](const Stage<CT, UNROLL, BITS> &st, int win, int buf) {
        const char *xb = x_lds + buf * x_buf_bytes + xr * geo.x_row_bytes;
        const uint32_t *szb = reinterpret_cast<const uint32_t *>(sz_lds + buf * sz_buf_bytes) + col * geo.sz_stride;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kbl = wave * UNROLL + u;             // block within the window
            f16x8 a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                a[t] = *reinterpret_cast<const f16x8 *>(xb + kbl * 256 + t * 64 + quarter * 16);
            const int gw = ((kbl << 7) + (quarter << 5)) >> gshift;
            uint32_t sz[CT];
#pragma unroll
            for (int t = 0; t < CT; ++t) sz[t] = szb[t * 16 * geo.sz_stride + gw];
            process_block<CT, FOLD, BITS>(acc, a, st.w[u], sz, wa.valid(win * WB + kbl));
        }
    };

    // Two register stages, two LDS buffers; the body is unrolled by two and
    // its loads are unconditional (past the end they are redirected), so the
    // compiler waits only for the older stage.
    Stage<CT, UNROLL, BITS> s0, s1;
    Coop<XC, SC> cp;
    coop_load(cp, 0);
    load_weights(s0, 0);
    coop_store(cp, 0);
    __syncthreads();
    for (int win = 0; win < nwin; win += 2) {
        coop_load(cp, win + 1);
        load_weights(s1, win + 1);
        compute(s0, win, 0);
        coop_store(cp, 1);
        __syncthreads();
        if (win + 1 >= nwin) break;
        coop_load(cp, win + 2);
        load_weights(s0, win + 2);
        compute(s1, win + 1, 1);
        coop_store(cp, 0);
        __syncthreads();
    }
    finish<SPLIT, CT>(acc, lds, y, m, n_out, row0, wave, lane);
}

// ---------------------------------------------------------------------------
// Launch planning.
// ---------------------------------------------------------------------------
constexpr size_t kMaxLds = 160 * 1024;     // per workgroup on gfx950

Geometry make_geometry(int m, int n_out, int n_in, int group_shift, int bits)
{
    Geometry g;
    g.m = m;
    g.n_out = n_out;
    g.n_in = n_in;
    g.group_shift = group_shift;
    g.words_per_row = n_in * bits / 32;
    g.groups_per_row = group_shift >= 31 ? 1 : n_in >> group_shift;   // 31: one group per row
    g.kblocks = (n_in + 127) >> 7;
    g.last_full_quarter = ((n_in - ((g.kblocks - 1) << 7)) >> 5) - 1;
    g.sz_stride = 0;
    g.x_row_bytes = 0;
    g.sz_vector = 0;
    g.groups = 0;
    return g;
}

// Kernel names in the form profilers print them, for the configuration query.
template <int SPLIT, int CT, int UNROLL, int DEPTH, bool FOLD, int BITS, bool PAIRED>
const char *resident_name()
{
    static const std::string s = "gemv_resident_kernel<" + std::to_string(SPLIT) + ", " + std::to_string(CT) +
                                 ", " + std::to_string(UNROLL) + ", " + std::to_string(DEPTH) + ", " +
                                 (FOLD ? "true" : "false") + ", " + std::to_string(BITS) + ", " +
                                 (PAIRED ? "true" : "false") + ">";
    return s.c_str();
}

template <int SPLIT, int CT, int UNROLL, bool FOLD, int MMAX, int BITS>
const char *window_name()
{
    static const std::string s = "gemv_window_kernel<" + std::to_string(SPLIT) + ", " + std::to_string(CT) + ", " +
                                 std::to_string(UNROLL) + ", " + (FOLD ? "true" : "false") + ", " +
                                 std::to_string(MMAX) + ", " + std::to_string(BITS) + ">";
    return s.c_str();
}

template <typename K>
hipError_t allow_full_lds(K kernel)
{
    // once per kernel instantiation (thread-safe static initialization)
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                                    (int)kMaxLds);
    return e;
}

template <int SPLIT, int CT, int UNROLL, int DEPTH, bool FOLD, int BITS = 4, bool PAIRED = false>
bool plan_resident(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                   const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                   uint16_t *y, hipStream_t stream, const char **query, hipError_t *err)
{
    static_assert(SPLIT >= CT || SPLIT == 1, "the LDS reduction assigns one wave per tile");
    Geometry g = make_geometry(m, n_out, n_in, group_shift, BITS);
    g.sz_stride = g.groups_per_row | 1;
    g.x_row_bytes = g.kblocks * 256 + 16;
    g.sz_vector = ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(zeros)) & 15) == 0 &&
                  (16 * CT * g.groups_per_row) % 8 == 0;
    const size_t x_bytes = (size_t)m * g.x_row_bytes;
    const size_t part = SPLIT > 1 ? (size_t)SPLIT * CT * 1024 : 0;
    const size_t lds = (x_bytes > part ? x_bytes : part) + (size_t)16 * CT * g.sz_stride * 4;
    if (lds > kMaxLds) return false;
    *err = hipSuccess;
    if (query) {
        *query = resident_name<SPLIT, CT, UNROLL, DEPTH, FOLD, BITS, PAIRED>();
        return true;
    }
    auto kernel = gemv_resident_kernel<SPLIT, CT, UNROLL, DEPTH, FOLD, BITS, PAIRED>;
    if (lds > 64 * 1024) {
        const hipError_t e = allow_full_lds(kernel);
        if (e != hipSuccess) {
            *err = e;
            return true;
        }
    }
    const int tiles = (n_out + 15) / 16;
    const dim3 grid((unsigned)((tiles + CT - 1) / CT)), block(64 * SPLIT);
    kernel<<<grid, block, lds, stream>>>(x, qweight, scales, zeros, y, g);
    *err = hipGetLastError();
    return true;
}

template <int NC, int RW, int W>
bool plan_rowstream(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                    const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                    uint16_t *y, hipStream_t stream, const char **query, hipError_t *err)
{
    static_assert(RW == 1 || RW == 2 || RW == 4 || RW == 8, "one storing lane per row");
    // m = 1, groups of at least 32 codes (or one per row), NC chunks of 2048
    // codes per row, and scale and zero-point arrays the staging reads as
    // 4-byte words
    if (m != 1 || group_shift < 5 || (n_in & 31) != 0 || (n_in + 2047) / 2048 != NC) return false;
    if (((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(zeros)) & 3) != 0) return false;
    Geometry g = make_geometry(m, n_out, n_in, group_shift, 4);
    constexpr int R = W * RW;
    const size_t lds = (size_t)NC * 64 * (kRsSlot + 4) + 2 * (size_t)((R * g.groups_per_row + 7) & ~7) * 2;
    if (lds > kMaxLds) return false;
    *err = hipSuccess;
    if (query) {
        static const std::string name = "gemv_rowstream_kernel<" + std::to_string(NC) + ", " + std::to_string(RW) +
                                        ", " + std::to_string(W) + ">";
        *query = name.c_str();
        return true;
    }
    auto kernel = gemv_rowstream_kernel<NC, RW, W>;
    if (lds > 64 * 1024) {
        const hipError_t e = allow_full_lds(kernel);
        if (e != hipSuccess) {
            *err = e;
            return true;
        }
    }
    kernel<<<dim3((unsigned)((n_out + R - 1) / R)), dim3(64 * W), lds, stream>>>(x, qweight, scales, zeros, y, g);
    *err = hipGetLastError();
    return true;
}

template <int NC, int W>
bool plan_rowstream8(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                     const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                     uint16_t *y, hipStream_t stream, const char **query, hipError_t *err)
{
    // m = 1, groups of at least 32 codes (or one per row), NC chunks of 1024
    // codes per row, and scale and zero-point arrays the staging reads as
    // 4-byte words
    if (m != 1 || group_shift < 5 || (n_in & 31) != 0 || (n_in + 1023) / 1024 != NC) return false;
    if (((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(zeros)) & 3) != 0) return false;
    Geometry g = make_geometry(m, n_out, n_in, group_shift, 8);
    const size_t lds = (size_t)NC * 64 * (kRs8Slot + 4) + 2 * (size_t)((W * g.groups_per_row + 7) & ~7) * 2;
    if (lds > kMaxLds) return false;
    *err = hipSuccess;
    if (query) {
        static const std::string name = "gemv_rowstream8_kernel<" + std::to_string(NC) + ", " + std::to_string(W) + ">";
        *query = name.c_str();
        return true;
    }
    auto kernel = gemv_rowstream8_kernel<NC, W>;
    if (lds > 64 * 1024) {
        const hipError_t e = allow_full_lds(kernel);
        if (e != hipSuccess) {
            *err = e;
            return true;
        }
    }
    kernel<<<dim3((unsigned)((n_out + W - 1) / W)), dim3(64 * W), lds, stream>>>(x, qweight, scales, zeros, y, g);
    *err = hipGetLastError();
    return true;
}

template <int SPLIT, int CT, int UNROLL, int DEPTH, bool FOLD, bool PAIRED>
const char *persistent_name()
{
    static const std::string s = "gemv_persistent_kernel<" + std::to_string(SPLIT) + ", " + std::to_string(CT) +
                                 ", " + std::to_string(UNROLL) + ", " + std::to_string(DEPTH) + ", " +
                                 (FOLD ? "true" : "false") + ", " + (PAIRED ? "true" : "false") + ">";
    return s.c_str();
}

// Compute units of the current device (looked up once per device).
hipError_t device_cus(int *cus)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    *cus = v;
    return hipSuccess;
}

template <int SPLIT, int CT, int UNROLL, int DEPTH, bool FOLD, int BITS = 4, bool PAIRED = false>
bool plan_persistent(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                     const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                     uint16_t *y, hipStream_t stream, const char **query, hipError_t *err)
{
    static_assert(BITS == 4, "INT4 only");
    if (m > 8) return false;
    Geometry g = make_geometry(m, n_out, n_in, group_shift, BITS);
    constexpr int SB = SPLIT * UNROLL;
    const int nstages = (g.kblocks + SB - 1) / SB;
    if (nstages % DEPTH != 0) return false;
    g.sz_stride = g.groups_per_row | 1;
    g.x_row_bytes = g.kblocks * 256 + 16;
    g.sz_vector = ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(zeros)) & 15) == 0 &&
                  (16 * CT * g.groups_per_row) % 8 == 0;
    const int tiles = (n_out + 15) / 16;
    g.groups = (tiles + CT - 1) / CT;
    const size_t x_bytes = (size_t)m * g.x_row_bytes;
    const size_t sz = (size_t)16 * CT * g.sz_stride * 4, part = (size_t)SPLIT * CT * 512;
    const size_t lds = x_bytes + (sz > part ? sz : part);
    if (lds > kMaxLds) return false;
    *err = hipSuccess;
    if (query) {
        *query = persistent_name<SPLIT, CT, UNROLL, DEPTH, FOLD, PAIRED>();
        return true;
    }
    auto kernel = gemv_persistent_kernel<SPLIT, CT, UNROLL, DEPTH, FOLD, PAIRED>;
    if (lds > 64 * 1024) {
        const hipError_t e = allow_full_lds(kernel);
        if (e != hipSuccess) {
            *err = e;
            return true;
        }
    }
    // one workgroup per slot the device can hold at once: each then walks
    // its share of the tile groups
    int cus = 0, per_cu = 0;
    hipError_t e = device_cus(&cus);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kernel), 64 * SPLIT,
                                                         lds);
    if (e != hipSuccess) {
        *err = e;
        return true;
    }
    const int slots = cus * (per_cu > 0 ? per_cu : 1);
    const dim3 grid((unsigned)(g.groups < slots ? g.groups : slots)), block(64 * SPLIT);
    kernel<<<grid, block, lds, stream>>>(x, qweight, scales, zeros, y, g);
    *err = hipGetLastError();
    return true;
}

template <int SPLIT, int CT, int UNROLL, bool FOLD, int MMAX, int BITS = 4>
bool plan_window(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                 const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                 uint16_t *y, hipStream_t stream, const char **query, hipError_t *err)
{
    static_assert(SPLIT >= CT || SPLIT == 1, "the LDS reduction assigns one wave per tile");
    static_assert(SPLIT * UNROLL % 2 == 0, "a window must hold whole groups of 256");
    constexpr int WB = SPLIT * UNROLL;
    if (m > MMAX) return false;
    Geometry g = make_geometry(m, n_out, n_in, group_shift, BITS);
    g.sz_stride = ((WB * 128) >> group_shift) | 1;
    g.x_row_bytes = WB * 256 + 16;
    const size_t x_region = 2 * (size_t)m * g.x_row_bytes;
    const size_t part = SPLIT > 1 ? (size_t)SPLIT * CT * 1024 : 0;
    const size_t lds = (x_region > part ? x_region : part) + 2 * (size_t)16 * CT * g.sz_stride * 4;
    if (lds > kMaxLds) return false;
    *err = hipSuccess;
    if (query) {
        *query = window_name<SPLIT, CT, UNROLL, FOLD, MMAX, BITS>();
        return true;
    }
    auto kernel = gemv_window_kernel<SPLIT, CT, UNROLL, FOLD, MMAX, BITS>;
    if (lds > 64 * 1024) {
        const hipError_t e = allow_full_lds(kernel);
        if (e != hipSuccess) {
            *err = e;
            return true;
        }
    }
    const int tiles = (n_out + 15) / 16;
    const dim3 grid((unsigned)((tiles + CT - 1) / CT)), block(64 * SPLIT);
    kernel<<<grid, block, lds, stream>>>(x, qweight, scales, zeros, y, g);
    *err = hipGetLastError();
    return true;
}

// Configurations chosen from measured sweeps on MI355X over the decode
// shapes (7B and 70B projections, m = 1 and 8, INT4 and INT8); other shapes
// fall through to the nearest rule.  One row of x takes the row-streaming
// kernels (INT4 14-31 %, INT8 12-32 % faster than the MFMA kernels on every
// such shape swept, 4096 to 16384 codes per row, grouped or per-channel)
// unless the scale or zero-point array is only 2-byte aligned or rows are
// longer than 16384 codes.  Paired INT4 loads pay on rows of 8192
// codes and more (9-26 % on the 70B and 8192x28672 shapes); on the
// 4096-wide 7B linears, whose launches are short and dependent, they
// measured the same as the fragment-order loads, which are kept there.
// INT8 rows are twice as long in bytes and paired loads pay on every
// measured shape (3-36 %).  Every rule ends in a configuration that always
// fits.
template <bool FOLD, int BITS>
hipError_t dispatch(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                    const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                    uint16_t *y, hipStream_t stream, const char **query)
{
    hipError_t e = hipSuccess;
    const int kblocks = (n_in + 127) >> 7;
    const int tiles = (n_out + 15) / 16;
#define Q4_RES(S, C, U, D) \
    if (plan_resident<S, C, U, D, FOLD, BITS>(x, qweight, scales, zeros, m, n_out, n_in, group_shift, y, stream, query, &e)) return e
#define Q4_PAIR(S, C, U, D) \
    if (plan_resident<S, C, U, D, FOLD, BITS, true>(x, qweight, scales, zeros, m, n_out, n_in, group_shift, y, stream, query, &e)) return e
#define Q4_WIN(S, C, U, MM) \
    if (plan_window<S, C, U, FOLD, MM, BITS>(x, qweight, scales, zeros, m, n_out, n_in, group_shift, y, stream, query, &e)) return e
#define Q4_RS(NC) \
    case NC: \
        if (plan_rowstream<NC, 1, 8>(x, qweight, scales, zeros, m, n_out, n_in, group_shift, y, stream, query, &e)) return e; \
        break
#define Q8_RS(NC) \
    case NC: \
        if (plan_rowstream8<NC, 8>(x, qweight, scales, zeros, m, n_out, n_in, group_shift, y, stream, query, &e)) return e; \
        break
    // one token and rows of up to 16384 codes: one wave per row (8 rows per
    // workgroup measured best on every such shape swept)
    if (m == 1) {
        if constexpr (BITS == 4) {
            switch ((n_in + 2047) / 2048) {
                Q4_RS(1); Q4_RS(2); Q4_RS(3); Q4_RS(4); Q4_RS(5); Q4_RS(6); Q4_RS(7); Q4_RS(8);
            default: break;
            }
        } else {
            switch ((n_in + 1023) / 1024) {
                Q8_RS(1); Q8_RS(2); Q8_RS(3); Q8_RS(4); Q8_RS(5); Q8_RS(6); Q8_RS(7); Q8_RS(8);
                Q8_RS(9); Q8_RS(10); Q8_RS(11); Q8_RS(12); Q8_RS(13); Q8_RS(14); Q8_RS(15); Q8_RS(16);
            default: break;
            }
        }
    }
    if (kblocks >= 16) {
        if constexpr (BITS == 8) {
            // twice the bytes per code: fewer waves per tile keep more
            // workgroups in flight per CU; paired loads throughout
            if (m == 1) {
                if (tiles <= 256 && kblocks >= 64) Q4_PAIR(8, 1, 1, 3);
                if (tiles <= 256) Q4_PAIR(8, 1, 1, 2);
                if (kblocks >= 128) Q4_PAIR(8, 1, 1, 3);
                if (tiles <= 768) Q4_PAIR(4, 1, 1, 2);
                Q4_PAIR(4, 2, 1, 1);
            }
            if (m <= 4) Q4_RES(8, 1, 1, 2);
            if (tiles >= 640) Q4_PAIR(8, 4, 1, 1);
            Q4_PAIR(8, 2, 1, 2);
        } else if (!FOLD) {
            if (m == 1) {
                if (tiles <= 256 && kblocks >= 64) Q4_RES(8, 1, 1, 3);
                if (kblocks >= 128 && tiles >= 512) Q4_PAIR(16, 1, 2, 1);
                if (tiles <= 768) Q4_RES(8, 1, 1, 2);
                Q4_RES(4, 2, 1, 2);
            }
            Q4_RES(16, 1, 1, 4);
        } else if (m == 1) {
            if (tiles <= 256 && kblocks >= 64) Q4_RES(8, 1, 1, 3);
            if (kblocks >= 128 && tiles >= 512) Q4_PAIR(8, 1, 2, 2);
            if (tiles <= 768) Q4_RES(8, 1, 1, 2);
            if (kblocks >= 64) Q4_PAIR(4, 2, 2, 2);
            Q4_RES(4, 2, 1, 2);
        } else {
            // many tile groups (n_out of 32768 and more): persistent
            // workgroups stage x once each and walk several groups
            if (tiles >= 2048 && m <= 8 &&
                plan_persistent<8, 4, 2, 1, FOLD, 4, true>(x, qweight, scales, zeros, m, n_out, n_in, group_shift, y,
                                                           stream, query, &e))
                return e;
            if (tiles >= 640) Q4_PAIR(8, 4, 2, 1);
            if (tiles >= 256) Q4_RES(8, 2, 1, 2);
            Q4_RES(8, 1, 1, 2);
        }
        if (m <= 8) Q4_WIN(16, 2, 1, 8);
        Q4_WIN(8, 2, 1, 16);
    }
    Q4_RES(4, 1, 1, 2);
    Q4_WIN(2, 1, 1, 16);
#undef Q4_RES
#undef Q4_PAIR
#undef Q4_WIN
#undef Q4_RS
#undef Q8_RS
    return hipErrorInvalidValue;                // unreachable: the last window always fits
}

}  // namespace

hipError_t q4_launch_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, int bits, uint16_t *y, hipStream_t stream, const char **query)
{
    // group k of a row is k >> shift; a per-channel group of any other
    // length than a power of two uses shift 31 (every k in group 0)
    int shift = 0;
    while ((1 << shift) < group_size) ++shift;
    if ((1 << shift) != group_size) shift = 31;
    if (bits == 8)
        return dispatch<false, 8>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream, query);
    // The fold applies s and z once per 128-wide block after summing raw
    // codes, subtracting z * sum(x) from the code sum; with one scale per
    // row (per-channel) most codes sit at z and that subtraction would
    // cancel terms far larger than the result, so per-channel weights take
    // the exact-subtraction form.
    return (group_size == 128 || group_size == 256)
               ? dispatch<true, 4>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream, query)
               : dispatch<false, 4>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream, query);
}
