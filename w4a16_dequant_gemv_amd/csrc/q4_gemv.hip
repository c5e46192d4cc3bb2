// q4_gemv.hip -- decode-shaped W4A16 linear layer, y[m][n] = sum_k x[m][k] w'[n][k]
// for 1 <= m <= 16, with w' = s (code - z) formed in registers.
//
// [Kern] §4: the dequantization is fused into the product, the fp16 weights
// are never materialized in memory.  [Guide] §1.2: at decode sizes every
// weight byte is read once per call and the arithmetic intensity is a few
// FLOP per byte, so the kernel is bound by HBM bandwidth; its job is to keep
// enough 16-byte loads in flight and to spend few VALU operations per weight.
//
// Mapping onto the matrix cores.  One v_mfma_f32_16x16x32_f16 takes a 16x32
// A block (rows = the m rows of x, zero-padded to 16) and a 32x16 B block
// (columns = 16 output channels).  Lane l supplies row/column l % 16 and
// eight k values chosen by l / 16, the same eight for A and B.  A wave
// covers 16 output channels; in one 128-wide k block, lane (col c, quarter
// q) loads the 16 bytes (32 codes) of channel c at k = kb + 32q .. kb+32q+31
// and feeds them to four MFMAs, one packed word each.  The unpacking yields
// codes in the pair order (c0,c4),(c1,c5),(c2,c6),(c3,c7); the x values are
// permuted the same way, which leaves the dot product unchanged.  All 32
// codes of a lane lie in one group (group sizes are multiples of 32).
//
// Work split.  A workgroup of SPLIT waves owns 16 output channels; wave w
// takes a contiguous range of k blocks, and the SPLIT partial 16x16 results
// are summed in LDS in a fixed order (deterministic).  UNROLL k blocks are
// loaded before any is consumed so that each lane keeps UNROLL 16-byte
// weight loads in flight.
#include "q4_device.h"
#include "q4_launch.h"

namespace {

template <int SPLIT, int UNROLL>
__global__ __launch_bounds__(64 * SPLIT) void gemv_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, int m, int n_out, int n_in, int group_shift,
    int kblocks_per_wave)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;      // output channel within the tile / row of x
    const int quarter = lane >> 4;  // which 32-wide slice of a 128-wide k block

    const int n = blockIdx.x * 16 + col;
    const bool n_ok = n < n_out;
    const int words_per_row = n_in >> 3;
    const int groups_per_row = n_in >> group_shift;
    const uint32_t *wrow = qweight + (int64_t)(n_ok ? n : 0) * words_per_row;
    const uint16_t *srow = scales + (int64_t)(n_ok ? n : 0) * groups_per_row;
    const uint16_t *zrow = zeros + (int64_t)(n_ok ? n : 0) * groups_per_row;

    const bool m_ok = col < m;
    const uint16_t *xrow = x + (int64_t)(m_ok ? col : 0) * n_in;

    const int kblocks = (n_in + 127) >> 7;
    const int kb_begin = wave * kblocks_per_wave;
    const int kb_end = min(kblocks, kb_begin + kblocks_per_wave);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb0 = kb_begin; kb0 < kb_end; kb0 += UNROLL) {
        u32x4 wv[UNROLL];
        uint16_t sv[UNROLL], zv[UNROLL];
        u32x4 xv[UNROLL][4];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int k = ((kb0 + u) << 7) + (quarter << 5);
            const bool k_ok = (kb0 + u < kb_end) && (k < n_in);
            wv[u] = u32x4{0u, 0u, 0u, 0u};
            sv[u] = 0;
            zv[u] = 0;
            if (n_ok && k_ok) {
                wv[u] = *reinterpret_cast<const u32x4 *>(wrow + (k >> 3));
                sv[u] = srow[k >> group_shift];
                zv[u] = zrow[k >> group_shift];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xv[u][j] = u32x4{0u, 0u, 0u, 0u};
                if (m_ok && k_ok) xv[u][j] = *reinterpret_cast<const u32x4 *>(xrow + k + 8 * j);
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const _Float16 s = bitcast<_Float16>(sv[u]);
            const _Float16 zb = bitcast<_Float16>(zv[u]) + (_Float16)1024.0f;
            const f16x2 scale = {s, s};
            const f16x2 bias = {zb, zb};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f16x8 b = dequant8_f16(wv[u][j], bias, scale);
                const f16x8 a = pair_order(xv[u][j]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
            }
        }
    }

    // Lane l holds rows 4*(l/16) + r (r = 0..3) of column l % 16.
    if (SPLIT > 1) {
        __shared__ f32x4 partial[SPLIT][64];
        partial[wave][lane] = acc;
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 1; w < SPLIT; ++w) acc += partial[w][lane];
    }
    if (!n_ok) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * quarter + r;
        if (row < m) y[(int64_t)row * n_out + n] = bitcast<uint16_t>((_Float16)acc[r]);
    }
}

template <int SPLIT>
hipError_t launch_split(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                        const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                        uint16_t *y, hipStream_t stream)
{
    const int kblocks = (n_in + 127) >> 7;
    const int per_wave = (kblocks + SPLIT - 1) / SPLIT;
    const dim3 grid((unsigned)((n_out + 15) / 16)), block(64 * SPLIT);
    gemv_kernel<SPLIT, 4><<<grid, block, 0, stream>>>(x, qweight, scales, zeros, y, m, n_out,
                                                      n_in, group_shift, per_wave);
    return hipGetLastError();
}

}  // namespace

hipError_t q4_launch_gemv(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, uint16_t *y, hipStream_t stream)
{
    int shift = 0;
    while ((1 << shift) < group_size) ++shift;
    const int kblocks = (int)((n_in + 127) >> 7);
    // Enough k blocks per wave to keep several loads in flight, enough waves
    // per channel tile to fill the machine when n_out is small.
    if (kblocks >= 32)
        return launch_split<8>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream);
    if (kblocks >= 16)
        return launch_split<4>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream);
    if (kblocks >= 8)
        return launch_split<2>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream);
    return launch_split<1>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream);
}
