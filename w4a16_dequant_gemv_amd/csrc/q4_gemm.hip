// q4_gemm.hip -- prefill-shaped W4A16 linear layer, y = x W'^T for large m.
//
// [Guide] §2.3: W4A16 turns the INT4 weights back into FP16 before the
// matrix product, so at prefill sizes the layer is bound by the fp16 matrix
// cores, not by memory.  The kernel therefore dequantizes each packed weight
// tile once into LDS as fp16 and lets every wave of the workgroup reuse it
// from there with v_mfma_f32_32x32x16_f16 (fp32 accumulation).
//
// Tiling.  A workgroup computes a BM x BN tile of y with WAVES_M x WAVES_N
// waves; each wave owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile made of 32x32
// MFMA tiles.  Per BK-wide k step the workgroup
//   * loads the x tile (BM x BK fp16, 16-byte chunks, 8 lanes per 128-byte
//     row run) and the packed weight tile (BN x BK codes, 16 bytes = 32 codes
//     per lane, all in one group) into registers,
//   * stores x into LDS and the dequantized weights s (c - z) as fp16 into
//     LDS, both in the pair order produced by the code unpacking,
//   * runs the MFMAs out of LDS while the next tile's global loads are in
//     flight.
// LDS rows are padded by 8 halves (16 bytes) so the 32 rows read by one
// 16-byte-per-lane fragment load fall on distinct bank groups.
//
// The grid is linear; workgroup ids are dealt round-robin to the eight XCDs,
// so ids are remapped to give each XCD a contiguous band of tiles, and tiles
// are walked column-band by column-band so consecutive workgroups on an XCD
// share weight tiles in its L2.
#include "q4_device.h"
#include "q4_launch.h"

namespace {

constexpr int kXcds = 8;

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, int m, int n_out, int n_in, int group_shift,
    int tiles_m, int tiles_n)
{
    constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    constexpr int WT_M = BM / WAVES_M, WT_N = BN / WAVES_N;
    constexpr int TM = WT_M / 32, TN = WT_N / 32;
    constexpr int LDK = BK + 8;
    constexpr int A_CHUNKS = BM * BK / 8 / THREADS;     // 16-byte x chunks per lane
    constexpr int B_SLICES = BN * BK / 32 / THREADS;    // 16-byte code slices per lane
    static_assert(A_CHUNKS * THREADS * 8 == BM * BK, "x tile does not split evenly");
    static_assert(B_SLICES * THREADS * 32 == BN * BK, "weight tile does not split evenly");
    static_assert(TM * 32 == WT_M && TN * 32 == WT_N, "wave tile not a multiple of 32");

    __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDK];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[BN * LDK];

    // --- tile selection (XCD-aware) ---
    const int tiles = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int per_xcd = (tiles + kXcds - 1) / kXcds;
    const int xcd = bid % kXcds;
    int t = xcd * per_xcd + bid / kXcds;
    // The last band may be short; ids past the end fold back onto the tiles
    // no band covered (bands are contiguous, so this is a bijection).
    if (tiles % kXcds != 0) {
        const int full = tiles % kXcds;       // bands with per_xcd tiles
        t = (xcd < full) ? xcd * per_xcd + bid / kXcds
                         : full * per_xcd + (xcd - full) * (per_xcd - 1) + bid / kXcds;
    }
    const int tile_n = t / tiles_m;
    const int tile_m = t % tiles_m;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / WAVES_N, wave_n = wave % WAVES_N;

    const int words_per_row = n_in >> 3;
    const int groups_per_row = n_in >> group_shift;

    // --- per-lane global load coordinates ---
    int a_row[A_CHUNKS], a_col[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int c = tid + i * THREADS;
        a_row[i] = c / (BK / 8);
        a_col[i] = (c % (BK / 8)) * 8;
    }
    int b_row[B_SLICES], b_col[B_SLICES];
#pragma unroll
    for (int i = 0; i < B_SLICES; ++i) {
        const int c = tid + i * THREADS;
        b_row[i] = c / (BK / 32);
        b_col[i] = (c % (BK / 32)) * 32;
    }

    u32x4 a_reg[A_CHUNKS];
    u32x4 b_reg[B_SLICES];
    uint16_t s_reg[B_SLICES], z_reg[B_SLICES];

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int r = m0 + a_row[i], k = k0 + a_col[i];
            a_reg[i] = u32x4{0u, 0u, 0u, 0u};
            if (r < m && k < n_in)
                a_reg[i] = *reinterpret_cast<const u32x4 *>(x + (int64_t)r * n_in + k);
        }
#pragma unroll
        for (int i = 0; i < B_SLICES; ++i) {
            const int r = n0 + b_row[i], k = k0 + b_col[i];
            b_reg[i] = u32x4{0u, 0u, 0u, 0u};
            s_reg[i] = 0;
            z_reg[i] = 0;
            if (r < n_out && k < n_in) {
                b_reg[i] = *reinterpret_cast<const u32x4 *>(qweight + (int64_t)r * words_per_row + (k >> 3));
                s_reg[i] = scales[(int64_t)r * groups_per_row + (k >> group_shift)];
                z_reg[i] = zeros[(int64_t)r * groups_per_row + (k >> group_shift)];
            }
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i)
            *reinterpret_cast<f16x8 *>(&As[a_row[i] * LDK + a_col[i]]) = pair_order(a_reg[i]);
#pragma unroll
        for (int i = 0; i < B_SLICES; ++i) {
            const _Float16 s = bitcast<_Float16>(s_reg[i]);
            const _Float16 zb = bitcast<_Float16>(z_reg[i]) + (_Float16)1024.0f;
            const f16x2 scale = {s, s}, bias = {zb, zb};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f16x8 *>(&Bs[b_row[i] * LDK + b_col[i] + 8 * j]) =
                    dequant8_f16(b_reg[i][j], bias, scale);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ktiles = (n_in + BK - 1) / BK;
    load_tile(0);
    for (int kt = 0; kt < ktiles; ++kt) {
        store_tile();
        __syncthreads();
        if (kt + 1 < ktiles) load_tile((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kk = ks * 16 + 8 * (lane >> 5);
            f16x8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const f16x8 *>(
                    &As[(wave_m * WT_M + i * 32 + (lane & 31)) * LDK + kk]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *reinterpret_cast<const f16x8 *>(
                    &Bs[(wave_n * WT_N + j * 32 + (lane & 31)) * LDK + kk]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // Lane l, register r of a 32x32 tile: column l % 32,
    // row 8 * (r / 4) + 4 * (l / 32) + r % 4.
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wave_n * WT_N + j * 32 + (lane & 31);
            if (col >= n_out) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wave_m * WT_M + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < m) y[(int64_t)row * n_out + col] = bitcast<uint16_t>((_Float16)acc[i][j][r]);
            }
        }
}

}  // namespace

hipError_t q4_launch_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, uint16_t *y, hipStream_t stream)
{
    constexpr int BM = 128, BN = 128, BK = 64;
    int shift = 0;
    while ((1 << shift) < group_size) ++shift;
    const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n_out + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(256);
    gemm_kernel<BM, BN, BK, 2, 2><<<grid, block, 0, stream>>>(
        x, qweight, scales, zeros, y, (int)m, (int)n_out, (int)n_in, shift, tiles_m, tiles_n);
    return hipGetLastError();
}
