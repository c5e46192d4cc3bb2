// q4_gemm.hip -- prefill-shaped W4A16 linear layer, y = x W'^T for large m.
//
// [Guide] §2.3: W4A16 turns the INT4 weights back into FP16 before the
// matrix product, so at prefill sizes the layer is bound by the fp16 matrix
// cores, not by memory.  The kernel dequantizes each packed weight tile once
// into LDS as fp16 and lets every wave of the workgroup reuse it from there
// with v_mfma_f32_32x32x16_f16 (fp32 accumulation).
//
// Tiling.  A workgroup computes a BM x BN tile of y (BM rows of x, BN output
// channels) with WM x WN waves, one wave per SIMD; each wave owns a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles.  k advances in steps
// of 64 = four MFMA substeps of 16.
//
// Software pipeline (one wave per SIMD, so every latency has to be covered
// by the wave's own instruction stream):
//   * three LDS stages: step k computes from stage k%3 while its stores fill
//     stage (k+2)%3 and stage (k+1)%3, published by the previous barrier,
//     already serves the first fragments of step k+1; one barrier per step;
//   * two fragment register sets: substep s+1's A/B fragments are read from
//     LDS while substep s runs its MFMAs;
//   * three global register sets: the x chunks and packed words of step
//     k+2 are loaded during step k-3 and written to LDS during step k (x
//     unchanged, weights dequantized to fp16 s * (c - z)), a quarter per
//     substep, each quarter's registers reloaded right after with step
//     k+5's data, so every load has about three steps to arrive;
//   * scheduling group barriers interleave each substep's LDS reads, LDS
//     writes, dequantization arithmetic and global loads between its MFMAs.
// The stage and register-set rotations both have period three, so the loop
// is unrolled three times and every LDS address is a lane constant plus an
// immediate.  Global loads are buffer loads: a per-tile resource, a
// lane-constant 32-bit offset and a uniform per-step offset.  The pipelined
// loop covers the full 64-wide steps; n_in % 64 == 32 leaves one 32-wide
// step, done afterwards without pipelining.
//
// LDS rows are 128 bytes (64 halves); the eight 16-byte chunks of row r are
// stored at chunk ^ swz(r) (gemm_tile.h) so that fragment reads (16 rows, one
// chunk each), x stores (whole rows) and weight stores (8 rows, two half-rows
// of 4 chunks each) all hit distinct 16-byte bank groups, whether the lanes
// are served 8 at a time over 32 banks or 16 at a time over 64 banks.
//
// The grid is linear; workgroup ids are dealt round-robin to the eight XCDs,
// so ids are remapped to give each XCD a contiguous range of tiles.  Tiles
// are numbered in bands of kGroupM row tiles, walked output-column by
// output-column inside a band, so an XCD's range covers few row tiles of x
// (BM rows x n_in fp16 each, the larger operand) and many column tiles of
// the packed weights (BN rows x n_in/2 bytes each), which its L2 shares.
#include <type_traits>

#include "gemm_tile.h"
#include "q4_device.h"
#include "q4_launch.h"

namespace {

// Eight codes of one packed word -> eight fp16 weights s * (c - z) in
// natural order (c0, c1), (c2, c3), ...: the codes are split into even and
// odd nibbles, byte-permuted next to a zero byte and OR-ed into the half
// 1024 (0x6400); (1024 + c) - (1024 + z) is exact and the product with s is
// the only rounding.
__device__ __forceinline__ u32x4 dequant_word_natural(uint32_t w, f16x2 bias, f16x2 scale)
{
    const uint32_t lo = w & 0x0F0F0F0Fu;           // c0 c2 c4 c6
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;    // c1 c3 c5 c7
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u;
    r[1] = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u;
    r[2] = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u;
    r[3] = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = bitcast<uint32_t>((bitcast<f16x2>(r[j]) - bias) * scale);
    return r;
}

// Four codes of one INT8 word -> four fp16 weights s * (c - z) in natural
// order, as two dwords (c0, c1), (c2, c3): each byte is placed next to a zero
// byte and OR-ed into the half 1024; (1024 + c) - (1024 + z) is exact for
// codes up to 255 and the product with s is the only rounding.
__device__ __forceinline__ u32x2 dequant_byte_word(uint32_t w, f16x2 bias, f16x2 scale)
{
    u32x2 r;
    r[0] = __builtin_amdgcn_perm(0u, w, 0x0C010C00u) | 0x64006400u;
    r[1] = __builtin_amdgcn_perm(0u, w, 0x0C030C02u) | 0x64006400u;
#pragma unroll
    for (int j = 0; j < 2; ++j) r[j] = bitcast<uint32_t>((bitcast<f16x2>(r[j]) - bias) * scale);
    return r;
}

template <int I, int N, int NDSR, int NDSW, int NVMEM, int NVALU>
__device__ __forceinline__ void interleave()
{
    if constexpr (I < N) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if constexpr (I < NDSR) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        if constexpr (NVALU > 0) __builtin_amdgcn_sched_group_barrier(kSgValu, NVALU, 0);
        if constexpr (I >= N - NDSW) __builtin_amdgcn_sched_group_barrier(kSgDsWrite, 1, 0);
        if constexpr (I < NVMEM) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 1, 0);
        interleave<I + 1, N, NDSR, NDSW, NVMEM, NVALU>();
    }
}

// PAIR_SZ: the two lanes of each lane pair dequantize slices of the same
// row and group (every case but INT4 with groups of 32), so the even lane
// loads the scale, the odd lane the zero-point, and a DPP swap gives each
// lane both: one 2-byte gather per slice and step instead of two.
template <int BM, int BN, int WM, int WN, int BITS, bool PAIR_SZ>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, int m, int n_out, int n_in, int group_shift,
    int tiles_m, int tiles_n)
{
    constexpr int BK = 64, KSUB = BK / 16;
    constexpr int NW = WM * WN, THREADS = 64 * NW;
    constexpr int WT_M = BM / WM, WT_N = BN / WN;
    constexpr int TM = WT_M / 32, TN = WT_N / 32;
    // A 16-byte slice of packed codes holds 128/BITS codes (32 INT4, 16 INT8),
    // i.e. CHS fp16 LDS chunks; a row's 64 codes per step are SPR slices.
    constexpr int SPR = BITS / 2, CPS = 128 / BITS, CHS = CPS / 8;
    constexpr int A_CHUNKS = BM * 8 / THREADS;         // 16-byte x chunks per lane per step
    constexpr int B_SLICES = BN * SPR / THREADS;       // 16-byte code slices per lane per step
    constexpr int A_PART = A_CHUNKS / KSUB;            // x chunks stored per substep
    constexpr int B_PART = B_SLICES;                   // packed words dequantized per substep
    static_assert(A_CHUNKS * THREADS == BM * 8 && A_PART * KSUB == A_CHUNKS,
                  "x tile does not split evenly");
    static_assert(B_SLICES * THREADS == BN * SPR, "weight tile does not split evenly");
    static_assert(BITS == 4 || (BITS == 8 && B_PART % 2 == 0), "INT8 stores pair words into chunks");
    static_assert(TM * 32 == WT_M && TN * 32 == WT_N, "wave tile not a multiple of 32");
    static_assert(THREADS % 128 == 0, "row swizzles assume 16-row lane strides");
    constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
    static_assert(kStages * STAGE <= 160 * 1024, "stages exceed LDS");
    extern __shared__ __attribute__((aligned(16))) char smem[];   // [kStages][A | B]

    // --- tile selection (XCD-aware) ---
    int tile_m, tile_n;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;
    const int words_per_row = n_in * BITS / 32;
    const int groups_per_row = group_shift >= 31 ? 1 : n_in >> group_shift;   // 31: one group per row
    const int ksteps = n_in / BK;                       // full 64-wide steps

    // Per-tile buffer resources covering the tile's rows; lanes add constant
    // 32-bit byte offsets (a tile spans at most 256 rows of at most 2^20
    // halves, so every offset stays below 2^30).  Rows past m or n_out read
    // the last row: they are never stored.
    const int rows_m = min(BM, m - m0), rows_n = min(BN, n_out - n0);
    const char *xg = reinterpret_cast<const char *>(x + (int64_t)m0 * n_in);
    const char *wg = reinterpret_cast<const char *>(qweight + (int64_t)n0 * words_per_row);
    const char *sg = reinterpret_cast<const char *>(scales + (int64_t)n0 * groups_per_row);
    const char *zg = reinterpret_cast<const char *>(zeros + (int64_t)n0 * groups_per_row);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(xg), (short)0, rows_m * n_in * 2, kBufferFlags);
    const __amdgpu_buffer_rsrc_t wr_ = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(wg), (short)0, rows_n * words_per_row * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(sg), (short)0, rows_n * groups_per_row * 2, kBufferFlags);
    const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(zg), (short)0, rows_n * groups_per_row * 2, kBufferFlags);
    uint32_t xoff[A_CHUNKS], woff[B_SLICES], soff[B_SLICES];
    const uint16_t *szp[B_SLICES];                      // PAIR_SZ: this lane's scale or zero-point row
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int c = tid + i * THREADS;                   // row c/8, chunk c%8
        const int r = min(c >> 3, m - 1 - m0);
        xoff[i] = (uint32_t)r * (uint32_t)n_in * 2u + (uint32_t)(c & 7) * 16u;
    }
#pragma unroll
    for (int i = 0; i < B_SLICES; ++i) {
        const int c = tid + i * THREADS;                   // row c/SPR, slice c%SPR of the step
        const int r = min(c / SPR, n_out - 1 - n0);
        woff[i] = (uint32_t)r * (uint32_t)words_per_row * 4u + (uint32_t)(c % SPR) * 16u;
        soff[i] = ((uint32_t)r * (uint32_t)groups_per_row + (uint32_t)(((c % SPR) * CPS) >> group_shift)) * 2u;
        szp[i] = reinterpret_cast<const uint16_t *>(((c & 1) ? zg : sg) + soff[i]);
    }
    // LDS byte offsets within a stage: x chunk i of this lane, weight chunk
    // j of slice i, fragment rows.  Rows of chunk i differ by multiples of 16
    // from those of chunk 0, so they share its swizzle.
    static_assert((THREADS / SPR) % 16 == 0, "weight rows of slice i must keep slice 0's swizzle");
    const int a_row = tid >> 3, b_row = tid / SPR, b_part = tid % SPR;
    const uint32_t a_st = a_row * 128 + (((tid & 7) ^ swz(a_row)) * 16);
    uint32_t b_st[CHS];
#pragma unroll
    for (int j = 0; j < CHS; ++j) b_st[j] = A_BYTES + b_row * 128 + (((b_part * CHS + j) ^ swz(b_row)) * 16);
    constexpr int B_ROW_STEP = THREADS / SPR * 128;     // LDS bytes between the rows of slices i and i+1
    const int frow = lane & 31, fkg = lane >> 5, fswz = swz(frow);
    const uint32_t fa = (wave_m * WT_M + frow) * 128, fb = A_BYTES + (wave_n * WT_N + frow) * 128;

    // Register type of the raw scale/zero bits.  Chosen so that no masking
    // or packing of the loaded halves is placed at the loop's back edge,
    // where it would wait for loads issued in the same step.
    using SzBits = std::conditional_t<PAIR_SZ, uint16_t, uint32_t>;
    struct Regs {
        u32x4 a[A_CHUNKS];
        u32x4 w[B_SLICES];
        SzBits s[B_SLICES], z[B_SLICES];               // raw fp16 bits (PAIR_SZ: z unused)
    };
    struct Frag {
        f16x8 a[TM], b[TN];
    };

    // Global loads of step kt (kt < ksteps): x chunks of substep part p, or
    // the packed words with their scales and zero-points.
    auto load_a = [&](Regs &g, int kt, int p) {
#pragma unroll
        for (int q = 0; q < A_PART; ++q) {
            const int i = p * A_PART + q;
            g.a[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[i], kt * (BK * 2), 0);
        }
    };
    auto load_b = [&](Regs &g, int kt) {
        const int gk = ((kt * BK) >> group_shift) * 2;
#pragma unroll
        for (int i = 0; i < B_SLICES; ++i) {
            g.w[i] = __builtin_amdgcn_raw_buffer_load_b128(wr_, woff[i], kt * (BK * BITS / 8), 0);
            if constexpr (PAIR_SZ) {
                g.s[i] = szp[i][gk >> 1];
            } else {
                g.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff[i], gk, 0);
                g.z[i] = __builtin_amdgcn_raw_buffer_load_b16(zr, soff[i], gk, 0);
            }
        }
    };
    // Scale and biased zero-point of slice i (PAIR_SZ: swapped in from the
    // partner lane).
    auto scale_bias = [&](const Regs &g, int i, f16x2 &scale, f16x2 &bias) {
        uint32_t sb, zb;
        if constexpr (PAIR_SZ) {
            const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)g.s[i], 0xB1, 0xF, 0xF, false);
            sb = (tid & 1) ? other : g.s[i];
            zb = (tid & 1) ? g.s[i] : other;
        } else {
            sb = g.s[i];
            zb = g.z[i];
        }
        const _Float16 sv = bitcast<_Float16>((uint16_t)sb);
        const _Float16 zv = bitcast<_Float16>((uint16_t)zb) + (_Float16)1024.0f;
        scale = f16x2{sv, sv};
        bias = f16x2{zv, zv};
    };
    auto load_all = [&](Regs &g, int kt) {
#pragma unroll
        for (int p = 0; p < KSUB; ++p) load_a(g, kt, p);
        load_b(g, kt);
    };
    // Part p of writing a step's registers into the stage at byte offset buf.
    auto store_part = [&](const Regs &g, uint32_t buf, int p) {
#pragma unroll
        for (int q = 0; q < A_PART; ++q) {
            const int i = p * A_PART + q;
            *reinterpret_cast<u32x4 *>(smem + buf + a_st + i * THREADS * 16) = g.a[i];
        }
        if (BITS == 4) {
#pragma unroll
            for (int q = 0; q < B_PART; ++q) {
                const int wd = p * B_PART + q, i = wd >> 2, j = wd & 3;
                f16x2 scale, bias;
                scale_bias(g, i, scale, bias);
                *reinterpret_cast<u32x4 *>(smem + buf + b_st[j] + i * B_ROW_STEP) =
                    dequant_word_natural(g.w[i][j], bias, scale);
            }
        } else {
            // two INT8 words (eight codes) make one fp16 chunk
#pragma unroll
            for (int q = 0; q < B_PART; q += 2) {
                const int wd = p * B_PART + q, i = wd >> 2, j = wd & 3;
                f16x2 scale, bias;
                scale_bias(g, i, scale, bias);
                const u32x2 lo = dequant_byte_word(g.w[i][j], bias, scale);
                const u32x2 hi = dequant_byte_word(g.w[i][j + 1], bias, scale);
                *reinterpret_cast<u32x4 *>(smem + buf + b_st[j >> 1] + i * B_ROW_STEP) =
                    u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    };
    auto store_all = [&](const Regs &g, uint32_t buf) {
#pragma unroll
        for (int p = 0; p < KSUB; ++p) store_part(g, buf, p);
    };
    // Fragments of MFMA substep ks: lane (row l % 32, k group l / 32) reads
    // logical chunk 2*ks + l/32 of its row.
    auto read_frag = [&](Frag &f, uint32_t buf, int ks) {
        const uint32_t cofs = ((2 * ks + fkg) ^ fswz) * 16;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            f.a[i] = *reinterpret_cast<const f16x8 *>(smem + buf + fa + cofs + i * 32 * 128);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            f.b[j] = *reinterpret_cast<const f16x8 *>(smem + buf + fb + cofs + j * 32 * 128);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
    };

    constexpr int NMFMA = TM * TN, NFRAG = TM + TN;
    constexpr int VALU_PER_SUBSTEP = B_PART * 20;
    constexpr int NVALU = (VALU_PER_SUBSTEP + NMFMA - 1) / NMFMA;

    if (ksteps > 0) {
        Regs R[3];
        Frag f0, f1;
        const int kmax = ksteps - 1;
        // The prologue issues its loads in the loop's own order, pinned by
        // scheduling barriers, so the wait counts the compiler places at the
        // loop head stay three steps deep.
        load_all(R[0], 0);
        __builtin_amdgcn_sched_barrier(0);
        load_all(R[1], min(1, kmax));
        __builtin_amdgcn_sched_barrier(0);
        load_all(R[2], min(2, kmax));
        __builtin_amdgcn_sched_barrier(0);
        store_all(R[0], 0);
        __builtin_amdgcn_sched_barrier(0);
        load_all(R[0], min(3, kmax));
        __builtin_amdgcn_sched_barrier(0);
        store_all(R[1], STAGE);
        __builtin_amdgcn_sched_barrier(0);
        load_all(R[1], min(4, kmax));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        read_frag(f0, 0, 0);

        // Step k with k % 3 == J: MFMAs of step k from stage J (substep 0's
        // fragments already in f0), step k+2's registers (set (J+2) % 3)
        // into stage (J+2) % 3, that set reloaded with step k+5, and step
        // k+1's first fragments read from stage (J+1) % 3.
        auto step = [&](auto J_, int k) {
            constexpr int J = decltype(J_)::value;
            constexpr uint32_t cur = J * STAGE, nxt = ((J + 1) % 3) * STAGE, wr = ((J + 2) % 3) * STAGE;
            Regs &g = R[(J + 2) % 3];
            const int kl = min(k + 5, kmax);
            read_frag(f1, cur, 1);
            store_part(g, wr, 0);
            load_a(g, kl, 0);
            mma(f0);
            interleave<0, NMFMA, NFRAG, A_PART + B_PART, A_PART, NVALU>();
            __builtin_amdgcn_sched_barrier(0);
            read_frag(f0, cur, 2);
            store_part(g, wr, 1);
            load_a(g, kl, 1);
            mma(f1);
            interleave<0, NMFMA, NFRAG, A_PART + B_PART, A_PART, NVALU>();
            __builtin_amdgcn_sched_barrier(0);
            read_frag(f1, cur, 3);
            store_part(g, wr, 2);
            load_a(g, kl, 2);
            mma(f0);
            interleave<0, NMFMA, NFRAG, A_PART + B_PART, A_PART, NVALU>();
            __builtin_amdgcn_sched_barrier(0);
            read_frag(f0, nxt, 0);
            store_part(g, wr, 3);
            load_a(g, kl, 3);
            load_b(g, kl);
            mma(f1);
            interleave<0, NMFMA, NFRAG, A_PART + B_PART, A_PART + (PAIR_SZ ? 2 : 3) * B_SLICES, NVALU>();
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        int k = 0;
        for (; k + 3 <= ksteps; k += 3) {
            step(I0{}, k);
            step(I1{}, k + 1);
            step(I2{}, k + 2);
        }
        if (k < ksteps) step(I0{}, k);
        if (k + 1 < ksteps) step(I1{}, k + 1);
    }

    if (n_in & (BK - 1)) {
        // Final 32-wide step at k = 64 * ksteps: x chunks 0..3 and weight
        // half 0 of every row, computed by substeps 0 and 1 only.  Every wave
        // finished reading the real data of every stage before the last
        // barrier, so stage 0 is free.
        const int kt = ksteps;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i)
            if ((tid & 7) < 4)
                *reinterpret_cast<u32x4 *>(smem + a_st + i * THREADS * 16) =
                    __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[i], kt * (BK * 2), 0);
        if (b_part < SPR / 2) {                 // the slices of k = 0 .. 31 of the step
            const int gk = ((kt * BK) >> group_shift) * 2;
#pragma unroll
            for (int i = 0; i < B_SLICES; ++i) {
                const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(wr_, woff[i], kt * (BK * BITS / 8), 0);
                const _Float16 sv = bitcast<_Float16>(__builtin_amdgcn_raw_buffer_load_b16(sr, soff[i], gk, 0));
                const _Float16 zb = bitcast<_Float16>(__builtin_amdgcn_raw_buffer_load_b16(zr, soff[i], gk, 0)) +
                                    (_Float16)1024.0f;
                const f16x2 scale = {sv, sv}, bias = {zb, zb};
                if (BITS == 4) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<u32x4 *>(smem + b_st[j] + i * B_ROW_STEP) =
                            dequant_word_natural(w[j], bias, scale);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        const u32x2 lo = dequant_byte_word(w[j], bias, scale);
                        const u32x2 hi = dequant_byte_word(w[j + 1], bias, scale);
                        *reinterpret_cast<u32x4 *>(smem + b_st[j >> 1] + i * B_ROW_STEP) =
                            u32x4{lo[0], lo[1], hi[0], hi[1]};
                    }
                }
            }
        }
        __syncthreads();
        Frag f;
        read_frag(f, 0, 0);
        mma(f);
        read_frag(f, 0, 1);
        mma(f);
    }

    // The MFMAs take the weight fragment as their first operand, so tile
    // (i, j) holds y^T: lane l, register r is output channel
    // 8 * (r / 4) + 4 * (l / 32) + r % 4 of the tile's 32, for x row l % 32.
    // The fp16 results go through LDS (row-major, rows padded to YS bytes,
    // each lane writing its runs of 4 consecutive channels as 8 bytes), then
    // every thread stores 16-byte pieces of whole rows, 16 lanes per 256
    // bytes, so y is written in full cache lines.  The stages are free: every
    // wave passed the last barrier (or the tail step's) after its last LDS
    // read, and the barrier below orders the rest.
    constexpr int YS = BN * 2 + 16;
    static_assert(BM * YS <= kStages * STAGE, "output tile exceeds LDS");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wave_m * WT_M + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int c = wave_n * WT_N + j * 32 + 8 * rq + 4 * (lane >> 5);
                const f16x2 lo = {(_Float16)acc[i][j][4 * rq], (_Float16)acc[i][j][4 * rq + 1]};
                const f16x2 hi = {(_Float16)acc[i][j][4 * rq + 2], (_Float16)acc[i][j][4 * rq + 3]};
                const u32x2 v = {bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
                *reinterpret_cast<u32x2 *>(smem + r * YS + c * 2) = v;
            }
    }
    __syncthreads();
    constexpr int CPR = BN / 8;                          // 16-byte pieces per row
    constexpr int RPP = THREADS / CPR;                   // rows per pass
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
hipError_t allow_lds(K kernel, size_t bytes)
{
    if (bytes <= 64 * 1024) return hipSuccess;
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                                    160 * 1024);
    return e;
}

template <int BM, int BN, int WM, int WN, int BITS, bool PAIR_SZ>
hipError_t launch_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                       const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                       uint16_t *y, hipStream_t stream)
{
    const int tiles_m = (m + BM - 1) / BM, tiles_n = (n_out + BN - 1) / BN;
    const size_t lds = kStages * (size_t)(BM + BN) * 128;
    auto kernel = gemm_kernel<BM, BN, WM, WN, BITS, PAIR_SZ>;
    const hipError_t e = allow_lds(kernel, lds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * WM * WN);
    kernel<<<grid, block, lds, stream>>>(x, qweight, scales, zeros, y, m, n_out, n_in, group_shift,
                                         tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t q4_launch_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, int bits, uint16_t *y, hipStream_t stream)
{
    // group k of a row is k >> shift; a per-channel group of any other
    // length than a power of two uses shift 31 (every k in group 0)
    int shift = 0;
    while ((1 << shift) < group_size) ++shift;
    if ((1 << shift) != group_size) shift = 31;
    if (bits == 8)
        return launch_gemm<256, 128, 4, 1, 8, true>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in,
                                                    shift, y, stream);
    // INT4 slices hold 32 codes: with groups of 32 the two slices of a row
    // step belong to different groups
    if (group_size == 32)
        return launch_gemm<256, 128, 4, 1, 4, false>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in,
                                                     shift, y, stream);
    return launch_gemm<256, 128, 4, 1, 4, true>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift,
                                                y, stream);
}
