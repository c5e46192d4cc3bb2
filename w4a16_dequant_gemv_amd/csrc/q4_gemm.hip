// q4_gemm.hip -- prefill-shaped W4A16 linear layer, y = x W'^T for large m.
//
// [Guide] §2.3: W4A16 turns the INT4 weights back into FP16 before the
// matrix product, so at prefill sizes the layer is bound by the fp16 matrix
// cores, not by memory.  The kernel dequantizes each packed weight tile once
// into LDS as fp16 and lets every wave of the workgroup reuse it from there
// with v_mfma_f32_16x16x32_f16 (fp32 accumulation; on gfx950 it measured
// about 7 % faster here than v_mfma_f32_32x32x16_f16 with the same operand
// bytes per flop).
//
// Tiling.  A workgroup computes a BM x BN tile of y (BM rows of x, BN output
// channels); k advances in steps of 64 = two MFMA substeps of 32.
//
// Warp specialization.  The workgroup has eight waves, two per SIMD: four
// consumers, each owning BM/4 x BN of the tile as 16x16 MFMA tiles, whose
// instruction streams are only LDS fragment reads and MFMAs; and four
// producers, which bring x and the packed weights of each step into LDS,
// the weights dequantized to fp16 s * (c - z).  The SIMD interleaves the
// two waves it holds, so the dequantization arithmetic and the load waits
// of the producer overlap the consumer's MFMAs without sharing one
// instruction stream.
//
// Pipeline.  Three LDS stages; one barrier per step, shared by both roles:
//   * consumers compute step k from stage k%3 (two fragment register sets,
//     substep 1's fragments read while substep 0 runs its MFMAs) and read
//     step k+1's first fragments from stage (k+1)%3 before the barrier;
//   * producers fill stage (k+2)%3 during step k: x by direct global->LDS
//     loads (buffer_load ... lds: no registers, no LDS store instructions,
//     which gfx950 executes at well under half its LDS read rate), weights
//     from one of three register sets loaded three steps earlier, which is
//     then reloaded with step k+5 (scales and zero-points: see SZV below).
//     Before the barrier a producer waits only until the step's x loads
//     (and every older load) have landed, leaving the new weight loads in
//     flight; a barrier that waited for every load would empty the pipeline
//     each step.
// Both rotations have period three, so the loop is unrolled three times and
// every LDS address is a lane constant plus an immediate.  Global loads are
// buffer loads: a per-tile resource, a lane-constant 32-bit offset and a
// uniform per-step offset.  The pipelined loop covers the full 64-wide
// steps; n_in % 64 == 32 leaves one 32-wide step, done afterwards without
// pipelining.
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
#include <string>
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

constexpr int kConsumers = 4, kProducers = 4;
constexpr int kGemmThreads = 64 * (kConsumers + kProducers);

// PAIR_SZ: the two lanes of each lane pair dequantize slices of the same
// row and group (every case but INT4 with groups of 32), so the even lane
// loads the scale, the odd lane the zero-point, and a DPP swap gives each
// lane both: one 2-byte gather per slice and step instead of two.
// SZV > 1 (with PAIR_SZ, groups of 64..256): the lane loads the raw bits of
// SZV consecutive groups of its row at once, once every 2^sz_log2p steps
// (the steps those groups span), and keeps them in registers.  Gathering 2
// bytes per step instead, each wave instruction touching a line per row, made
// up a sixth of the workgroup's L2 requests and about 15 % of the step time.
template <int BM, int BN, int BITS, bool PAIR_SZ, int SZV = 1>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ y, int m, int n_out, int n_in, int group_shift,
    int tiles_m, int tiles_n, int sz_log2p)
{
    static_assert(SZV == 1 || (PAIR_SZ && (SZV == 2 || SZV == 8)), "scale vectors of 2 or 8 groups");
    constexpr int BK = 64;
    constexpr int PT = 64 * kProducers;                 // producer threads
    constexpr int WT_M = BM / kConsumers, WT_N = BN;    // consumer wave tile
    constexpr int TM = WT_M / 16, TN = WT_N / 16;       // 16x16 MFMA tiles per wave
    // A 16-byte slice of packed codes holds 128/BITS codes (32 INT4, 16 INT8),
    // i.e. CHS fp16 LDS chunks; a row's 64 codes per step are SPR slices.
    constexpr int SPR = BITS / 2, CPS = 128 / BITS, CHS = CPS / 8;
    constexpr int A_CHUNKS = BM * 8 / PT;               // 16-byte x chunks per producer lane (32-wide tail step)
    constexpr int B_SLICES = BN * SPR / PT;             // 16-byte code slices per producer lane per step
    static_assert(A_CHUNKS * PT == BM * 8, "x tile does not split evenly");
    static_assert(B_SLICES * PT == BN * SPR, "weight tile does not split evenly");
    static_assert(TM * 16 == WT_M && TN * 16 == WT_N, "wave tile not a multiple of 16");
    static_assert(PT % 128 == 0 && (PT / SPR) % 16 == 0, "row swizzles assume 16-row lane strides");
    static_assert(BM == 64 * kProducers, "each producer wave loads 64 rows of x per step");
    constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
    static_assert(kStages == 3, "the loop is unrolled for three stages");
    static_assert(kStages * STAGE <= 160 * 1024, "stages exceed LDS");
    extern __shared__ __attribute__((aligned(16))) char smem[];   // [kStages][A | B]

    // --- tile selection (XCD-aware) ---
    int tile_m, tile_n;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ksteps = n_in / BK;                       // full 64-wide steps

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

    if (wave < kConsumers) {
        // ---------------- consumer: fragments and MFMAs ----------------
        struct Frag {
            f16x8 a[TM], b[TN];
        };
        const int frow = lane & 15, fkg = lane >> 4, fswz = swz(frow);
        const uint32_t fa = (wave * WT_M + frow) * 128, fb = A_BYTES + frow * 128;
        // Fragments of MFMA substep ks (32 k): lane (row l % 16, k group
        // l / 16) reads logical chunk 4*ks + l/16 of its row.
        auto read_frag = [&](Frag &f, uint32_t buf, int ks) {
            const uint32_t cofs = ((4 * ks + fkg) ^ fswz) * 16;
#pragma unroll
            for (int i = 0; i < TM; ++i)
                f.a[i] = *reinterpret_cast<const f16x8 *>(smem + buf + fa + cofs + i * 16 * 128);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                f.b[j] = *reinterpret_cast<const f16x8 *>(smem + buf + fb + cofs + j * 16 * 128);
        };
        auto mma = [&](const Frag &f) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
        };
        constexpr int NMFMA = TM * TN, NFRAG = TM + TN;
        if (ksteps > 0) {
            __syncthreads();                            // stages 0 and 1 written
            Frag f0, f1;
            read_frag(f0, 0, 0);
            // Step k with k % 3 == J: MFMAs from stage J (substep 0's
            // fragments already in f0), then step k+1's first fragments
            // from stage (J+1) % 3, published by the previous barrier.
            auto step = [&](auto J_) {
                constexpr int J = decltype(J_)::value;
                constexpr uint32_t cur = J * STAGE, nxt = ((J + 1) % 3) * STAGE;
                read_frag(f1, cur, 1);
                mma(f0);
                interleave<0, NMFMA, NFRAG, 0, 0, 0>();
                __builtin_amdgcn_sched_barrier(0);
                read_frag(f0, nxt, 0);
                mma(f1);
                interleave<0, NMFMA, NFRAG, 0, 0, 0>();
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
            };
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            int k = 0;
            for (; k + 3 <= ksteps; k += 3) {
                step(I0{});
                step(I1{});
                step(I2{});
            }
            if (k < ksteps) step(I0{});
            if (k + 1 < ksteps) step(I1{});
        }
        if (n_in & (BK - 1)) {
            __syncthreads();                            // the producers' 32-wide step is in stage 0
            Frag f;
            read_frag(f, 0, 0);
            mma(f);
        }
    } else {
        // ---------------- producer: global loads, dequantization, LDS stores ----------------
        const int ptid = tid - 64 * kConsumers;
        const int words_per_row = n_in * BITS / 32;
        const int groups_per_row = group_shift >= 31 ? 1 : n_in >> group_shift;   // 31: one group per row
        // Per-tile buffer resources covering the tile's rows; lanes add
        // constant 32-bit byte offsets (a tile spans at most 256 rows of at
        // most 2^20 halves, so every offset stays below 2^30).  Rows past m
        // or n_out read the last row: they are never stored.
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
        const uint16_t *szp[B_SLICES];                  // PAIR_SZ: this lane's scale or zero-point row
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = ptid + i * PT;                // row c/8, chunk c%8
            const int r = min(c >> 3, m - 1 - m0);
            xoff[i] = (uint32_t)r * (uint32_t)n_in * 2u + (uint32_t)(c & 7) * 16u;
        }
#pragma unroll
        for (int i = 0; i < B_SLICES; ++i) {
            const int c = ptid + i * PT;                // row c/SPR, slice c%SPR of the step
            const int r = min(c / SPR, n_out - 1 - n0);
            woff[i] = (uint32_t)r * (uint32_t)words_per_row * 4u + (uint32_t)(c % SPR) * 16u;
            soff[i] = ((uint32_t)r * (uint32_t)groups_per_row + (uint32_t)(((c % SPR) * CPS) >> group_shift)) * 2u;
            szp[i] = reinterpret_cast<const uint16_t *>(((c & 1) ? zg : sg) + soff[i]);
        }
        // x of a full step goes global -> LDS directly (no registers, no
        // LDS store instructions): direct load j of producer wave pw fills
        // tile rows pw*64 + 8j .. +8 whole, lane i landing at LDS row i/8,
        // physical chunk i%8, so the lane loads the logical chunk that the
        // row's swizzle places there.
        typedef __attribute__((address_space(3))) char lds_char;
        const int pw = wave - kConsumers;
        uint32_t xdoff[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = pw * 64 + 8 * j + (lane >> 3);
            xdoff[j] = (uint32_t)min(r, m - 1 - m0) * (uint32_t)n_in * 2u + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
        }
        auto load_x = [&](uint32_t buf, int kt) {
            // (the offsets are passed as int explicitly: with an implicit
            // conversion this toolchain's host pass dropped the kernel's launch stub)
            lds_char *dst = (lds_char *)smem + buf + pw * 64 * 128;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void *)(dst + j * 8 * 128),
                                                         16, (int)xdoff[j], kt * (BK * 2), 0, 0);
        };
        // LDS byte offsets within a stage: x chunk i of this lane (32-wide
        // tail step only), weight chunk j of slice i.  Rows of chunk (slice)
        // i differ by multiples of 16 from those of chunk (slice) 0, so they
        // share its swizzle.
        const int a_row = ptid >> 3, b_row = ptid / SPR, b_part = ptid % SPR;
        const uint32_t a_st = a_row * 128 + (((ptid & 7) ^ swz(a_row)) * 16);
        uint32_t b_st[CHS];
#pragma unroll
        for (int j = 0; j < CHS; ++j) b_st[j] = A_BYTES + b_row * 128 + (((b_part * CHS + j) ^ swz(b_row)) * 16);
        constexpr int B_ROW_STEP = PT / SPR * 128;      // LDS bytes between the rows of slices i and i+1

        // Register type of the raw scale/zero bits, chosen so that no masking
        // or packing of the loaded halves waits on loads of the same step.
        using SzBits = std::conditional_t<PAIR_SZ, uint16_t, uint32_t>;
        using SzVec = std::conditional_t<SZV == 8, u32x4, uint32_t>;   // SZV raw halves
        struct Regs {
            u32x4 w[B_SLICES];
            SzBits s[B_SLICES], z[B_SLICES];            // raw fp16 bits (PAIR_SZ: z unused; SZV > 1: unused)
            SzVec v[B_SLICES];                          // SZV > 1: the groups from step kt on, if loaded
        };
        constexpr int W_LOADS = B_SLICES * (SZV > 1 ? 1 : PAIR_SZ ? 2 : 3);   // per load_w (SZV > 1: without the vector)
        // SZV > 1: data step kt loads a new vector when kt is a multiple of
        // 2^sz_log2p (a new run of SZV groups begins there).
        const int sz_mask = (1 << sz_log2p) - 1;
        auto sz_due = [&](int kt) { return SZV > 1 && (kt & sz_mask) == 0; };
        // Weight loads of step kt (kt < ksteps).
        auto load_w = [&](Regs &g, int kt) {
            const int gk = ((kt * BK) >> group_shift) * 2;
#pragma unroll
            for (int i = 0; i < B_SLICES; ++i) {
                g.w[i] = __builtin_amdgcn_raw_buffer_load_b128(wr_, woff[i], kt * (BK * BITS / 8), 0);
                if constexpr (SZV > 1) {
                    (void)gk;
                } else if constexpr (PAIR_SZ) {
                    g.s[i] = szp[i][gk >> 1];
                } else {
                    g.s[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff[i], gk, 0);
                    g.z[i] = __builtin_amdgcn_raw_buffer_load_b16(zr, soff[i], gk, 0);
                }
            }
            if constexpr (SZV > 1) {
                if (sz_due(kt)) {
                    const int first = (kt >> sz_log2p) * SZV;           // first group of the run
#pragma unroll
                    for (int i = 0; i < B_SLICES; ++i) g.v[i] = *reinterpret_cast<const SzVec *>(szp[i] + first);
                }
            }
        };
        // SZV > 1: the run of groups that the steps being stored use, and
        // this lane's raw scale (or zero-point) bits of slice i at step kt.
        SzVec cur[B_SLICES];
        auto sz_bits = [&](const Regs &g, int i, int kt) -> uint32_t {
            if constexpr (SZV > 1) {
                const int e = ((kt * BK) >> group_shift) & (SZV - 1);   // group within the run
                uint32_t d;
                if constexpr (SZV == 8) d = cur[i][e >> 1];
                else d = cur[i];
                return (d >> (16 * (e & 1))) & 0xFFFFu;
            } else {
                return g.s[i];
            }
        };
        // Scale and biased zero-point (1024 + z) of slice i as fp16 pairs.
        auto scale_bias = [&](const Regs &g, int i, int kt, f16x2 &scale, f16x2 &bias) {
            uint32_t sb, zb;
            if constexpr (PAIR_SZ) {
                const uint32_t own = sz_bits(g, i, kt);
                const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);
                sb = (tid & 1) ? other : own;
                zb = (tid & 1) ? own : other;
            } else {
                sb = g.s[i];
                zb = g.z[i];
            }
            const _Float16 sv = bitcast<_Float16>((uint16_t)sb);
            const _Float16 zv = bitcast<_Float16>((uint16_t)zb) + (_Float16)1024.0f;
            scale = f16x2{sv, sv};
            bias = f16x2{zv, zv};
        };
        // Dequantized slice i (packed words w) into its CHS chunks.
        auto store_slice = [&](uint32_t buf, int i, const u32x4 &w, f16x2 scale, f16x2 bias) {
            if constexpr (BITS == 4) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u32x4 *>(smem + buf + b_st[j] + i * B_ROW_STEP) =
                        dequant_word_natural(w[j], bias, scale);
            } else {
                // two INT8 words (eight codes) make one fp16 chunk
#pragma unroll
                for (int j = 0; j < 4; j += 2) {
                    const u32x2 lo = dequant_byte_word(w[j], bias, scale);
                    const u32x2 hi = dequant_byte_word(w[j + 1], bias, scale);
                    *reinterpret_cast<u32x4 *>(smem + buf + b_st[j >> 1] + i * B_ROW_STEP) =
                        u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            }
        };
        // Data step kt (stores go in increasing kt, so cur holds the run
        // that the last due step loaded).
        auto store_w = [&](const Regs &g, uint32_t buf, int kt) {
            if constexpr (SZV > 1) {
                if (sz_due(kt)) {
#pragma unroll
                    for (int i = 0; i < B_SLICES; ++i) cur[i] = g.v[i];
                }
            }
#pragma unroll
            for (int i = 0; i < B_SLICES; ++i) {
                f16x2 scale, bias;
                scale_bias(g, i, kt, scale, bias);
                store_slice(buf, i, g.w[i], scale, bias);
            }
        };
        // Wait until at most n vector-memory operations remain, n being the
        // loads of the last one or two load_w calls (their scale vectors
        // included when due); the count is an immediate, so each possible n
        // has its own wait.
        auto wait_left = [&](int n) {
            if (n == W_LOADS) wait_vmem<W_LOADS>();
            else if (n == W_LOADS + B_SLICES) wait_vmem<W_LOADS + B_SLICES>();
            else if (n == 2 * W_LOADS) wait_vmem<2 * W_LOADS>();
            else if (n == 2 * W_LOADS + B_SLICES) wait_vmem<2 * W_LOADS + B_SLICES>();
            else wait_vmem<2 * W_LOADS + 2 * B_SLICES>();
        };
        auto vec_loads = [&](int kt) { return sz_due(kt) ? B_SLICES : 0; };
        if (ksteps > 0) {
            Regs R[3];
            const int kmax = ksteps - 1;
            load_x(0, 0);
            load_x(STAGE, min(1, kmax));
            // The prologue issues its loads in the loop's own order, pinned
            // by scheduling barriers, so the wait counts the compiler places
            // in the loop stay three steps deep.
            load_w(R[0], 0);
            __builtin_amdgcn_sched_barrier(0);
            load_w(R[1], min(1, kmax));
            __builtin_amdgcn_sched_barrier(0);
            load_w(R[2], min(2, kmax));
            __builtin_amdgcn_sched_barrier(0);
            store_w(R[0], 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            load_w(R[0], min(3, kmax));
            __builtin_amdgcn_sched_barrier(0);
            store_w(R[1], STAGE, min(1, kmax));
            __builtin_amdgcn_sched_barrier(0);
            load_w(R[1], min(4, kmax));
            __builtin_amdgcn_sched_barrier(0);
            wait_left(2 * W_LOADS + vec_loads(min(3, kmax)) + vec_loads(min(4, kmax)));
            barrier_keep_vmem();
            // Step k with k % 3 == J: step k+2's registers (set (J+2) % 3)
            // into stage (J+2) % 3, which the consumers finished reading
            // before the previous barrier, then that set reloaded with step
            // k+5.  Steps past the last reload and rewrite the last step.
            auto step = [&](auto J_, int k) {
                constexpr int J = decltype(J_)::value;
                constexpr uint32_t wr = ((J + 2) % 3) * STAGE;
                Regs &g = R[(J + 2) % 3];
                load_x(wr, min(k + 2, kmax));
                __builtin_amdgcn_sched_barrier(0);
                store_w(g, wr, min(k + 2, kmax));
                __builtin_amdgcn_sched_barrier(0);
                load_w(g, min(k + 5, kmax));
                __builtin_amdgcn_sched_barrier(0);
                wait_left(W_LOADS + vec_loads(min(k + 5, kmax)));   // this step's x (and every older load) landed
                barrier_keep_vmem();
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
            // half 0 of every row, computed by substeps 0 and 1 only.  The
            // consumers finished reading the real data of every stage before
            // the last barrier, so stage 0 is free.
            const int kt = ksteps;
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i)
                if ((ptid & 7) < 4)
                    *reinterpret_cast<u32x4 *>(smem + a_st + i * PT * 16) =
                        __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[i], kt * (BK * 2), 0);
            if (b_part < SPR / 2) {                     // the slices of k = 0 .. 31 of the step
                const int gk = ((kt * BK) >> group_shift) * 2;
#pragma unroll
                for (int i = 0; i < B_SLICES; ++i) {
                    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(wr_, woff[i], kt * (BK * BITS / 8), 0);
                    const _Float16 sv = bitcast<_Float16>(__builtin_amdgcn_raw_buffer_load_b16(sr, soff[i], gk, 0));
                    const _Float16 zb = bitcast<_Float16>(__builtin_amdgcn_raw_buffer_load_b16(zr, soff[i], gk, 0)) +
                                        (_Float16)1024.0f;
                    store_slice(0, i, w, f16x2{sv, sv}, f16x2{zb, zb});
                }
            }
            __syncthreads();
        }
    }

    // The MFMAs take the weight fragment as first operand, so tile (i, j)
    // holds y^T: lane l, register r is output channel 4 * (l / 16) + r of
    // the tile's 16, for x row l % 16.  The consumers write their fp16
    // results to LDS (row-major, rows padded to YS bytes, each lane writing
    // its 4 consecutive channels as 8 bytes), then all threads store 16-byte
    // pieces of whole rows, 16 lanes per 256-byte row, so y is written in
    // full cache lines.  Every wave passed the last barrier after its last
    // read of a stage, and the barrier below orders the rest.
    constexpr int YS = BN * 2 + 16;
    static_assert(BM * YS <= kStages * STAGE, "output tile exceeds LDS");
    __syncthreads();
    if (wave < kConsumers) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wave * WT_M + i * 16 + (lane & 15);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int c = j * 16 + 4 * (lane >> 4);
                const f16x2 lo = {(_Float16)acc[i][j][0], (_Float16)acc[i][j][1]};
                const f16x2 hi = {(_Float16)acc[i][j][2], (_Float16)acc[i][j][3]};
                *reinterpret_cast<u32x2 *>(smem + r * YS + c * 2) = u32x2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
            }
        }
    }
    __syncthreads();
    constexpr int CPR = BN / 8;                          // 16-byte pieces per row
    constexpr int RPP = kGemmThreads / CPR;              // rows per pass
    static_assert(CPR * RPP == kGemmThreads && BM % RPP == 0, "output tile does not split evenly");
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

template <int BM, int BN, int BITS, bool PAIR_SZ, int SZV = 1>
hipError_t launch_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                       const uint16_t *zeros, int m, int n_out, int n_in, int group_shift,
                       uint16_t *y, hipStream_t stream, const char **query)
{
    if (query) {
        // the kernel's name in the form profilers print it
        static const std::string s = "gemm_kernel<" + std::to_string(BM) + ", " + std::to_string(BN) + ", " +
                                     std::to_string(BITS) + ", " + (PAIR_SZ ? "true" : "false") + ", " +
                                     std::to_string(SZV) + ">";
        *query = s.c_str();
        return hipSuccess;
    }
    const int tiles_m = (m + BM - 1) / BM, tiles_n = (n_out + BN - 1) / BN;
    const size_t lds = kStages * (size_t)(BM + BN) * 128;
    // steps per run of SZV groups: SZV << (group_shift - 6), a power of two
    int sz_log2p = 0;
    if (SZV > 1) sz_log2p = (SZV == 8 ? 3 : 1) + group_shift - 6;
    auto kernel = gemm_kernel<BM, BN, BITS, PAIR_SZ, SZV>;
    static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    kernel<<<dim3((unsigned)(tiles_m * tiles_n)), dim3(kGemmThreads), lds, stream>>>(
        x, qweight, scales, zeros, y, m, n_out, n_in, group_shift, tiles_m, tiles_n, sz_log2p);
    return hipGetLastError();
}

// Slices of one row and group per lane pair (PAIR_SZ): scale vectors of 8
// groups where the rows' runs of groups are 16-byte aligned, else of 2 where
// 4-byte aligned, for groups of 64 to 256 (a run then spans whole steps);
// otherwise one gather per step.
template <int BITS>
hipError_t launch_paired(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                         const uint16_t *zeros, int m, int n_out, int n_in, int shift, uint16_t *y,
                         hipStream_t stream, const char **query)
{
    const int groups = shift >= 31 ? 1 : n_in >> shift;
    const uintptr_t a = reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(zeros);
    if (shift >= 6 && shift <= 8 && groups % 8 == 0 && (a & 15) == 0)
        return launch_gemm<256, 128, BITS, true, 8>(x, qweight, scales, zeros, m, n_out, n_in, shift, y, stream, query);
    if (shift >= 6 && shift <= 8 && groups % 2 == 0 && (a & 3) == 0)
        return launch_gemm<256, 128, BITS, true, 2>(x, qweight, scales, zeros, m, n_out, n_in, shift, y, stream, query);
    return launch_gemm<256, 128, BITS, true>(x, qweight, scales, zeros, m, n_out, n_in, shift, y, stream, query);
}

}  // namespace

hipError_t q4_launch_gemm(const uint16_t *x, const uint32_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, int64_t m, int64_t n_out, int64_t n_in,
                          int group_size, int bits, uint16_t *y, hipStream_t stream, const char **query)
{
    // group k of a row is k >> shift; a per-channel group of any other
    // length than a power of two uses shift 31 (every k in group 0)
    int shift = 0;
    while ((1 << shift) < group_size) ++shift;
    if ((1 << shift) != group_size) shift = 31;
    if (bits == 8)
        return launch_paired<8>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream, query);
    // INT4 slices hold 32 codes: with groups of 32 the two slices of a row
    // step belong to different groups
    if (group_size == 32)
        return launch_gemm<256, 128, 4, false>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y,
                                               stream, query);
    return launch_paired<4>(x, qweight, scales, zeros, (int)m, (int)n_out, (int)n_in, shift, y, stream, query);
}
