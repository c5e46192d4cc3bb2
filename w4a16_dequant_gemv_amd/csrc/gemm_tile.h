// gemm_tile.h -- device helpers shared by the LDS-staged MFMA GEMM kernels
// (W4A16 / W8A16 in q4_gemm.hip, W8A8 in w8a8.hip): the XCD-aware tile order,
// the LDS chunk swizzle, buffer-resource flags, scheduling-group patterns and
// the waits that let direct global->LDS loads stay in flight across barriers.
#pragma once

#include <hip/hip_runtime.h>

constexpr int kXcds = 8;
constexpr int kStages = 3;
constexpr int kGroupM = 2;
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format).
constexpr int kBufferFlags = 0x00020000;

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100,
              kSgDsWrite = 0x200;

// Tile of workgroup `bid`.  Workgroup ids are dealt round-robin to the eight
// XCDs, so ids are remapped to give each XCD a contiguous range of tiles
// (XCDs 0..extra-1 own one more); tiles are numbered in bands of kGroupM row
// tiles, walked column by column inside a band, so an XCD's range covers few
// row tiles of x and its L2 shares them.
__device__ __forceinline__ void xcd_tile(int bid, int tiles_m, int tiles_n, int &tile_m, int &tile_n)
{
    const int tiles = tiles_m * tiles_n;
    const int xcd = bid % kXcds, local = bid / kXcds;
    const int per_xcd = tiles / kXcds, extra = tiles % kXcds;
    const int t = xcd < extra ? xcd * (per_xcd + 1) + local
                              : extra * (per_xcd + 1) + (xcd - extra) * per_xcd + local;
    const int band = t / (kGroupM * tiles_n);
    const int band_m = min(kGroupM, tiles_m - band * kGroupM);
    const int in_band = t - band * kGroupM * tiles_n;
    tile_n = in_band / band_m;
    tile_m = band * kGroupM + in_band % band_m;
}

// Chunk permutation of LDS row r, a function of r & 15.  Its low two bits
// differ across any 4 consecutive rows and across the 4 even (or 4 odd) rows
// of an aligned group of 8; the whole value differs across any aligned group
// of 8 rows and across the 8 even (or 8 odd) rows of an aligned group of 16.
__device__ __forceinline__ int swz(int r)
{
    return ((r ^ (r >> 2)) & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
}

// Scheduling pattern of one substep: each of its N MFMAs is followed by one
// LDS read (the first NDSR slots), NVALU vector ALU instructions, one LDS
// write (the last NDSW slots) and one global load (the first NVMEM slots).
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

// Wait until at most N vector-memory operations of this wave are
// outstanding (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt 7 and
// lgkmcnt 15 mean no wait on those); the empty asm statements keep the
// compiler from moving memory accesses across the wait.
template <int N>
__device__ __forceinline__ void wait_vmem()
{
    static_assert(N >= 0 && N < 64, "the vector-memory counter has six bits");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
    asm volatile("" ::: "memory");
}

// Workgroup barrier that waits for this wave's LDS operations only
// (lgkmcnt 0), leaving its vector-memory loads, direct LDS loads included,
// in flight; __syncthreads() would wait for all of them.
__device__ __forceinline__ void barrier_keep_vmem()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
