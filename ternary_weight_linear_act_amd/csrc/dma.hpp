// Shared pieces of the pipelined GEMMs: direct global->LDS loads
// (global_load_lds: the data never passes through VGPRs), the explicit vmcnt
// wait and a bare barrier that go with them, and the XCD-aware tile placement.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace bl {

constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glob_void_t;

__device__ __forceinline__ void dma16(const void *gsrc, uint8_t *ldst)
{
    __builtin_amdgcn_global_load_lds((glob_void_t *)gsrc, (lds_void_t *)ldst, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Tile placement over the 8 XCDs (each has its own L2): when the tile grid
// splits evenly into 4 x 2 regions, one region per XCD; otherwise tiles are
// dealt round-robin with consecutive logical tiles on one XCD.
__host__ __device__ inline bool xcd_regions(int64_t tiles_m, int64_t tiles_n)
{
    return tiles_m % 4 == 0 && tiles_n >= 2;
}

__host__ __device__ inline int64_t xcd_grid(int64_t tiles_m, int64_t tiles_n)
{
    if (xcd_regions(tiles_m, tiles_n)) return kXcds * (tiles_m / 4) * ((tiles_n + 1) / 2);
    return (tiles_m * tiles_n + kXcds - 1) / kXcds * kXcds;
}

// Output tile (m_tile, n_tile) of workgroup b under the placement above;
// false for a workgroup past the last tile.
__device__ __forceinline__ bool xcd_tile(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t *m_tile,
                                         int64_t *n_tile)
{
    if (xcd_regions(tiles_m, tiles_n)) {
        // each XCD owns one of 4 x 2 blocks of the tile grid: a quarter of the
        // activation rows and half of the weight columns stay in its L2
        const int64_t x = b % kXcds, j = b / kXcds;
        const int64_t mc = tiles_m / 4;
        const int64_t nlo = tiles_n * (x / 4) / 2, nhi = tiles_n * (x / 4 + 1) / 2;
        *m_tile = (x % 4) * mc + j % mc;
        *n_tile = nlo + j / mc;
        return *n_tile < nhi;
    }
    const int64_t per_xcd = (tiles_m * tiles_n + kXcds - 1) / kXcds;
    const int64_t tile = (b % kXcds) * per_xcd + b / kXcds;
    *m_tile = tile % tiles_m;
    *n_tile = tile / tiles_m;
    return tile < tiles_m * tiles_n;
}

}  // namespace bl
