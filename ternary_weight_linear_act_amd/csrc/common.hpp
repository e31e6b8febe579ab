// Internal helpers shared by the HIP kernels of libbitlinear (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bitlinear.h"

namespace bl {

// ---------------------------------------------------------------------------
// Packed code layout: 16 two-bit codes per little-endian 32-bit word, code j
// at bit 8*(j%4) + 2*(j/4); code = ternary + 1 (I2_S mapping 00=-1, 01=0,
// 10=+1).  (w >> 2*s) & 0x03030303 yields codes 4s..4s+3 in byte lanes 0..3.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int code_bit(int j) { return 8 * (j & 3) + 2 * (j >> 2); }

constexpr uint32_t kCodeMask = 0x03030303u;

// bytes per row of each region
__host__ __device__ inline int64_t dense_row_bytes(int64_t K) { return K / 4; }
__host__ __device__ inline int64_t nm_value_row_bytes(int64_t K, int n, int m) { return K * n / m / 4; }
__host__ __device__ inline int64_t nm_mask_row_bytes(int64_t K) { return K / 8; }

enum class Pattern { Dense, NM24, NM68 };

// Decode one 64-weight superblock of an N:M row into 4 dense code words
// (pruned positions get code 1, i.e. weight 0).
//   2:4: vals = 2 words (32 kept codes), masks = 2 words (16 nibbles)
//   6:8: vals = 3 words (48 kept codes), masks = 2 words (8 bytes)
// Every group keeps exactly N codes, so group g's kept codes are the run
// N*g .. N*g+N-1 of the value stream: all word/field indices are compile-time
// constants and only the position inside the group depends on the mask.
template <Pattern P>
__device__ __forceinline__ void decode_superblock(const uint32_t *vals, const uint32_t *masks,
                                                  uint32_t dense[4])
{
    constexpr int M = (P == Pattern::NM24) ? 4 : 8;
    constexpr int N = (P == Pattern::NM24) ? 2 : 6;
#pragma unroll
    for (int d = 0; d < 4; ++d) dense[d] = 0;
#pragma unroll
    for (int g = 0; g < 64 / M; ++g) {
        uint32_t mk;
        if (M == 4) mk = (masks[g >> 3] >> (4 * (g & 7))) & 0xFu;
        else        mk = (masks[g >> 2] >> (8 * (g & 3))) & 0xFFu;
        // this group's kept codes as a linear run, kept code r at bits 2r
        uint32_t lin = 0;
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const int c = N * g + r;
            lin |= ((vals[c >> 4] >> code_bit(c & 15)) & 3u) << (2 * r);
        }
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const int p = g * M + i;
            const uint32_t below = __builtin_popcount(mk & ((1u << i) - 1u));
            const uint32_t code = ((mk >> i) & 1u) ? ((lin >> (2 * below)) & 3u) : 1u;
            dense[p >> 4] |= code << code_bit(p & 15);
        }
    }
}

// ---------------------------------------------------------------------------
// Whole-wave reductions on DPP lane moves (no LDS round trips): xor 1 and
// xor 2 inside quads, rotations by 4 and 8 inside rows of 16, then the four
// row results are read into scalars.  Every lane must be active.  The result
// is wave-uniform.  Max is order-free; the integer sum is exact.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp_move(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = fmaxf(v, __int_as_float(dpp_move<kDppQuadXor1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<kDppQuadXor2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<kDppRowRor4>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<kDppRowRor8>(__float_as_int(v))));
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ int wave_sum_dpp(int v)
{
    v += dpp_move<kDppQuadXor1>(v);
    v += dpp_move<kDppQuadXor2>(v);
    v += dpp_move<kDppRowRor4>(v);
    v += dpp_move<kDppRowRor8>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

}  // namespace bl
