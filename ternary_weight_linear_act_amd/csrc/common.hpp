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
__host__ __device__ __forceinline__ void decode_superblock(const uint32_t *vals, const uint32_t *masks,
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
// Faster N:M decode.  The interleaved code layout above is a 4 x 4 matrix of
// 2-bit cells (byte = row); its transpose is the linear layout, code j at
// bits 2j.  In linear order a group's kept codes form a short run, and the
// dense group is that run with code 01 inserted at the pruned positions:
//  - 2:4 (16 groups per superblock): a 256-entry table, indexed by the keep
//    nibble and the 4 bits of the two kept codes, gives the group's 8 bits;
//  - 6:8 (8 groups): the two pruned positions p < q come from the zero bits
//    of the keep byte, and 01 is inserted at p, then at q.
// Same results as decode_superblock (the exhaustive and random checks in the
// test suite compare the two paths through the forward kernels).
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ uint32_t code_transpose(uint32_t x)
{
    uint32_t t = (x ^ (x >> 6)) & 0x00CC00CCu;
    x ^= t ^ (t << 6);
    t = (x ^ (x >> 12)) & 0x0000F0F0u;
    x ^= t ^ (t << 12);
    return x;
}

// code 01 inserted at position p (0..7) of a linear run of 2-bit codes
__host__ __device__ __forceinline__ uint32_t insert_zero_code(uint32_t run, uint32_t p)
{
    const uint32_t lo = run & ((1u << (2 * p)) - 1u);
    return lo | (1u << (2 * p)) | ((run >> (2 * p)) << (2 * p + 2));
}

// entry idx of the 2:4 table: keep nibble idx & 15, kept codes idx >> 4
__host__ __device__ inline uint8_t nm24_table_entry(uint32_t idx)
{
    const uint32_t keep = idx & 15u, run = idx >> 4;
    uint32_t pruned[2] = {0, 0}, np = 0;
    for (uint32_t i = 0; i < 4; ++i)
        if (!((keep >> i) & 1u) && np < 2) pruned[np++] = i;
    if (np != 2) return 0x55;                      // not a 2:4 mask: never produced by the packer
    return (uint8_t)insert_zero_code(insert_zero_code(run, pruned[0]), pruned[1]);
}

template <Pattern P>
__host__ __device__ __forceinline__ void decode_superblock_fast(const uint32_t *vals, const uint32_t *masks,
                                                                 uint32_t dense[4], const uint8_t *table24)
{
    if constexpr (P == Pattern::NM24) {
        const uint32_t v[2] = {code_transpose(vals[0]), code_transpose(vals[1])};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t vw = v[d >> 1], mw = masks[d >> 1];
            uint32_t lin = 0;
#pragma unroll
            for (int gl = 0; gl < 4; ++gl) {
                const int off = 16 * (d & 1) + 4 * gl;
                const uint32_t idx = ((mw >> off) & 15u) | (((vw >> off) & 15u) << 4);
                lin |= (uint32_t)table24[idx] << (8 * gl);
            }
            dense[d] = code_transpose(lin);
        }
    } else {
        const uint64_t lo = (uint64_t)code_transpose(vals[0]) | ((uint64_t)code_transpose(vals[1]) << 32);
        const uint64_t hi = (uint64_t)code_transpose(vals[1]) | ((uint64_t)code_transpose(vals[2]) << 32);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t lin = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int g = 2 * d + h, off = 12 * g;
                const uint32_t run = (uint32_t)((off + 12 <= 64 ? lo >> off : hi >> (off - 32)) & 0xFFFu);
                const uint32_t pm = ~(masks[g >> 2] >> (8 * (g & 3))) & 0xFFu;
                const uint32_t p = __builtin_ctz(pm | 0x80u), q = 31 - __builtin_clz(pm | 1u);
                lin |= insert_zero_code(insert_zero_code(run, p), q) << (16 * h);
            }
            dense[d] = code_transpose(lin);
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
constexpr int kDppRowMirror = 0x140;       // lane i <- lane 15 - i within each row of 16
constexpr int kDppRowHalfMirror = 0x141;   // lane i <- lane 7 - i within each half row of 8

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

// ---------------------------------------------------------------------------
// One-token N:M dot product without decoding to dense codes (the one-token
// decode kernel).  A value word's 16 kept codes c = t + 1 become 64 * t as
// signed bytes: (c - 1) mod 4 per 2-bit field by an add that cannot carry out
// of its field, then each field moved to the top of its byte.  Byte b of u[s]
// holds kept code 4s + b of the word, the order of the packed layout.
// ---------------------------------------------------------------------------
__host__ __device__ inline void nm_tbytes(uint32_t V, uint32_t u[4])
{
    const uint32_t t2 = ((V & 0x55555555u) + 0x55555555u) ^ (~V & 0xAAAAAAAAu);
    u[0] = (t2 << 6) & 0xC0C0C0C0u;
    u[1] = (t2 << 4) & 0xC0C0C0C0u;
    u[2] = (t2 << 2) & 0xC0C0C0C0u;
    u[3] = t2 & 0xC0C0C0C0u;
}

// Byte-permute selectors (v_perm_b32: values 0-3 pick a byte of the second
// source, 4-7 of the first, 12 gives a zero byte) that spread a group's kept
// t-bytes over its positions; pruned positions get zero bytes.
//   2:4: entry i = the mask byte of groups 2h, 2h+1 (even group in the low
//        nibble).  Source: the word whose bytes 0-1 are the even group's kept
//        t-bytes and 2-3 the odd group's.  lo / hi select the even / odd
//        group's 4 positions.
//   6:8: entry i = mask byte | (group parity << 8).  Sources: the two t-byte
//        words holding the group's 6 kept codes, which start at byte 0 of the
//        first (even group) or byte 2 (odd).  lo / hi: positions 0-3 / 4-7.
constexpr int nm_sel_entries(Pattern p) { return p == Pattern::NM24 ? 256 : 512; }

template <Pattern P>
__host__ __device__ inline void nm_sel_entry(int i, uint32_t *lo, uint32_t *hi)
{
    uint64_t sel = 0x0C0C0C0C0C0C0C0Cull;
    if (P == Pattern::NM24) {
        for (int half = 0; half < 2; ++half) {
            const int m = (i >> (4 * half)) & 15;
            for (int p = 0, k = 0; p < 4; ++p)
                if ((m >> p) & 1) {
                    const int sh = 8 * (4 * half + p);
                    if (k < 2) sel = (sel & ~(0xFFull << sh)) | ((uint64_t)(2 * half + k) << sh);
                    ++k;
                }
        }
    } else {
        const int m = i & 0xFF, base = ((i >> 8) & 1) ? 2 : 0;
        for (int p = 0, k = 0; p < 8; ++p)
            if ((m >> p) & 1) {
                if (k < 6) sel = (sel & ~(0xFFull << (8 * p))) | ((uint64_t)(base + k) << (8 * p));
                ++k;
            }
    }
    *lo = (uint32_t)sel;
    *hi = (uint32_t)(sel >> 32);
}

// Half H (0 or 1) of a superblock: positions 32H .. 32H+31 as 64 * t signed
// bytes (t = 0 where pruned), e[j] = positions 32H + 4j .. +3.  vals points
// at value word H; 2:4 reads that word (groups 8H .. 8H+7), 6:8 reads words
// H and H+1 (groups 4H .. 4H+3).  mask = mask word H.  tab:
// nm_sel_entries(P) (lo, hi) word pairs.  OPS::perm(s0, s1, sel) is
// v_perm_b32 on the GPU (an emulation in the host check).
template <Pattern P, class OPS, int H>
__host__ __device__ inline void nm_expand_half(const uint32_t *vals, uint32_t mask, const uint32_t *tab, uint32_t *e)
{
    if constexpr (P == Pattern::NM24) {
        uint32_t u[4];
        nm_tbytes(vals[0], u);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t i = (mask >> (8 * s)) & 0xFFu;
            e[2 * s] = OPS::perm(u[s], u[s], tab[2 * i]);
            e[2 * s + 1] = OPS::perm(u[s], u[s], tab[2 * i + 1]);
        }
    } else {
        uint32_t u[8];                                   // t-byte words 4H .. 4H+7
        nm_tbytes(vals[0], u);
        nm_tbytes(vals[1], u + 4);
#pragma unroll
        for (int gl = 0; gl < 4; ++gl) {
            const int g = 4 * H + gl;
            const uint32_t i = ((mask >> (8 * gl)) & 0xFFu) | ((uint32_t)(g & 1) << 8);
            const int d = ((3 * g) >> 1) - 4 * H;         // first word of the group's 6 kept codes
            e[2 * gl] = OPS::perm(u[d + 1], u[d], tab[2 * i]);
            e[2 * gl + 1] = OPS::perm(u[d + 1], u[d], tab[2 * i + 1]);
        }
    }
}

// The whole superblock: e[j] = positions 4j .. 4j+3.
template <Pattern P, class OPS>
__host__ __device__ inline void nm_expand_superblock(const uint32_t *vals, const uint32_t *masks,
                                                     const uint32_t *tab, uint32_t *e)
{
    nm_expand_half<P, OPS, 0>(vals, masks[0], tab, e);
    nm_expand_half<P, OPS, 1>(vals + 1, masks[1], tab, e + 8);
}

// acc[0..3] += 64 * sum over the superblock's 64 positions of t * x, with x
// the superblock's activation bytes (16 words of 4 int8).  OPS::dot4(a, b,
// acc) is v_dot4_i32_i8 on the GPU.
template <Pattern P, class OPS>
__host__ __device__ inline void nm_dot_superblock(const uint32_t *vals, const uint32_t *masks, const uint32_t *tab,
                                                  const int32_t *xw, int *acc)
{
    uint32_t e[16];
    nm_expand_superblock<P, OPS>(vals, masks, tab, e);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j & 3] = OPS::dot4((int)e[j], xw[j], acc[j & 3]);
}

#if defined(__HIP_DEVICE_COMPILE__)
// v_perm_b32 and v_dot4_i32_i8 for nm_expand_superblock / nm_dot_superblock
struct DeviceOps {
    __device__ static uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) { return __builtin_amdgcn_perm(s0, s1, sel); }
    __device__ static int dot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }
};
#else
struct DeviceOps {
    __device__ static uint32_t perm(uint32_t, uint32_t, uint32_t);
    __device__ static int dot4(int, int, int);
};
#endif

// ---------------------------------------------------------------------------
// Per-token absmax int8 activation quantisation ("BitNet b1.58 2B4T Technical
// Report 요약 설명", sec. 2; "BitNet 논문 분석: 1-Bit LLM의 시대", section
// "Absmean 양자화 함수"): g = max|x|, s = fl32(127/g), q = rne(fl32(x*s)).
//
// A row with g < 2^-100 is first scaled by 2^100 (exact: |x| <= g), since
// fl32(127/g) overflows to +inf once g < 127/FLT_MAX; wherever the unscaled s
// is finite this gives the same q.  With that, |fl32(x*s)| <= 127 * (1 +
// 2^-23) * (1 + 2^-24) < 127.5 for finite x, so the clamp to [-128, 127]
// never binds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float act_prescale(float g) { return g < 0x1p-100f ? 0x1p100f : 1.0f; }

// s for the (prescaled) row; 0 for an all-zero row, whose codes are then 0
__device__ __forceinline__ float act_scale(float g, float up) { return g == 0.0f ? 0.0f : 127.0f / (g * up); }

// rne(fl32(x*s)) for |x*s| < 2^22: adding 1.5 * 2^23 rounds half to even
// onto the unit bits of the sum, which hold the integer in two's complement,
// so the sum's low byte is the int8 code.  The product is rounded on its
// own (no contraction: the library is built with -ffp-contract=off).
__device__ __forceinline__ uint32_t act_round_bits(float x, float s) { return __float_as_uint(x * s + 0x1.8p23f); }

// four codes packed little-endian into one word; *sum receives their sum
__device__ __forceinline__ uint32_t act_quant4(float x0, float x1, float x2, float x3, float s, int *sum)
{
    const uint32_t b0 = act_round_bits(x0, s), b1 = act_round_bits(x1, s);
    const uint32_t b2 = act_round_bits(x2, s), b3 = act_round_bits(x3, s);
    *sum = (int)(b0 + b1 + b2 + b3 - 4u * 0x4B400000u);
    return (b0 & 0xFFu) | ((b1 & 0xFFu) << 8) | ((b2 & 0xFFu) << 16) | (b3 << 24);
}


// ---------------------------------------------------------------------------
// Transform of an activation row before the quantiser, for the steps either
// side of a BitNet linear ("BitNet b1.58 2B4T Technical Report 요약 설명",
// sec. 2: squared ReLU in the feed-forward network, subln; "BitNet 논문
// 분석: 1-Bit LLM의 시대", section "Absmean 양자화 함수": BitLinear_b158
// normalises its input with an RMSNorm before activation_quant).
//   kTrGate: h = fl32(fl32(r * r) * up), r = max(x, 0)   (else h = x)
//   kTrNorm: RMSNorm with weight gamma.  Its per-row factor 1/rms divides
//            out of the absmax codes, so the codes are those of
//            v = fl32(h * gamma) and 1/rms goes into the scale:
//            rinv = 1 / sqrt(sum h^2 / K + eps) in binary64 (each square
//            exact), x_scale = fl32(max|v| / 127 * rinv).
// Only the sum's order differs between evaluations: its relative error is at
// most K * 2^-53 (non-negative terms), far below binary32's half-ulp, so
// x_scale can differ from an in-order evaluation by one ulp at most.
// ---------------------------------------------------------------------------
constexpr int kTrGate = 1, kTrNorm = 2;

struct ActTransform {
    const float *up;      // M x K, kTrGate
    const float *gamma;   // K, kTrNorm
    float eps;
};

__device__ __forceinline__ float act_gate(float x, float u)
{
    const float r = fmaxf(x, 0.0f);
    return (r * r) * u;
}

__device__ __forceinline__ double act_rinv(double ss, int64_t K, float eps)
{
    return 1.0 / sqrt(ss / (double)K + (double)eps);
}

__device__ __forceinline__ float act_norm_scale(float g, double rinv)
{
    return g == 0.0f ? 0.0f : (float)((double)g / 127.0 * rinv);
}

// Whole-wave binary64 sum on the same DPP lane moves as the reductions above
// (each half of the double moved on its own).  The association differs from
// lane to lane, but the four row results read out are fixed by the lane
// values, so the sum is deterministic and wave-uniform.
template <int CTRL>
__device__ __forceinline__ double dpp_move_f64(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)dpp_move<CTRL>((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)dpp_move<CTRL>((int)(uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_move_f64<kDppQuadXor1>(v);
    v += dpp_move_f64<kDppQuadXor2>(v);
    v += dpp_move_f64<kDppRowRor4>(v);
    v += dpp_move_f64<kDppRowRor8>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

}  // namespace bl
