// Decode GEMV: y[m, n] = sum_k Xq[m, k] * W_eff[n, k] for a handful of tokens.
//
// "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 5.1: the packed ternary
// weights (four per byte) are what moves from HBM, which is the point of the
// packing; "BitNet 논문 분석: 1-Bit LLM의 시대", section "Absmean 양자화 함수":
// the product is an integer linear of the ternary weights with the int8
// activations, rescaled by the weight and activation scales.
//
// MI355X design: the weight stream is the only large operand, so each lane
// owns 16-byte chunks (64 weights) of a row and keeps U of them in flight
// with plain dwordx4 loads; LPR lanes share a row so a load instruction reads
// LPR*16 contiguous bytes per row.  Codes are unpacked in registers with one
// shift and one AND per 4 weights -- (word >> 2s) & 0x03030303 puts 4 codes in
// the 4 byte lanes -- and fed to v_dot4_i32_i8 against 4 activation bytes.
// The codes are c = t + 1 in {0,1,2}, so the lanes accumulate sum c*q and the
// epilogue subtracts the activation row sum: sum t*q = sum c*q - sum q
// (exact in int32).  The LPR partial sums are combined with xor shuffles and
// one lane per (row, token) applies the dequant scale.
#include "kernels.hpp"

namespace bl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dot4(uint32_t codes, int32_t x, int acc)
{
    return __builtin_amdgcn_sdot4((int)codes, x, acc, false);
}

// 64 weights (4 code words) against 64 activation bytes (16 dwords)
__device__ __forceinline__ int dot64(const uint32_t w[4], const i32x4 x[4], int acc)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t word = w[q];
        acc = dot4(word & kCodeMask, x[q][0], acc);
        acc = dot4((word >> 2) & kCodeMask, x[q][1], acc);
        acc = dot4((word >> 4) & kCodeMask, x[q][2], acc);
        acc = dot4((word >> 6) & kCodeMask, x[q][3], acc);
    }
    return acc;
}

// Load chunk c (64 weights) of row n as 4 dense code words.
template <Pattern P>
__device__ __forceinline__ void load_chunk(const uint8_t *__restrict__ packed, int64_t N, int64_t K,
                                           int64_t n, int64_t c, uint32_t w[4])
{
    if (P == Pattern::Dense) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(packed + n * (K / 4) + c * 16);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else {
        constexpr int GM = (P == Pattern::NM24) ? 4 : 8;
        constexpr int GN = (P == Pattern::NM24) ? 2 : 6;
        constexpr int VW = 64 * GN / GM / 16;
        const int64_t vrow = nm_value_row_bytes(K, GN, GM);
        const uint32_t *vp = reinterpret_cast<const uint32_t *>(packed + n * vrow + c * (VW * 4));
        const uint32_t *mp = reinterpret_cast<const uint32_t *>(packed + N * vrow + n * (K / 8) + c * 8);
        uint32_t vals[VW], masks[2];
#pragma unroll
        for (int v = 0; v < VW; ++v) vals[v] = vp[v];
        masks[0] = mp[0];
        masks[1] = mp[1];
        decode_superblock<P>(vals, masks, w);
    }
}

// MT tokens, LPR lanes per weight row, U chunks in flight per lane.
template <Pattern P, int MT, int LPR, int U>
__global__ __launch_bounds__(256) void gemv_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ x_scale, const int32_t *__restrict__ x_rowsum,
    const uint8_t *__restrict__ packed, const float *__restrict__ w_scale, int64_t M, int64_t N,
    int64_t K, float *__restrict__ Y, int32_t *__restrict__ acc_out)
{
    constexpr int RPW = 64 / LPR;                       // rows per wave
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t n = wave * RPW + lane / LPR;
    const int j = lane % LPR;
    const int64_t C = K / 64;                           // chunks per row

    int acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0;

    if (n < N) {
        for (int64_t c0 = j; c0 < C; c0 += (int64_t)LPR * U) {
            uint32_t w[U][4];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + (int64_t)u * LPR;
                if (c < C) load_chunk<P>(packed, N, K, n, c, w[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + (int64_t)u * LPR;
                if (c < C) {
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const i32x4 *xp = reinterpret_cast<const i32x4 *>(Xq + (int64_t)t * K + c * 64);
                        i32x4 x[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) x[q] = xp[q];
                        acc[t] = dot64(w[u], x, acc[t]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) acc[t] += __shfl_xor(acc[t], off, 64);
    }
    if (n < N && j == 0) {
        const float beta = w_scale[0];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < M) {
                const int a = acc[t] - x_rowsum[t];
                Y[(int64_t)t * N + n] = (float)a * (beta * x_scale[t]);
                if (acc_out) acc_out[(int64_t)t * N + n] = a;
            }
        }
    }
}

template <Pattern P, int MT, int LPR, int U>
hipError_t launch(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                  const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                  hipStream_t stream)
{
    constexpr int kBlock = 256;
    constexpr int rows_per_block = kBlock / LPR;
    const int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_kernel<P, MT, LPR, U>), dim3((unsigned)blocks), dim3(kBlock), 0, stream, Xq,
                       xs, rs, packed, w_scale, M, N, K, Y, acc);
    return hipGetLastError();
}

template <Pattern P>
hipError_t dispatch_mt(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                       const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                       hipStream_t stream)
{
    switch (M) {
    case 1: return launch<P, 1, 8, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
    case 2: return launch<P, 2, 8, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
    case 3: return launch<P, 3, 8, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
    default: return launch<P, 4, 8, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
    }
}

}  // namespace

// Decode GEMV for 1 <= M <= 4 tokens.
hipError_t launch_gemv(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                       const float *w_scale, Pattern p, int64_t M, int64_t N, int64_t K, float *Y,
                       int32_t *acc, hipStream_t stream)
{
    switch (p) {
    case Pattern::Dense: return dispatch_mt<Pattern::Dense>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
    case Pattern::NM24: return dispatch_mt<Pattern::NM24>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
    case Pattern::NM68: return dispatch_mt<Pattern::NM68>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace bl
