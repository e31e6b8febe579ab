// Pack time: absmean ternarisation, optional N:M magnitude mask, 2-bit packing.
//
// "BitNet 논문 분석: 1-Bit LLM의 시대", section "Absmean 양자화 함수"
// (weight_quant_ternary): beta = mean |W| over the whole matrix, then
// t = clamp(round(W / (beta + 1e-5)), -1, 1).  "BitNet b1.58 2B4T Technical
// Report 요약 설명", sec. 5.1: four ternary weights per int8; the I2_S code
// ("bitnet.cpp 추론 프레임워크") maps -1, 0, +1 to 00, 01, 10.
// "Sparse-BitNet ..." review, sec. 3.2: the N:M mask keeps the N largest
// |latent weight| per block of M and is applied after ternarisation, with
// beta taken over the full, unmasked matrix.
//
// beta is accumulated in binary64 in a fixed order -- each row k-ascending,
// then the row sums n-ascending -- so the result does not depend on the launch
// shape.  Pack is offline (weights are packed once and stored packed), so the
// ordered sums favour reproducibility over speed.
#include "kernels.hpp"

namespace bl {
namespace {

constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void row_abs_sum_kernel(const float *__restrict__ W, int64_t N,
                                                             int64_t K, double *__restrict__ rowsum)
{
    const int64_t n = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (n >= N) return;
    const float4 *w4 = reinterpret_cast<const float4 *>(W + n * K);
    double s = 0.0;
    for (int64_t i = 0; i < K / 4; ++i) {
        const float4 v = w4[i];
        s += fabs((double)v.x);
        s += fabs((double)v.y);
        s += fabs((double)v.z);
        s += fabs((double)v.w);
    }
    rowsum[n] = s;
}

__global__ void beta_kernel(const double *__restrict__ rowsum, int64_t N, int64_t K,
                            float *__restrict__ w_scale)
{
    if (blockIdx.x != 0 || threadIdx.x != 0) return;
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n) total += rowsum[n];
    w_scale[0] = (float)(total / (double)(N * K));
}

__device__ __forceinline__ uint32_t ternary_code(float w, float d)
{
    float r = rintf(w / d);                    // IEEE binary32 division, half to even
    r = fminf(fmaxf(r, -1.0f), 1.0f);
    return (uint32_t)((int)r + 1);
}

// One thread per 16-weight word; rows are contiguous and K % 16 == 0, so word
// i covers floats [16 i, 16 i + 16) of the row-major matrix.
__global__ __launch_bounds__(kBlock) void pack_dense_kernel(const float *__restrict__ W, int64_t words,
                                                            const float *__restrict__ w_scale,
                                                            uint32_t *__restrict__ out)
{
    const float d = w_scale[0] + 1e-5f;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * kBlock) {
        const float4 *w4 = reinterpret_cast<const float4 *>(W + i * 16);
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = w4[q];
            word |= ternary_code(v.x, d) << code_bit(4 * q + 0);
            word |= ternary_code(v.y, d) << code_bit(4 * q + 1);
            word |= ternary_code(v.z, d) << code_bit(4 * q + 2);
            word |= ternary_code(v.w, d) << code_bit(4 * q + 3);
        }
        out[i] = word;
    }
}

// One thread per (row, 64-weight superblock).  Within each group of M the kept
// set is {i : rank(i) < N}, rank(i) = #{j : |w_j| > |w_i|} +
// #{j < i : |w_j| == |w_i|}: the N largest magnitudes, ties to the lower k.
template <Pattern P>
__global__ __launch_bounds__(kBlock) void pack_nm_kernel(const float *__restrict__ W, int64_t N,
                                                         int64_t K, const float *__restrict__ w_scale,
                                                         uint8_t *__restrict__ out)
{
    constexpr int GM = (P == Pattern::NM24) ? 4 : 8;     // group size M
    constexpr int GN = (P == Pattern::NM24) ? 2 : 6;     // kept per group N
    constexpr int VW = 64 * GN / GM / 16;                // value words per superblock
    const int64_t sbs = K / 64;
    const int64_t vrow = nm_value_row_bytes(K, GN, GM);
    const int64_t mrow = nm_mask_row_bytes(K);
    const float d = w_scale[0] + 1e-5f;
    for (int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x; idx < N * sbs;
         idx += (int64_t)gridDim.x * kBlock) {
        const int64_t n = idx / sbs, sb = idx % sbs;
        const float4 *w4 = reinterpret_cast<const float4 *>(W + n * K + sb * 64);
        float w[64];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float4 v = w4[q];
            w[4 * q + 0] = v.x;
            w[4 * q + 1] = v.y;
            w[4 * q + 2] = v.z;
            w[4 * q + 3] = v.w;
        }
        uint32_t vals[VW];
        uint32_t masks[2] = {0u, 0u};
#pragma unroll
        for (int v = 0; v < VW; ++v) vals[v] = 0u;
#pragma unroll
        for (int g = 0; g < 64 / GM; ++g) {
            uint32_t mk = 0u;
#pragma unroll
            for (int i = 0; i < GM; ++i) {
                const float mi = fabsf(w[g * GM + i]);
                int rank = 0;
#pragma unroll
                for (int j = 0; j < GM; ++j) {
                    const float mj = fabsf(w[g * GM + j]);
                    rank += (mj > mi) || (j < i && mj == mi);
                }
                mk |= (rank < GN ? 1u : 0u) << i;
            }
            // kept codes of this group as a linear run (kept code r at bits 2r)
            uint32_t lin = 0u;
#pragma unroll
            for (int i = 0; i < GM; ++i) {
                const uint32_t below = __builtin_popcount(mk & ((1u << i) - 1u));
                const uint32_t code = ternary_code(w[g * GM + i], d);
                lin |= ((mk >> i) & 1u) ? (code << (2 * below)) : 0u;
            }
#pragma unroll
            for (int r = 0; r < GN; ++r) {
                const int c = GN * g + r;                    // kept-code index in the superblock
                vals[c >> 4] |= ((lin >> (2 * r)) & 3u) << code_bit(c & 15);
            }
            if (GM == 4) masks[g >> 3] |= mk << (4 * (g & 7));
            else         masks[g >> 2] |= mk << (8 * (g & 3));
        }
        uint32_t *vout = reinterpret_cast<uint32_t *>(out + n * vrow + sb * (VW * 4));
#pragma unroll
        for (int v = 0; v < VW; ++v) vout[v] = vals[v];
        uint32_t *mout = reinterpret_cast<uint32_t *>(out + N * vrow + n * mrow + sb * 8);
        mout[0] = masks[0];
        mout[1] = masks[1];
    }
}

unsigned grid_for(int64_t items)
{
    int64_t blocks = (items + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;          // grid-stride beyond this
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_absmean(const float *W, int64_t N, int64_t K, double *rowsum, float *w_scale,
                          hipStream_t stream)
{
    hipLaunchKernelGGL(row_abs_sum_kernel, dim3((unsigned)((N + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                       stream, W, N, K, rowsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(beta_kernel, dim3(1), dim3(64), 0, stream, rowsum, N, K, w_scale);
    return hipGetLastError();
}

hipError_t launch_pack(const float *W, int64_t N, int64_t K, Pattern p, const float *w_scale,
                       uint8_t *packed, hipStream_t stream)
{
    switch (p) {
    case Pattern::Dense: {
        const int64_t words = N * K / 16;
        hipLaunchKernelGGL(pack_dense_kernel, dim3(grid_for(words)), dim3(kBlock), 0, stream, W, words,
                           w_scale, reinterpret_cast<uint32_t *>(packed));
        break;
    }
    case Pattern::NM24:
        hipLaunchKernelGGL(pack_nm_kernel<Pattern::NM24>, dim3(grid_for(N * (K / 64))), dim3(kBlock), 0,
                           stream, W, N, K, w_scale, packed);
        break;
    case Pattern::NM68:
        hipLaunchKernelGGL(pack_nm_kernel<Pattern::NM68>, dim3(grid_for(N * (K / 64))), dim3(kBlock), 0,
                           stream, W, N, K, w_scale, packed);
        break;
    }
    return hipGetLastError();
}

}  // namespace bl
