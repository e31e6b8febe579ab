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
// shape.  Pack is offline (weights are packed once and stored packed); the
// ordered sums are dependent chains of binary64 adds, so only their loads are
// spread over the workgroup.
#include "kernels.hpp"

namespace bl {
namespace {

constexpr int kBlock = 256;

// Row sums: a workgroup takes kSumRows rows; the whole workgroup stages
// column chunks of them in LDS with coalesced loads, and thread r adds row
// r's chunk in k order (the ordered sum is a chain of dependent binary64
// adds; the loads around it are what this layout speeds up: 11008 x 2048
// took 190-290 us with one thread per row reading its own row).
constexpr int kSumRows = 32, kSumCols = 256;

__global__ __launch_bounds__(kBlock) void row_abs_sum_kernel(const float *__restrict__ W, int64_t N,
                                                             int64_t K, double *__restrict__ rowsum)
{
    // row stride kSumCols + 1 words: thread r reads bank (r + c) % 64 at column c
    constexpr int kPer = kSumRows * kSumCols / kBlock;             // staged floats per thread
    __shared__ float tile[kSumRows * (kSumCols + 1)];
    const int64_t n0 = (int64_t)blockIdx.x * kSumRows;
    const int rows = (int)min((int64_t)kSumRows, N - n0);
    const int t = threadIdx.x;
    // the next chunk in registers while the current one is summed
    float pre[kPer];
    auto fetch = [&](int64_t k0) {
        const int cols = (int)min((int64_t)kSumCols, K - k0);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = t + j * kBlock, r = i / kSumCols, c = i % kSumCols;
            pre[j] = (r < rows && c < cols) ? W[(n0 + r) * K + k0 + c] : 0.0f;
        }
    };
    fetch(0);
    double s = 0.0;
    for (int64_t k0 = 0; k0 < K; k0 += kSumCols) {
        const int cols = (int)min((int64_t)kSumCols, K - k0);
        __syncthreads();                                           // the previous chunk is consumed
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = t + j * kBlock;
            tile[(i / kSumCols) * (kSumCols + 1) + i % kSumCols] = pre[j];
        }
        __syncthreads();
        if (k0 + kSumCols < K) fetch(k0 + kSumCols);
        if (t < rows) {
            // 16 LDS reads ahead of each 16 adds: only the adds form the chain
            const float *row = tile + t * (kSumCols + 1);
            int c = 0;
            for (; c + 16 <= cols; c += 16) {
                float v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = row[c + j];
#pragma unroll
                for (int j = 0; j < 16; ++j) s += fabs((double)v[j]);
            }
            for (; c < cols; ++c) s += fabs((double)row[c]);
        }
    }
    if (t < rows) rowsum[n0 + t] = s;
}

// The row sums in n order, by one thread, from LDS chunks filled by all.
constexpr int kBetaChunk = 4096;

__global__ __launch_bounds__(kBlock) void beta_kernel(const double *__restrict__ rowsum, int64_t N, int64_t K,
                                                      float *__restrict__ w_scale)
{
    __shared__ double part[kBetaChunk];
    double total = 0.0;
    for (int64_t n0 = 0; n0 < N; n0 += kBetaChunk) {
        const int cnt = (int)min((int64_t)kBetaChunk, N - n0);
        __syncthreads();
        for (int i = threadIdx.x; i < cnt; i += kBlock) part[i] = rowsum[n0 + i];
        __syncthreads();
        if (threadIdx.x == 0) {
            int i = 0;
            for (; i + 16 <= cnt; i += 16) {
                double v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = part[i + j];
#pragma unroll
                for (int j = 0; j < 16; ++j) total += v[j];
            }
            for (; i < cnt; ++i) total += part[i];
        }
    }
    if (threadIdx.x == 0) w_scale[0] = (float)(total / (double)(N * K));
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

// N:M-masked weights in the dense layout, for any N <= M with M in {4, 8,
// 16}: the mask of pack_nm_kernel (the N largest magnitudes per group of M,
// ties to the lower k), the kept weights' codes c = t + 1 and code 1 (t = 0)
// at the pruned positions, 16 codes per word.  One thread per (row,
// 64-weight superblock).
template <int GM>
__global__ __launch_bounds__(kBlock) void pack_nm_dense_kernel(const float *__restrict__ W, int64_t N, int64_t K,
                                                               int gn, const float *__restrict__ w_scale,
                                                               uint32_t *__restrict__ out)
{
    const int64_t sbs = K / 64;
    const float d = w_scale[0] + 1e-5f;
    for (int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x; idx < N * sbs;
         idx += (int64_t)gridDim.x * kBlock) {
        const float4 *w4 = reinterpret_cast<const float4 *>(W + idx * 64);   // row n, superblock sb: contiguous
        float w[64];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float4 v = w4[q];
            w[4 * q + 0] = v.x;
            w[4 * q + 1] = v.y;
            w[4 * q + 2] = v.z;
            w[4 * q + 3] = v.w;
        }
        uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < 64 / GM; ++g) {
#pragma unroll
            for (int i = 0; i < GM; ++i) {
                const float mi = fabsf(w[g * GM + i]);
                int rank = 0;
#pragma unroll
                for (int j = 0; j < GM; ++j) {
                    const float mj = fabsf(w[g * GM + j]);
                    rank += (mj > mi) || (j < i && mj == mi);
                }
                const int k = g * GM + i;
                const uint32_t code = rank < gn ? ternary_code(w[k], d) : 1u;
                words[k >> 4] |= code << code_bit(k & 15);
            }
        }
        uint4 *o = reinterpret_cast<uint4 *>(out + idx * 4);
        *o = make_uint4(words[0], words[1], words[2], words[3]);
    }
}

// 2:4 weights in the trit-packed storage: per group of 4 inputs the mask of
// pack_nm_kernel (the two largest |w|, ties to the lower k), kept inputs
// i0 < i1, and one 6-bit code 9 p + 3 c(i0) + c(i1), with c = t + 1 and p the
// index of (i0, i1) in (0,1) (0,2) (0,3) (1,2) (1,3) (2,3).  The 16 codes of
// 64 consecutive inputs form one 96-bit little-endian string (group g at bit
// 6 g), 12 bytes; a row is its K / 64 strings in k order, rows back to back,
// so string i of the matrix sits at byte 12 i.  One thread per string.
__global__ __launch_bounds__(kBlock) void pack_trit24_kernel(const float *__restrict__ W, int64_t strings,
                                                             const float *__restrict__ w_scale,
                                                             uint32_t *__restrict__ out)
{
    const float d = w_scale[0] + 1e-5f;
    for (int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x; idx < strings;
         idx += (int64_t)gridDim.x * kBlock) {
        const float4 *w4 = reinterpret_cast<const float4 *>(W + idx * 64);
        uint32_t words[3] = {0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            const float4 v = w4[g];
            const float w[4] = {v.x, v.y, v.z, v.w};
            uint32_t mk = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float mi = fabsf(w[i]);
                int rank = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float mj = fabsf(w[j]);
                    rank += (mj > mi) || (j < i && mj == mi);
                }
                mk |= (rank < 2 ? 1u : 0u) << i;
            }
            // the ranks are a permutation of 0..3: exactly two bits are set
            const int i0 = __builtin_ctz(mk), i1 = 31 - __builtin_clz(mk);
            const uint32_t p = (uint32_t)(i0 == 0 ? i1 - 1 : i0 == 1 ? i1 + 1 : 5);
            uint32_t c0 = 0u, c1 = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t c = ternary_code(w[i], d);
                c0 = (i == i0) ? c : c0;
                c1 = (i == i1) ? c : c1;
            }
            const uint32_t code = 9u * p + 3u * c0 + c1;
            const int bit = 6 * g, wi = bit >> 5, o = bit & 31;
            words[wi] |= code << o;
            if (o > 26) words[wi + 1] |= code >> (32 - o);
        }
        uint32_t *o = out + idx * 3;
        o[0] = words[0];
        o[1] = words[1];
        o[2] = words[2];
    }
}

unsigned grid_for(int64_t items)
{
    int64_t blocks = (items + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;          // grid-stride beyond this
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_pack_nm_dense(const float *W, int64_t N, int64_t K, int n, int m, const float *w_scale,
                                uint8_t *packed, hipStream_t stream)
{
    uint32_t *o = reinterpret_cast<uint32_t *>(packed);
    const dim3 grid(grid_for(N * (K / 64)));
    switch (m) {
    case 4: hipLaunchKernelGGL(pack_nm_dense_kernel<4>, grid, dim3(kBlock), 0, stream, W, N, K, n, w_scale, o); break;
    case 8: hipLaunchKernelGGL(pack_nm_dense_kernel<8>, grid, dim3(kBlock), 0, stream, W, N, K, n, w_scale, o); break;
    case 16: hipLaunchKernelGGL(pack_nm_dense_kernel<16>, grid, dim3(kBlock), 0, stream, W, N, K, n, w_scale, o); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pack_trit24(const float *W, int64_t N, int64_t K, const float *w_scale, uint8_t *packed,
                              hipStream_t stream)
{
    const int64_t strings = N * (K / 64);
    hipLaunchKernelGGL(pack_trit24_kernel, dim3(grid_for(strings)), dim3(kBlock), 0, stream, W, strings, w_scale,
                       reinterpret_cast<uint32_t *>(packed));
    return hipGetLastError();
}

hipError_t launch_absmean(const float *W, int64_t N, int64_t K, double *rowsum, float *w_scale,
                          hipStream_t stream)
{
    hipLaunchKernelGGL(row_abs_sum_kernel, dim3((unsigned)((N + kSumRows - 1) / kSumRows)), dim3(kBlock), 0,
                       stream, W, N, K, rowsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(beta_kernel, dim3(1), dim3(kBlock), 0, stream, rowsum, N, K, w_scale);
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
