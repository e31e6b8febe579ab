// Per-token absmax int8 activation quantisation.
//
// "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 2 Architecture: each
// token's activations become 8-bit integers scaled by that token's absolute
// maximum; "BitNet 논문 분석: 1-Bit LLM의 시대", section "Absmean 양자화 함수"
// (activation_quant): round, then clamp to the int8 range.  Scale 127/max|x|
// computed once per row, then multiplied in; round half to even (the
// arithmetic and the tiny-row rule are in common.hpp).
//
// One workgroup per row.  Pass 1 reads the row with 16-byte loads and reduces
// |x| to the row maximum (exact, order-free) through DPP lane moves and LDS.
// Pass 2 re-reads the row (L2-resident), quantises, stores four int8 per
// 32-bit store and reduces the int32 row sum the forward kernels need.
// Optionally the row is transformed first (ReLU^2 gate, RMSNorm; see
// common.hpp): the same two passes over the transformed values, with the
// norm's sum of squares reduced in binary64 beside max|v|.
#include "kernels.hpp"

namespace bl {
namespace {

constexpr int kQuantBlock = 256;
constexpr int kWaves = kQuantBlock / 64;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// TR: the row transform (kTrGate, kTrNorm bits; common.hpp).  Pass 1 forms
// the transformed row v (and h's sum of squares for the norm) and reduces
// max|v|; pass 2 forms v again (same operations, same values) and quantises.
template <int TR>
__global__ __launch_bounds__(kQuantBlock) void quant_act_kernel(
    const float *__restrict__ X, ActTransform tr, int64_t K, int8_t *__restrict__ Xq,
    float *__restrict__ x_scale, int32_t *__restrict__ x_rowsum)
{
    __shared__ float s_max[kWaves];
    __shared__ int s_sum[kWaves];
    __shared__ double s_ss[kWaves];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(X + row * K);
    const f32x4 *u4 = reinterpret_cast<const f32x4 *>((TR & kTrGate) ? tr.up + row * K : X);
    const f32x4 *g4 = reinterpret_cast<const f32x4 *>((TR & kTrNorm) ? tr.gamma : X);
    int *q4 = reinterpret_cast<int *>(Xq + row * K);
    const int64_t n4 = K / 4;

    // h (gated row) and v (what the codes are taken from) of entries 4i..4i+3
    auto row4 = [&](int64_t i, f32x4 &h) -> f32x4 {
        h = x4[i];
        if constexpr ((TR & kTrGate) != 0) {
            const f32x4 u = u4[i];
#pragma unroll
            for (int c = 0; c < 4; ++c) h[c] = act_gate(h[c], u[c]);
        }
        f32x4 v = h;
        if constexpr ((TR & kTrNorm) != 0) {
            const f32x4 gm = g4[i];
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = h[c] * gm[c];
        }
        return v;
    };

    float g = 0.0f;
    double ss = 0.0;
    for (int64_t i = tid; i < n4; i += kQuantBlock) {
        f32x4 h;
        const f32x4 v = row4(i, h);
        g = fmaxf(g, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        if constexpr ((TR & kTrNorm) != 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) ss += (double)h[c] * (double)h[c];
        }
    }
    g = wave_max_dpp(g);
    if (lane == 0) s_max[wave] = g;
    if constexpr ((TR & kTrNorm) != 0) {
        ss = wave_sum_f64(ss);
        if (lane == 0) s_ss[wave] = ss;
    }
    __syncthreads();
    g = s_max[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) g = fmaxf(g, s_max[w]);

    int sum = 0;
    const float up = act_prescale(g);
    const float s = act_scale(g, up);        // IEEE binary32 division
    for (int64_t i = tid; i < n4; i += kQuantBlock) {
        f32x4 h;
        f32x4 v = row4(i, h);
        if (up != 1.0f) v *= up;              // row-uniform, rare
        int s4;
        q4[i] = (int)act_quant4(v[0], v[1], v[2], v[3], s, &s4);
        sum += s4;
    }
    sum = wave_sum_dpp(sum);
    if (lane == 0) s_sum[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += s_sum[w];
        if constexpr ((TR & kTrNorm) != 0) {
            double t = 0.0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) t += s_ss[w];
            x_scale[row] = act_norm_scale(g, act_rinv(t, K, tr.eps));
        } else {
            x_scale[row] = (g == 0.0f) ? 0.0f : g / 127.0f;
        }
        if (x_rowsum) x_rowsum[row] = total;
    }
}

// ---------------------------------------------------------------------------
// 4-bit activations after an online Hadamard transform (the BitNet v2
// summary: the H-BitLinear transforms the activations, then quantises them to
// 4 bits).  Blocks of B inputs (a power of two dividing K, B <= kHChunk) are
// multiplied by the Sylvester Hadamard matrix with radix-2 butterflies, stage
// h = 1, 2, 4, ..., B/2 turning every pair (i, i + h), i & h == 0, into
// (a + b, a - b) in binary32: each value depends on its two inputs only, so
// any schedule of a stage gives the same bits.  The stages h < 8 run in
// registers on 8 consecutive values per thread, the rest in LDS.  The
// codes are the 4-bit absmax ones, 7 / max|v| (the factor 1/sqrt(B) of the
// orthonormal transform divides out of them and goes into the scale),
// stored one per int8.  Rows longer than one LDS chunk are transformed twice
// (once for the maximum, once to quantise): no scratch memory is needed.
// ---------------------------------------------------------------------------
constexpr int kHChunk = 8192;             // floats of a row transformed at a time

__device__ void hadamard_chunk(const float *__restrict__ x, int len, int64_t B, float *s_v)
{
    const int tid = threadIdx.x;
    for (int gi = tid; gi < len / 8; gi += kQuantBlock) {
        const f32x4 lo = reinterpret_cast<const f32x4 *>(x)[2 * gi], hi = reinterpret_cast<const f32x4 *>(x)[2 * gi + 1];
        float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int h = 1; h < 8; h *= 2) {
            if (h >= B) break;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (!(i & h)) {
                    const float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
        }
        reinterpret_cast<f32x4 *>(s_v)[2 * gi] = f32x4{v[0], v[1], v[2], v[3]};
        reinterpret_cast<f32x4 *>(s_v)[2 * gi + 1] = f32x4{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();
    for (int64_t h = 8; h < B; h *= 2) {
        for (int p = tid; p < len / 2; p += kQuantBlock) {
            const int i = ((p & ~(int)(h - 1)) << 1) | (p & (int)(h - 1));
            const float a = s_v[i], b = s_v[i + h];
            s_v[i] = a + b;
            s_v[i + h] = a - b;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kQuantBlock) void quant_act_h4_kernel(
    const float *__restrict__ X, int64_t K, int64_t B, int8_t *__restrict__ Xq, float *__restrict__ x_scale,
    int32_t *__restrict__ x_rowsum)
{
    __shared__ __attribute__((aligned(16))) float s_v[kHChunk];
    __shared__ float s_max[kWaves];
    __shared__ int s_sum[kWaves];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *x = X + row * K;
    const int64_t chunk = (int64_t)kHChunk / B * B;
    const bool one = K <= chunk;

    float g = 0.0f;
    for (int64_t c0 = 0; c0 < K; c0 += chunk) {
        const int len = (int)min(chunk, K - c0);
        hadamard_chunk(x + c0, len, B, s_v);
        for (int i = tid; i < len; i += kQuantBlock) g = fmaxf(g, fabsf(s_v[i]));
        if (!one) __syncthreads();
    }
    g = wave_max_dpp(g);
    if (lane == 0) s_max[wave] = g;
    __syncthreads();
    g = s_max[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) g = fmaxf(g, s_max[w]);

    const float up = act_prescale(g);
    const float s = (g == 0.0f) ? 0.0f : 7.0f / (g * up);
    int sum = 0;
    int *q4 = reinterpret_cast<int *>(Xq + row * K);
    for (int64_t c0 = 0; c0 < K; c0 += chunk) {
        const int len = (int)min(chunk, K - c0);
        if (!one) hadamard_chunk(x + c0, len, B, s_v);
        for (int i = tid; i < len / 4; i += kQuantBlock) {
            f32x4 v = reinterpret_cast<const f32x4 *>(s_v)[i];
            if (up != 1.0f) v *= up;              // row-uniform, rare
            int s4;
            q4[c0 / 4 + i] = (int)act_quant4(v[0], v[1], v[2], v[3], s, &s4);
            sum += s4;
        }
        if (!one) __syncthreads();
    }
    sum = wave_sum_dpp(sum);
    if (lane == 0) s_sum[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += s_sum[w];
        x_scale[row] = (g == 0.0f) ? 0.0f : (float)((double)g / 7.0 / sqrt((double)B));
        if (x_rowsum) x_rowsum[row] = total;
    }
}

}  // namespace

hipError_t launch_quant_act_h4(const float *X, int64_t M, int64_t K, int64_t B, int8_t *Xq, float *x_scale,
                               int32_t *x_rowsum, hipStream_t stream)
{
    if (M == 0) return hipSuccess;
    if (B < 1 || B > kHChunk || (B & (B - 1)) || K % B || K % 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_act_h4_kernel, dim3((unsigned)M), dim3(kQuantBlock), 0, stream, X, K, B, Xq, x_scale,
                       x_rowsum);
    return hipGetLastError();
}

hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *x_scale,
                            int32_t *x_rowsum, hipStream_t stream)
{
    return launch_quant_act_ex(X, ActTransform{nullptr, nullptr, 0.0f}, M, K, Xq, x_scale, x_rowsum, stream);
}

hipError_t launch_quant_act_ex(const float *X, ActTransform tr, int64_t M, int64_t K, int8_t *Xq,
                               float *x_scale, int32_t *x_rowsum, hipStream_t stream)
{
    if (M == 0) return hipSuccess;
    const int t = (tr.up ? kTrGate : 0) | (tr.gamma ? kTrNorm : 0);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)M), dim3(kQuantBlock), 0, stream, X, tr, K, Xq, x_scale,
                           x_rowsum);
    };
    switch (t) {
    case 0: go(quant_act_kernel<0>); break;
    case kTrGate: go(quant_act_kernel<kTrGate>); break;
    case kTrNorm: go(quant_act_kernel<kTrNorm>); break;
    default: go(quant_act_kernel<kTrGate | kTrNorm>); break;
    }
    return hipGetLastError();
}

}  // namespace bl
