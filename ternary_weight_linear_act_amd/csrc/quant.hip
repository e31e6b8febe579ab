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
#include "kernels.hpp"

namespace bl {
namespace {

constexpr int kQuantBlock = 256;
constexpr int kWaves = kQuantBlock / 64;

__global__ __launch_bounds__(kQuantBlock) void quant_act_kernel(
    const float *__restrict__ X, int64_t K, int8_t *__restrict__ Xq,
    float *__restrict__ x_scale, int32_t *__restrict__ x_rowsum)
{
    __shared__ float s_max[kWaves];
    __shared__ int s_sum[kWaves];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float4 *x4 = reinterpret_cast<const float4 *>(X + row * K);
    int *q4 = reinterpret_cast<int *>(Xq + row * K);
    const int64_t n4 = K / 4;

    float g = 0.0f;
    for (int64_t i = tid; i < n4; i += kQuantBlock) {
        const float4 v = x4[i];
        g = fmaxf(g, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    g = wave_max_dpp(g);
    if (lane == 0) s_max[wave] = g;
    __syncthreads();
    g = s_max[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) g = fmaxf(g, s_max[w]);

    int sum = 0;
    const float up = act_prescale(g);
    const float s = act_scale(g, up);        // IEEE binary32 division
    if (up == 1.0f) {
        for (int64_t i = tid; i < n4; i += kQuantBlock) {
            const float4 v = x4[i];
            int s4;
            q4[i] = (int)act_quant4(v.x, v.y, v.z, v.w, s, &s4);
            sum += s4;
        }
    } else {
        for (int64_t i = tid; i < n4; i += kQuantBlock) {
            const float4 v = x4[i];
            int s4;
            q4[i] = (int)act_quant4(v.x * up, v.y * up, v.z * up, v.w * up, s, &s4);
            sum += s4;
        }
    }
    sum = wave_sum_dpp(sum);
    if (lane == 0) s_sum[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += s_sum[w];
        x_scale[row] = (g == 0.0f) ? 0.0f : g / 127.0f;
        if (x_rowsum) x_rowsum[row] = total;
    }
}

}  // namespace

hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *x_scale,
                            int32_t *x_rowsum, hipStream_t stream)
{
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)M), dim3(kQuantBlock), 0, stream, X, K, Xq,
                       x_scale, x_rowsum);
    return hipGetLastError();
}

}  // namespace bl
