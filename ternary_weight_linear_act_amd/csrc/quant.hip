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
template <int TR, int BLOCK = kQuantBlock>
__global__ __launch_bounds__(BLOCK) void quant_act_kernel(
    const float *__restrict__ X, ActTransform tr, int64_t K, int8_t *__restrict__ Xq,
    float *__restrict__ x_scale, int32_t *__restrict__ x_rowsum)
{
    constexpr int W = BLOCK / 64;
    __shared__ float s_max[W];
    __shared__ int s_sum[W];
    __shared__ double s_ss[W];
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
    for (int64_t i = tid; i < n4; i += BLOCK) {
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
    for (int w = 1; w < W; ++w) g = fmaxf(g, s_max[w]);

    int sum = 0;
    const float up = act_prescale(g);
    const float s = act_scale(g, up);        // IEEE binary32 division
    for (int64_t i = tid; i < n4; i += BLOCK) {
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
        for (int w = 0; w < W; ++w) total += s_sum[w];
        if constexpr ((TR & kTrNorm) != 0) {
            double t = 0.0;
#pragma unroll
            for (int w = 0; w < W; ++w) t += s_ss[w];
            x_scale[row] = act_norm_scale(g, act_rinv(t, K, tr.eps));
        } else {
            x_scale[row] = (g == 0.0f) ? 0.0f : g / 127.0f;
        }
        if (x_rowsum) x_rowsum[row] = total;
    }
}

// The plain quantiser with the row held in registers between its two steps
// (NV float4 per thread, K <= 4 NV BLOCK): the row is read once, where the
// two-pass form reads it again (from L2 if it is still there, else from the
// Infinity Cache or HBM).  Same arithmetic, same results.
template <int BLOCK, int NV>
__device__ __forceinline__ void quant_act_reg_body(const float *__restrict__ X, int64_t K,
                                                   int8_t *__restrict__ Xq, float *__restrict__ x_scale,
                                                   int32_t *__restrict__ x_rowsum, int64_t row)
{
    constexpr int W = BLOCK / 64;
    __shared__ float s_max[W];
    __shared__ int s_sum[W];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(X + row * K);
    int *q4 = reinterpret_cast<int *>(Xq + row * K);
    const int64_t n4 = K / 4;

    // every load first (entries past the row re-read its last one and count as 0)
    f32x4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int64_t i = tid + (int64_t)j * BLOCK;
        const f32x4 a = x4[i < n4 ? i : n4 - 1];
        v[j] = (i < n4) ? a : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float g = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        g = fmaxf(g, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
    g = wave_max_dpp(g);
    if (lane == 0) s_max[wave] = g;
    __syncthreads();
    g = s_max[0];
#pragma unroll
    for (int w = 1; w < W; ++w) g = fmaxf(g, s_max[w]);

    int sum = 0;
    const float up = act_prescale(g);
    const float s = act_scale(g, up);        // IEEE binary32 division
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int64_t i = tid + (int64_t)j * BLOCK;
        if (i < n4) {
            f32x4 a = v[j];
            if (up != 1.0f) a *= up;          // row-uniform, rare
            int s4;
            q4[i] = (int)act_quant4(a[0], a[1], a[2], a[3], s, &s4);
            sum += s4;
        }
    }
    sum = wave_sum_dpp(sum);
    if (lane == 0) s_sum[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) total += s_sum[w];
        x_scale[row] = (g == 0.0f) ? 0.0f : g / 127.0f;
        if (x_rowsum) x_rowsum[row] = total;
    }
}

template <int BLOCK, int NV>
__global__ __launch_bounds__(BLOCK) void quant_act_reg_kernel(const float *__restrict__ X, int64_t K,
                                                             int8_t *__restrict__ Xq, float *__restrict__ x_scale,
                                                             int32_t *__restrict__ x_rowsum)
{
    quant_act_reg_body<BLOCK, NV>(X, K, Xq, x_scale, x_rowsum, blockIdx.x);
}

// Several independent inputs quantised in one launch: group g's rows are
// workgroups [row_start[g], row_start[g + 1]), each quantised exactly as
// quant_act_reg_kernel does (the row's maximum is exact, codes and row sums
// are integers: the thread count does not change a bit).  The argument is
// read in place in the kernel-argument segment (indexed by the group, a copy
// would live in scratch memory).
template <int BLOCK, int NV>
__global__ __launch_bounds__(BLOCK) void quant_act_multi_kernel(QuantGroupArgs)
{
    const QuantGroupArgs &qa = *(const QuantGroupArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    int gi = 0;
#pragma unroll
    for (int i = 1; i < kMaxQuantGroups; ++i)
        if ((int64_t)blockIdx.x >= qa.row_start[i]) gi = i;   // entries past ngroups: the row count
    quant_act_reg_body<BLOCK, NV>(qa.X[gi], qa.K[gi], qa.Xq[gi], qa.x_scale[gi], qa.x_rowsum[gi],
                                  (int64_t)blockIdx.x - qa.row_start[gi]);
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

// ---------------------------------------------------------------------------
// The same quantiser with each block held by one wave in registers, for
// B = 64 V (V = 1 .. 16 values per lane) and rows of at most 16 waves of
// 16 / V blocks (K / B <= 16 * (16 / V), so K <= 16384).  Lane l
// holds the V consecutive values l V .. l V + V - 1 of a block: the stages
// h < V pair values inside the lane, the stages h = V d (d = 1 .. 32) pair
// lane l with lane l ^ d, the lower element taking a + b and the upper one
// a - b as in the LDS form -- the same binary32 operations on the same
// operands.  Wave w of W takes blocks w, w + W, ...: no LDS pass and no
// barrier between stages, one barrier for the row maximum, and the row is
// read once.  The exchanges inside rows of 16 lanes are DPP moves; only
// d = 16 and 32 go through ds_bpermute.
// ---------------------------------------------------------------------------
constexpr int kH4Slots = 16;               // register values per lane

// the value of lane l ^ D: DPP moves inside rows of 16 lanes (D = 4: the
// half-row mirror, i -> i ^ 7, then i -> i ^ 3 in quads; D = 8: the row
// mirror, i -> i ^ 15, then the half-row mirror), ds_bpermute across rows
constexpr int kDppQuadXor3 = 0x1B;   // quad_perm [3, 2, 1, 0]
template <int D>
__device__ __forceinline__ float lane_xor(float v)
{
    const int b = __float_as_int(v);
    if constexpr (D == 1) return __int_as_float(dpp_move<kDppQuadXor1>(b));
    if constexpr (D == 2) return __int_as_float(dpp_move<kDppQuadXor2>(b));
    if constexpr (D == 4) return __int_as_float(dpp_move<kDppQuadXor3>(dpp_move<kDppRowHalfMirror>(b)));
    if constexpr (D == 8) return __int_as_float(dpp_move<kDppRowHalfMirror>(dpp_move<kDppRowMirror>(b)));
    return __shfl_xor(v, D);
}

// stage h = V D of one block: lane l pairs with lane l ^ D
template <int V, int D>
__device__ __forceinline__ void lane_stage(float (&v)[V], int lane)
{
    const bool upper = (lane & D) != 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const float o = lane_xor<D>(v[j]);
        v[j] = upper ? o - v[j] : v[j] + o;
    }
}

template <int V>
__global__ __launch_bounds__(1024) void quant_act_h4_wave_kernel(
    const float *__restrict__ X, int64_t K, int8_t *__restrict__ Xq, float *__restrict__ x_scale,
    int32_t *__restrict__ x_rowsum)
{
    constexpr int NB = kH4Slots / V;       // blocks per wave at most
    constexpr int B = 64 * V;
    __shared__ float s_max[16];
    __shared__ int s_sum[16];
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    const int nblk = (int)(K / B);
    const float *x = X + row * K + lane * V;

    float v[NB][V];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int blk = wave + i * W;
        if (blk < nblk) {
            const float *src = x + (int64_t)blk * B;
            if constexpr (V >= 4) {
#pragma unroll
                for (int j = 0; j < V; j += 4) {
                    const f32x4 t = *reinterpret_cast<const f32x4 *>(src + j);
                    v[i][j] = t[0]; v[i][j + 1] = t[1]; v[i][j + 2] = t[2]; v[i][j + 3] = t[3];
                }
            } else {
#pragma unroll
                for (int j = 0; j < V; ++j) v[i][j] = src[j];
            }
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j) v[i][j] = 0.0f;
        }
    }

    float g = 0.0f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (wave + i * W >= nblk) continue;              // wave-uniform
#pragma unroll
        for (int h = 1; h < V; h *= 2)
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (!(j & h)) {
                    const float a = v[i][j], b = v[i][j + h];
                    v[i][j] = a + b;
                    v[i][j + h] = a - b;
                }
        lane_stage<V, 1>(v[i], lane);
        lane_stage<V, 2>(v[i], lane);
        lane_stage<V, 4>(v[i], lane);
        lane_stage<V, 8>(v[i], lane);
        lane_stage<V, 16>(v[i], lane);
        lane_stage<V, 32>(v[i], lane);
#pragma unroll
        for (int j = 0; j < V; ++j) g = fmaxf(g, fabsf(v[i][j]));
    }
    g = wave_max_dpp(g);
    if (lane == 0) s_max[wave] = g;
    __syncthreads();
    g = s_max[0];
    for (int w = 1; w < W; ++w) g = fmaxf(g, s_max[w]);

    const float up = act_prescale(g);
    const float s = (g == 0.0f) ? 0.0f : 7.0f / (g * up);
    int sum = 0;
    int8_t *q = Xq + row * K + lane * V;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int blk = wave + i * W;
        if (blk >= nblk) continue;
        if (up != 1.0f) {                                 // row-uniform, rare
#pragma unroll
            for (int j = 0; j < V; ++j) v[i][j] *= up;
        }
        int8_t *dst = q + (int64_t)blk * B;
        if constexpr (V >= 4) {
#pragma unroll
            for (int j = 0; j < V; j += 4) {
                int s4;
                *reinterpret_cast<uint32_t *>(dst + j) = act_quant4(v[i][j], v[i][j + 1], v[i][j + 2], v[i][j + 3], s, &s4);
                sum += s4;
            }
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const uint32_t b = act_round_bits(v[i][j], s);
                dst[j] = (int8_t)(b & 0xFFu);
                sum += (int)(b - 0x4B400000u);
            }
        }
    }
    sum = wave_sum_dpp(sum);
    if (lane == 0) s_sum[wave] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        int total = 0;
        for (int w = 0; w < W; ++w) total += s_sum[w];
        x_scale[row] = (g == 0.0f) ? 0.0f : (float)((double)g / 7.0 / sqrt((double)B));
        if (x_rowsum) x_rowsum[row] = total;
    }
}

// Waves per row: for few rows as many as there are blocks (up to 16), for the
// row's latency; from 256 rows the fewest that hold the row, but at least 8
// (measured at 2048 x 6912, B = 256: 7 waves 18.3 us, 8 waves 16.6, 16
// waves 18.6; at 2048 x 2560: 3 waves 7.9, 8 waves 8.8, 10 waves 10.4).
// One row of 6912, B = 256: 3.8 us (the LDS form: 9.5 us).
template <int V>
hipError_t launch_h4_wave(const float *X, int64_t M, int64_t K, int8_t *Xq, float *x_scale, int32_t *x_rowsum,
                          hipStream_t stream)
{
    constexpr int NB = kH4Slots / V;
    const int nblk = (int)(K / (64 * V));
    int W = nblk < 16 ? nblk : 16;
    if (M >= 256) {
        W = (nblk + NB - 1) / NB;
        if (W < 8) W = nblk < 8 ? nblk : 8;
    }
    hipLaunchKernelGGL(quant_act_h4_wave_kernel<V>, dim3((unsigned)M), dim3(64 * W), 0, stream, X, K, Xq, x_scale,
                       x_rowsum);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// BitNet a4.8's hybrid activations ("BitNet 논문 분석: 1-Bit LLM의 시대",
// section "BitNet a4.8: 하이브리드 양자화 전략": the largest values of the
// activation tensor are split off and kept at 8 bits, the rest is quantised
// to 4 bits, each part with its own scale).  Per token row x and a
// caller-given outlier count T: S = the T largest |x| (equal magnitudes: the
// lower k first); hi = x on S, lo = x off S; hi gets the 8-bit quantiser
// (127 / max|hi|), lo the 4-bit one (7 / max|lo|, codes in [-7, 7]), both
// with the tiny-row rule of common.hpp.  Row 2m of Xq receives token m's hi
// codes, row 2m + 1 its lo codes, with scales max/127 and max/7.
//
// One workgroup per row, the row in registers.  S is found by a radix
// select over the bit patterns of |x| (for finite values their order as
// unsigned integers is the order of the magnitudes): three passes of 11, 10
// and 10 bits, most significant first, each a histogram in LDS of the keys
// that match the digits found so far, then a suffix scan over the bins that
// finds the digit holding the T-th largest key.  After the last pass the
// threshold key t and the number r of keys equal to t that belong to S are
// known; keys above t are in S.  When fewer than all the keys equal to t
// belong to S (ties at the threshold), the first r in k order are taken: a
// block-wide exclusive count of the equal keys in k order.
// ---------------------------------------------------------------------------
template <int BLOCK>
__device__ __forceinline__ int block_exclusive_count(int v, int *s_tmp, int *total)
{
    constexpr int W = BLOCK / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    if (lane == 63) s_tmp[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const int t = s_tmp[w];
        before += (w < wave) ? t : 0;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

template <int BLOCK, int NV>
__global__ __launch_bounds__(BLOCK) void quant_act_a48_kernel(const float *__restrict__ X, int64_t K, int64_t T,
                                                             int8_t *__restrict__ Xq, float *__restrict__ x_scale,
                                                             int32_t *__restrict__ x_rowsum)
{
    constexpr int W = BLOCK / 64;
    __shared__ int s_hist[2048];
    __shared__ int s_pick[2];
    __shared__ int s_tmp[W];
    __shared__ float s_max[2][W];
    __shared__ int s_sum[2][W];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(X + row * K);
    const int64_t n4 = K / 4;

    f32x4 v[NV];
    uint32_t key[NV][4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int64_t i = tid + (int64_t)j * BLOCK;
        const f32x4 a = x4[i < n4 ? i : n4 - 1];
        v[j] = (i < n4) ? a : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) key[j][c] = __float_as_uint(v[j][c]) & 0x7FFFFFFFu;
    }

    // radix select of the T-th largest key (1 <= T < K; T = 0 selects none,
    // T = K all): digits of 11, 10 and 10 bits, most significant first (the
    // keys' top bits are the exponent: 11 bits spread a row's values over
    // enough bins to keep the LDS atomics from piling onto a few addresses)
    uint32_t thr = 0xFFFFFFFFu;        // keys > thr are selected
    int rank = 0;                      // keys == thr to select, in k order
    bool ties_split = false;
    if (T > 0 && T < K) {
        uint32_t prefix = 0u, mask = 0u;
        int r = (int)T;
        int eq_count = 0;
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 20 : pass == 1 ? 10 : 0;
            const int nbins = pass == 0 ? 2048 : 1024;
            for (int b = tid; b < nbins; b += BLOCK) s_hist[b] = 0;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int64_t i = tid + (int64_t)j * BLOCK;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (i < n4 && (key[j][c] & mask) == prefix)
                        atomicAdd(&s_hist[(key[j][c] >> shift) & (uint32_t)(nbins - 1)], 1);
            }
            __syncthreads();
            if (wave == 0) {
                // lane l holds bins [l * per, l * per + per): suffix sums over
                // the lanes find the lane whose bins hold the r-th largest
                // key, then the lanes take one bin each of that lane's range
                const int per = nbins / 64;
                int own = 0;
                // rotated by the lane, so that the 64 lanes' reads spread over the banks
                for (int c = 0; c < per; ++c) own += s_hist[lane * per + ((c + lane) & (per - 1))];
                int incl = own;           // keys in bins of lanes >= lane
#pragma unroll
                for (int d = 1; d < 64; d *= 2) {
                    const int o = __shfl_down(incl, d, 64);
                    if (lane + d < 64) incl += o;
                }
                const int above = incl - own;
                const unsigned long long hit = __ballot(above < r && r <= incl);   // exactly one lane
                const int tl = __ffsll(hit) - 1;
                const int above_t = __shfl(above, tl, 64);
                const int h = lane < per ? s_hist[tl * per + lane] : 0;
                int incl2 = h;
#pragma unroll
                for (int d = 1; d < 64; d *= 2) {
                    const int o = __shfl_down(incl2, d, 64);
                    if (lane + d < 64) incl2 += o;
                }
                const int above2 = above_t + incl2 - h;
                if (lane < per && above2 < r && r <= above2 + h) {
                    s_pick[0] = tl * per + lane;
                    s_pick[1] = r - above2;
                }
            }
            __syncthreads();
            const int digit = s_pick[0];
            r = s_pick[1];
            eq_count = s_hist[digit];
            prefix |= (uint32_t)digit << shift;
            mask |= (uint32_t)(nbins - 1) << shift;
            __syncthreads();
        }
        thr = prefix;
        rank = r;
        ties_split = rank < eq_count;  // workgroup-uniform
    }

    // selection flags; ties at the threshold split in k order when needed
    uint32_t selbits[NV];
    {
        int base = 0;                  // equal keys in earlier j blocks
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t i = tid + (int64_t)j * BLOCK;
            uint32_t sb = 0;
            int eqn = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool in = i < n4;
                const bool above = T >= K ? true : (T > 0 && key[j][c] > thr);
                const bool eq = T > 0 && T < K && key[j][c] == thr;
                if (in && above) sb |= 1u << c;
                if (in && eq) eqn++;
            }
            if (ties_split) {
                int tot = 0;
                const int before = base + block_exclusive_count<BLOCK>(eqn, s_tmp, &tot);
                int seen = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bool eq = i < n4 && key[j][c] == thr;
                    if (eq && before + seen < rank) sb |= 1u << c;
                    seen += eq ? 1 : 0;
                }
                base += tot;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (i < n4 && T > 0 && T < K && key[j][c] == thr) sb |= 1u << c;
            }
            selbits[j] = sb;
        }
    }

    // the two maxima
    float gh = 0.0f, gl = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float a = fabsf(v[j][c]);
            if ((selbits[j] >> c) & 1u) gh = fmaxf(gh, a);
            else gl = fmaxf(gl, a);
        }
    gh = wave_max_dpp(gh);
    gl = wave_max_dpp(gl);
    if (lane == 0) {
        s_max[0][wave] = gh;
        s_max[1][wave] = gl;
    }
    __syncthreads();
    gh = s_max[0][0];
    gl = s_max[1][0];
#pragma unroll
    for (int w = 1; w < W; ++w) {
        gh = fmaxf(gh, s_max[0][w]);
        gl = fmaxf(gl, s_max[1][w]);
    }
    const float uph = act_prescale(gh), upl = act_prescale(gl);
    const float sh = act_scale(gh, uph);                       // 127 / (g * up)
    const float sl = gl == 0.0f ? 0.0f : 7.0f / (gl * upl);     // 7 / (g * up)

    int *qh4 = reinterpret_cast<int *>(Xq + (2 * row) * K);
    int *ql4 = reinterpret_cast<int *>(Xq + (2 * row + 1) * K);
    int sumh = 0, suml = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int64_t i = tid + (int64_t)j * BLOCK;
        uint32_t wh = 0, wl = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool sel = (selbits[j] >> c) & 1u;
            const uint32_t bh = act_round_bits(v[j][c] * uph, sh);
            const uint32_t bl = act_round_bits(v[j][c] * upl, sl);
            const int ch = sel ? (int)(bh - 0x4B400000u) : 0;
            const int cl = sel ? 0 : (int)(bl - 0x4B400000u);
            wh |= ((uint32_t)ch & 0xFFu) << (8 * c);
            wl |= ((uint32_t)cl & 0xFFu) << (8 * c);
            sumh += ch;
            suml += cl;
        }
        if (i < n4) {
            qh4[i] = (int)wh;
            ql4[i] = (int)wl;
        }
    }
    sumh = wave_sum_dpp(sumh);
    suml = wave_sum_dpp(suml);
    if (lane == 0) {
        s_sum[0][wave] = sumh;
        s_sum[1][wave] = suml;
    }
    __syncthreads();
    if (tid == 0) {
        int th = 0, tl = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            th += s_sum[0][w];
            tl += s_sum[1][w];
        }
        x_scale[2 * row] = (gh == 0.0f) ? 0.0f : gh / 127.0f;
        x_scale[2 * row + 1] = (gl == 0.0f) ? 0.0f : gl / 7.0f;
        if (x_rowsum) {
            x_rowsum[2 * row] = th;
            x_rowsum[2 * row + 1] = tl;
        }
    }
}

// y[m, n] = Y2[2m, n] + Y2[2m + 1, n]: the rescaled outlier and 4-bit parts
__global__ __launch_bounds__(256) void a48_combine_kernel(const float *__restrict__ Y2, int64_t M, int64_t N,
                                                          float *__restrict__ Y)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx - m * N;
    Y[idx] = Y2[(2 * m) * N + n] + Y2[(2 * m + 1) * N + n];
}

}  // namespace

// The row in registers: up to 8 float4 per thread with 256 threads (K <=
// 8192), 4 with 1024; 1024 threads per row for up to 512 rows of K >= 4096
// (latency), else 256 (many rows side by side).  hipErrorNotSupported past
// K = 16384.
hipError_t launch_quant_act_a48(const float *X, int64_t M, int64_t K, int64_t T, int8_t *Xq, float *x_scale,
                                int32_t *x_rowsum, hipStream_t stream, const char **name)
{
    if (M == 0) return hipSuccess;
    auto go = [&](auto kern, int threads) {
        hipLaunchKernelGGL(kern, dim3((unsigned)M), dim3(threads), 0, stream, X, K, T, Xq, x_scale, x_rowsum);
        return hipGetLastError();
    };
    const int64_t nv256 = (K / 4 + 255) / 256, nv1024 = (K / 4 + 1023) / 1024;
    const bool wide = (M <= 512 && K >= 4096) || K > 8192;
    *name = wide ? "quant_act_a48_1024" : "quant_act_a48_256";
    if (!wide) {
        if (nv256 <= 1) return go(quant_act_a48_kernel<256, 1>, 256);
        if (nv256 <= 2) return go(quant_act_a48_kernel<256, 2>, 256);
        if (nv256 <= 4) return go(quant_act_a48_kernel<256, 4>, 256);
        return go(quant_act_a48_kernel<256, 8>, 256);
    }
    if (nv1024 <= 2) return go(quant_act_a48_kernel<1024, 2>, 1024);
    if (nv1024 <= 4) return go(quant_act_a48_kernel<1024, 4>, 1024);
    return hipErrorNotSupported;
}

hipError_t launch_a48_combine(const float *Y2, int64_t M, int64_t N, float *Y, hipStream_t stream)
{
    if (M == 0) return hipSuccess;
    const int64_t blocks = (M * N + 255) / 256;
    hipLaunchKernelGGL(a48_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, Y2, M, N, Y);
    return hipGetLastError();
}

hipError_t launch_quant_act_h4(const float *X, int64_t M, int64_t K, int64_t B, int8_t *Xq, float *x_scale,
                               int32_t *x_rowsum, hipStream_t stream, const char **name)
{
    if (M == 0) return hipSuccess;
    if (B < 1 || B > kHChunk || (B & (B - 1)) || K % B || K % 8) return hipErrorInvalidValue;
    // one block per wave in registers where it fits (64 <= B <= 1024 and at
    // most 16 waves of 16 / (B / 64) blocks each)
    if (B >= 64 && B <= 1024 && K / B <= 16 * (kH4Slots / (B / 64))) {
        *name = "quant_act_h4_wave";
        switch (B) {
        case 64: return launch_h4_wave<1>(X, M, K, Xq, x_scale, x_rowsum, stream);
        case 128: return launch_h4_wave<2>(X, M, K, Xq, x_scale, x_rowsum, stream);
        case 256: return launch_h4_wave<4>(X, M, K, Xq, x_scale, x_rowsum, stream);
        case 512: return launch_h4_wave<8>(X, M, K, Xq, x_scale, x_rowsum, stream);
        default: return launch_h4_wave<16>(X, M, K, Xq, x_scale, x_rowsum, stream);
        }
    }
    *name = "quant_act_h4";
    hipLaunchKernelGGL(quant_act_h4_kernel, dim3((unsigned)M), dim3(kQuantBlock), 0, stream, X, K, B, Xq, x_scale,
                       x_rowsum);
    return hipGetLastError();
}

hipError_t launch_quant_act_multi(QuantGroupArgs qa, hipStream_t stream)
{
    if (qa.ngroups < 1 || qa.ngroups > kMaxQuantGroups) return hipErrorNotSupported;
    int64_t rows = 0, n4max = 0;
    for (int g = 0; g < qa.ngroups; ++g) {
        qa.row_start[g] = rows;
        rows += qa.M[g];
        if (qa.K[g] / 4 > n4max) n4max = qa.K[g] / 4;
    }
    for (int g = qa.ngroups; g <= kMaxQuantGroups; ++g) qa.row_start[g] = rows;
    if (rows == 0) return hipSuccess;
    if (rows > (1LL << 31) - 1) return hipErrorNotSupported;
    // the single-input rule: 1024 threads per row for up to a few hundred
    // long rows, else 256; the row in registers (at most 4 or 8 float4 per
    // thread)
    const bool wide = rows <= 512 && n4max >= 1024;
    const int threads = wide ? 1024 : kQuantBlock;
    const int64_t nv = (n4max + threads - 1) / threads;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)rows), dim3(threads), 0, stream, qa);
        return hipGetLastError();
    };
    if (wide) {
        if (nv <= 1) return go(quant_act_multi_kernel<1024, 1>);
        if (nv <= 2) return go(quant_act_multi_kernel<1024, 2>);
        if (nv <= 4) return go(quant_act_multi_kernel<1024, 4>);
    } else {
        if (nv <= 1) return go(quant_act_multi_kernel<kQuantBlock, 1>);
        if (nv <= 2) return go(quant_act_multi_kernel<kQuantBlock, 2>);
        if (nv <= 4) return go(quant_act_multi_kernel<kQuantBlock, 4>);
        if (nv <= 8) return go(quant_act_multi_kernel<kQuantBlock, 8>);
    }
    return hipErrorNotSupported;
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
    // up to a few hundred long rows: 1024 threads per row for the row's
    // latency (measured with 256: one row of 6912 3.7 -> 2.6 us, 8 and 64
    // rows of 11008 5.3 -> 3.2-3.4 us; 255 rows of 6912 3.4 us against 4.5
    // at 256 rows with 256 threads); many rows are bandwidth-bound: 256
    const bool wide = M <= 512 && K >= 4096;
    auto go = [&](auto kern, int threads) {
        hipLaunchKernelGGL(kern, dim3((unsigned)M), dim3(threads), 0, stream, X, tr, K, Xq, x_scale, x_rowsum);
    };
    if (t == 0) {
        // the row in registers where it fits: at most 8 (256 threads) or 4
        // (1024 threads) float4 per thread
        const int threads = wide ? 1024 : kQuantBlock;
        const int64_t nv = (K / 4 + threads - 1) / threads;
        auto reg = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)M), dim3(threads), 0, stream, X, K, Xq, x_scale, x_rowsum);
            return hipGetLastError();
        };
        if (wide) {
            if (nv <= 1) return reg(quant_act_reg_kernel<1024, 1>);
            if (nv <= 2) return reg(quant_act_reg_kernel<1024, 2>);
            if (nv <= 4) return reg(quant_act_reg_kernel<1024, 4>);
        } else {
            if (nv <= 1) return reg(quant_act_reg_kernel<kQuantBlock, 1>);
            if (nv <= 2) return reg(quant_act_reg_kernel<kQuantBlock, 2>);
            if (nv <= 4) return reg(quant_act_reg_kernel<kQuantBlock, 4>);
            if (nv <= 8) return reg(quant_act_reg_kernel<kQuantBlock, 8>);
        }
    }
    if (wide) {
        switch (t) {
        case 0: go(quant_act_kernel<0, 1024>, 1024); break;
        case kTrGate: go(quant_act_kernel<kTrGate, 1024>, 1024); break;
        case kTrNorm: go(quant_act_kernel<kTrNorm, 1024>, 1024); break;
        default: go(quant_act_kernel<kTrGate | kTrNorm, 1024>, 1024); break;
        }
    } else {
        switch (t) {
        case 0: go(quant_act_kernel<0>, kQuantBlock); break;
        case kTrGate: go(quant_act_kernel<kTrGate>, kQuantBlock); break;
        case kTrNorm: go(quant_act_kernel<kTrNorm>, kQuantBlock); break;
        default: go(quant_act_kernel<kTrGate | kTrNorm>, kQuantBlock); break;
        }
    }
    return hipGetLastError();
}

}  // namespace bl
