// Fused decode forward: per-token absmax int8 quantisation of the fp32
// activations plus the skinny MFMA contraction of one or more projections that
// share those activations (q/k/v, or gate/up), all in one launch.
//
// Same arithmetic as the separate calls: "BitNet b1.58 2B4T Technical Report
// 요약 설명", sec. 2 (per-token absmax 8-bit activations) and sec. 5.1 (packed
// weights, unpacked on chip); "BitNet 논문 분석: 1-Bit LLM의 시대", section
// "Absmean 양자화 함수" (activation_quant, integer linear, rescale).  The
// quantised values, row sums and scales are bit-identical to
// bitlinear_quant_act's, so the outputs equal the unfused path's bit for bit.
//
// Why fuse: a decode BitLinear moves a few MB, so on MI355X a launch's fixed
// cost (dispatch, first HBM round trip, completion) is comparable to the
// transfer itself.  Fusing the activation quantisation removes one launch per
// projection group, and serving several projections in one grid removes the
// rest.  Each workgroup recomputes max|x| over the whole activation row from
// L2 (M x K x 4 bytes, M <= 4), which costs far less than a launch.
//
// Workgroup layout: it owns ROWS rows of one projection; KS waves split K as in
// the skinny kernel.  Order of work: (1) all KS waves issue the loads of the
// fp32 activation rows (read once, into registers), (2) then the wave's weight
// loads; (3) as soon as the activations arrive -- the weights still in flight
// -- reduce max|x| per token through DPP lane moves and LDS, quantise the
// registers to int8 into a block-shared LDS row and reduce the int32 row sums;
// (4) stage the weights in LDS; (5) MFMA, reduce across waves, epilogue.
#pragma once

#include "skinny_impl.hpp"

namespace bl {

namespace fused {

using skinny::i32x4;
using skinny::u32x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
using skinny::unpack_word;
using skinny::RawChunk;
using skinny::load_raw_chunk;
using skinny::decode_chunk;
using skinny::fill_nm24_table;

template <int KS, int CMAX, int MT, int ROWS>
struct FusedLds {
    static constexpr int kStride = (CMAX + 1) * 16;          // weight row stride
    static constexpr int kW = ROWS * kStride;                 // per wave
    static constexpr int kZero = 256;                         // zero block (token rows >= M)
};

// KS waves split K; at most CMAX chunks per wave; at most MT (<= 4) tokens
// per workgroup: more tokens run in tiles of MT along the grid's y (each tile
// quantises its own token rows and re-reads the weights, mostly from L2);
// ROWS weight rows per workgroup: 16 (one MFMA column block), 32 (two), or 8
// (the MFMA's columns 8..15 repeat rows 0..7 and are not stored: twice the
// workgroups for short matrices).  The activation row (K bytes per token, plus
// 3 zero chunks) is shared in LDS and sized at launch (dynamic LDS).
template <Pattern P, int KS, int CMAX, int MT, int ROWS>
__global__ __launch_bounds__(64 * KS) void fused_kernel(const float *__restrict__ X, int64_t M, int64_t K,
                                                        FusedProjArgs args, float *__restrict__ x_scale_out)
{
    static_assert(CMAX % 4 == 0 && MT >= 1 && MT <= 4, "config");
    static_assert(ROWS == 8 || ROWS == 16 || ROWS == 32, "rows per workgroup");
    using L = FusedLds<KS, CMAX, MT, ROWS>;
    constexpr int RG = (ROWS + 15) / 16;                      // MFMA column blocks
    constexpr int WLOADS = (ROWS * CMAX + 63) / 64;
    constexpr int T = 64 * KS;
    __shared__ __attribute__((aligned(16))) uint8_t s_w[KS][L::kW];
    __shared__ __attribute__((aligned(16))) uint8_t s_zero[L::kZero];
    __shared__ float s_max[MT][KS];
    __shared__ int s_sum[MT][KS];
    __shared__ i32x4 s_part[RG][KS > 1 ? KS - 1 : 1][64];
    __shared__ uint8_t s_nm24[P == Pattern::NM24 ? 256 : 1];
    extern __shared__ __attribute__((aligned(16))) uint8_t s_x[];   // MT x (K + 192) int8

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, q = lane >> 4;
    // token tile blockIdx.y: tokens MT y .. MT y + MT - 1 of the call
    const int64_t t0 = (int64_t)blockIdx.y * MT;
    X += t0 * K;
    if (x_scale_out) x_scale_out += t0;
    const int mt = (int)min(M - t0, (int64_t)MT);
    const int64_t xstride = K + 192;

    // which projection and which rows
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxFusedProj; ++i)
        if ((int)blockIdx.x >= args.block_start[i]) p = i;       // entries past nproj: the block count
    const int64_t N = args.N[p];
    const uint8_t *packed = args.packed[p];
    const int64_t n0 = (int64_t)(blockIdx.x - args.block_start[p]) * ROWS;
    const float beta = args.w_scale[p][0];

    const int64_t C = K / 64;
    const int64_t c_lo = C * wave / KS;
    const int cw = (int)(C * (wave + 1) / KS - c_lo);
    uint8_t *lw = s_w[wave];

    // every argument the kernel reads in SGPRs now: a scalar load left pending
    // would make the compiler wait for all outstanding memory operations
    asm volatile("" ::"s"(X), "s"(packed), "s"(args.w_scale[p]), "s"(args.Y[p]), "s"(args.acc[p]));

    // (1) the fp32 activation rows first, read once into registers (XR float4
    //     per thread per token covers K: K/4 = 16 C <= 16 KS CMAX = XR T):
    //     waiting for them below leaves the weight loads in flight
    constexpr int XR = CMAX / 4;
    const int64_t n4 = K / 4;
    f32x4 xr[MT][XR];                  // ext vectors: an array of HIP's float4 structs
    float g[MT];                       // can end up in scratch memory
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const f32x4 *x4 = reinterpret_cast<const f32x4 *>(X + (int64_t)min(m, mt - 1) * K);
#pragma unroll
        for (int j = 0; j < XR; ++j) {
            const int64_t i = tid + (int64_t)j * T;
            const f32x4 a = x4[i < n4 ? i : 0];
            xr[m][j] = (m < mt && i < n4) ? a : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // (2) weight loads of this wave, all in flight
    RawChunk<P> w[WLOADS];
    int w_off[WLOADS];
    const float inv_cw = 1.0f / (float)cw;
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
        const int f = i * 64 + lane;
        const int row = (int)(((float)f + 0.5f) * inv_cw);
        const int col = f - row * cw;
        // lanes past the wave's ROWS x cw chunks re-read the wave's first chunk
        // (a line it fetches anyway) rather than another workgroup's rows
        const int64_t n = min(n0 + (row < ROWS ? row : 0), N - 1);
        w_off[i] = (row < ROWS) ? row * L::kStride + col * 16 : -1;
        w[i] = load_raw_chunk<P>(packed, N, K, n, c_lo + (row < ROWS ? col : 0));
    }

    __builtin_amdgcn_sched_barrier(0);
    fill_nm24_table<P>(s_nm24, tid, T);              // ready after the barrier below

    // (3a) max |x| per token over the whole row
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < XR; ++j) {
            const f32x4 a = xr[m][j];
            v = fmaxf(v, fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3]))));
        }
        v = wave_max_dpp(v);
        if (lane == 0) s_max[m][wave] = v;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float v = s_max[m][0];
#pragma unroll
        for (int k2 = 1; k2 < KS; ++k2) v = fmaxf(v, s_max[m][k2]);
        g[m] = v;
    }

    // (3b) quantise into LDS, row sums
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int sum = 0;
        if (m < mt) {
            uint32_t *q4 = reinterpret_cast<uint32_t *>(s_x + m * xstride);
            const float up = act_prescale(g[m]);
            const float s = act_scale(g[m], up);
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                const int64_t i = tid + (int64_t)j * T;
                const f32x4 a = xr[m][j] * up;             // up = 1 unless max|x| < 2^-100
                int s4;
                const uint32_t packed4 = act_quant4(a[0], a[1], a[2], a[3], s, &s4);
                if (i < n4) {
                    sum += s4;
                    q4[i] = packed4;
                }
            }
            // 3 zero chunks after the row
            if (tid < 48) q4[n4 + tid] = 0;
        }
        sum = wave_sum_dpp(sum);
        if (lane == 0) s_sum[m][wave] = sum;
    }
    if (tid < L::kZero / 16) reinterpret_cast<u32x4 *>(s_zero)[tid] = u32x4{0u, 0u, 0u, 0u};

    // (4) weights to LDS
#pragma unroll
    for (int i = 0; i < WLOADS; ++i)
        if (w_off[i] >= 0) *reinterpret_cast<u32x4 *>(lw + w_off[i]) = decode_chunk<P>(w[i], s_nm24);
    __syncthreads();

    int rs[4];
    float xsc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * q + v;
        int tot = 0;
        float gm = 0.0f;
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
            if (mm == m) {
#pragma unroll
                for (int k2 = 0; k2 < KS; ++k2) tot += s_sum[mm][k2];
                gm = g[mm];
            }
        rs[v] = tot;
        xsc[v] = (gm == 0.0f) ? 0.0f : gm / 127.0f;
    }
    if (x_scale_out && blockIdx.x == 0 && tid < mt) {
        float gm = 0.0f;
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
            if (mm == tid) gm = g[mm];
        x_scale_out[tid] = (gm == 0.0f) ? 0.0f : gm / 127.0f;
    }

    // (5) MFMA phase: column block g covers weight rows 16 g + r (ROWS == 8:
    // rows r & 7, the upper half repeating the lower)
    const uint8_t *arow = (r < mt) ? s_x + r * xstride + (c_lo + q) * 64 : s_zero;
    const int astep = (r < mt) ? 256 : 0;
    i32x4 acc[RG][4];
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[g2][t] = i32x4{0, 0, 0, 0};
    const int steps = (cw + 3) / 4;
    for (int s = 0; s < steps; ++s) {
        i32x4 a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // past this wave's range the activation bytes belong to the next
            // wave's range or the zero tail: mask them with the column test
            const i32x4 a0 = *reinterpret_cast<const i32x4 *>(arow + s * astep + 16 * t);
            a[t] = (4 * s + q < cw) ? a0 : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int g2 = 0; g2 < RG; ++g2) {
            const int wr = (ROWS == 8) ? (r & 7) : 16 * g2 + r;
            const u32x4 b = *reinterpret_cast<const u32x4 *>(lw + wr * L::kStride + q * 16 + s * 64);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[g2][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], unpack_word(b[t]), acc[g2][t], 0, 0, 0);
        }
    }
    i32x4 sum[RG];
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2) sum[g2] = (acc[g2][0] + acc[g2][1]) + (acc[g2][2] + acc[g2][3]);
    if (KS > 1) {
        if (wave > 0) {
#pragma unroll
            for (int g2 = 0; g2 < RG; ++g2) s_part[g2][wave - 1][lane] = sum[g2];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int g2 = 0; g2 < RG; ++g2)
#pragma unroll
            for (int w2 = 1; w2 < KS; ++w2) sum[g2] += s_part[g2][w2 - 1][lane];
    }

    float *Y = args.Y[p] + t0 * N;
    int32_t *acc_out = args.acc[p] ? args.acc[p] + t0 * N : nullptr;
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2) {
        const int64_t nn = n0 + 16 * g2 + r;
        if ((ROWS == 8 && r >= 8) || nn >= N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * q + v;
            if (m < mt) {
                const int av = sum[g2][v] - rs[v];
                Y[(int64_t)m * N + nn] = (float)av * (beta * xsc[v]);
                if (acc_out) acc_out[(int64_t)m * N + nn] = av;
            }
        }
    }
}

template <Pattern P, int KS, int CMAX, int MT, int ROWS>
hipError_t launch_fused(const float *X, int64_t M, int64_t K, const FusedProjArgs &args, int blocks,
                        float *x_scale, hipStream_t stream)
{
    const size_t dyn = (size_t)MT * (size_t)(K + 192);
    hipLaunchKernelGGL((fused_kernel<P, KS, CMAX, MT, ROWS>), dim3((unsigned)blocks, (unsigned)((M + MT - 1) / MT)),
                       dim3(64 * KS), dyn, stream, X, M, K, args, x_scale);
    return hipGetLastError();
}

}  // namespace fused
}  // namespace bl
