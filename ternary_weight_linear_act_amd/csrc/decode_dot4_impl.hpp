#pragma once

// Decode forward for one token (M = 1) on packed int8 dot products, with or
// without the activation quantisation fused in, for one or more projections
// that share the activations.
//
// "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 2 (per-token absmax
// 8-bit activations) and sec. 5.1 (the packed weights, four per byte, are
// what moves from HBM; they are unpacked on chip); "BitNet 논문 분석: 1-Bit
// LLM의 시대", section "Absmean 양자화 함수" (activation_quant, the integer
// linear of ternary weights and int8 activations, the rescale).  Same
// arithmetic as bitlinear_quant_act + bitlinear_forward, bit for bit.
//
// Why not the MFMA kernel at M = 1: with one token the MFMA's 16 token rows
// are 15/16 padding, and staging the weights through LDS into the MFMA
// operand layout is a second pass over every weight byte.  Here a weight
// chunk (16 bytes = 64 codes) goes from the load straight into 16
// v_dot4_i32_iu8 against the activation bytes, read from LDS.
//
// Layout: LPR lanes share a weight row, lane j takes chunks j, j + LPR, ...
// (so a load instruction reads LPR * 16 contiguous bytes of each row), every
// load of the lane is issued up front, the activations first.  A workgroup is
// 4 waves, 256 / LPR rows.  The LPR partial sums meet through DPP lane moves;
// no barrier follows the loads but the one that publishes the int8
// activations, which the weights are most likely still in flight for.
// Codes are c = t + 1, so the sums are sum c*q and the epilogue subtracts the
// activation row sum.
#include "fused_impl.hpp"

namespace bl {
namespace dot4 {

using skinny::i32x4;
using skinny::u32x4;
using skinny::RawChunk;
using skinny::load_raw_chunk;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxK = 16384;                 // activation row in LDS and registers

template <int LPR>
__device__ __forceinline__ int lanes_sum(int v)
{
    v += dpp_move<kDppQuadXor1>(v);
    v += dpp_move<kDppQuadXor2>(v);
    if (LPR >= 8) v += dpp_move<kDppRowHalfMirror>(v);
    if (LPR >= 16) v += dpp_move<kDppRowMirror>(v);
    if (LPR >= 32) v += __shfl_xor(v, 16, 64);
    if (LPR >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// FUSED: X is the fp32 activation row (quantised here; x_scale_out, if not
// NULL, receives its scale); otherwise Xq / x_scale / x_rowsum are the
// quantised row.  args.block_start[i] is the first workgroup of projection i.
// U = chunks per lane, fixed at compile time so that every load is issued
// unconditionally (a load under a branch makes the compiler wait for it at
// the join); the host guarantees K <= 64 * U * LPR.  W waves per workgroup,
// W * 64 / LPR rows.
// One projection of a workgroup: its packed weights, scale, outputs, rows.
struct ProjView {
    const uint8_t *packed;
    const float *w_scale;
    float *Y;
    int32_t *acc;
    int64_t N;
};

// What a workgroup resolves once its input-row loads are issued: its
// projection, its block of RB rows there, and x_scale_out (non-NULL for the
// one workgroup that writes the scale).
struct ProjSel {
    ProjView v;
    int64_t row_block;
    float *x_scale_out;
};

// `resolve()` returns the workgroup's ProjSel.  It is called after the input
// row's loads are issued, so that their scalar loads (which return out of
// order: any use waits for all) do not hold the row loads back.  Only threads
// below 64 * W may enter.
template <Pattern P, int LPR, int U, bool FUSED, int W = 4, int TR = 0, class Resolve>
__device__ __forceinline__ void decode_dot4_body(
    const float *__restrict__ X, const int8_t *__restrict__ Xq, const float *__restrict__ x_scale,
    const int32_t *__restrict__ x_rowsum, int64_t K, const Resolve &resolve, const ActTransform &tr)
{
    static_assert(TR == 0 || FUSED, "the row transform belongs to the fused form");
    constexpr bool GATE = (TR & kTrGate) != 0, NORM = (TR & kTrNorm) != 0;
    constexpr int RPW = 64 / LPR, RB = W * RPW, kThreads = 64 * W;
    extern __shared__ __attribute__((aligned(16))) uint8_t s_x[];      // K int8 activations
    __shared__ float s_max[W];
    __shared__ int s_sum[W];
    __shared__ double s_ss[NORM ? W : 1];
    __shared__ uint32_t s_sel[P == Pattern::Dense ? 1 : 2 * nm_sel_entries(P)];   // N:M byte selectors

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t C = K / 64;
    // 1. activations first: they need only the input row (an argument of the
    //    launch), not the projection's pointers, whose scalar loads may still
    //    be in flight where the workgroup's lookup is deep.  16-byte loads,
    //    enough for K = 64 * U * LPR (indices past the row re-read element 0
    //    and are never used)
    asm volatile("" ::"s"(X), "s"(Xq), "s"(tr.up), "s"(tr.gamma));
    constexpr int XR = FUSED ? (16 * U * LPR + kThreads - 1) / kThreads : (4 * U * LPR + kThreads - 1) / kThreads;
    const int64_t n4 = K / 4, n16 = K / 16;
    f32x4 xf[FUSED ? XR : 1];          // ext vectors: HIP's float4 / uint4 structs
    u32x4 xb[FUSED ? 1 : XR];          // in an array are not kept in registers
    f32x4 uf[GATE ? XR : 1];           // the gate's second operand (up)
    f32x4 gf[NORM ? XR : 1];           // the RMSNorm weight
#pragma unroll
    for (int t = 0; t < XR; ++t) {
        const int64_t i = tid + (int64_t)t * kThreads;
        if constexpr (FUSED) xf[t] = reinterpret_cast<const f32x4 *>(X)[i < n4 ? i : 0];
        else xb[t] = reinterpret_cast<const u32x4 *>(Xq)[i < n16 ? i : 0];
        if constexpr (GATE) uf[t] = reinterpret_cast<const f32x4 *>(tr.up)[i < n4 ? i : 0];
        if constexpr (NORM) gf[t] = reinterpret_cast<const f32x4 *>(tr.gamma)[i < n4 ? i : 0];
    }
    __builtin_amdgcn_sched_barrier(0);

    const ProjSel sel = resolve();
    const ProjView &v = sel.v;
    const int64_t row_block = sel.row_block;
    float *__restrict__ x_scale_out = sel.x_scale_out;
    const int64_t N = v.N;
    const uint8_t *packed = v.packed;
    const int64_t row = row_block * RB + wave * RPW + lane / LPR;
    const int j = lane % LPR;
    float *Y = v.Y;
    int32_t *acc_out = v.acc;
    const float *w_scale = v.w_scale;
    // every argument read later in SGPRs now (a pending scalar load would make
    // the compiler wait for all outstanding memory operations at its use)
    asm volatile("" ::"s"(x_scale), "s"(x_rowsum), "s"(packed), "s"(Y), "s"(acc_out), "s"(w_scale),
                 "s"(x_scale_out));

    // 0. the scalars the epilogue needs, issued before the weights: read at
    //    the end, each would cost a full memory round trip there
    const float wsc = w_scale[0];
    float xsc = 0.0f;
    int rs = 0;
    if constexpr (!FUSED) {
        xsc = x_scale[0];
        rs = x_rowsum[0];
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. the lane's weight chunks (rows past N re-read row N - 1 and chunks
    //    past the row re-read chunk C - 1; neither is used)
    RawChunk<P> w[U];
    const int64_t r = min(row, N - 1);
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load_raw_chunk<P>(packed, N, K, r, min((int64_t)(j + u * LPR), C - 1));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (P != Pattern::Dense)                 // ready after the barrier below
        for (int i = tid; i < nm_sel_entries(P); i += kThreads) nm_sel_entry<P>(i, &s_sel[2 * i], &s_sel[2 * i + 1]);

    // 3. the int8 activations into LDS, with their scale and row sum
    double ss = 0.0;                   // the norm's sum of squares, then its block total
    float xg = 0.0f;                   // max|v| of the normalised row
    if constexpr (FUSED) {
        // the transformed row (common.hpp): h = ReLU(x)^2 * up, then the codes
        // are taken from h * gamma and the norm's sum of squares from h
        if constexpr (TR != 0) {
#pragma unroll
            for (int t = 0; t < XR; ++t) {
                f32x4 h = xf[t];
                if constexpr (GATE) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) h[c] = act_gate(h[c], uf[t][c]);
                }
                if constexpr (NORM) {
                    double sq = 0.0;
#pragma unroll
                    for (int c = 0; c < 4; ++c) sq += (double)h[c] * (double)h[c];
                    ss += (tid + (int64_t)t * kThreads < n4) ? sq : 0.0;
#pragma unroll
                    for (int c = 0; c < 4; ++c) h[c] = h[c] * gf[t][c];
                }
                xf[t] = h;
            }
        }
        // branch-free: entries past the row (re-reads of element 0) are
        // masked out of the max and the sum and never stored
        float g = 0.0f;
#pragma unroll
        for (int t = 0; t < XR; ++t) {
            const f32x4 a = xf[t];
            const float m = fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3])));
            g = fmaxf(g, tid + (int64_t)t * kThreads < n4 ? m : 0.0f);
        }
        g = wave_max_dpp(g);
        if (lane == 0) s_max[wave] = g;
        if constexpr (NORM) {
            ss = wave_sum_f64(ss);
            if (lane == 0) s_ss[wave] = ss;
        }
        __syncthreads();
        g = s_max[0];
#pragma unroll
        for (int i = 1; i < W; ++i) g = fmaxf(g, s_max[i]);
        const float up = act_prescale(g);
        const float s = act_scale(g, up);
        if (up != 1.0f) {                              // workgroup-uniform, rare
#pragma unroll
            for (int t = 0; t < XR; ++t) xf[t] *= up;
        }
        int sum = 0;
        uint32_t *q4 = reinterpret_cast<uint32_t *>(s_x);
#pragma unroll
        for (int t = 0; t < XR; ++t) {
            const int64_t i = tid + (int64_t)t * kThreads;
            const f32x4 a = xf[t];
            int s4;
            const uint32_t packed4 = act_quant4(a[0], a[1], a[2], a[3], s, &s4);
            const bool in = i < n4;
            sum += in ? s4 : 0;
            if (in) q4[i] = packed4;
        }
        sum = wave_sum_dpp(sum);
        if (lane == 0) s_sum[wave] = sum;
        __syncthreads();
        rs = s_sum[0];
#pragma unroll
        for (int i = 1; i < W; ++i) rs += s_sum[i];
        if constexpr (NORM) {
            // the binary64 division chain of the scale waits until after the
            // dot products (only the epilogue reads it)
            double t = s_ss[0];
#pragma unroll
            for (int i = 1; i < W; ++i) t += s_ss[i];
            ss = t;
            xg = g;
        } else {
            xsc = (g == 0.0f) ? 0.0f : g / 127.0f;
            if (x_scale_out && tid == 0) x_scale_out[0] = xsc;
        }
    } else {
#pragma unroll
        for (int t = 0; t < XR; ++t) {
            const int64_t i = tid + (int64_t)t * kThreads;
            if (i < n16) reinterpret_cast<u32x4 *>(s_x)[i] = xb[t];
        }
        __syncthreads();
    }

    // 4. dot products, branch-free (a branch per chunk would make the
    //    compiler wait for every weight load at the first one), 16 v_dot4
    //    per chunk against 64 activation bytes; chunks past the row (c >= C,
    //    last round only) contribute nothing.
    int acc;
    if constexpr (P == Pattern::Dense) {
        // In word w, code pair s of each byte is (w >> 2s) & 0x03; pairs 1
        // and 2 are taken in place (masks 0x0C, 0x30: the code times 4 or
        // 16, still a positive int8) into accumulators of their own, divided
        // back exactly at the end; pair 3 is shifted down (times 64 would not
        // fit an int8).
        int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = j + u * LPR;
            const bool in = c < C;
            const i32x4 *xp = reinterpret_cast<const i32x4 *>(s_x + (in ? c : C - 1) * 64);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const i32x4 xx = xp[q];
                const uint32_t word = in ? w[u].w[q] : 0u;
                a0 = __builtin_amdgcn_sdot4((int)(word & kCodeMask), xx[0], a0, false);
                a1 = __builtin_amdgcn_sdot4((int)(word & (kCodeMask << 2)), xx[1], a1, false);
                a2 = __builtin_amdgcn_sdot4((int)(word & (kCodeMask << 4)), xx[2], a2, false);
                a3 = __builtin_amdgcn_sdot4((int)((word >> 6) & kCodeMask), xx[3], a3, false);
            }
        }
        // a1 = 4 * S1 and a2 = 16 * S2 exactly, so the shifts are exact;
        // |a2| <= 16 * 2 * 127 * K / 4 < 2^31 for K <= 16384
        acc = a0 + (a1 >> 2) + (a2 >> 4) + a3;
    } else {
        // N:M: the kept codes are not decoded to dense words; each group's
        // kept weights, as 64 * t bytes, are spread over its positions by a
        // byte permute (nm_dot_superblock), pruned positions 0.  Chunks past
        // the row get code 1 (t = 0) everywhere.
        int a4[4] = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = j + u * LPR;
            const bool in = c < C;
            const i32x4 *xp = reinterpret_cast<const i32x4 *>(s_x + (in ? c : C - 1) * 64);
            int32_t xw[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const i32x4 xx = xp[q];
                xw[4 * q] = xx[0]; xw[4 * q + 1] = xx[1]; xw[4 * q + 2] = xx[2]; xw[4 * q + 3] = xx[3];
            }
            uint32_t vals[RawChunk<P>::kVals];
#pragma unroll
            for (int v = 0; v < RawChunk<P>::kVals; ++v) vals[v] = in ? w[u].w[v] : 0x55555555u;
            nm_dot_superblock<P, DeviceOps>(vals, w[u].w + RawChunk<P>::kVals, s_sel, xw, a4);
        }
        // every term is 64 * t * x: the shift is exact; |sum| <= 64 * 128 * K < 2^31
        acc = (a4[0] + a4[1] + a4[2] + a4[3]) >> 6;
    }
    acc = lanes_sum<LPR>(acc);
    if constexpr (NORM) {
        xsc = act_norm_scale(xg, act_rinv(ss, K, tr.eps));
        if (x_scale_out && tid == 0) x_scale_out[0] = xsc;
    }
    if (j == 0 && row < N) {
        // dense codes are t + 1: subtract the activation row sum
        const int av = (P == Pattern::Dense) ? acc - rs : acc;
        Y[row] = (float)av * (wsc * xsc);
        if (acc_out) acc_out[row] = av;
    }
}

template <Pattern P, int LPR, int U, bool FUSED, int W = 4, int TR = 0>
__global__ __launch_bounds__(64 * W) void decode_dot4_kernel(
    const float *__restrict__ X, const int8_t *__restrict__ Xq, const float *__restrict__ x_scale,
    const int32_t *__restrict__ x_rowsum, int64_t K, FusedProjArgs args, float *__restrict__ x_scale_out,
    ActTransform tr)
{
    // entries past the last projection hold the block count, so no test of
    // nproj is needed: without one the table loads issue together rather
    // than one round trip each
    // the input row's pointers, K and the table in the first batch of
    // argument loads; the projection's pointers are read in resolve(), after
    // the row loads are issued
    asm volatile("" ::"s"(X), "s"(Xq), "s"(K), "s"(tr.up), "s"(tr.gamma));
    const int block = (int)blockIdx.x;
    int p = 0, first = 0;
#pragma unroll
    for (int i = 1; i < kMaxFusedProj; ++i)
        if (block >= args.block_start[i]) {
            p = i;
            first = args.block_start[i];
        }
    asm volatile("" ::"s"(p), "s"(first));
    const auto resolve = [&]() {
        return ProjSel{ProjView{args.packed[p], args.w_scale[p], args.Y[p], args.acc[p], args.N[p]},
                       (int64_t)(block - first), block == 0 ? x_scale_out : nullptr};
    };
    decode_dot4_body<P, LPR, U, FUSED, W, TR>(X, Xq, x_scale, x_rowsum, K, resolve, tr);
}

}  // namespace dot4

// The host rule of the one-token kernel's configuration, for K and the
// projections of one input group: lanes per row, the fewest of 8, 16, 32, 64
// that keep a lane's chunks U <= 5, or <= 7 with the quantisation fused in
// (<= 4 at 64 lanes, K <= 16384).  The fused kernel reads and quantises the
// whole fp32 row in every workgroup, so it prefers fewer, fuller workgroups:
// at 8 lanes per row it takes 8 waves (64 rows) per workgroup where 4 waves
// would need more than 320 workgroups (gate+up of a 2B FFN: 432 -> 216,
// 4.1 -> 4.0 us), except with a row transform (trb != 0), where 4 waves
// measured faster (RMSNorm on gate+up 5.35 -> 5.13 us).
struct Dot4Config {
    int lpr;          // lanes per weight row
    int u;            // chunks of 64 codes per lane
    bool w8;          // 8 waves per workgroup (else 4)
    int64_t rb;       // weight rows per workgroup
};

inline Dot4Config dot4_config(int64_t K, bool fused, int trb, const FusedProjArgs &args)
{
    const int64_t C = K / 64;
    const int64_t umax = fused ? 7 : 5;
    int lpr = 8;
    while (lpr < 64 && (C + lpr - 1) / lpr > umax) lpr *= 2;
    const int u = (int)((C + lpr - 1) / lpr);
    int64_t b4 = 0;
    for (int i = 0; i < args.nproj; ++i) b4 += (args.N[i] + 31) / 32;
    const bool w8 = fused && lpr == 8 && b4 > 320 && trb == 0;
    return Dot4Config{lpr, u, w8, (w8 ? 8 : 4) * (64 / lpr)};
}

// Fills args.block_start for rows of `rb` per workgroup; returns the
// workgroup count.
inline int64_t dot4_block_starts(FusedProjArgs &args, int64_t rb)
{
    int64_t blocks = 0;
    for (int i = 0; i < args.nproj; ++i) {
        args.block_start[i] = (int32_t)blocks;
        blocks += (args.N[i] + rb - 1) / rb;
    }
    for (int i = args.nproj; i <= kMaxFusedProj; ++i) args.block_start[i] = (int32_t)blocks;
    return blocks;
}

using Dot4Fn = void (*)(dim3, size_t, hipStream_t, const float *, const int8_t *, const float *, const int32_t *,
                        int64_t, const FusedProjArgs &, float *, const ActTransform &);

// The fused kernel with a row transform (tr_bits = kTrGate | kTrNorm bits,
// not 0), built in a translation unit of its own; nullptr for a
// configuration that does not exist.
Dot4Fn pick_dot4_tr(Pattern p, int tr_bits, bool w8, int lpr, int u);

namespace {

using Fn = Dot4Fn;

template <Pattern P, int LPR, int U, bool FUSED, int W = 4, int TR = 0>
void launch(dim3 grid, size_t lds, hipStream_t stream, const float *X, const int8_t *Xq, const float *xs,
            const int32_t *rs, int64_t K, const FusedProjArgs &args, float *x_scale_out, const ActTransform &tr)
{
    hipLaunchKernelGGL((dot4::decode_dot4_kernel<P, LPR, U, FUSED, W, TR>), grid, dim3(64 * W), lds, stream, X, Xq,
                       xs, rs, K, args, x_scale_out, tr);
}

// Fused, 8 lanes per row, 8 waves (64 rows per workgroup)
template <Pattern P, int TR = 0>
Fn pick_w8(int u)
{
    switch (u) {
    case 1: return launch<P, 8, 1, true, 8, TR>;
    case 2: return launch<P, 8, 2, true, 8, TR>;
    case 3: return launch<P, 8, 3, true, 8, TR>;
    case 4: return launch<P, 8, 4, true, 8, TR>;
    case 5: return launch<P, 8, 5, true, 8, TR>;
    case 6: return launch<P, 8, 6, true, 8, TR>;
    case 7: return launch<P, 8, 7, true, 8, TR>;
    default: return nullptr;
    }
}

// The (lanes per row, chunks per lane) pairs the host rule below can pick:
// plain U <= 5 (<= 4 at 64 lanes), fused U <= 7 (4 at 64 lanes).
template <Pattern P, bool FUSED, int TR = 0>
Fn pick(int lpr, int u)
{
    switch (lpr * 16 + u) {
    case 8 * 16 + 1: return launch<P, 8, 1, FUSED, 4, TR>;
    case 8 * 16 + 2: return launch<P, 8, 2, FUSED, 4, TR>;
    case 8 * 16 + 3: return launch<P, 8, 3, FUSED, 4, TR>;
    case 8 * 16 + 4: return launch<P, 8, 4, FUSED, 4, TR>;
    case 8 * 16 + 5: return launch<P, 8, 5, FUSED, 4, TR>;
    case 16 * 16 + 4: return launch<P, 16, 4, FUSED, 4, TR>;
    case 16 * 16 + 5: return launch<P, 16, 5, FUSED, 4, TR>;
    case 32 * 16 + 4: return launch<P, 32, 4, FUSED, 4, TR>;
    case 32 * 16 + 5: return launch<P, 32, 5, FUSED, 4, TR>;
    case 64 * 16 + 4: return launch<P, 64, 4, FUSED, 4, TR>;
    default: break;
    }
    if constexpr (FUSED) {
        switch (lpr * 16 + u) {
        case 8 * 16 + 6: return launch<P, 8, 6, true, 4, TR>;
        case 8 * 16 + 7: return launch<P, 8, 7, true, 4, TR>;
        case 16 * 16 + 6: return launch<P, 16, 6, true, 4, TR>;
        case 16 * 16 + 7: return launch<P, 16, 7, true, 4, TR>;
        case 32 * 16 + 6: return launch<P, 32, 6, true, 4, TR>;
        case 32 * 16 + 7: return launch<P, 32, 7, true, 4, TR>;
        default: return nullptr;
        }
    } else {
        switch (lpr * 16 + u) {
        case 16 * 16 + 3: return launch<P, 16, 3, false>;
        case 32 * 16 + 3: return launch<P, 32, 3, false>;
        case 64 * 16 + 3: return launch<P, 64, 3, false>;
        default: return nullptr;
        }
    }
}


}  // namespace
}  // namespace bl
