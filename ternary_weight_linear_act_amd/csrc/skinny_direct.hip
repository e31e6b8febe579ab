// Skinny MFMA forward (5 to 64 tokens) with the packed weights taken straight
// from the load registers as the MFMA's B operand: no staging of the weights
// in LDS.
//
// "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 5.1: the packed ternary
// weights (four per byte) are what moves from HBM and are unpacked on chip;
// "BitNet 논문 분석: 1-Bit LLM의 시대", section "Absmean 양자화 함수": the
// integer linear of the ternary weights with the int8 activations, then the
// rescale by the weight and activation scales.  Same arithmetic as the
// staged skinny kernel (skinny_impl.hpp), bit for bit.
//
// The lane <-> k mapping of that kernel already gives lane (r, q) = (lane %
// 16, lane / 16) exactly one 16-byte chunk per 256-wide step: chunk 4 s + q
// of weight row r, whose four words feed the four MFMAs of the step.  Here
// the lane loads that chunk itself, so the weights go HBM -> VGPR -> MFMA
// with no LDS round trip and no wait for the other lanes' stores; each load
// instruction covers half of a 128-byte line of 16 rows, and the next step's
// instruction the other half.  The activations (the wave's K range of MT
// token rows, 3 zero chunks after it) are staged in LDS as in the staged
// kernel.  RG column blocks of 16 weight rows per wave share the activation
// reads.  KS waves split K; their partial sums meet in LDS.
//
// Where it is used (measured on MI355X against the staged kernel, dense
// weights, us): gate + up of a 3B block (2 x 11008 rows, K = 2048) at 8
// tokens 7.0 -> 6.3; gate + up of a 2B FFN (2 x 6912, K = 2560) at 8 tokens
// 7.2 -> 6.2; the 3B down projection (11008 -> 2048) at 8 tokens 7.6 -> 6.2;
// q, k, v of a 3B block at 64 tokens (one grouped launch) 6.8 -> 5.3.  At 4
// tokens and for narrow projections (<= 2560 rows) at 8-16 tokens the staged
// kernel measured as fast or faster.  Wide projections at 9-64 tokens take
// the form with several token tiles per workgroup (skinny_direct_tiles.hip) first.
#include <stdio.h>

#include "kernels.hpp"
#include "skinny_impl.hpp"

namespace bl {
namespace skinny_direct {

using skinny::i32x4;
using skinny::u32x4;
using skinny::RawChunk;
using skinny::load_raw_chunk;
using skinny::decode_chunk;
using skinny::unpack_word;

template <int KS, int CMAX, int MT, int RG>
struct Lds {
    static constexpr int kXStride = (CMAX + 3) * 64;               // activation row (3 zero chunks)
    static constexpr int kWave = MT * kXStride + 64;               // + the zero block of token rows >= M
    static constexpr int kBytes = KS * kWave + (KS > 1 ? KS - 1 : 1) * RG * 64 * 16;
};

// Dense weights only.  1 <= M - 16 y <= MT tokens per tile (tiles of 16
// along y when M > 16, then MT == 16); the host keeps KS <= K / 64 and
// K / 64 <= KS * CMAX.
// `bx`, `by`: the workgroup's column block (within this launch's share of the
// grid) and token tile; `smem`: Lds<KS, CMAX, MT, RG>::kBytes of LDS.  Only
// waves below KS may enter.
template <int KS, int CMAX, int MT, int RG>
__device__ __forceinline__ void skinny_direct_body(const int8_t *__restrict__ Xq, const float *__restrict__ x_scale,
                                                   const int32_t *__restrict__ x_rowsum, const FusedProjArgs &args,
                                                   int64_t M, int64_t K, int bx, int by, uint8_t *smem)
{
    static_assert(CMAX % 4 == 0 && MT >= 1 && MT <= 16, "config");
    using L = Lds<KS, CMAX, MT, RG>;
    constexpr int SMAX = CMAX / 4;                                 // 256-wide steps per wave
    constexpr int XLOADS = (MT * CMAX * 4 + 63) / 64;
    auto s_x = reinterpret_cast<uint8_t (*)[L::kWave]>(smem);                       // [KS][kWave]
    auto s_part = reinterpret_cast<i32x4 (*)[RG][64]>(smem + KS * L::kWave);        // [KS - 1][RG][64]

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int p = proj_of_block(args, bx);
    const int64_t N = args.N[p];
    const uint8_t *packed = args.packed[p];
    const float *w_scale = args.w_scale[p];
    const int64_t n0 = (int64_t)(bx - args.block_start[p]) * 16 * RG;
    const int64_t t0 = (int64_t)by * 16;                           // token tile
    Xq += t0 * K;
    x_scale += t0;
    x_rowsum += t0;
    float *Y = args.Y[p] + t0 * N;
    int32_t *acc_out = args.acc[p] ? args.acc[p] + t0 * N : nullptr;
    const int mt = (int)min(M - t0, (int64_t)MT);
    const int64_t C = K / 64;
    const int64_t c_lo = C * wave / KS;
    const int cw = (int)(C * (wave + 1) / KS - c_lo);              // 1 <= cw <= CMAX
    uint8_t *lx = s_x[wave];
    uint8_t *lz = lx + MT * L::kXStride;
    // every kernel argument in SGPRs now: a scalar load left pending would make
    // the compiler wait for all outstanding memory operations at its first use
    asm volatile("" ::"s"(Xq), "s"(x_scale), "s"(x_rowsum), "s"(packed), "s"(w_scale), "s"(Y), "s"(acc_out));

    // 1. the wave's activation range first (consecutive lanes, consecutive bytes)
    u32x4 x[XLOADS];
    int x_off[XLOADS];
    const int xw = cw * 4;                                         // 16-byte pieces per token
    const float inv_xw = 1.0f / (float)xw;
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int f = i * 64 + lane;
        const int m = (int)(((float)f + 0.5f) * inv_xw);
        const int piece = f - m * xw;
        x_off[i] = (m < mt) ? m * L::kXStride + piece * 16 : -1;
        x[i] = *reinterpret_cast<const u32x4 *>(Xq + (int64_t)min(m, mt - 1) * K + c_lo * 64 +
                                                (m < mt ? piece : 0) * 16);
    }
    const float beta = w_scale[0];
    int rs[4];
    float xsc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = min(4 * q + v, mt - 1);
        rs[v] = x_rowsum[m];
        xsc[v] = x_scale[m];
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. every weight chunk of the lane, all in flight: step s, column block g
    //    takes chunk 4 s + q of row 16 g + r (unconditional: chunks past the
    //    wave's range re-read its last one, rows past N re-read row N - 1)
    RawChunk<Pattern::Dense> w[SMAX][RG];
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int64_t n = min(n0 + 16 * g + r, N - 1);
            w[s][g] = load_raw_chunk<Pattern::Dense>(packed, N, K, n, c_lo + min(4 * s + q, cw - 1));
        }
    __builtin_amdgcn_sched_barrier(0);

    // 3. activations to LDS: 3 zero chunks after each row, the zero block
    for (int f = lane; f < mt * 12 + 4; f += 64) {
        const int off = (f < mt * 12) ? (f / 12) * L::kXStride + (cw * 4 + f % 12) * 16
                                      : MT * L::kXStride + (f - mt * 12) * 16;
        *reinterpret_cast<u32x4 *>(lx + off) = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < XLOADS; ++i)
        if (x_off[i] >= 0) *reinterpret_cast<u32x4 *>(lx + x_off[i]) = x[i];
    // the wave reads only its own staging area: its own stores, completed
    __builtin_amdgcn_s_waitcnt(0xc07f);                            // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();

    // 4. MFMA: per step, the four activation words of the lane's chunk (zero
    //    past the wave's range: the zero chunks) against each column block's
    //    weight words, as they arrive (in-order load waits)
    const uint8_t *arow = (r < mt) ? lx + r * L::kXStride + q * 64 : lz;
    const int astep = (r < mt) ? 256 : 0;
    i32x4 acc[RG][4];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[g][t] = i32x4{0, 0, 0, 0};
    const int steps = (cw + 3) / 4;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
        if (s < steps) {                                           // wave-uniform
            i32x4 a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const i32x4 *>(arow + s * astep + 16 * t);
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                const u32x4 b = decode_chunk<Pattern::Dense>(w[s][g], nullptr);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[g][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], unpack_word(b[t]), acc[g][t], 0, 0, 0);
            }
        }
    }
    i32x4 sum[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) sum[g] = (acc[g][0] + acc[g][1]) + (acc[g][2] + acc[g][3]);

    // 5. the KS partial sums meet in LDS
    if (KS > 1) {
        if (wave > 0) {
#pragma unroll
            for (int g = 0; g < RG; ++g) s_part[wave - 1][g][lane] = sum[g];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int w2 = 1; w2 < KS; ++w2) sum[g] += s_part[w2 - 1][g][lane];
    }

    // 6. epilogue: offset-code correction, dequant scale; lane (r, q) holds
    //    tokens 4 q .. 4 q + 3 of weight row 16 g + r
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int64_t nn = n0 + 16 * g + r;
        if (nn >= N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * q + v;
            if (m < mt) {
                const int av = sum[g][v] - rs[v];
                Y[(int64_t)m * N + nn] = (float)av * (beta * xsc[v]);
                if (acc_out) acc_out[(int64_t)m * N + nn] = av;
            }
        }
    }
}

template <int KS, int CMAX, int MT, int RG>
__global__ __launch_bounds__(64 * KS) void skinny_direct_kernel(const int8_t *__restrict__ Xq,
                                                                const float *__restrict__ x_scale,
                                                                const int32_t *__restrict__ x_rowsum,
                                                                FusedProjArgs args, int64_t M, int64_t K)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    skinny_direct_body<KS, CMAX, MT, RG>(Xq, x_scale, x_rowsum, args, M, K, (int)blockIdx.x, (int)blockIdx.y, smem);
}

// Several inputs in one launch (workgroups of 512 threads: a configuration
// with KS waves runs them in waves 0 .. KS - 1, the others end at once; a
// barrier waits only for the waves that have not ended).  The argument is
// read in place in the kernel-argument segment (indexed by the group, a copy
// would live in scratch memory).
#define BL_DIRECT_CASE(ID, KS, CMAX, MT, RG)                                                                    \
    case ID:                                                                                                    \
        if (wave < (KS))                                                                                        \
            skinny_direct_body<KS, CMAX, MT, RG>(da.Xq[gi], da.x_scale[gi], da.x_rowsum[gi], da.args[gi], da.M, \
                                                 da.K[gi], blk, 0, smem);                                       \
        return;

__global__ __launch_bounds__(512) void skinny_direct_multi_kernel(DirectMultiArgs)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const DirectMultiArgs &da = *(const DirectMultiArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    // the configuration and first block selected with the group from values
    // read with the table (loaded from the selected index instead, they cost
    // a second scalar round trip)
    int cfgs[kMaxInputGroups], firsts[kMaxInputGroups];
#pragma unroll
    for (int i = 0; i < kMaxInputGroups; ++i) {
        cfgs[i] = da.cfg[i];
        firsts[i] = da.group_start[i];
    }
    int gi = 0, cfg = cfgs[0], first = firsts[0];
#pragma unroll
    for (int i = 1; i < kMaxInputGroups; ++i)
        if ((int)blockIdx.x >= firsts[i]) {   // entries past ngroups: the block count
            gi = i;
            cfg = cfgs[i];
            first = firsts[i];
        }
    const int blk = (int)blockIdx.x - first;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    switch (cfg) {
        BL_DIRECT_CASE(0, 4, 8, 8, 1)
        BL_DIRECT_CASE(1, 4, 8, 8, 2)
        BL_DIRECT_CASE(2, 2, 20, 8, 1)
        BL_DIRECT_CASE(3, 8, 24, 8, 1)
    default: return;
    }
}

#undef BL_DIRECT_CASE

}  // namespace skinny_direct

namespace {

thread_local char g_name[80];

template <int KS, int CMAX, int MT, int RG>
hipError_t launch(const int8_t *Xq, const float *xs, const int32_t *rs, FusedProjArgs args, int64_t M, int64_t K,
                  hipStream_t stream, const char **name, bool query)
{
    static_assert(skinny_direct::Lds<KS, CMAX, MT, RG>::kBytes <= 160 * 1024, "LDS");
    const int64_t C = K / 64;
    if (C < KS || C > (int64_t)KS * CMAX || (M > 16 && MT != 16) || (M <= 16 && M > MT))
        return hipErrorNotSupported;
    int64_t blocks = 0;
    for (int i = 0; i < args.nproj; ++i) {
        args.block_start[i] = (int32_t)blocks;
        blocks += (args.N[i] + 16 * RG - 1) / (16 * RG);
    }
    for (int i = args.nproj; i <= kMaxFusedProj; ++i) args.block_start[i] = (int32_t)blocks;
    if (blocks > (1LL << 30)) return hipErrorNotSupported;
    snprintf(g_name, sizeof g_name, "skinny_direct_dense_ks%d_c%d_mt%d_rg%d%s", KS, CMAX, MT, RG,
             args.nproj > 1 ? "_grouped" : "");
    *name = g_name;
    if (query) return hipSuccess;
    auto kern = skinny_direct::skinny_direct_kernel<KS, CMAX, MT, RG>;
    constexpr size_t lds = skinny_direct::Lds<KS, CMAX, MT, RG>::kBytes;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks, (unsigned)((M + 15) / 16)), dim3(64 * KS), lds, stream, Xq, xs,
                       rs, args, M, K);
    return hipGetLastError();
}

}  // namespace

// The measured cases of the file comment (dense weights; args.nproj >= 1);
// hipErrorNotSupported (nothing launched) for every other shape.
hipError_t launch_skinny_direct(const int8_t *Xq, const float *xs, const int32_t *rs, const FusedProjArgs &args,
                                Pattern p, int64_t M, int64_t K, hipStream_t stream, const char **name, bool query)
{
    if (p != Pattern::Dense || args.nproj < 1 || args.nproj > kMaxFusedProj) return hipErrorNotSupported;
    int64_t rows = 0;
    for (int i = 0; i < args.nproj; ++i) rows += args.N[i];
    const int64_t C = K / 64;
    const bool wide = rows >= 8192;
    if (M >= 5 && M <= 8 && C >= 8 && C <= 32 && wide)
        return launch<4, 8, 8, 2>(Xq, xs, rs, args, M, K, stream, name, query);
    if (M >= 5 && M <= 8 && C > 32 && C <= 40 && wide)
        return launch<2, 20, 8, 1>(Xq, xs, rs, args, M, K, stream, name, query);
    if (M >= 5 && M <= 8 && C > 128 && C <= 192)
        return launch<8, 24, 8, 1>(Xq, xs, rs, args, M, K, stream, name, query);
    if (M >= 17 && M <= kSkinnyMaxM && args.nproj >= 2 && C >= 8 && C <= 32)
        return launch<4, 8, 16, 1>(Xq, xs, rs, args, M, K, stream, name, query);
    return hipErrorNotSupported;
}

// The multi-input launch at 5-8 tokens.  Each group's configuration (KS
// waves splitting K, CMAX chunks per wave, RG blocks of 16 weight rows per
// wave): K <= 2048 (at most 32 chunks) KS = 4, RG = 2 from 8192 rows in all
// (the single-input rule's), else RG = 1; 33-40 chunks KS = 2 (the
// single-input rule's); 41-192 chunks KS = 8 (the single-input rule's from
// 129 chunks).  Groups take the grid in order of decreasing K, as in the
// one-token multi-input launch.
hipError_t launch_skinny_direct_multi(DirectMultiArgs da, hipStream_t stream, const char **name, bool query)
{
    thread_local char g_mname[160];
    if (da.ngroups < 1 || da.ngroups > kMaxInputGroups || da.M < 5 || da.M > 8) return hipErrorNotSupported;
    {
        // decreasing K, stable
        DirectMultiArgs in = da;
        int order[kMaxInputGroups];
        for (int g = 0; g < da.ngroups; ++g) order[g] = g;
        for (int i = 1; i < da.ngroups; ++i)
            for (int j = i; j > 0 && in.K[order[j]] > in.K[order[j - 1]]; --j) {
                const int t = order[j];
                order[j] = order[j - 1];
                order[j - 1] = t;
            }
        for (int g = 0; g < da.ngroups; ++g) {
            const int o = order[g];
            da.Xq[g] = in.Xq[o];
            da.x_scale[g] = in.x_scale[o];
            da.x_rowsum[g] = in.x_rowsum[o];
            da.K[g] = in.K[o];
            da.args[g] = in.args[o];
        }
    }
    static const int kKS[4] = {4, 4, 2, 8}, kRG[4] = {1, 2, 1, 1};
    static const size_t kLds[4] = {skinny_direct::Lds<4, 8, 8, 1>::kBytes, skinny_direct::Lds<4, 8, 8, 2>::kBytes,
                                   skinny_direct::Lds<2, 20, 8, 1>::kBytes, skinny_direct::Lds<8, 24, 8, 1>::kBytes};
    int64_t blocks = 0;
    size_t lds = 0;
    int len = snprintf(g_mname, sizeof g_mname, "skinny_direct_multi_dense");
    for (int g = 0; g < da.ngroups; ++g) {
        FusedProjArgs &a = da.args[g];
        if (a.nproj < 1 || a.nproj > kMaxFusedProj) return hipErrorNotSupported;
        const int64_t C = da.K[g] / 64;
        int64_t rows = 0;
        for (int i = 0; i < a.nproj; ++i) rows += a.N[i];
        int cfg;
        if (C >= 4 && C <= 32) cfg = rows >= 8192 ? 1 : 0;
        else if (C >= 33 && C <= 40) cfg = 2;
        else if (C >= 41 && C <= 192) cfg = 3;
        else return hipErrorNotSupported;
        da.cfg[g] = cfg;
        da.group_start[g] = (int32_t)blocks;
        for (int i = 0; i < a.nproj; ++i) {
            a.block_start[i] = (int32_t)(blocks - da.group_start[g]);
            blocks += (a.N[i] + 16 * kRG[cfg] - 1) / (16 * kRG[cfg]);
        }
        for (int i = a.nproj; i <= kMaxFusedProj; ++i) a.block_start[i] = (int32_t)(blocks - da.group_start[g]);
        if (blocks > (1LL << 30)) return hipErrorNotSupported;
        if (kLds[cfg] > lds) lds = kLds[cfg];
        if (len < (int)sizeof g_mname)
            len += snprintf(g_mname + len, sizeof g_mname - len, "%sks%d_rg%d_p%d", g ? "+" : "_", kKS[cfg], kRG[cfg],
                            a.nproj);
    }
    for (int g = da.ngroups; g <= kMaxInputGroups; ++g) da.group_start[g] = (int32_t)blocks;
    *name = g_mname;
    if (query) return hipSuccess;
    auto kern = skinny_direct::skinny_direct_multi_kernel;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(512), lds, stream, da);
    return hipGetLastError();
}

}  // namespace bl
