// Few-token forward (9 to 64 tokens) over wide projections: the packed
// weights straight from the load registers into the MFMA operand, as in the
// direct-load skinny kernel, with TT tiles of 16 tokens sharing every weight
// fragment a lane loads.
//
// "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 5.1: the packed ternary
// weights (four per byte) are what moves from HBM and are unpacked on chip;
// "BitNet 논문 분석: 1-Bit LLM의 시대", section "Absmean 양자화 함수": the
// integer linear of the ternary weights with the int8 activations, then the
// rescale by the weight and activation scales.  Same arithmetic as the other
// skinny kernels, bit for bit.
//
// Workgroup: KS = 4 waves, 16 * RG weight rows, TT * 16 token rows.  Wave w
// takes the w-th quarter of K's 64-wide chunks: its activation range of the
// tile's token rows is staged in LDS by coalesced loads, and lane (r, q) loads
// chunk 4 s + q of weight row 16 g + r for step s and column block g (64
// bytes of each of 16 rows per load instruction), which is its B operand for
// the step's four MFMAs against every token tile.  Codes of chunks past the
// wave's range are masked to 0 (zero products: the offset code 0 times any
// activation), so K needs no padding.  The four partial tiles of each output
// tile meet in LDS, in the activation area, at the tile's owner wave, which
// applies the offset-code correction and the dequant scale.  Token groups
// (16 * TT tokens each) of one row block run on one XCD (workgroup ids 8
// apart), so a later group's weight reads can hit that XCD's L2.  Counted
// HBM traffic at 64 tokens: 1.07x the algorithmic bytes with two groups
// (gate + up of a 3B block), 1.5-1.6x with four, where the non-temporal
// weight loads leave little in L2 (cached loads measured slower all the same).
//
// Where it is used (dense weights; a call's projections together; measured
// on MI355X against the library's previous kernel for the shape, us):
//   9-16 tokens, >= 6912 rows (TT 1, RG 2): gate + up of a 3B block (2 x 11008,
//     K 2048) at 16 tokens 7.6 -> 6.9; a 2B FFN's gate + up (2 x 6912, K 2560)
//     14.5 -> 6.8; one 6912-row projection 8.0 -> 5.3
//   17-32 tokens, >= 13824 rows (TT 1, RG 4): 3B gate + up at 32 tokens
//     10.4 -> 8.7; 2B gate + up 21.1 -> 9.2
//   17-32 tokens, 6912-13823 rows (TT 1, RG 2): 11008 rows at 32 tokens
//     8.3 -> 6.4; 6912 rows 10.5 -> 6.3
//   33-64 tokens, >= 16384 rows, K <= 2048 (TT 2, RG 6): 3B gate + up at 64
//     tokens 16.0 -> 11.4, at 48 15.8 -> 11.1
//   33-64 tokens, 6912-13823 rows (TT 1, RG 4): 11008 rows at 64 tokens
//     8.9 -> 8.2; 6912 rows (K 2560) 9.5 -> 8.5
//   17-64 tokens, 2560-6911 rows (TT 1, RG 2): 2560 x 2560 at 64 tokens
//     10.1 -> 6.0, at 17 6.7 -> 4.9; 3072 x 3072 at 48 tokens 10.6 -> 5.9;
//     5120 rows (K 2048) at 32 tokens 9.4 -> 5.2; q, k, v of a 3B block
//     (2560 rows in all) at 64 tokens 5.4 -> 5.0
//   33-64 tokens, 2048-2559 rows (TT 1, RG 2): 2048 x 2048 at 64 tokens
//     4.6 -> 4.3 (at 17-32 tokens the staged kernel is as fast)
// Non-temporal stores of Y, whole token rows from an LDS tile: the outputs
// leave in one burst at the end.
#include <stdio.h>

#include "kernels.hpp"
#include "skinny_impl.hpp"

namespace bl {
namespace skinny_direct_tiles {

using skinny::i32x4;
using skinny::u32x4;

constexpr int KS = 4;

template <int TT, int RG, int S>
struct Lds {
    static constexpr int kRow = S * 256 + 16;                      // staged token row (16-byte pad: banks)
    static constexpr int kWave = TT * 16 * kRow;
    static constexpr int kAct = KS * kWave;
    static constexpr int kPart = (KS - 1) * TT * RG * 64 * 16;     // [tile][slot][lane] i32x4
    static constexpr int kYRow = 16 * RG + 4;                      // staged output row (words, padded)
    static constexpr int kY = TT * 16 * kYRow * 4;                 // the Y tile, then the acc tile, after
    static constexpr int kBytes = kAct > kPart + 2 * kY ? kAct : kPart + 2 * kY;   // the partials
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Dense weights.  ty = ceil(M / (16 TT)) token groups (M <= 64) and `parts`
// K parts (1 unless SPLIT); grid = ceil(blocks / 8) * 8 * ty * parts.  The
// host keeps KS <= (chunks of a K part) <= 4 * S * KS.  SPLIT (one
// projection): each workgroup writes the raw int32 sums of its K part to
// ws[part][m][n] (M x N per part) and split_epilogue_kernel finishes.
// `id`: the workgroup's index within this launch's share of the grid (a
// multiple of 8 from the grid's start, so that ids 8 apart still share an
// XCD); `smem`: Lds<TT, RG, S>::kBytes + 512 bytes of LDS.
template <int TT, int RG, int S, bool SPLIT>
__device__ __forceinline__ void skinny_direct_tiles_body(const int8_t *__restrict__ Xq,
                                                         const float *__restrict__ x_scale,
                                                         const int32_t *__restrict__ x_rowsum,
                                                         const FusedProjArgs &args, int64_t M, int64_t K,
                                                         int32_t parts, int32_t *__restrict__ ws, int id,
                                                         uint8_t *smem)
{
    using L = Lds<TT, RG, S>;
    constexpr int XLOADS = TT * 16 * S * 16 / 64;                 // 16-byte pieces per lane
    uint8_t *s_x = smem;
    int32_t *s_rs = reinterpret_cast<int32_t *>(smem + L::kBytes);
    float *s_xs = reinterpret_cast<float *>(smem + L::kBytes + 256);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, q = lane >> 4;

    // workgroup id -> (row block, token group, K part): ids 8 apart share an XCD
    const int ty = (int)((M + 16 * TT - 1) / (16 * TT));
    const int ny = SPLIT ? ty * parts : ty;
    const int yy = (id / 8) % ny;
    const int bx = (id / (8 * ny)) * 8 + id % 8;
    const int by = yy % ty;
    const int kp = SPLIT ? yy / ty : 0;
    if (bx >= args.block_start[args.nproj]) return;                // whole workgroup, before any barrier
    const int p = proj_of_block(args, bx);
    const int64_t N = args.N[p];
    const uint8_t *packed = args.packed[p];
    const float *w_scale = args.w_scale[p];
    const int64_t t0 = (int64_t)by * TT * 16;
    Xq += t0 * K;
    x_scale += t0;
    x_rowsum += t0;
    const int64_t mg = M - t0;                                     // tokens of this group (>= 1)
    float *Y = args.Y[p] + t0 * N;
    int32_t *acc_out = args.acc[p] ? args.acc[p] + t0 * N : nullptr;
    const int64_t n0 = (int64_t)(bx - args.block_start[p]) * 16 * RG;
    const int64_t C = K / 64;
    const int64_t cp_lo = SPLIT ? C * kp / parts : 0;              // the part's chunks
    const int64_t cp = SPLIT ? C * (kp + 1) / parts - cp_lo : C;
    const int64_t c_lo = cp_lo + cp * wave / KS;
    const int cw = (int)(cp_lo + cp * (wave + 1) / KS - c_lo);     // 1 <= cw <= 4 S
    uint8_t *lx = s_x + wave * L::kWave;
    // every kernel argument in SGPRs now: a scalar load left pending would make
    // the compiler wait for all outstanding memory operations at its first use
    asm volatile("" ::"s"(Xq), "s"(x_scale), "s"(x_rowsum), "s"(packed), "s"(w_scale), "s"(Y), "s"(acc_out));

    // 1. the wave's activation range: consecutive lanes, consecutive 16-byte
    //    pieces of a token row (rows past the group are not staged: they only
    //    feed outputs that are not stored)
    const int mt = (int)min(mg, (int64_t)(TT * 16));
    u32x4 x[XLOADS];
    int x_off[XLOADS];
    const int xw = cw * 4;
    const float inv_xw = 1.0f / (float)xw;
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int f = i * 64 + lane;
        const int m = (int)(((float)f + 0.5f) * inv_xw);           // exact: f < 2^24
        const int piece = f - m * xw;
        x_off[i] = (m < mt) ? m * L::kRow + piece * 16 : -1;
        x[i] = *reinterpret_cast<const u32x4 *>(Xq + (int64_t)min(m, mt - 1) * K + c_lo * 64 +
                                                (m < mt ? piece : 0) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. every weight chunk of the lane, all in flight (chunks past the range
    //    re-read its last one, rows past N re-read row N - 1)
    u32x4 w[S][RG];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int64_t n = min(n0 + 16 * g + r, N - 1);
            w[s][g] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(packed + n * (K / 4) + (c_lo + min(4 * s + q, cw - 1)) * 16));
        }
    // the epilogue's per-token values last: waited for only at the end
    const int mrow = min(lane, (int)mg - 1);
    const int rs_l = x_rowsum[mrow];
    const float xs_l = x_scale[mrow];
    const float beta = w_scale[0];
    __builtin_amdgcn_sched_barrier(0);

    // 3. activations to LDS; the wave reads only its own area
#pragma unroll
    for (int i = 0; i < XLOADS; ++i)
        if (x_off[i] >= 0) *reinterpret_cast<u32x4 *>(lx + x_off[i]) = x[i];
    __builtin_amdgcn_s_waitcnt(0xc07f);                            // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();

    // 4. MFMA: per step and token tile, the lane's four activation words
    //    against each column block's weight words, as the weights arrive
    i32x4 acc[TT][RG];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int g = 0; g < RG; ++g) acc[tt][g] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bool live = 4 * s + q < cw;
        const uint32_t cm = live ? kCodeMask : 0u;
        const int aoff = r * L::kRow + (live ? (4 * s + q) * 64 : 0);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            i32x4 a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const i32x4 *>(lx + tt * 16 * L::kRow + aoff + 16 * t);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const uint32_t wv = w[s][g][t];
                    i32x4 b;
                    b[0] = (int)(wv & cm);
                    b[1] = (int)((wv >> 2) & cm);
                    b[2] = (int)((wv >> 4) & cm);
                    b[3] = (int)((wv >> 6) & cm);
                    acc[tt][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b, acc[tt][g], 0, 0, 0);
                }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 5. partial tiles to their owner wave (tile j = tt RG + g, owner j % KS),
    //    in the activation area once every wave is done with it
    __syncthreads();
    if (wave == 0) {
        s_rs[lane] = rs_l;
        s_xs[lane] = xs_l;
    }
    i32x4 *part = reinterpret_cast<i32x4 *>(s_x);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int j = tt * RG + g, owner = j % KS;
            if (owner != wave) part[(j * (KS - 1) + wave - (wave > owner ? 1 : 0)) * 64 + lane] = acc[tt][g];
        }
    __syncthreads();

    // 6. epilogue: lane (r, q) holds tokens 4 q .. 4 q + 3 of the token tile,
    //    weight row 16 g + r.  Y goes to an LDS tile first and leaves as
    //    whole token rows of 16 RG outputs (16-byte non-temporal stores where
    //    N and Y allow): the fragment layout would write 64-byte pieces of
    //    four rows per instruction (3B gate + up at 64 tokens 11.3 -> 10.5 us).
    float *yt = reinterpret_cast<float *>(s_x + L::kPart);
    int32_t *at = reinterpret_cast<int32_t *>(s_x + L::kPart + L::kY);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int j = tt * RG + g;
            if (j % KS != wave) continue;
            i32x4 sum = acc[tt][g];
#pragma unroll
            for (int sl = 0; sl < KS - 1; ++sl) sum += part[(j * (KS - 1) + sl) * 64 + lane];
            const int64_t n = n0 + 16 * g + r;
            if constexpr (!SPLIT) {
                int av[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 16 * tt + 4 * q + v;
                    av[v] = sum[v] - s_rs[m];
                    yt[m * L::kYRow + 16 * g + r] = (float)av[v] * (beta * s_xs[m]);
                }
                if (acc_out) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) at[(16 * tt + 4 * q + v) * L::kYRow + 16 * g + r] = av[v];
                }
                continue;
            }
            if (n >= N) continue;
            if constexpr (SPLIT) {
                int32_t *wp = ws + ((int64_t)kp * M + t0) * N + n;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 16 * tt + 4 * q + v;
                    if (m < mg) wp[(int64_t)m * N] = sum[v];
                }
                continue;
            }
        }
    if constexpr (!SPLIT) {
        __syncthreads();
        constexpr int W4 = 4 * RG;                                 // 16-byte pieces per token row
        const int ncols = (int)min((int64_t)(16 * RG), N - n0);
        const int mrows = (int)min(mg, (int64_t)(TT * 16));
        const bool vec = (N % 4 == 0) && (reinterpret_cast<uintptr_t>(Y) % 16 == 0);
#pragma unroll
        for (int i0 = 0; i0 < TT * 16 * W4; i0 += 64 * KS) {
            const int i = i0 + threadIdx.x;
            const int m = i / W4, c = 4 * (i % W4);
            if (i >= TT * 16 * W4 || m >= mrows) continue;
            const float *src = yt + m * L::kYRow + c;
            float *dst = Y + (int64_t)m * N + n0 + c;
            if (vec && c + 4 <= ncols) {
                __builtin_nontemporal_store(*reinterpret_cast<const f32x4 *>(src), reinterpret_cast<f32x4 *>(dst));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c + e < ncols) __builtin_nontemporal_store(src[e], dst + e);
            }
        }
        if (acc_out) {
            for (int i = threadIdx.x; i < mrows * 16 * RG; i += 64 * KS) {
                const int m = i / (16 * RG), c = i % (16 * RG);
                if (c < ncols) acc_out[(int64_t)m * N + n0 + c] = at[m * L::kYRow + c];
            }
        }
    }
}

template <int TT, int RG, int S, bool SPLIT>
__global__ __launch_bounds__(64 * KS) void skinny_direct_tiles_kernel(const int8_t *__restrict__ Xq,
                                                                      const float *__restrict__ x_scale,
                                                                      const int32_t *__restrict__ x_rowsum,
                                                                      FusedProjArgs args, int64_t M, int64_t K,
                                                                      int32_t parts, int32_t *__restrict__ ws)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    skinny_direct_tiles_body<TT, RG, S, SPLIT>(Xq, x_scale, x_rowsum, args, M, K, parts, ws, (int)blockIdx.x, smem);
}

// Several quantised inputs in one launch (9-64 tokens each): group g's
// workgroups are [group_start[g], group_start[g + 1]) (multiples of 8: each
// group keeps the one-input kernel's XCD placement) and run configuration
// cfg[g] (as numbered by tiles_config).  The argument is read in place in the
// kernel-argument segment (indexed by the group, a copy would live in
// scratch memory).
#define BL_TILES_CASE(ID, TT, RG, S)                                                                            \
    case ID:                                                                                                    \
        skinny_direct_tiles_body<TT, RG, S, false>(da.Xq[gi], da.x_scale[gi], da.x_rowsum[gi], da.args[gi], da.M,  \
                                                   da.K[gi], 1, nullptr, id, smem);                            \
        return;

__global__ __launch_bounds__(64 * KS) void skinny_direct_tiles_multi_kernel(DirectMultiArgs)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const DirectMultiArgs &da = *(const DirectMultiArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    int gi = 0;
#pragma unroll
    for (int i = 1; i < kMaxInputGroups; ++i)
        if ((int)blockIdx.x >= da.group_start[i]) gi = i;   // entries past ngroups: the block count
    const int id = (int)blockIdx.x - da.group_start[gi];
    switch (da.cfg[gi]) {
        BL_TILES_CASE(0, 1, 2, 2)
        BL_TILES_CASE(1, 1, 2, 3)
        BL_TILES_CASE(2, 1, 4, 2)
        BL_TILES_CASE(3, 1, 4, 3)
        BL_TILES_CASE(4, 2, 6, 2)
    default: return;
    }
}

#undef BL_TILES_CASE

// Sum of the K parts' int32 partials (integer sums: exact in any order),
// offset-code correction and dequant scale; one output per thread.
__global__ __launch_bounds__(256) void split_epilogue_kernel(const float *__restrict__ x_scale,
                                                             const int32_t *__restrict__ x_rowsum,
                                                             const float *__restrict__ w_scale, int64_t M, int64_t N,
                                                             int32_t parts, const int32_t *__restrict__ ws,
                                                             float *__restrict__ Y, int32_t *__restrict__ acc_out)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N;
    int acc = 0;
    for (int o = 0; o < parts; ++o) acc += ws[(int64_t)o * M * N + idx];
    const int av = acc - x_rowsum[m];
    Y[idx] = (float)av * (w_scale[0] * x_scale[m]);
    if (acc_out) acc_out[idx] = av;
}

}  // namespace skinny_direct_tiles

namespace {

thread_local char g_name[80];

// Dynamic LDS past 64 KB must be allowed per kernel.
hipError_t allow_lds(const void *kern, size_t bytes)
{
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int TT, int RG, int S>
hipError_t launch(const int8_t *Xq, const float *xs, const int32_t *rs, FusedProjArgs args, int64_t M, int64_t K,
                  hipStream_t stream, const char **name, bool query)
{
    using L = skinny_direct_tiles::Lds<TT, RG, S>;
    static_assert(L::kBytes + 512 <= 160 * 1024, "LDS");
    constexpr int KS = skinny_direct_tiles::KS;
    const int64_t C = K / 64;
    const int64_t ty = (M + 16 * TT - 1) / (16 * TT);
    if (C < KS || C > (int64_t)4 * S * KS || ty < 1 || ty > 4) return hipErrorNotSupported;
    int64_t blocks = 0;
    for (int i = 0; i < args.nproj; ++i) {
        args.block_start[i] = (int32_t)blocks;
        blocks += (args.N[i] + 16 * RG - 1) / (16 * RG);
    }
    for (int i = args.nproj; i <= kMaxFusedProj; ++i) args.block_start[i] = (int32_t)blocks;
    const int64_t grid = (blocks + 7) / 8 * 8 * ty;
    if (grid > (1LL << 30)) return hipErrorNotSupported;
    snprintf(g_name, sizeof g_name, "skinny_direct_tiles_dense_t%d_rg%d_s%d%s", TT, RG, S, args.nproj > 1 ? "_grouped" : "");
    *name = g_name;
    if (query) return hipSuccess;
    auto kern = skinny_direct_tiles::skinny_direct_tiles_kernel<TT, RG, S, false>;
    const hipError_t e = allow_lds((const void *)kern, L::kBytes + 512);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KS), (size_t)(L::kBytes + 512), stream, Xq, xs, rs, args,
                       M, K, 1, nullptr);
    return hipGetLastError();
}

// One projection with K split into `parts` parts over the workgroups: int32
// partials (parts x M x N) in the caller's workspace, then the epilogue kernel.
template <int TT, int RG, int S>
hipError_t launch_split(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                        const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, int parts,
                        Scratch &scratch, hipStream_t stream, const char **name)
{
    using L = skinny_direct_tiles::Lds<TT, RG, S>;
    static_assert(L::kBytes + 512 <= 160 * 1024, "LDS");
    constexpr int KS = skinny_direct_tiles::KS;
    const int64_t C = K / 64;
    const int64_t ty = (M + 16 * TT - 1) / (16 * TT);
    // every K part holds between KS and 4 S KS chunks
    if (parts < 2 || C / parts < KS || (C + parts - 1) / parts > (int64_t)4 * S * KS || ty < 1 || ty > 4)
        return hipErrorNotSupported;
    const int64_t blocks = (N + 16 * RG - 1) / (16 * RG);
    const int64_t grid = (blocks + 7) / 8 * 8 * ty * parts;
    if (grid > (1LL << 30) || blocks > (1LL << 30)) return hipErrorNotSupported;
    snprintf(g_name, sizeof g_name, "skinny_direct_tiles_dense_t%d_rg%d_s%d_splitk%d", TT, RG, S, parts);
    *name = g_name;
    if (!scratch.take((size_t)parts * (size_t)(M * N) * 4)) return scratch.query ? hipSuccess : hipErrorOutOfMemory;
    FusedProjArgs args = {};
    args.nproj = 1;
    args.packed[0] = packed;
    args.w_scale[0] = w_scale;
    args.N[0] = N;
    args.Y[0] = Y;
    args.acc[0] = acc;
    args.block_start[0] = 0;
    for (int i = 1; i <= kMaxFusedProj; ++i) args.block_start[i] = (int32_t)blocks;
    int32_t *ws = reinterpret_cast<int32_t *>(scratch.ptr);
    {
        using LS = skinny_direct_tiles::Lds<TT, RG, S>;
        auto kern = skinny_direct_tiles::skinny_direct_tiles_kernel<TT, RG, S, true>;
        const hipError_t e0 = allow_lds((const void *)kern, LS::kBytes + 512);
        if (e0 != hipSuccess) return e0;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KS), (size_t)(LS::kBytes + 512), stream, Xq, xs, rs,
                           args, M, K, (int32_t)parts, ws);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(skinny_direct_tiles::split_epilogue_kernel, dim3((unsigned)((M * N + 255) / 256)), dim3(256), 0,
                       stream, xs, rs, w_scale, M, N, (int32_t)parts, ws, Y, acc);
    return hipGetLastError();
}

template <int TT, int RG>
hipError_t launch_k(const int8_t *Xq, const float *xs, const int32_t *rs, const FusedProjArgs &args, int64_t M,
                    int64_t K, hipStream_t stream, const char **name, bool query)
{
    if (K / 64 <= 32) return launch<TT, RG, 2>(Xq, xs, rs, args, M, K, stream, name, query);
    return launch<TT, RG, 3>(Xq, xs, rs, args, M, K, stream, name, query);
}

}  // namespace

namespace {

// The measured cases of the file comment (dense weights, 9-64 tokens, K 256 to
// 3072): the configuration <TT, RG, S> as 0: <1, 2, 2>, 1: <1, 2, 3>,
// 2: <1, 4, 2>, 3: <1, 4, 3>, 4: <2, 6, 2>; -1 for every other shape.
int tiles_config(int64_t M, int64_t K, int64_t rows)
{
    const int64_t C = K / 64;
    if (M < 9 || M > 64 || C < skinny_direct_tiles::KS || C > 48 || rows < 2048) return -1;
    const int s3 = C <= 32 ? 0 : 1;                                // S = 2 up to 32 chunks, else 3
    if (rows < 6912) return M >= (rows < 2560 ? 33 : 17) ? 0 + s3 : -1;
    if (M <= 16) return 0 + s3;
    if (M <= 32) return rows >= 13824 ? 2 + s3 : 0 + s3;
    if (rows < 13824) return 2 + s3;
    if (rows >= 16384 && C <= 32) return 4;
    return -1;
}

}  // namespace

hipError_t launch_skinny_direct_tiles(const int8_t *Xq, const float *xs, const int32_t *rs, const FusedProjArgs &args,
                               Pattern p, int64_t M, int64_t K, hipStream_t stream, const char **name, bool query)
{
    if (p != Pattern::Dense || args.nproj < 1 || args.nproj > kMaxFusedProj) return hipErrorNotSupported;
    int64_t rows = 0;
    for (int i = 0; i < args.nproj; ++i) rows += args.N[i];
    switch (tiles_config(M, K, rows)) {
    case 0: return launch<1, 2, 2>(Xq, xs, rs, args, M, K, stream, name, query);
    case 1: return launch<1, 2, 3>(Xq, xs, rs, args, M, K, stream, name, query);
    case 2: return launch<1, 4, 2>(Xq, xs, rs, args, M, K, stream, name, query);
    case 3: return launch<1, 4, 3>(Xq, xs, rs, args, M, K, stream, name, query);
    case 4: return launch<2, 6, 2>(Xq, xs, rs, args, M, K, stream, name, query);
    default: return hipErrorNotSupported;
    }
}

// One dense projection at 9-64 tokens with K too deep for one workgroup's
// staging (49 to 384 chunks of 64) and 1024 to 4096 weight rows (2560 past
// 32 tokens): K split into ceil(C / 48) parts over the workgroups, int32
// partials in the caller's workspace (parts x M x N), then one elementwise
// pass.  Measured on MI355X against the few-token GEMM with K split (us):
// 2560 x 6912 at 16 tokens 11.9 -> 7.8, at 32 12.5 -> 9.5, at 64 15.7 ->
// 11.6; 2048 x 11008 at 9 tokens 11.3 -> 7.9, at 32 11.3 -> 10.1, at 64
// 12.4 -> 12.2; 4096 x 11008 at 16 tokens 15.8 -> 10.8 (at 64: 18.8
// against 20.5, hence the narrower row range there).  The forward tries the
// staged skinny kernel first (1024 x 4096 at 16-64 tokens: 4.5 us there).
// hipErrorNotSupported (nothing launched) for every other shape.
hipError_t launch_skinny_direct_tiles_split(const int8_t *Xq, const float *xs, const int32_t *rs,
                                            const uint8_t *packed, const float *w_scale, Pattern p, int64_t M,
                                            int64_t N, int64_t K, float *Y, int32_t *acc, Scratch &scratch,
                                            hipStream_t stream, const char **name)
{
    const int64_t C = K / 64;
    if (p != Pattern::Dense || M < 9 || M > 64 || C <= 48 || C > 384 || N < 1024 || N > (M <= 32 ? 4096 : 2560))
        return hipErrorNotSupported;
    const int parts = (int)((C + 47) / 48);
    if (M <= 32)
        return launch_split<1, 2, 3>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, parts, scratch, stream, name);
    return launch_split<2, 4, 3>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, parts, scratch, stream, name);
}

// The multi-input launch at 9-64 tokens: every group must fit the one-input
// rule (tiles_config).
hipError_t launch_skinny_direct_tiles_multi(DirectMultiArgs da, hipStream_t stream, const char **name, bool query)
{
    thread_local char g_mname[160];
    if (da.ngroups < 1 || da.ngroups > kMaxInputGroups) return hipErrorNotSupported;
    static const int kTT[5] = {1, 1, 1, 1, 2}, kRG[5] = {2, 2, 4, 4, 6}, kS[5] = {2, 3, 2, 3, 2};
    static const size_t kLds[5] = {
        skinny_direct_tiles::Lds<1, 2, 2>::kBytes + 512, skinny_direct_tiles::Lds<1, 2, 3>::kBytes + 512,
        skinny_direct_tiles::Lds<1, 4, 2>::kBytes + 512, skinny_direct_tiles::Lds<1, 4, 3>::kBytes + 512,
        skinny_direct_tiles::Lds<2, 6, 2>::kBytes + 512};
    int64_t grid = 0;
    size_t lds = 0;
    int len = snprintf(g_mname, sizeof g_mname, "skinny_direct_tiles_multi_dense");
    for (int g = 0; g < da.ngroups; ++g) {
        FusedProjArgs &a = da.args[g];
        if (a.nproj < 1 || a.nproj > kMaxFusedProj) return hipErrorNotSupported;
        int64_t rows = 0;
        for (int i = 0; i < a.nproj; ++i) rows += a.N[i];
        const int cfg = tiles_config(da.M, da.K[g], rows);
        if (cfg < 0) return hipErrorNotSupported;
        da.cfg[g] = cfg;
        int64_t blocks = 0;
        for (int i = 0; i < a.nproj; ++i) {
            a.block_start[i] = (int32_t)blocks;
            blocks += (a.N[i] + 16 * kRG[cfg] - 1) / (16 * kRG[cfg]);
        }
        for (int i = a.nproj; i <= kMaxFusedProj; ++i) a.block_start[i] = (int32_t)blocks;
        const int64_t ty = (da.M + 16 * kTT[cfg] - 1) / (16 * kTT[cfg]);
        da.group_start[g] = (int32_t)grid;
        grid += (blocks + 7) / 8 * 8 * ty;
        if (grid > (1LL << 30)) return hipErrorNotSupported;
        if (kLds[cfg] > lds) lds = kLds[cfg];
        if (len < (int)sizeof g_mname)
            len += snprintf(g_mname + len, sizeof g_mname - len, "%st%d_rg%d_s%d_p%d", g ? "+" : "_", kTT[cfg],
                            kRG[cfg], kS[cfg], a.nproj);
    }
    for (int g = da.ngroups; g <= kMaxInputGroups; ++g) da.group_start[g] = (int32_t)grid;
    *name = g_mname;
    if (query) return hipSuccess;
    auto kern = skinny_direct_tiles::skinny_direct_tiles_multi_kernel;
    const hipError_t e = allow_lds((const void *)kern, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * skinny_direct_tiles::KS), lds, stream, da);
    return hipGetLastError();
}

}  // namespace bl
