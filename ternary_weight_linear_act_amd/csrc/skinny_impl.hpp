// Skinny forward for decode (1 <= M <= 16 tokens) on v_mfma_i32_16x16x64_i8.
//
// "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 5.1: the packed ternary
// weights (four per byte) are what moves from HBM, and the GPU kernel brings
// them into on-chip shared memory, unpacks them and computes against the
// 8-bit activations; "BitNet 논문 분석: 1-Bit LLM의 시대", section "Absmean
// 양자화 함수": integer linear of the ternary weights with the int8
// activations, then the rescale by the weight and activation scales.
//
// Why MFMA for M = 1: a 16x16x64 MFMA takes the activations as its A operand
// (token rows, zero-padded to 16) and 16 weight rows as its B operand, so one
// 64-byte slice of the activation vector serves 16 weight rows -- the
// activation traffic drops 16x compared with a per-row dot-product loop, and
// the VALU only unpacks codes: (word >> 2s) & 0x03030303 puts 4 codes in the
// 4 byte lanes, already in the order the B operand wants.
//
// Data flow of one wave: it owns 16 weight rows and a K range of cw chunks
// (a chunk = 64 weights = 16 packed bytes).
//  1. Load: every global load of the wave is issued up front, the
//     activations first (so that staging them waits for nothing else), then
//     the weights, in pairs: load 2j + h brings rows 8h .. 8h+7, chunks 8j .. 8j+7
//     (8 lanes read 128 contiguous bytes of a row, a full cache line), so
//     each pair completes two 256-wide steps for all 16 rows.  The M x cw
//     activation chunks are read with consecutive lanes on consecutive bytes.
//     Weight rows are staged in LDS with a stride of (8 * pairs + 1) * 16
//     bytes, an odd number of 16-byte units, so the MFMA-side reads (lane r of 16
//     reads row r) hit 16 distinct 4-bank groups.  Activation rows get 3
//     zero chunks after their last one, and a 64-byte zero block serves the
//     token rows >= M, so the MFMA loop needs no selects.
//  2. MFMA, pipelined with the loads: as soon as pair j has landed (in-order
//     vmcnt waits) it is written to LDS and its two steps run, while later
//     pairs are still in flight.  Per 256-wide step s, lane (r, q) = (lane % 16, lane / 16) reads
//     chunk 4 s + q of weight row r; MFMA t uses word t: B holds
//     k = 64 (4 s + q) + 16 t + (0..15) for weight row r, A the same k for
//     token r.  Four accumulators (one per t) keep the MFMAs independent, so
//     the dependent-MFMA latency is paid once per four.  Lane (r, q) ends with
//     C[4 q + v][r], v = 0..3: token 4 q + v of weight row r.
//  3. KS waves of a workgroup split K; their partial sums meet in LDS.  The
//     epilogue subtracts the activation row sum (codes are c = t + 1) and
//     applies beta * x_scale.
// Memory operations are branch-free (addresses clamped into range, unused
// values dropped), so the compiler issues all loads of a wave back to back.
#pragma once

#include "common.hpp"

namespace bl {

// Projections served by one launch (q/k/v, or gate/up, sharing their
// activations): per projection its packed weights, beta, output rows and
// outputs; block_start[i] is the first workgroup of projection i.
constexpr int kMaxFusedProj = 8;

struct FusedProjArgs {
    const uint8_t *packed[kMaxFusedProj];
    const float *w_scale[kMaxFusedProj];
    float *Y[kMaxFusedProj];
    int32_t *acc[kMaxFusedProj];
    int64_t N[kMaxFusedProj];
    int32_t block_start[kMaxFusedProj + 1];
    int32_t nproj;
};

// Several input groups in one one-token launch (decode_multi.hip): group g
// is the fp32 row X[g] of K[g] inputs with the projections args[g]; its
// workgroups are [group_start[g], group_start[g + 1]) of the grid and run
// configuration cfg[g] of the kernel's menu.
constexpr int kMaxInputGroups = 4;

struct MultiGroupArgs {
    const float *X[kMaxInputGroups];
    float *x_scale_out[kMaxInputGroups];
    int64_t K[kMaxInputGroups];
    int32_t cfg[kMaxInputGroups];
    int32_t group_start[kMaxInputGroups + 1];
    int32_t ngroups;
    FusedProjArgs args[kMaxInputGroups];
};

// Several quantised inputs in one launch of the direct-load skinny kernel
// (skinny_direct.hip), M tokens each: group g reads Xq[g] (M x K[g]) with
// the projections args[g]; its workgroups are [group_start[g],
// group_start[g + 1]) and run configuration cfg[g] of the kernel's menu.
struct DirectMultiArgs {
    const int8_t *Xq[kMaxInputGroups];
    const float *x_scale[kMaxInputGroups];
    const int32_t *x_rowsum[kMaxInputGroups];
    int64_t K[kMaxInputGroups];
    int32_t cfg[kMaxInputGroups];
    int32_t group_start[kMaxInputGroups + 1];
    int32_t ngroups;
    int64_t M;
    FusedProjArgs args[kMaxInputGroups];
};

// the projection of workgroup `block`
__device__ __forceinline__ int proj_of_block(const FusedProjArgs &args, int block)
{
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxFusedProj; ++i)
        if (block >= args.block_start[i]) p = i;   // entries past nproj hold the block count: loads issue together
    return p;
}

namespace skinny {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 unpack_word(uint32_t w)
{
    i32x4 b;
    b[0] = (int)(w & kCodeMask);
    b[1] = (int)((w >> 2) & kCodeMask);
    b[2] = (int)((w >> 4) & kCodeMask);
    b[3] = (int)((w >> 6) & kCodeMask);
    return b;
}

// Chunk c (64 weights) of row n as raw packed words: dense = 4 code words;
// N:M = the superblock's kept-code words, then its 2 mask words.  Loading
// the raw words and decoding them later (decode_chunk) keeps every load of a
// wave in flight at once: a decode right after each load would wait for it.
template <Pattern P>
struct RawChunk {
    static constexpr int kVals = (P == Pattern::Dense) ? 4 : (P == Pattern::NM24 ? 2 : 3);
    static constexpr int kWords = (P == Pattern::Dense) ? 4 : kVals + 2;
    uint32_t w[kWords];
};

template <Pattern P>
__device__ __forceinline__ RawChunk<P> load_raw_chunk(const uint8_t *__restrict__ packed, int64_t N, int64_t K,
                                                      int64_t n, int64_t c)
{
    RawChunk<P> r;
    if constexpr (P == Pattern::Dense) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(packed + n * (K / 4) + c * 16));
        r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
    } else {
        constexpr int GM = (P == Pattern::NM24) ? 4 : 8;
        constexpr int GN = (P == Pattern::NM24) ? 2 : 6;
        constexpr int VW = RawChunk<P>::kVals;
        const int64_t vrow = nm_value_row_bytes(K, GN, GM);
        const uint32_t *vp = reinterpret_cast<const uint32_t *>(packed + n * vrow + c * (VW * 4));
        const uint32_t *mp = reinterpret_cast<const uint32_t *>(packed + N * vrow + n * (K / 8) + c * 8);
#pragma unroll
        for (int v = 0; v < VW; ++v) r.w[v] = vp[v];
        r.w[VW] = mp[0];
        r.w[VW + 1] = mp[1];
    }
    return r;
}

// table24: the 2:4 decode table in LDS (fill_nm24_table), unused otherwise
template <Pattern P>
__device__ __forceinline__ u32x4 decode_chunk(const RawChunk<P> &r, const uint8_t *table24)
{
    if constexpr (P == Pattern::Dense) {
        return u32x4{r.w[0], r.w[1], r.w[2], r.w[3]};
    } else {
        uint32_t w[4];
        decode_superblock_fast<P>(r.w, r.w + RawChunk<P>::kVals, w, table24);
        return u32x4{w[0], w[1], w[2], w[3]};
    }
}

// fill the 256-byte 2:4 decode table (all threads of the workgroup; the
// caller places a barrier before the first decode)
template <Pattern P>
__device__ __forceinline__ void fill_nm24_table(uint8_t *table24, int tid, int nthreads)
{
    if constexpr (P == Pattern::NM24)
        for (int i = tid; i < 256; i += nthreads) table24[i] = nm24_table_entry((uint32_t)i);
}

// LDS bytes of one wave's staging area
template <int CMAX, int MT>
struct SkinnyLds {
    static constexpr int kStride = (8 * ((CMAX + 7) / 8) + 1) * 16;   // weight row stride (whole pairs)
    static constexpr int kXStride = (CMAX + 3) * 64;         // activation row stride (3 zero chunks)
    static constexpr int kW = 16 * kStride;
    static constexpr int kX = MT * kXStride;
    static constexpr int kZero = 64;                          // zero block for token rows >= M
    static constexpr int kBytes = kW + kX + kZero;
};

// KS waves per workgroup split K; each wave covers at most CMAX chunks; at
// most MT tokens (M <= MT <= 16).  One or more projections that share the
// activations (args), 16 weight rows per workgroup.
template <Pattern P, int KS, int CMAX, int MT>
__global__ __launch_bounds__(64 * KS) void skinny_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ x_scale, const int32_t *__restrict__ x_rowsum,
    FusedProjArgs args, int64_t M, int64_t K)
{
    static_assert(CMAX % 4 == 0 && MT >= 1 && MT <= 16, "config");
    using L = SkinnyLds<CMAX, MT>;
    constexpr int XLOADS = (MT * CMAX * 4 + 63) / 64;
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[KS][L::kBytes];
    __shared__ i32x4 s_part[KS > 1 ? KS - 1 : 1][64];
    __shared__ uint8_t s_nm24[P == Pattern::NM24 ? 256 : 1];

    // the wave index is wave-uniform: say so, so that branches on it are scalar
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int p = proj_of_block(args, (int)blockIdx.x);
    const int64_t N = args.N[p];
    const uint8_t *packed = args.packed[p];
    const float *w_scale = args.w_scale[p];
    const int64_t n0 = (int64_t)(blockIdx.x - args.block_start[p]) * 16;
    // token tile blockIdx.y: rows 16 y .. 16 y + 15 of the call's M (then
    // MT = 16); the tiles share nothing, and re-read the weights from L2
    const int64_t t0 = (int64_t)blockIdx.y * 16;
    Xq += t0 * K;
    x_scale += t0;
    x_rowsum += t0;
    float *Y = args.Y[p] + t0 * N;
    int32_t *acc_out = args.acc[p] ? args.acc[p] + t0 * N : nullptr;
    M = min(M - t0, (int64_t)MT);
    const int64_t C = K / 64;
    const int mt = (int)M;                           // 1 <= M <= MT
    // this wave's chunk range [c_lo, c_lo + cw), 1 <= cw <= CMAX (the host keeps KS <= C)
    const int64_t c_lo = C * wave / KS;
    const int cw = (int)(C * (wave + 1) / KS - c_lo);
    uint8_t *lw = s_stage[wave];
    uint8_t *lx = lw + L::kW;
    uint8_t *lz = lx + L::kX;

    // every kernel argument in SGPRs now: a scalar load left pending would make
    // the compiler wait for all outstanding memory operations at its first use
    asm volatile("" ::"s"(Xq), "s"(x_scale), "s"(x_rowsum), "s"(packed), "s"(w_scale), "s"(Y), "s"(acc_out));

    // 1a. activations first: waiting for them later leaves the weights in flight
    u32x4 x[XLOADS];
    int x_off[XLOADS];
    const int xw = cw * 4;                           // 16-byte pieces per token
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
    // epilogue operands
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

    // 1b. all weight loads of the wave, in pairs (see above)
    constexpr int PAIRS = (CMAX + 7) / 8;
    const int pairs = (cw + 7) / 8;
    const int lrow = lane >> 3, lcol = lane & 7;
    RawChunk<P> w[PAIRS][2];
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // unconditional (pairs past this wave's range re-read its last
            // chunk), so the compiler can count outstanding loads exactly
            const int col = 8 * j + lcol;
            const int64_t n = min(n0 + 8 * h + lrow, N - 1);
            w[j][h] = load_raw_chunk<P>(packed, N, K, n, c_lo + min(col, cw - 1));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (P == Pattern::NM24) {
        fill_nm24_table<P>(s_nm24, threadIdx.x, 64 * KS);
        __syncthreads();
    }
    // zero chunks after each activation row (12 pieces of 16 bytes), and the zero block
    for (int f = lane; f < mt * 12 + 4; f += 64) {
        const int off = (f < mt * 12) ? (f / 12) * L::kXStride + (cw * 4 + f % 12) * 16
                                      : L::kX + (f - mt * 12) * 16;
        *reinterpret_cast<u32x4 *>(lx + off) = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < XLOADS; ++i)
        if (x_off[i] >= 0) *reinterpret_cast<u32x4 *>(lx + x_off[i]) = x[i];

    // 2. per pair: stage in LDS, then its two steps of MFMAs (4 accumulators)
    const uint8_t *brow = lw + r * L::kStride + q * 16;
    const uint8_t *arow = (r < mt) ? lx + r * L::kXStride + q * 64 : lz;
    const int astep = (r < mt) ? 256 : 0;
    i32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = i32x4{0, 0, 0, 0};
    const int steps = (cw + 3) / 4;
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
        if (j < pairs) {                                     // wave-uniform
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<u32x4 *>(lw + (8 * h + lrow) * L::kStride + (8 * j + lcol) * 16) =
                    decode_chunk<P>(w[j][h], s_nm24);
            __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): staged
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int s = 2 * j + s2;
                if (s < steps) {
                    // chunks >= cw: the weight slot holds a repeated chunk but the
                    // activation slot is zero, so the product is zero
                    const u32x4 b = *reinterpret_cast<const u32x4 *>(brow + s * 64);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const i32x4 a = *reinterpret_cast<const i32x4 *>(arow + s * astep + 16 * t);
                        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, unpack_word(b[t]), acc[t], 0, 0, 0);
                    }
                }
            }
        }
    }
    i32x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);

    // 3. combine the KS partial sums
    if (KS > 1) {
        if (wave > 0) s_part[wave - 1][lane] = sum;
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w2 = 1; w2 < KS; ++w2) sum += s_part[w2 - 1][lane];
    }

    // 4. epilogue: offset-code correction, dequant scale
    const int64_t nn = n0 + r;
    if (nn >= N) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * q + v;
        if (m < mt) {
            const int av = sum[v] - rs[v];
            Y[(int64_t)m * N + nn] = (float)av * (beta * xsc[v]);
            if (acc_out) acc_out[(int64_t)m * N + nn] = av;
        }
    }
}

// args.block_start filled by the caller (16 weight rows per workgroup);
// `blocks` workgroups along x, the 16-token tiles along y
template <Pattern P, int KS, int CMAX, int MT>
hipError_t launch_skinny(const int8_t *Xq, const float *xs, const int32_t *rs, const FusedProjArgs &args,
                         int64_t blocks, int64_t M, int64_t K, hipStream_t stream)
{
    hipLaunchKernelGGL((skinny_kernel<P, KS, CMAX, MT>), dim3((unsigned)blocks, (unsigned)((M + 15) / 16)),
                       dim3(64 * KS), 0, stream, Xq, xs, rs, args, M, K);
    return hipGetLastError();
}

}  // namespace skinny
}  // namespace bl
