// Prefill GEMM for 2:4 weights on gfx950's sparse matrix cores
// (v_smfmac_i32_32x32x64_i8): Y[m, n] = (sum_k Xq[m, k] * W_eff[n, k]) *
// beta * x_scale[m].
//
// "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to Semi-Structured
// Sparsity" (review), sec. 4 and 5.3: the speedups come from hardware that
// skips the pruned half of a 2:4 weight block.  The sparse MFMA takes a
// 2:4-sparse operand as its kept values plus a 2-bit position per value, and
// issues a 32 x 32 x 64 product in about the time of a dense 32 x 32 x 32 one
// (measured here at 1.8 times the dense int8 rate).  The 2:4 groups run along
// K, so the weights are the sparse operand (A: 32 weight rows) and the
// activations the dense one (B: 32 tokens); the output fragment is
// transposed (weight rows x tokens).
//
// Operand layouts of v_smfmac_i32_32x32x64_i8 (determined on the device with
// random operands), lane l, h = l / 32:
//   A (sparse, 16 bytes): row l % 32, the kept values of k in [32h, 32h + 32)
//     in increasing k -- eight groups of four, two values each; index VGPR:
//     2 bits per value, its position in its group;
//   B (dense, 32 bytes): column l % 32, bytes 0-15 = k in [16h, 16h + 16),
//     bytes 16-31 = k in [32 + 16h, 48 + 16h);
//   D: column l % 32, rows 8 (v / 4) + 4h + (v % 4), as the dense 32x32 MFMA.
// The packed 2:4 format (include/bitlinear.h) holds, per row and 64 inputs,
// two 32-bit words of kept codes (the 16 of k < 32, then the 16 of k >= 32)
// and two mask words (eight 4-bit group masks each), so a lane's A fragment
// is one value word and one mask word:
//   codes c = t + 1 -> t bytes by one byte permute per four codes
//     ((w >> 2s) & 0x03030303 holds codes 4s .. 4s + 3);
//   mask nibble (two bits set) -> position nibble i0 | i1 << 2 by a byte
//     permute: the six valid masks differ in their low three bits, which index
//     an 8-entry table.
// The values are t in {-1, 0, +1}: no offset-code row sum is subtracted.
//
// Tiling: a workgroup owns BM tokens x 256 weight rows (BM = 256 or 128),
// eight waves (two per SIMD).  K runs in 128-wide slices through an LDS ring
// of S stages filled by direct loads: per slice BM x 128 bytes of activations
// (128-byte rows, 16-byte pieces XOR-swizzled by row) and 8 KB of packed
// weights (values, masks: 16 bytes per row each).  Per slice and wave: 2
// k-steps of sparse MFMAs; the first group has the second k-step's activation
// reads and weight expansions issued between its MFMAs, the second the next
// slice's reads.  K % 128 == 0 (other K take the t-byte GEMM).
//
// The kernel is VALU-bound: per slice a SIMD issues 1024 cycles of sparse
// MFMA but, with 64-token wave tiles, about 1400 cycles of VALU, most of it
// the expansion of each weight fragment in every wave that shares it
// (variants built from a copy of the sources: without the expansion -4.5 us,
// without the MFMAs at all -10 us, on 2048 x 6912 x 2560).  A fragment's
// expansion is reused once per 32 tokens of the wave tile, so the waves take
// tall tiles: 128 tokens x 64 rows (BM = 256, 2 x 4 waves, S = 3) or 128 x 32
// (BM = 128, 1 x 8 waves, S = 4).  Measured against 64 x 128 wave tiles:
// 2048 x 6912 x 2560 43.2 -> 40.0 us, 4096 x 8192 x 4096 119 -> 109 us
// (dense: 43.5 and 133 us); BM = 128 for tile counts that leave the chip
// half empty at BM = 256, e.g. 1000 x 8000 x 2560 59.5 -> 33.8 us (dense
// 28.4) and 2048 x 2560 x 6912 79 -> 46 us (dense 50.8).
#include "dma.hpp"
#include "kernels.hpp"

namespace bl {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSBK = 128;                 // K per slice
constexpr int kBN = 256;                  // weight rows per workgroup
constexpr int kSV = kBN * 16;             // value bytes per stage (masks the same)

// code c -> t byte (c = 0, 1, 2 -> 0xFF, 0x00, 0x01)
constexpr uint32_t kCodeToT = 0x000100FFu;
// mask nibble & 7 -> position nibble i0 | i1 << 2:
// 1 (1001) -> 12, 2 (1010) -> 13, 3 (0011) -> 4, 4 (1100) -> 14, 5 (0101) -> 8, 6 (0110) -> 9
constexpr uint32_t kIdxLo = 0x040D0C00u, kIdxHi = 0x0009080Eu;

__device__ __forceinline__ void expand24(uint32_t vw, uint32_t mw, i32x4 &a, int &ix)
{
    a[0] = (int)__builtin_amdgcn_perm(0u, kCodeToT, vw & 0x03030303u);
    a[1] = (int)__builtin_amdgcn_perm(0u, kCodeToT, (vw >> 2) & 0x03030303u);
    a[2] = (int)__builtin_amdgcn_perm(0u, kCodeToT, (vw >> 4) & 0x03030303u);
    a[3] = (int)__builtin_amdgcn_perm(0u, kCodeToT, (vw >> 6) & 0x03030303u);
    const uint32_t lo = __builtin_amdgcn_perm(kIdxHi, kIdxLo, mw & 0x07070707u);
    const uint32_t hi = __builtin_amdgcn_perm(kIdxHi, kIdxLo, (mw >> 4) & 0x07070707u);
    ix = (int)(lo | (hi << 4));
}

// BM tokens x 256 weight rows per workgroup; WM x WN waves (tokens x weight
// rows), each owning (BM / WM) x (256 / WN).
template <int BM, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_nm24_sparse_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ x_scale, const uint8_t *__restrict__ packed,
    const float *__restrict__ w_scale, int64_t M, int64_t N, int64_t K, float *__restrict__ Y,
    int32_t *__restrict__ acc_out)
{
    static_assert(S >= 3, "the pipeline needs S >= 3");
    constexpr int kBM = BM;
    constexpr int kSA = kBM * kSBK;                   // activation bytes per stage
    constexpr int kStage = kSA + 2 * kSV;
    constexpr int NW = WM * WN, T = 64 * NW;
    constexpr int kTM = kBM / WM, kTN = kBN / WN;
    constexpr int kFM = kTM / 32, kFN = kTN / 32;
    constexpr int A_PER_W = kSA / 1024 / NW;         // activation loads per wave and slice
    constexpr int W_PER_W = 8 / NW;                   // weight loads (4 KB values + 4 KB masks)
    static_assert(kSA / 1024 % NW == 0 && 8 % NW == 0, "loads must split evenly over the waves");
    constexpr int kLoadsPerSlice = A_PER_W + W_PER_W;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    float *s_sc = reinterpret_cast<float *>(smem + S * kStage);

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int h = lane >> 5, li = lane & 31;

    const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
    int64_t mt, nt;
    if (!xcd_tile(blockIdx.x, tiles_m, tiles_n, &mt, &nt)) return;
    const int64_t m0 = mt * kBM, n0 = nt * kBN;
    const float beta = w_scale[0];
    for (int i = tid; i < kBM; i += T) s_sc[i] = beta * x_scale[min(m0 + i, M - 1)];

    const int64_t slices = K / kSBK;
    const int64_t vrow = K / 8;                       // value (and mask) bytes per weight row
    // per-lane sources: activation instruction jj covers rows 8 jj .. + 7,
    // lane = row (lane / 8), slot lane % 8, which holds logical piece
    // slot ^ (row & 7); weight instruction q: 64 rows of the values (q < 4) or
    // the masks (q >= 4), one row per lane
    const int8_t *a_src[A_PER_W];
#pragma unroll
    for (int j = 0; j < A_PER_W; ++j) {
        const int row = (wave * A_PER_W + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (row & 7);
        a_src[j] = Xq + min(m0 + row, M - 1) * K + 16 * c;
    }
    const uint8_t *w_src[W_PER_W];
#pragma unroll
    for (int j = 0; j < W_PER_W; ++j) {
        const int q = wave * W_PER_W + j;
        const int64_t wr = min(n0 + 64 * (q % 4) + lane, N - 1);
        w_src[j] = packed + (q / 4) * N * vrow + wr * vrow;
    }

    auto issue = [&](int64_t sl) {
        uint8_t *st = smem + (sl % S) * kStage;
        const int64_t k0 = sl * kSBK;
#pragma unroll
        for (int j = 0; j < A_PER_W; ++j) dma16(a_src[j] + k0, st + (wave * A_PER_W + j) * 1024);
#pragma unroll
        for (int j = 0; j < W_PER_W; ++j) dma16(w_src[j] + k0 / 8, st + kSA + (wave * W_PER_W + j) * 1024);
    };

    // operands of k-step s (0, 1) of a slice
    auto read_tok = [&](int64_t sl, int s, i32x8 (&dst)[kFM]) {
        const uint8_t *st = smem + (sl % S) * kStage;
#pragma unroll
        for (int fm = 0; fm < kFM; ++fm) {
            const int r = wm * kTM + fm * 32 + li;
            const i32x4 lo = *reinterpret_cast<const i32x4 *>(st + r * kSBK + 16 * ((4 * s + h) ^ (r & 7)));
            const i32x4 hi = *reinterpret_cast<const i32x4 *>(st + r * kSBK + 16 * ((4 * s + 2 + h) ^ (r & 7)));
            dst[fm] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    // a weight fragment's words for both k-steps of a slice: the row's 16
    // value bytes and 16 mask bytes (consecutive rows, so the 16-byte reads
    // are free of bank conflicts), of which lane half h takes words h, 2 + h
    auto read_w = [&](int64_t sl, uint32_t (&vw)[kFN][2], uint32_t (&mw)[kFN][2]) {
        const uint8_t *st = smem + (sl % S) * kStage;
#pragma unroll
        for (int fn = 0; fn < kFN; ++fn) {
            const int r = wn * kTN + fn * 32 + li;
            const i32x4 v4 = *reinterpret_cast<const i32x4 *>(st + kSA + r * 16);
            const i32x4 m4 = *reinterpret_cast<const i32x4 *>(st + kSA + kSV + r * 16);
            vw[fn][0] = (uint32_t)(h ? v4[1] : v4[0]);
            vw[fn][1] = (uint32_t)(h ? v4[3] : v4[2]);
            mw[fn][0] = (uint32_t)(h ? m4[1] : m4[0]);
            mw[fn][1] = (uint32_t)(h ? m4[3] : m4[2]);
        }
    };

    i32x16 acc[kFM][kFN];
#pragma unroll
    for (int x = 0; x < kFM; ++x)
#pragma unroll
        for (int y = 0; y < kFN; ++y)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[x][y][v] = 0;
    auto mfma_grp = [&](const i32x8 (&tk)[kFM], const i32x4 (&wa)[kFN], const int (&wi)[kFN]) {
#pragma unroll
        for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
            for (int fm = 0; fm < kFM; ++fm)
                acc[fm][fn] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(wa[fn], tk[fm], acc[fm][fn], wi[fn], 0, 0);
    };
    // one MFMA, then one LDS read while reads remain, then NV VALU operations
    auto interleave = [](auto nrc, auto nvc) {
        constexpr int NR = decltype(nrc)::value, NV = decltype(nvc)::value;
#pragma unroll
        for (int i = 0; i < kFM * kFN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
        }
    };
    // group 0 reads the k-step-1 activations and expands the k-step-1
    // weights (already in registers) between its MFMAs; group 1 reads the
    // next slice's operands
    using G0 = std::integral_constant<int, 2 * kFM>;
    using G0V = std::integral_constant<int, (18 * kFN + kFM * kFN - 1) / (kFM * kFN)>;
    using G1 = std::integral_constant<int, 2 * kFM + 2 * kFN>;
    using G1V = std::integral_constant<int, 0>;

    // prologue: S-1 slices in flight, slice 0 resident, k-step 0 operands ready
#pragma unroll
    for (int sl = 0; sl < S - 1; ++sl)
        if (sl < slices) issue(sl);
    if (S - 2 < slices) wait_vm<kLoadsPerSlice * (S - 2)>();
    else wait_vm<0>();
    block_barrier();
    i32x8 tk0[kFM], tk1[kFM];
    i32x4 wa0[kFN], wa1[kFN];
    int wi0[kFN], wi1[kFN];
    uint32_t vw[kFN][2], mw[kFN][2];
    read_tok(0, 0, tk0);
    read_w(0, vw, mw);
#pragma unroll
    for (int fn = 0; fn < kFN; ++fn) expand24(vw[fn][0], mw[fn][0], wa0[fn], wi0[fn]);
    asm volatile("" ::"s"(Y), "s"(acc_out));

    auto slice = [&](int64_t it, bool steady) {
        __builtin_amdgcn_sched_barrier(0);
        mfma_grp(tk0, wa0, wi0);
        read_tok(it, 1, tk1);
#pragma unroll
        for (int fn = 0; fn < kFN; ++fn) expand24(vw[fn][1], mw[fn][1], wa1[fn], wi1[fn]);
        interleave(G0(), G0V());
        __builtin_amdgcn_sched_barrier(0);
        const bool more = steady || it + 1 < slices;
        if (steady) {
            wait_vm<kLoadsPerSlice * (S - 3)>();      // slice it+1 landed (this wave's loads)
            block_barrier();                          // ... and every wave's
            issue(it + S - 1);                        // into the stage of slice it-1
        } else if (more) {
            if (it + S - 2 < slices) wait_vm<kLoadsPerSlice * (S - 3)>();
            else wait_vm<0>();
            block_barrier();
            if (it + S - 1 < slices) issue(it + S - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_grp(tk1, wa1, wi1);
        if (more) {
            read_w(it + 1, vw, mw);
            read_tok(it + 1, 0, tk0);
        }
        interleave(G1(), G1V());
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
#pragma unroll
            for (int fn = 0; fn < kFN; ++fn) expand24(vw[fn][0], mw[fn][0], wa0[fn], wi0[fn]);
        }
    };
    int64_t it = 0;
    for (; it + S <= slices; ++it) slice(it, true);
    for (; it < slices; ++it) slice(it, false);

    // epilogue: fragment (fm, fn) holds tokens m = .. + li and weight rows
    // n = .. + 8 (v / 4) + 4h + v % 4 -- four consecutive n per v / 4
    const bool vec = (m0 + kBM <= M) && (n0 + kBN <= N) && (N % 4 == 0) && !acc_out;
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm) {
        const int lm = wm * kTM + fm * 32 + li;
        const int64_t m = m0 + lm;
        const float sc = s_sc[lm];
#pragma unroll
        for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wn * kTN + fn * 32 + 8 * q + 4 * h;
                f32x4 y;
#pragma unroll
                for (int r = 0; r < 4; ++r) y[r] = (float)acc[fm][fn][4 * q + r] * sc;
                if (vec) {
                    *reinterpret_cast<f32x4 *>(Y + m * N + n) = y;
                } else if (m < M) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) {
                            Y[m * N + n + r] = y[r];
                            if (acc_out) acc_out[m * N + n + r] = acc[fm][fn][4 * q + r];
                        }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// 2:4 weights at 1-16 tokens on the sparse matrix cores
// (v_smfmac_i32_16x16x128_i8).  The weights are the sparse A operand (16
// rows per workgroup), the tokens the dense B operand (16 columns, zero past
// M): lane l holds weight row l % 16 and, as B, token l % 16; q = l / 16.
//   A: the kept values of k in [32q, 32q + 32) of a 128-wide step -- one
//      value word and one mask word of the packed row (expand24);
//   B: bytes 0-15 = k in [16q, 16q + 16), bytes 16-31 = k in [64 + 16q,
//      80 + 16q) of the step, read straight from Xq (L2-resident);
//   D: token l % 16, weight rows 4q .. 4q + 3.
// The workgroup's KS waves take consecutive runs of at most U steps of K;
// every load of a wave is issued before its first MFMA; wave 0 adds the
// other waves' partial sums (LDS) and applies beta * x_scale.  The values
// are t in {-1, 0, +1}: no row sum is subtracted.  K % 128 == 0.
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(1024) void skinny_nm24_smfmac_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ x_scale, const uint8_t *__restrict__ packed,
    const float *__restrict__ w_scale, int64_t M, int64_t N, int64_t K, float *__restrict__ Y,
    int32_t *__restrict__ acc_out)
{
    __shared__ i32x4 s_part[16][64];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = blockDim.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t T = K / 128;
    const int64_t s0 = T * wave / KS;
    const int cnt = (int)(T * (wave + 1) / KS - s0);            // 1 .. U steps, wave-uniform
    const int64_t n = min(n0 + r, N - 1);
    const uint32_t *vrow = reinterpret_cast<const uint32_t *>(packed) + n * (K / 32);
    const uint32_t *mrow = reinterpret_cast<const uint32_t *>(packed + N * (K / 8)) + n * (K / 32);
    const bool tok = r < M;
    const int8_t *xrow = Xq + (tok ? r : 0) * K;

    // every load first: steps past this wave's run re-read its last step and
    // contribute zero activations
    uint32_t vw[U], mw[U];
    i32x4 blo[U], bhi[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t st = s0 + min(u, cnt - 1);
        vw[u] = vrow[4 * st + q];
        mw[u] = mrow[4 * st + q];
        blo[u] = *reinterpret_cast<const i32x4 *>(xrow + 128 * st + 16 * q);
        bhi[u] = *reinterpret_cast<const i32x4 *>(xrow + 128 * st + 64 + 16 * q);
    }
    __builtin_amdgcn_sched_barrier(0);
    i32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool live = tok && u < cnt;
        i32x8 b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[j] = live ? blo[u][j] : 0;
            b[4 + j] = live ? bhi[u][j] : 0;
        }
        i32x4 a;
        int ix;
        expand24(vw[u], mw[u], a, ix);
        acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, acc, ix, 0, 0);
    }
    if (KS > 1) {
        if (wave > 0) s_part[wave][lane] = acc;
        __syncthreads();
        if (wave != 0) return;
        for (int w = 1; w < KS; ++w) acc += s_part[w][lane];
    }
    if (!tok) return;
    const float sc = w_scale[0] * x_scale[r];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t nn = n0 + 4 * q + v;
        if (nn < N) {
            Y[(int64_t)r * N + nn] = (float)acc[v] * sc;
            if (acc_out) acc_out[(int64_t)r * N + nn] = acc[v];
        }
    }
}

template <int U>
hipError_t launch_skinny_sparse(const int8_t *Xq, const float *xs, const uint8_t *packed, const float *w_scale,
                                int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream,
                                bool query)
{
    const int64_t T = K / 128;
    const int64_t KS = (T + U - 1) / U;
    if (KS > 16) return hipErrorNotSupported;
    if (query) return hipSuccess;
    hipLaunchKernelGGL(skinny_nm24_smfmac_kernel<U>, dim3((unsigned)((N + 15) / 16)), dim3((unsigned)(64 * KS)), 0,
                       stream, Xq, xs, packed, w_scale, M, N, K, Y, acc);
    return hipGetLastError();
}

template <int BM, int WM, int WN, int S>
hipError_t launch_sparse(const int8_t *Xq, const float *xs, const uint8_t *packed, const float *w_scale, int64_t M,
                         int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream)
{
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + kBN - 1) / kBN;
    const int64_t grid = xcd_grid(tiles_m, tiles_n);
    const size_t lds = (size_t)S * (BM * kSBK + 2 * kSV) + 4 * BM;
    auto kern = gemm_nm24_sparse_kernel<BM, WM, WN, S>;
    const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), lds, stream, Xq, xs, packed, w_scale, M, N, K,
                       Y, acc);
    return hipGetLastError();
}

}  // namespace

// 2:4 weights at 1 <= M <= 16 tokens, K % 128 == 0 and K <= 16384;
// hipErrorNotSupported otherwise.  At most 4 steps of 128 per wave up to
// K = 8192 (16 waves), 8 beyond (measured: 4 is as fast or faster).  With
// `query` set, launches nothing and returns hipSuccess where it would launch.
hipError_t launch_skinny_nm24_smfmac(const int8_t *Xq, const float *xs, const uint8_t *packed, const float *w_scale,
                                     int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream,
                                     bool query)
{
    if (K % 128 != 0 || M < 1 || M > 16 || K > 16384) return hipErrorNotSupported;
    if (K <= 8192) return launch_skinny_sparse<4>(Xq, xs, packed, w_scale, M, N, K, Y, acc, stream, query);
    return launch_skinny_sparse<8>(Xq, xs, packed, w_scale, M, N, K, Y, acc, stream, query);
}

// 2:4 weights, K % 128 == 0; hipErrorNotSupported otherwise.  tile_m: 256
// or 128 tokens per workgroup.
hipError_t launch_gemm_nm24_sparse(const int8_t *Xq, const float *xs, const uint8_t *packed, const float *w_scale,
                                   int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream,
                                   int tile_m)
{
    if (K % kSBK != 0 || M < 1) return hipErrorNotSupported;
    if (tile_m == 128) return launch_sparse<128, 1, 8, 4>(Xq, xs, packed, w_scale, M, N, K, Y, acc, stream);
    return launch_sparse<256, 2, 4, 3>(Xq, xs, packed, w_scale, M, N, K, Y, acc, stream);
}

}  // namespace bl
