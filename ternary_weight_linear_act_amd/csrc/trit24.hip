// Forward on 2:4 weights in the trit-packed storage (written by
// launch_pack_trit24): per group of 4 inputs one 6-bit code 9 p + 3 a + b,
// p the index of the kept pair (i0, i1) in (0,1) (0,2) (0,3) (1,2) (1,3)
// (2,3), a and b the codes t + 1 of the ternary weights at i0 and i1; the 16
// codes of 64 inputs in a 96-bit little-endian string (group g at bit 6 g),
// 12 bytes, rows of K / 64 strings.  1.5 bits per weight, against 2 for the
// 2:4 values + masks and for the dense codes.
//
// "Sparse-BitNet ..." review, sec. 3.2: 2:4 keeps two of every four inputs;
// "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 5.1 and section
// "I2_S 커널의 내부 동작" of the bitnet.cpp page: the weights move packed and
// are unpacked on chip, and TL2 indexes a pair of ternary weights by its
// 3 x 3 = 9 combinations, as a and b do here.  The arithmetic after the
// unpack is the 2:4 forward's: the same acc, bit for bit, and the same Y.
//
// One token (K <= 16384): trit24_decode_kernel, the one-token dot4 kernel's
// layout (LPR lanes per weight row, U strings per lane, every load issued up
// front, int8 activations in LDS) with a 64-entry table in LDS that maps a
// code to its four weights as signed bytes (codes 54-63, which the packer
// never writes, to zeros), so a group costs a field extract, a table read and
// one v_dot4 against the activation word of the group; no row sum is needed.
// More tokens: the strings are expanded to the dense 2-bit codes in the
// caller's workspace, then the dense forward runs on them.
#include <stdio.h>

#include "kernels.hpp"

namespace bl {
namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef int i32x4v __attribute__((ext_vector_type(4)));

constexpr int kDecodeMaxK = 16384;
constexpr int kWaves = 4, kThreads = 64 * kWaves;

// Kept pair p = c / 9 of code c: 8 * i0 and 8 * i1, one nibble per pair (in
// units of 8 bits), and the codes a, b = t + 1 of its two weights.
struct TritGroup {
    uint32_t lo, hi, a, b;
};

__device__ __forceinline__ TritGroup trit_group(uint32_t c)
{
    const uint32_t p = c / 9u, v = c - 9u * p, a = v / 3u;
    return TritGroup{(0x211000u >> (4u * p)) & 0xFu, (0x332321u >> (4u * p)) & 0xFu, a, v - 3u * a};
}

// The four weights of code c as signed bytes t (0 at the pruned inputs); codes
// past 53, which the packer never writes, give zeros.
__device__ __forceinline__ uint32_t trit_signed_bytes(uint32_t c)
{
    if (c > 53u) return 0u;
    const TritGroup g = trit_group(c);
    return (((g.a - 1u) & 0xFFu) << (8u * g.lo)) | (((g.b - 1u) & 0xFFu) << (8u * g.hi));
}

// The same as the dense codes t + 1, one per byte (1 at the pruned inputs):
// the two kept bytes of 0x01010101 are cleared (no borrow: each is 1), then
// set to a and b.
__device__ __forceinline__ uint32_t trit_code_bytes(uint32_t c)
{
    if (c > 53u) return 0x01010101u;
    const TritGroup g = trit_group(c);
    return 0x01010101u - (1u << (8u * g.lo)) - (1u << (8u * g.hi)) + (g.a << (8u * g.lo)) + (g.b << (8u * g.hi));
}

// Code of group g (0..15) of the 96-bit string w[0..2].
template <int G>
__device__ __forceinline__ uint32_t trit_code(const uint32_t *w)
{
    constexpr int bit = 6 * G, wi = bit >> 5, o = bit & 31;
    if constexpr (o <= 26) return (w[wi] >> o) & 63u;
    else return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], o) & 63u;
}

// One thread per string: 12 bytes in, the 16 bytes of dense codes out (code
// of input k at bit code_bit(k % 16) of word k / 16 of the 64-input chunk).
__global__ __launch_bounds__(256) void trit24_expand_kernel(const uint32_t *__restrict__ packed, int64_t strings,
                                                            u32x4v *__restrict__ dense)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= strings) return;
    const uint32_t w[3] = {packed[3 * i], packed[3 * i + 1], packed[3 * i + 2]};
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#define TRIT_GROUP(G) d[(G) >> 2] |= trit_code_bytes(trit_code<G>(w)) << (2 * ((G) & 3));
    TRIT_GROUP(0) TRIT_GROUP(1) TRIT_GROUP(2) TRIT_GROUP(3) TRIT_GROUP(4) TRIT_GROUP(5) TRIT_GROUP(6)
    TRIT_GROUP(7) TRIT_GROUP(8) TRIT_GROUP(9) TRIT_GROUP(10) TRIT_GROUP(11) TRIT_GROUP(12) TRIT_GROUP(13)
    TRIT_GROUP(14) TRIT_GROUP(15)
#undef TRIT_GROUP
    dense[i] = u32x4v{d[0], d[1], d[2], d[3]};
}

// Sum over each aligned group of LPR lanes (8 to 64), the total in every lane
// of the group: quad exchanges, then mirrors within 8 and 16 lanes, then
// swaps across rows of 16.
template <int LPR>
__device__ __forceinline__ int row_lanes_sum(int v)
{
    v += dpp_move<kDppQuadXor1>(v);
    v += dpp_move<kDppQuadXor2>(v);
    v += dpp_move<kDppRowHalfMirror>(v);
    if (LPR >= 16) v += dpp_move<kDppRowMirror>(v);
    if (LPR >= 32) v += __shfl_xor(v, 16, 64);
    if (LPR >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// One token.  LPR lanes share a weight row; lane j takes strings j, j + LPR,
// ... (U of them; the host guarantees K <= 64 U LPR), so a load instruction
// reads LPR * 12 contiguous bytes of each row.  A workgroup is 4 waves,
// 256 / LPR rows.  Strings past the row read as all-ones words, whose codes
// (63) contribute nothing.
template <int LPR, int U>
__global__ __launch_bounds__(kThreads) void trit24_decode_kernel(const int8_t *__restrict__ Xq,
                                                                 const float *__restrict__ x_scale,
                                                                 const uint8_t *__restrict__ packed,
                                                                 const float *__restrict__ w_scale, int64_t N,
                                                                 int64_t K, float *__restrict__ Y,
                                                                 int32_t *__restrict__ acc_out)
{
    constexpr int RPW = 64 / LPR, RB = kWaves * RPW;
    extern __shared__ __attribute__((aligned(16))) uint8_t s_x[];      // K int8 activations
    __shared__ uint32_t s_lut[64];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t row = (int64_t)blockIdx.x * RB + wave * RPW + lane / LPR;
    const int j = lane % LPR;
    const int C = (int)(K / 64);                // <= 256 strings (K <= 16384)
    asm volatile("" ::"s"(Xq), "s"(x_scale), "s"(packed), "s"(w_scale), "s"(Y), "s"(acc_out));
    const float wsc = w_scale[0];
    const float xsc = x_scale[0];
    __builtin_amdgcn_sched_barrier(0);

    // activations: 16-byte loads, enough for K = 64 U LPR (indices past the
    // row re-read element 0 and are never stored)
    constexpr int XR = (4 * U * LPR + kThreads - 1) / kThreads;
    const int n16 = C * 4;
    u32x4v xb[XR];
#pragma unroll
    for (int t = 0; t < XR; ++t) {
        const int i = tid + t * kThreads;
        xb[t] = reinterpret_cast<const u32x4v *>(Xq)[i < n16 ? i : 0];
    }
    __builtin_amdgcn_sched_barrier(0);

    // the lane's strings (rows past N re-read row N - 1 and strings past the
    // row re-read string C - 1; neither is used); 32-bit offsets within the
    // row (64-bit ones made the compiler tie the loads to the scale loads)
    uint32_t w[U][3];
    const uint32_t *rp = reinterpret_cast<const uint32_t *>(packed + min(row, N - 1) * (int64_t)(3 * C * 4));
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = min(j + u * LPR, C - 1);
#pragma unroll
        for (int i = 0; i < 3; ++i) w[u][i] = __builtin_nontemporal_load(rp + (3 * c + i));
    }
    __builtin_amdgcn_sched_barrier(0);

    if (tid < 64) s_lut[tid] = trit_signed_bytes((uint32_t)tid);
#pragma unroll
    for (int t = 0; t < XR; ++t) {
        const int i = tid + t * kThreads;
        if (i < n16) reinterpret_cast<u32x4v *>(s_x)[i] = xb[t];
    }
    __syncthreads();

    // dot products, branch-free: group g of a string against activation word
    // g of its 64-byte chunk
    int a[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = j + u * LPR;
        const bool in = c < C;
        const i32x4v *xp = reinterpret_cast<const i32x4v *>(s_x + (in ? c : C - 1) * 64);
        const uint32_t ws[3] = {in ? w[u][0] : ~0u, in ? w[u][1] : ~0u, in ? w[u][2] : ~0u};
        uint32_t codes[16];
        codes[0] = trit_code<0>(ws);   codes[1] = trit_code<1>(ws);   codes[2] = trit_code<2>(ws);
        codes[3] = trit_code<3>(ws);   codes[4] = trit_code<4>(ws);   codes[5] = trit_code<5>(ws);
        codes[6] = trit_code<6>(ws);   codes[7] = trit_code<7>(ws);   codes[8] = trit_code<8>(ws);
        codes[9] = trit_code<9>(ws);   codes[10] = trit_code<10>(ws); codes[11] = trit_code<11>(ws);
        codes[12] = trit_code<12>(ws); codes[13] = trit_code<13>(ws); codes[14] = trit_code<14>(ws);
        codes[15] = trit_code<15>(ws);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const i32x4v xx = xp[q];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                a[e] = __builtin_amdgcn_sdot4((int)s_lut[codes[4 * q + e]], xx[e], a[e], false);
        }
    }
    int acc = (a[0] + a[1]) + (a[2] + a[3]);
    acc = row_lanes_sum<LPR>(acc);
    if (j == 0 && row < N) {
        Y[row] = (float)acc * (wsc * xsc);
        if (acc_out) acc_out[row] = acc;
    }
}

using DecodeFn = void (*)(dim3, size_t, hipStream_t, const int8_t *, const float *, const uint8_t *, const float *,
                          int64_t, int64_t, float *, int32_t *);

template <int LPR, int U>
void launch_decode(dim3 grid, size_t lds, hipStream_t stream, const int8_t *Xq, const float *xs,
                   const uint8_t *packed, const float *w_scale, int64_t N, int64_t K, float *Y, int32_t *acc)
{
    hipLaunchKernelGGL((trit24_decode_kernel<LPR, U>), grid, dim3(kThreads), lds, stream, Xq, xs, packed, w_scale, N,
                       K, Y, acc);
}

// The (lanes per row, strings per lane) pairs of the host rule: the fewest
// lanes of 8, 16, 32, 64 that keep U <= 5.
DecodeFn pick_decode(int lpr, int u)
{
    switch (lpr * 16 + u) {
    case 8 * 16 + 1: return launch_decode<8, 1>;
    case 8 * 16 + 2: return launch_decode<8, 2>;
    case 8 * 16 + 3: return launch_decode<8, 3>;
    case 8 * 16 + 4: return launch_decode<8, 4>;
    case 8 * 16 + 5: return launch_decode<8, 5>;
    case 16 * 16 + 3: return launch_decode<16, 3>;
    case 16 * 16 + 4: return launch_decode<16, 4>;
    case 16 * 16 + 5: return launch_decode<16, 5>;
    case 32 * 16 + 3: return launch_decode<32, 3>;
    case 32 * 16 + 4: return launch_decode<32, 4>;
    case 32 * 16 + 5: return launch_decode<32, 5>;
    case 64 * 16 + 3: return launch_decode<64, 3>;
    case 64 * 16 + 4: return launch_decode<64, 4>;
    default: return nullptr;
    }
}

thread_local char g_name[160];

}  // namespace

hipError_t launch_forward_trit24(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                                 const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                                 Scratch &scratch, hipStream_t stream, const char **name)
{
    const int64_t C = K / 64;
    if (M == 1 && K <= kDecodeMaxK) {
        int lpr = 8;
        while (lpr < 64 && (C + lpr - 1) / lpr > 5) lpr *= 2;
        const int u = (int)((C + lpr - 1) / lpr);
        const DecodeFn f = pick_decode(lpr, u);
        const int64_t rb = kWaves * (64 / lpr);
        const int64_t blocks = (N + rb - 1) / rb;
        if (!f || blocks > (1LL << 30)) return hipErrorNotSupported;
        snprintf(g_name, sizeof g_name, "trit24_decode_lpr%d_u%d", lpr, u);
        *name = g_name;
        if (scratch.query) return hipSuccess;
        f(dim3((unsigned)blocks), (size_t)K, stream, Xq, xs, packed, w_scale, N, K, Y, acc);
        return hipGetLastError();
    }
    // the expanded rows first, then (256-byte aligned) whatever the dense
    // forward on them needs
    const size_t rows_bytes = ((size_t)N * (size_t)(K / 4) + 255) / 256 * 256;
    Scratch dense_need;
    dense_need.query = true;
    const char *dn = "";
    (void)launch_forward(Xq, xs, rs, nullptr, w_scale, Pattern::Dense, M, N, K, Y, acc, dense_need, stream, &dn);
    const bool go = scratch.take(rows_bytes + dense_need.need);
    if (!go && !scratch.query) return hipErrorOutOfMemory;
    Scratch dense_scratch;
    dense_scratch.query = scratch.query;
    if (go) {
        const int64_t strings = N * C;
        hipLaunchKernelGGL(trit24_expand_kernel, dim3((unsigned)((strings + 255) / 256)), dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t *>(packed), strings, reinterpret_cast<u32x4v *>(scratch.ptr));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        dense_scratch.ptr = scratch.ptr + rows_bytes;
        dense_scratch.bytes = scratch.bytes - rows_bytes;
    }
    const hipError_t e = launch_forward(Xq, xs, rs, scratch.ptr, w_scale, Pattern::Dense, M, N, K, Y, acc,
                                        dense_scratch, stream, &dn);
    snprintf(g_name, sizeof g_name, "trit24_expand+%s", dn);
    *name = g_name;
    return e;
}

}  // namespace bl
