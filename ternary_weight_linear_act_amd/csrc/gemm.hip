// Prefill GEMM on int8 MFMA: Y[m, n] = (sum_k Xq[m, k] * W_eff[n, k]) * beta * x_scale[m].
//
// "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 5.1: the GPU kernel
// brings the packed weights (four ternary per byte) from HBM into on-chip
// shared memory, unpacks them there and computes against 8-bit activations.
// With many tokens the contraction is dense, so on gfx950 it runs on
// v_mfma_i32_32x32x32_i8.
//
// Tiling: a workgroup owns a BM x BN output tile and walks K in 64-wide
// slices.  The activation tile (BM x 64 int8) and the *packed* weight tile
// (BN x 16 bytes) are staged in LDS, double-buffered: the global loads of
// slice i+1 are issued before the MFMAs of slice i and written to the other
// buffer afterwards, so there is one barrier per slice.  Each wave unpacks its
// weight fragments in registers right before the MFMA ((word >> 2s) &
// 0x03030303 gives four codes per 32-bit lane value, already in the byte order
// the B operand wants) -- LDS holds 2 bits per weight, not 8.  Codes are
// c = t + 1, so the int32 accumulators hold sum c*q and the fused epilogue
// subtracts the activation row sum before the dequant scale.
//
// LDS layouts are padded so MFMA-side reads are conflict-free: activation
// rows 80 bytes apart (16 consecutive rows start in 16 distinct 4-bank
// groups), packed weight rows 24 bytes apart (32 consecutive rows read 8-byte
// pairs from 32 distinct bank pairs).
//
// MFMA operand mapping (same for A and B, so any k permutation is harmless):
// lane l, half h = l / 32, k-step s in {0, 1} of a 64-wide slice holds the
// 16 consecutive k = 32 h + 16 s + (0..15); A row / B column = l % 32.
// Output: lane l holds column l % 32 and rows 8 (v / 4) + 4 h + (v % 4).
//
// Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs, so
// consecutive logical tiles (which share a weight column tile) are mapped to
// workgroups on the same XCD and reuse its L2; the pipelined dense kernel
// instead gives each XCD one block of a 4 x 2 partition of the tile grid when
// the grid allows it.
#include <algorithm>
#include <string_view>
#include <type_traits>

#include "dma.hpp"
#include "kernels.hpp"
#include "skinny_impl.hpp"

namespace bl {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;
constexpr int LDA = BK + 16;      // bytes per staged activation row
constexpr int LDB = 24;           // bytes per staged packed weight row (16 used)
constexpr int kCus = 256;                  // MI355X compute units
constexpr int64_t kTBytesMaxK = 1 << 18;   // N:M t-byte GEMM: 64 * 127 * K < 2^31

// Raw packed words of weight row n for the K slice starting at k0: dense = 4
// code words; N:M = the superblock's value words then its 2 mask words.
template <Pattern P>
struct RawSlice {
    static constexpr int kWords = (P == Pattern::Dense) ? 4 : (P == Pattern::NM24 ? 2 : 3) + 2;
    uint32_t w[kWords];
};

template <Pattern P>
__device__ __forceinline__ void load_raw(const uint8_t *__restrict__ packed, int64_t N, int64_t K, int64_t n,
                                         int64_t k0, RawSlice<P> &r)
{
    if (P == Pattern::Dense) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(packed + n * (K / 4) + k0 / 4);
        r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
    } else {
        constexpr int GM = (P == Pattern::NM24) ? 4 : 8;
        constexpr int GN = (P == Pattern::NM24) ? 2 : 6;
        constexpr int VW = 64 * GN / GM / 16;
        const int64_t vrow = nm_value_row_bytes(K, GN, GM);
        const int64_t sb = k0 / 64;
        const uint32_t *vp = reinterpret_cast<const uint32_t *>(packed + n * vrow + sb * (VW * 4));
        const uint32_t *mp = reinterpret_cast<const uint32_t *>(packed + N * vrow + n * (K / 8) + sb * 8);
#pragma unroll
        for (int v = 0; v < VW; ++v) r.w[v] = vp[v];
        r.w[VW] = mp[0];
        r.w[VW + 1] = mp[1];
    }
}

// 4 dense code words from a raw slice (N:M: decode the superblock; table24 is
// the 2:4 decode table in LDS)
template <Pattern P>
__device__ __forceinline__ u32x4 dense_words(const RawSlice<P> &r, const uint8_t *table24)
{
    if constexpr (P == Pattern::Dense) {
        return u32x4{r.w[0], r.w[1], r.w[2], r.w[3]};
    } else {
        constexpr int VW = RawSlice<P>::kWords - 2;
        uint32_t w[4];
        decode_superblock_fast<P>(r.w, r.w + VW, w, table24);
        return u32x4{w[0], w[1], w[2], w[3]};
    }
}

// N:M rows expanded to the dense code layout, one 64-weight chunk per thread
// (pruned positions get code 1, t = 0), so that the pipelined dense GEMM can
// run on them: one pass over the weights per call.
template <Pattern P>
__global__ __launch_bounds__(256) void nm_expand_dense_kernel(const uint8_t *__restrict__ packed, int64_t N,
                                                              int64_t K, uint8_t *__restrict__ dense)
{
    __shared__ uint8_t s_nm24[P == Pattern::NM24 ? 256 : 1];
    if constexpr (P == Pattern::NM24) {
        s_nm24[threadIdx.x] = nm24_table_entry((uint32_t)threadIdx.x);
        __syncthreads();
    }
    const int64_t C = K / 64;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N * C) return;
    const int64_t n = i / C, c = i - n * C;
    RawSlice<P> r;
    load_raw<P>(packed, N, K, n, c * 64, r);
    *reinterpret_cast<u32x4 *>(dense + n * (K / 4) + c * 16) = dense_words<P>(r, s_nm24);
}

__device__ __forceinline__ i32x4 unpack_word(uint32_t w)
{
    i32x4 b;
    b[0] = (int)(w & kCodeMask);
    b[1] = (int)((w >> 2) & kCodeMask);
    b[2] = (int)((w >> 4) & kCodeMask);
    b[3] = (int)((w >> 6) & kCodeMask);
    return b;
}

// Fused epilogue of one wave's FM x FN 32x32 fragments: acc - rowsum, times
// beta * x_scale, to Y (and acc_out).  Full tiles (the common case) take a
// branch-free path: one 64-bit row pointer per output row, the row sums and
// scales of 4 consecutive rows read from LDS with one 16-byte load each, and
// the column offsets folded into the store's immediate offset.  NT: the
// full tiles' outputs go out as non-temporal stores -- where every tile of the
// grid ends at once (one round of tiles over the compute units) their output
// leaves in one burst at the end, and streaming stores drain it faster
// (512 x 8960 x 1536: 17.2 -> 15.5 us; 1024 x 8192 x 2048: 23.5 -> 22.3 us).
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int TM, int TN, int FM, int FN, bool NT = false>
__device__ __forceinline__ void store_tile(const i32x16 (&acc)[FM][FN], const int *s_rs, const float *s_sc,
                                           int wm, int wn, int h, int li, int64_t m0, int64_t n0, int64_t M,
                                           int64_t N, bool full, float *__restrict__ Y,
                                           int32_t *__restrict__ acc_out)
{
    if (full && !acc_out) {
        float *yb = Y + (m0 + wm * TM + 4 * h) * N + (n0 + wn * TN + li);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int lr0 = wm * TM + fm * 32 + 8 * g + 4 * h;
                const i32x4 rs4 = *reinterpret_cast<const i32x4 *>(s_rs + lr0);
                const f32x4 sc4 = *reinterpret_cast<const f32x4 *>(s_sc + lr0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float *yr = yb + (int64_t)(fm * 32 + 8 * g + r) * N;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const float y = (float)(acc[fm][fn][4 * g + r] - rs4[r]) * sc4[r];
                        if constexpr (NT) __builtin_nontemporal_store(y, &yr[fn * 32]);
                        else yr[fn * 32] = y;
                    }
                }
            }
        }
        return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int lr = wm * TM + fm * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            const int64_t m = m0 + lr;
            if (m >= M) continue;
            const int rs = s_rs[lr];
            const float sc = s_sc[lr];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int64_t n = n0 + wn * TN + fn * 32 + li;
                if (n < N) {
                    const int av = acc[fm][fn][v] - rs;
                    Y[m * N + n] = (float)av * sc;
                    if (acc_out) acc_out[m * N + n] = av;
                }
            }
        }
    }
}

// BM x BN tile, WM x WN waves, each wave (BM/WM) x (BN/WN) of 32x32 fragments.
//
// TB (N:M only): instead of decoding each superblock to dense 2-bit words,
// its kept codes are spread over their positions as 64 * t signed bytes by
// byte permutes (nm_expand_superblock; pruned positions 0), staged in LDS as
// 64 bytes per row and slice (80 apart), and read straight into the B
// operand.  The accumulators then hold 64 * sum t*q: no row sum is
// subtracted, and the exact shift by 6 precedes the epilogue.  |acc| <= 64 *
// 127 * K, so the host uses it for K <= 2^18.
template <Pattern P, int BM, int BN, int WM, int WN, bool TB = false, bool SPLIT = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ x_scale, const int32_t *__restrict__ x_rowsum,
    const uint8_t *__restrict__ packed, const float *__restrict__ w_scale, int64_t M, int64_t N,
    int64_t K, float *__restrict__ Y, int32_t *__restrict__ acc_out, int32_t splits = 1,
    int32_t *__restrict__ ws = nullptr)
{
    constexpr int T = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;          // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;          // 32x32 fragments per wave
    static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "tile");
    static_assert(!TB || P != Pattern::Dense, "t-bytes are for N:M");
    constexpr int LB = TB ? 80 : LDB;                  // bytes per staged weight row
    constexpr int A_PIECES = BM * 4;                   // 16-byte pieces of an activation slice
    constexpr int A_PER_T = (A_PIECES + T - 1) / T;
    constexpr int B_PER_T = (BN + T - 1) / T;          // packed rows (16 bytes) per thread
    // TB: a work item is half a row's superblock (32 positions); items
    // [0, BN) are first halves, [BN, 2 BN) second halves, so the half is
    // wave-uniform (BN is a multiple of 64)
    constexpr int BH_PER_T = (2 * BN + T - 1) / T;
    constexpr int VWH = (P == Pattern::NM68) ? 2 : 1;  // value words of a half
    __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * LDA];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * LB];
    __shared__ __attribute__((aligned(16))) int s_rs[BM];
    __shared__ __attribute__((aligned(16))) float s_sc[BM];
    __shared__ uint8_t s_nm24[P == Pattern::NM24 && !TB ? 256 : 1];
    __shared__ uint32_t s_sel[TB ? 2 * nm_sel_entries(P) : 1];

    // the wave index is wave-uniform: say so, so that branches on it are scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int h = lane >> 5, li = lane & 31;
    if constexpr (TB) {
        for (int i = tid; i < nm_sel_entries(P); i += T) nm_sel_entry<P>(i, &s_sel[2 * i], &s_sel[2 * i + 1]);
        __syncthreads();
    } else if constexpr (P == Pattern::NM24) {
        for (int i = tid; i < 256; i += T) s_nm24[i] = nm24_table_entry((uint32_t)i);
        __syncthreads();
    }

    const int64_t tiles_m = (M + BM - 1) / BM;
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    // XCD-aware order: logical tile = xcd * per_xcd + index within the XCD
    const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
    // SPLIT: blockIdx.x = split * (per_xcd * kXcds) + tile workgroup, as in
    // the pipelined kernel's split-K form (same partial layout and epilogue)
    const int64_t split = SPLIT ? (int64_t)blockIdx.x / (per_xcd * kXcds) : 0;
    const int64_t b = (int64_t)blockIdx.x - split * per_xcd * kXcds;
    const int64_t tile = (b % kXcds) * per_xcd + b / kXcds;
    if (tile >= tiles) return;
    // consecutive logical tiles walk M first, so they share a weight column tile
    const int64_t m0 = (tile % tiles_m) * BM;
    const int64_t n0 = (tile / tiles_m) * BN;
    const float beta = w_scale[0];

    for (int i = tid; i < BM; i += T) {
        const int64_t m = min(m0 + i, M - 1);
        s_rs[i] = TB ? 0 : x_rowsum[m];               // t-bytes: no offset codes
        s_sc[i] = beta * x_scale[m];
    }

    // global -> register staging of one K slice
    u32x4 ra[A_PER_T];
    RawSlice<P> rb[TB ? 1 : B_PER_T];
    uint32_t hv[TB ? BH_PER_T : 1][VWH], hm[TB ? BH_PER_T : 1];
    auto load_slice = [&](int64_t k0) {
#pragma unroll
        for (int p = 0; p < A_PER_T; ++p) {
            const int idx = p * T + tid;
            const int row = idx >> 2, c = idx & 3;
            const int64_t m = min(m0 + row, M - 1);        // rows >= M: any finite data, never stored
            ra[p] = *reinterpret_cast<const u32x4 *>(Xq + m * K + k0 + 16 * c);
        }
        if constexpr (TB) {
            constexpr int GM = (P == Pattern::NM24) ? 4 : 8, GN = (P == Pattern::NM24) ? 2 : 6;
            constexpr int VW = 64 * GN / GM / 16;
            const int64_t vrow = nm_value_row_bytes(K, GN, GM), sb = k0 / 64;
#pragma unroll
            for (int p = 0; p < BH_PER_T; ++p) {
                const int idx = p * T + tid;
                if ((2 * BN) % T == 0 || idx < 2 * BN) {
                    const int h = idx / BN, row = idx % BN;
                    const int64_t n = min(n0 + row, N - 1);
                    const uint32_t *vp = reinterpret_cast<const uint32_t *>(packed + n * vrow + sb * (VW * 4)) + h;
#pragma unroll
                    for (int v = 0; v < VWH; ++v) hv[p][v] = vp[v];
                    hm[p] = reinterpret_cast<const uint32_t *>(packed + N * vrow + n * (K / 8) + sb * 8)[h];
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < B_PER_T; ++p) {
                const int row = p * T + tid;
                if (BN % T == 0 || row < BN) {             // whole waves
                    const int64_t n = min(n0 + row, N - 1);
                    load_raw<P>(packed, N, K, n, k0, rb[p]);
                }
            }
        }
    };
    auto store_slice = [&](int buf) {
#pragma unroll
        for (int p = 0; p < A_PER_T; ++p) {
            const int idx = p * T + tid;
            if (A_PIECES % T == 0 || idx < A_PIECES) {
                const int row = idx >> 2, c = idx & 3;
                *reinterpret_cast<u32x4 *>(sA[buf] + row * LDA + 16 * c) = ra[p];
            }
        }
        if constexpr (TB) {
#pragma unroll
            for (int p = 0; p < BH_PER_T; ++p) {
                const int idx = p * T + tid;
                if ((2 * BN) % T == 0 || idx < 2 * BN) {
                    const int h = idx / BN, row = idx % BN;          // h wave-uniform
                    uint32_t e[8];
                    if (h == 0) nm_expand_half<P, DeviceOps, 0>(hv[p], hm[p], s_sel, e);
                    else nm_expand_half<P, DeviceOps, 1>(hv[p], hm[p], s_sel, e);
                    u32x4 *dst = reinterpret_cast<u32x4 *>(sB[buf] + row * LB + 32 * h);
                    dst[0] = u32x4{e[0], e[1], e[2], e[3]};
                    dst[1] = u32x4{e[4], e[5], e[6], e[7]};
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < B_PER_T; ++p) {
                const int row = p * T + tid;
                if (BN % T == 0 || row < BN) {
                    const u32x4 d = dense_words<P>(rb[p], s_nm24);
                    u32x2 *dst = reinterpret_cast<u32x2 *>(sB[buf] + row * LDB);
                    dst[0] = u32x2{d[0], d[1]};
                    dst[1] = u32x2{d[2], d[3]};
                }
            }
        }
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int c = 0; c < FN; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][c][v] = 0;

    // this workgroup's K slices [sl0, sl0 + slices)
    const int64_t all_slices = K / BK;
    const int64_t sl0 = SPLIT ? all_slices * split / splits : 0;
    const int64_t slices = SPLIT ? all_slices * (split + 1) / splits - sl0 : all_slices;
    load_slice(sl0 * BK);
    store_slice(0);
    __syncthreads();

    for (int64_t it = 0; it < slices; ++it) {
        const int buf = (int)(it & 1);
        if (it + 1 < slices) load_slice((sl0 + it + 1) * BK);

        // B fragments: words 2h and 2h+1 of each row (k-steps s = 0, 1); all
        // fragments of the slice are read into distinct registers first
        // (t-bytes: the 32 bytes of those positions)
        u32x2 bw[FN];
        i32x4 bt[2][FN];
        i32x4 a[2][FM];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const uint8_t *brow = sB[buf] + (wn * TN + fn * 32 + li) * LB;
            if constexpr (TB) {
                bt[0][fn] = *reinterpret_cast<const i32x4 *>(brow + 32 * h);
                bt[1][fn] = *reinterpret_cast<const i32x4 *>(brow + 32 * h + 16);
            } else {
                bw[fn] = *reinterpret_cast<const u32x2 *>(brow + 8 * h);
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                a[s][fm] = *reinterpret_cast<const i32x4 *>(sA[buf] + (wm * TM + fm * 32 + li) * LDA + 32 * h + 16 * s);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            i32x4 bb[FN];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) bb[fn] = TB ? bt[s][fn] : unpack_word(bw[fn][s]);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[s][fm], bb[fn], acc[fm][fn], 0, 0, 0);
        }

        if (it + 1 < slices) store_slice(buf ^ 1);
        __syncthreads();
    }

    if constexpr (SPLIT) {                             // raw partials; the epilogue kernel finishes
        constexpr int E = FM * FN * 16;
        int32_t *mine = ws + (split * tiles + tile) * (int64_t)(E * T);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int v = 0; v < 16; ++v) mine[((fm * FN + fn) * 16 + v) * T + tid] = acc[fm][fn][v];
        return;
    }

    if constexpr (TB) {                                // 64 * sum t*q: exact
#pragma unroll
        for (int a2 = 0; a2 < FM; ++a2)
#pragma unroll
            for (int c = 0; c < FN; ++c)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a2][c][v] >>= 6;
    }

    // fused epilogue: offset-code correction and dequant scale
    store_tile<TM, TN, FM, FN>(acc, s_rs, s_sc, wm, wn, h, li, m0, n0, M, N,
                               (m0 + BM <= M) && (n0 + BN <= N), Y, acc_out);
}

// ---------------------------------------------------------------------------
// Dense path with a deeper pipeline: S-stage LDS ring filled by direct
// global->LDS loads (global_load_lds_dwordx4: the data never passes through
// VGPRs), so S-1 K slices are in flight while one is consumed; one barrier
// per slice.  Each wave issues the same number of loads per slice (A: BM/16
// instructions spread over the waves; B: BN / waves rows, one instruction per
// 64 rows or one half-wave instruction for 32), which keeps the vmcnt
// bookkeeping a compile-time constant.
//
// A direct load writes 64 consecutive 16-byte LDS slots per instruction, so
// the activation tile is stored unpadded, 64 bytes per row, with the 16-byte
// pieces XOR-swizzled: logical piece c of row r sits in slot c ^ ((r >> 2) & 3).
// The MFMA-side read of 16 consecutive rows at one logical piece then covers
// 16 distinct 4-bank groups.  Packed weight rows are 16 bytes apart.
//
// Schedule of one slice (two k-steps of 32), per wave:
//   MFMAs of k-step 0, each followed by one LDS read of the A fragments of
//     k-step 1; then unpack the weight codes of k-step 1
//   wait for slice i+1, barrier, issue the loads of slice i+S-1
//   MFMAs of k-step 1, each followed by one LDS read of the packed weights and
//     A fragments (k-step 0) of slice i+1; then unpack those weight codes
// A read issued right behind an MFMA runs while the matrix core works through
// the rest of the group, so its result is in registers when the next group
// starts (measured on 2048 x 6912 x 2560: 43.7 -> 40.3 us against issuing the
// reads after the whole group).  The barrier is a bare s_barrier with
// compiler-level fences: the wait for the direct loads is explicit (vmcnt),
// and the fragments a wave read from the stage being overwritten were
// consumed before it reached the barrier.
// ---------------------------------------------------------------------------
// SPLIT: the K slices are divided among `splits` workgroups per output tile
// (blockIdx.x = split * tile workgroups + tile workgroup); each writes its
// int32 partial tile to the workspace `ws` (element e of thread t at e * T + t)
// and the epilogue kernel below, launched next on the same stream, adds the
// partials (integer sums: the result does not depend on the order) and
// applies the dequant scale.  Used when there are too few output tiles to fill
// the chip (few tokens).  The kernel boundary makes the partials visible: no
// fence or counter is needed.
//
// The body is a device function of the workgroup's index within its grid
// (`bid`), so that a grouped launch can run several projections' grids as
// one (gemm_dma_grouped_kernel below).
template <int BM, int BN, int WM, int WN, int S, bool SPLIT, bool NT>
__device__ __forceinline__ void gemm_dma_tile(
    const int8_t *__restrict__ Xq, const float *__restrict__ x_scale, const int32_t *__restrict__ x_rowsum,
    const uint8_t *__restrict__ packed, const float *__restrict__ w_scale, int64_t M, int64_t N,
    int64_t K, float *__restrict__ Y, int32_t *__restrict__ acc_out, int32_t splits, int32_t *__restrict__ ws,
    int64_t bid)
{
    constexpr int NW = WM * WN;
    constexpr int T = 64 * NW;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "tile");
    constexpr int A_INSTR = BM / 16;                   // 1 KB (16 rows) per instruction
    static_assert(A_INSTR % NW == 0, "A loads must split evenly over the waves");
    constexpr int A_PER_W = A_INSTR / NW;
    constexpr int B_ROWS_W = BN / NW;                  // packed weight rows loaded per wave
    static_assert(BN % NW == 0 && (B_ROWS_W == 32 || B_ROWS_W % 64 == 0), "B loads per wave");
    constexpr int B_PER_W = (B_ROWS_W + 63) / 64;      // 32 rows: one half-wave instruction
    constexpr int LPS = A_PER_W + B_PER_W;             // loads per slice per wave
    static_assert(S >= 3, "the pipeline needs S >= 3");
    constexpr int SA = BM * 64, SB = BN * 16, STAGE = SA + SB;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int *s_rs = reinterpret_cast<int *>(smem + S * STAGE);
    float *s_sc = reinterpret_cast<float *>(smem + S * STAGE + 4 * BM);

    // the wave index is wave-uniform: say so, so that branches on it are scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int h = lane >> 5, li = lane & 31;

    const int64_t tiles_m = (M + BM - 1) / BM;
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
    const int64_t grid_tiles = per_xcd * kXcds;
    const int64_t split = SPLIT ? bid / grid_tiles : 0;
    const int64_t b = bid - split * grid_tiles;
    int64_t tile, m0, n0;
    if (!SPLIT && xcd_regions(tiles_m, tiles_n)) {
        // each XCD owns one of 4 x 2 blocks of the tile grid: a quarter of the
        // activation rows and half of the weight columns stay in its L2
        const int64_t x = b % kXcds, j = b / kXcds;
        const int64_t mc = tiles_m / 4;
        const int64_t nlo = tiles_n * (x / 4) / 2, nhi = tiles_n * (x / 4 + 1) / 2;
        const int64_t mt = (x % 4) * mc + j % mc, nt = nlo + j / mc;
        if (nt >= nhi) return;
        tile = nt * tiles_m + mt;
        m0 = mt * BM;
        n0 = nt * BN;
    } else {
        tile = (b % kXcds) * per_xcd + b / kXcds;
        if (tile >= tiles) return;
        m0 = (tile % tiles_m) * BM;
        n0 = (tile / tiles_m) * BN;
    }
    const float beta = w_scale[0];
    for (int i = tid; i < BM; i += T) {
        const int64_t m = min(m0 + i, M - 1);
        s_rs[i] = x_rowsum[m];
        s_sc[i] = beta * x_scale[m];
    }

    // this workgroup's K slices [sl0, sl0 + slices)
    const int64_t all_slices = K / BK;
    const int64_t sl0 = SPLIT ? all_slices * split / splits : 0;
    const int64_t slices = SPLIT ? all_slices * (split + 1) / splits - sl0 : all_slices;

    // per-lane global sources of this wave's loads (advance by k0 per slice)
    const int8_t *a_src[A_PER_W];
#pragma unroll
    for (int j = 0; j < A_PER_W; ++j) {
        const int jj = wave * A_PER_W + j;
        const int row = jj * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 2) & 3);
        a_src[j] = Xq + min(m0 + row, M - 1) * K + 16 * c;
    }
    const uint8_t *b_src[B_PER_W];
#pragma unroll
    for (int j = 0; j < B_PER_W; ++j)
        b_src[j] = packed + min(n0 + wave * B_ROWS_W + j * 64 + lane, N - 1) * (K / 4);

    auto issue = [&](int64_t sl) {
        uint8_t *st = smem + (sl % S) * STAGE;
        const int64_t k0 = (sl0 + sl) * BK;
#pragma unroll
        for (int j = 0; j < A_PER_W; ++j) dma16(a_src[j] + k0, st + (wave * A_PER_W + j) * 1024);
#pragma unroll
        for (int j = 0; j < B_PER_W; ++j)
            if (B_ROWS_W >= 64 || lane < 32) dma16(b_src[j] + k0 / 4, st + SA + (wave * B_ROWS_W + j * 64) * 16);
    };

    // fragment offsets within a stage: A row r, logical piece 2h + k-step;
    // B row of fragment fn, words 2h and 2h+1 (k-steps 0 and 1)
    int fa[2][FM];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = wm * TM + fm * 32 + li;
            fa[s2][fm] = r * 64 + 16 * ((2 * h + s2) ^ ((r >> 2) & 3));
        }
    const int fb = SA + (wn * TN + li) * 16 + 8 * h;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto read_a = [&](int64_t sl, auto s2c, i32x4 (&dst)[FM]) {
        constexpr int s2 = decltype(s2c)::value;
        const uint8_t *st = smem + (sl % S) * STAGE;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) dst[fm] = *reinterpret_cast<const i32x4 *>(st + fa[s2][fm]);
    };
    auto read_b = [&](int64_t sl, u32x2 (&dst)[FN]) {
        const uint8_t *st = smem + (sl % S) * STAGE;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) dst[fn] = *reinterpret_cast<const u32x2 *>(st + fb + fn * 32 * 16);
    };

    auto unpack = [&](const u32x2 (&bw)[FN], auto s2c, i32x4 (&bb)[FN]) {
        constexpr int s2 = decltype(s2c)::value;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) bb[fn] = unpack_word(bw[fn][s2]);
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[x][y][v] = 0;
    auto mfma_grp = [&](const i32x4 (&a)[FM], const i32x4 (&bb)[FN]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[fm], bb[fn], acc[fm][fn], 0, 0, 0);
    };
    // scheduling of one group: each of its MFMAs followed by one of NR LDS reads
    auto interleave = [](auto nrc) {
        constexpr int NR = decltype(nrc)::value;
#pragma unroll
        for (int i = 0; i < FM * FN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
            if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
    };

    // prologue: S-1 slices in flight, slice 0 resident, its k-step-0 operands in registers
#pragma unroll
    for (int sl = 0; sl < S - 1; ++sl)
        if (sl < slices) issue(sl);
    if (S - 2 < slices) wait_vm<LPS * (S - 2)>();
    else wait_vm<0>();
    block_barrier();
    i32x4 a0[FM], a1[FM], bb0[FN], bb1[FN];
    u32x2 bw[FN];
    read_a(0, I0(), a0);
    read_b(0, bw);
    unpack(bw, I0(), bb0);
    // the output pointers are read only by the epilogue: complete their scalar
    // loads here, or every LDS wait in the loop becomes a wait for everything
    asm volatile("" ::"s"(Y), "s"(acc_out), "s"(ws));

    // one slice; `steady`: slices it+1 .. it+S-1 exist (no guards needed)
    auto slice = [&](int64_t it, bool steady) {
        __builtin_amdgcn_sched_barrier(0);
        mfma_grp(a0, bb0);
        read_a(it, I1(), a1);
        interleave(std::integral_constant<int, FM>());
        __builtin_amdgcn_sched_barrier(0);
        unpack(bw, I1(), bb1);
        const bool more = steady || it + 1 < slices;
        if (steady) {
            wait_vm<LPS * (S - 3)>();                  // slice it+1 landed (this wave's loads)
            block_barrier();                           // ... and every wave's
            issue(it + S - 1);                         // into the stage of slice it-1
        } else if (more) {
            if (it + S - 2 < slices) wait_vm<LPS * (S - 3)>();
            else wait_vm<0>();
            block_barrier();
            if (it + S - 1 < slices) issue(it + S - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_grp(a1, bb1);
        if (more) {
            read_b(it + 1, bw);
            read_a(it + 1, I0(), a0);
        }
        interleave(std::integral_constant<int, FM + (FN + 1) / 2>());
        __builtin_amdgcn_sched_barrier(0);
        if (more) unpack(bw, I0(), bb0);
    };
    int64_t it = 0;
    for (; it + S <= slices; ++it) slice(it, true);
    for (; it < slices; ++it) slice(it, false);

    if constexpr (SPLIT) {
        constexpr int E = FM * FN * 16;
        int32_t *mine = ws + (split * tiles + tile) * (int64_t)(E * T);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int v = 0; v < 16; ++v) mine[((fm * FN + fn) * 16 + v) * T + tid] = acc[fm][fn][v];
        return;
    }
    store_tile<TM, TN, FM, FN, NT>(acc, s_rs, s_sc, wm, wn, h, li, m0, n0, M, N,
                                   (m0 + BM <= M) && (n0 + BN <= N), Y, acc_out);
}

template <int BM, int BN, int WM, int WN, int S, bool SPLIT, int OCC = 1, bool NT = false>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_dma_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ x_scale, const int32_t *__restrict__ x_rowsum,
    const uint8_t *__restrict__ packed, const float *__restrict__ w_scale, int64_t M, int64_t N,
    int64_t K, float *__restrict__ Y, int32_t *__restrict__ acc_out, int32_t splits, int32_t *__restrict__ ws)
{
    gemm_dma_tile<BM, BN, WM, WN, S, SPLIT, NT>(Xq, x_scale, x_rowsum, packed, w_scale, M, N, K, Y, acc_out, splits,
                                                ws, (int64_t)blockIdx.x);
}

// Several projections sharing the activations in one launch (no K split):
// workgroup b belongs to projection p (args.block_start) and runs block b -
// block_start[p] of that projection's own grid.  One launch for gate and up
// of a 3B block at 64 tokens: 17.4 -> 14.7 us against one per projection.
template <int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_grouped_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ x_scale, const int32_t *__restrict__ x_rowsum,
    FusedProjArgs args, int64_t M, int64_t K)
{
    const int p = proj_of_block(args, (int)blockIdx.x);
    gemm_dma_tile<BM, BN, WM, WN, S, false, false>(Xq, x_scale, x_rowsum, args.packed[p], args.w_scale[p], M,
                                                   args.N[p], K, args.Y[p], args.acc[p], 1, nullptr,
                                                   (int64_t)blockIdx.x - args.block_start[p]);
}

// Epilogue of the split-K GEMM, one thread per output element (m, n): find
// the element's slot in the GEMM kernel's per-thread fragment layout, add the
// `splits` partials (integers: order-free), subtract the row sum (TB: divide
// the 64 * t sums by 64 instead; no offset codes) and scale.
template <int BM, int BN, int WM, int WN, bool TB = false>
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(
    const float *__restrict__ x_scale, const int32_t *__restrict__ x_rowsum, const float *__restrict__ w_scale,
    int64_t M, int64_t N, int32_t splits, const int32_t *__restrict__ ws, float *__restrict__ Y,
    int32_t *__restrict__ acc_out)
{
    constexpr int T = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FN = TN / 32;
    constexpr int E = (TM / 32) * FN * 16;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx - m * N;
    const int64_t tiles_m = (M + BM - 1) / BM;
    const int64_t tiles = tiles_m * ((N + BN - 1) / BN);
    const int64_t tile = (n / BN) * tiles_m + m / BM;
    const int lr = (int)(m % BM), lc = (int)(n % BN);
    const int wave = (lr / TM) * WN + lc / TN;
    const int fm = (lr % TM) / 32, fn = (lc % TN) / 32;
    const int r32 = lr % 32;                      // row in the 32x32 fragment: 8 (v / 4) + 4 h + v % 4
    const int hh = (r32 >> 2) & 1, v = (r32 >> 3) * 4 + (r32 & 3);
    const int tid = wave * 64 + 32 * hh + (lc % 32);
    const int e = (fm * FN + fn) * 16 + v;
    int acc = 0;
    for (int64_t o = 0; o < splits; ++o) acc += ws[(o * tiles + tile) * (int64_t)(E * T) + (int64_t)e * T + tid];
    const int av = TB ? (acc >> 6) : acc - x_rowsum[m];
    Y[idx] = (float)av * (w_scale[0] * x_scale[m]);
    if (acc_out) acc_out[idx] = av;
}

template <int BM, int BN, int WM, int WN, int S, bool SPLIT = false, int OCC = 1, bool NT = false>
hipError_t launch_dma(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                      const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                      hipStream_t stream, int32_t splits = 1, int32_t *ws = nullptr)
{
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
    const int64_t grid = SPLIT ? per_xcd * kXcds * splits : xcd_grid(tiles_m, tiles_n);
    const size_t lds = (size_t)S * (BM * 64 + BN * 16) + 8 * BM;
    auto kern = gemm_dma_kernel<BM, BN, WM, WN, S, SPLIT, OCC, NT>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), lds, stream, Xq, xs, rs, packed, w_scale,
                       M, N, K, Y, acc, splits, ws);
    if (SPLIT) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t blocks = (M * N + 255) / 256;
        hipLaunchKernelGGL((splitk_epilogue_kernel<BM, BN, WM, WN>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           xs, rs, w_scale, M, N, splits, ws, Y, acc);
    }
    return hipGetLastError();
}

// Largest split-K partial-sum area (int32 partial tiles) a few-token GEMM
// takes from the caller's workspace: bounds the splits, so the workspace of
// such a call stays within 32 MiB.
constexpr int64_t kMaxSplitBytes = 32ll << 20;

// Few tokens (dense, M <= 64): BM x BN tiles over a deep ring, K split over
// enough workgroups to occupy every compute unit (none when the tiles alone
// do).
template <int BM, int BN, int WM, int WN>
hipError_t launch_few_tokens(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                             const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                             Scratch &scratch, hipStream_t stream, const char **name, const char *split_name,
                             const char *plain_name)
{
    constexpr int S = 8;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t slices = K / BK;
    int64_t splits = std::min<int64_t>((kCus + tiles - 1) / tiles, slices / 4);   // >= 4 slices each
    const int64_t per_split = tiles * (int64_t)BM * BN * 4;        // partial bytes per split
    splits = std::min<int64_t>(splits, kMaxSplitBytes / per_split);
    if (splits >= 2) {
        *name = split_name;
        if (!scratch.take((size_t)(splits * per_split))) return scratch.query ? hipSuccess : hipErrorOutOfMemory;
        return launch_dma<BM, BN, WM, WN, S, true>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream,
                                                   (int32_t)splits, reinterpret_cast<int32_t *>(scratch.ptr));
    }
    *name = plain_name;
    if (scratch.query) return hipSuccess;
    return launch_dma<BM, BN, WM, WN, S, false>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
}

// N:M t-byte GEMM with too few output tiles to fill the chip (few tokens,
// or few weight rows): K split over enough workgroups to occupy every compute
// unit, as for the dense few-token path; partials of 64 * t sums, exact.
// Returns hipErrorNotSupported when no split applies (the caller launches
// the unsplit kernel).
template <Pattern P, int BM, int BN, int WM, int WN>
hipError_t launch_tbytes_split(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                               const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                               Scratch &scratch, hipStream_t stream)
{
    if (K > kTBytesMaxK) return hipErrorNotSupported;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t slices = K / BK;
    int64_t splits = std::min<int64_t>((kCus + tiles - 1) / tiles, slices / 4);   // >= 4 slices each
    const int64_t per_split = tiles * (int64_t)BM * BN * 4;
    splits = std::min<int64_t>(splits, kMaxSplitBytes / per_split);
    if (splits < 2) return hipErrorNotSupported;
    if (!scratch.take((size_t)(splits * per_split))) return scratch.query ? hipSuccess : hipErrorOutOfMemory;
    int32_t *w = reinterpret_cast<int32_t *>(scratch.ptr);
    const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((gemm_kernel<P, BM, BN, WM, WN, true, true>), dim3((unsigned)(per_xcd * kXcds * splits)),
                       dim3(64 * WM * WN), 0, stream, Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, (int32_t)splits,
                       w);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t blocks = (M * N + 255) / 256;
    hipLaunchKernelGGL((splitk_epilogue_kernel<BM, BN, WM, WN, true>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       xs, rs, w_scale, M, N, (int32_t)splits, w, Y, acc);
    return hipGetLastError();
}

template <Pattern P, int BM, int BN, int WM, int WN>
hipError_t launch(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                  const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                  hipStream_t stream)
{
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
    const int64_t grid = per_xcd * kXcds;
    if constexpr (P != Pattern::Dense) {
        if (K <= kTBytesMaxK) {
            hipLaunchKernelGGL((gemm_kernel<P, BM, BN, WM, WN, true>), dim3((unsigned)grid), dim3(64 * WM * WN), 0,
                               stream, Xq, xs, rs, packed, w_scale, M, N, K, Y, acc);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_kernel<P, BM, BN, WM, WN>), dim3((unsigned)grid), dim3(64 * WM * WN), 0, stream,
                       Xq, xs, rs, packed, w_scale, M, N, K, Y, acc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nm24_sparse(const int8_t *Xq, const float *xs, const uint8_t *packed, const float *w_scale,
                                   int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream,
                                   int tile_m);

namespace {

template <Pattern P>
hipError_t dispatch(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                    const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                    Scratch &scratch, hipStream_t stream, const char **name)
{
    static const char *names[2][3][3] = {
        {{"", "", ""},
         {"gemm_nm24_256x256", "gemm_nm24_128x128", "gemm_nm24_64x128"},
         {"gemm_nm68_256x256", "gemm_nm68_128x128", "gemm_nm68_64x128"}},
        {{"", "", ""},
         {"gemm_nm24_256x256_tbytes", "gemm_nm24_128x128_tbytes", "gemm_nm24_64x128_tbytes"},
         {"gemm_nm68_256x256_tbytes", "gemm_nm68_128x128_tbytes", "gemm_nm68_64x128_tbytes"}}};
    const int pi = (int)P;
    const int tb = (P != Pattern::Dense && K <= kTBytesMaxK) ? 1 : 0;   // as launch() decides
    auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if constexpr (P == Pattern::Dense) {
        if (M > 64) {
            // pipelined kernel; tile size by a cost model measured on MI355X
            // over M = 256 .. 3072: one round of tiles over the 256 compute
            // units costs about 4 for 256 x 256, 2 for 128 x 256 (8 waves of
            // 64 x 64) and 1.35 for 128 x 128 (smaller tiles: more operand
            // traffic per MFMA).  E.g. 1000 x 8000 x 2560: 4 / 2 / 2.7, measured
            // 40 / 27 / 32 us; 3072 x 6912: 8 / 6 / 8.1, measured 75 / 64 / 78
            // us; 2048 x 6912: 4 / 4 / 5.4 (a tie, measured 43-44 us both).
            auto rounds = [&](int64_t t) { return (double)((t + kCus - 1) / kCus); };
            const double c256 = 4.0 * rounds(tiles(256, 256)), c12 = 2.0 * rounds(tiles(128, 256));
            const double c128 = 1.35 * rounds(tiles(128, 128));
            // too few 128 x 128 tiles for the chip (deep K, few weight rows:
            // 512 x 2560 x 6912 has 80): K split over enough workgroups, the
            // partial tiles in the workspace, as for few tokens
            if (tiles(128, 128) < kCus / 2 && K / BK >= 8) {
                const int64_t t = tiles(128, 128);
                int64_t splits = std::min<int64_t>((kCus + t - 1) / t, (K / BK) / 4);
                splits = std::min<int64_t>(splits, kMaxSplitBytes / (t * 128 * 128 * 4));
                if (splits >= 2) {
                    *name = "gemm_dense_splitk_128x128_w4_s4";
                    if (!scratch.take((size_t)(splits * t * 128 * 128 * 4)))
                        return scratch.query ? hipSuccess : hipErrorOutOfMemory;
                    return launch_dma<128, 128, 2, 2, 4, true>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream,
                                                               (int32_t)splits,
                                                               reinterpret_cast<int32_t *>(scratch.ptr));
                }
            }
            if (c256 <= c12 && c256 <= c128) {
                // six stages (120 KB of LDS): 2048 x 6912 x 2560 43.4 -> 42.7
                // us, 4096 x 8192 x 4096 124 -> 120 us against four; the
                // smaller tiles measured slower with more than four
                *name = "gemm_dense_dma_256x256_w8_s6";
                if (scratch.query) return hipSuccess;
                return launch_dma<256, 256, 2, 4, 6>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
            }
            // one round of tiles: streaming stores for the output (see store_tile)
            if (c12 <= c128) {
                *name = "gemm_dense_dma_128x256_w8_s4";
                if (scratch.query) return hipSuccess;
                if (tiles(128, 256) <= kCus)
                    return launch_dma<128, 256, 2, 4, 4, false, 1, true>(Xq, xs, rs, packed, w_scale, M, N, K, Y,
                                                                         acc, stream);
                return launch_dma<128, 256, 2, 4, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
            }
            *name = "gemm_dense_dma_128x128_w4_s4";
            if (scratch.query) return hipSuccess;
            if (tiles(128, 128) <= kCus)
                return launch_dma<128, 128, 2, 2, 4, false, 1, true>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc,
                                                                     stream);
            return launch_dma<128, 128, 2, 2, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
        }
        // narrow weight tiles: more workgroups from N, so fewer K splits (none
        // for wide N).  Measured against 128-wide tiles: at 64 tokens,
        // 2048 -> 11008 17.7 -> 10.2 us (one launch) and 2048 -> 2048 8.9 ->
        // 8.2 us; at 20-32 tokens, 1536 -> 8960 11.3 -> 7.6 us and 2048 ->
        // 11008 12.9 -> 8.2 us.  Deep K takes 64-wide tiles (11008 -> 2048 at
        // 64 tokens: 12.9 -> 12.5 us, where 32-wide ones take 14.4).
        // Narrow tiles take 32 tokens also at 33-64 tokens: twice the
        // workgroups of one-wave tiles, for a latency-bound chain of K slices
        // (64 x 11008 x 2048: 10.1 -> 8.5 us against 64 x 32 tiles; 48 x 8960
        // x 1536: 9.9 -> 7.5 us).
        const bool narrow = K <= 4096 || N >= 32 * kCus;
        if (narrow)
            return launch_few_tokens<32, 32, 1, 1>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, scratch, stream, name,
                                                   "gemm_dense_splitk_32x32", "gemm_dense_dma_32x32");
        if (M <= 32)
            return launch_few_tokens<32, 64, 1, 1>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, scratch, stream, name,
                                                   "gemm_dense_splitk_32x64", "gemm_dense_dma_32x64");
        return launch_few_tokens<64, 64, 2, 1>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, scratch, stream, name,
                                               "gemm_dense_splitk_64x64", "gemm_dense_dma_64x64");
    } else {
        // 65+ tokens where the sparse MFMA does not apply (6:8; 2:4 below 128
        // tokens or with K % 128 != 0): expand the rows to dense codes once
        // into the caller's workspace, then the pipelined dense GEMM.
        // Measured against the t-byte GEMM, 6:8 (dense beside it): 2048 x
        // 6912 x 2560 70 -> 52 us (48), 4096 x 8192 x 4096 218 -> 141 us
        // (137), 2048 x 2560 x 6912 88 -> 59 us (54), 128 x 8960 x 1536 18.0
        // -> 16.7 us (11.7).
        const bool sparse24 = P == Pattern::NM24 && M >= 128 && K % 128 == 0;
        if (M > 64 && !sparse24) {
            static const char *expand_names[3][4] = {
                {"", "", "", ""},
                {"gemm_nm24_expand_dense_256x256", "gemm_nm24_expand_dense_128x256", "gemm_nm24_expand_dense_128x128",
                 "gemm_nm24_expand_dense_splitk_128x128"},
                {"gemm_nm68_expand_dense_256x256", "gemm_nm68_expand_dense_128x256", "gemm_nm68_expand_dense_128x128",
                 "gemm_nm68_expand_dense_splitk_128x128"}};
            // the expanded rows first, then (256-byte aligned) whatever the
            // dense GEMM on them needs (K split: its partial tiles)
            const size_t rows_bytes = ((size_t)N * (size_t)(K / 4) + 255) / 256 * 256;
            Scratch dense_need;
            dense_need.query = true;
            const char *dn = "";
            (void)dispatch<Pattern::Dense>(Xq, xs, rs, nullptr, w_scale, M, N, K, Y, acc, dense_need, stream, &dn);
            const bool go = scratch.take(rows_bytes + dense_need.need);
            if (!go && !scratch.query) return hipErrorOutOfMemory;
            Scratch dense_scratch;
            dense_scratch.query = scratch.query;
            if (go) {
                const int64_t chunks = N * (K / 64);
                hipLaunchKernelGGL(nm_expand_dense_kernel<P>, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                                   stream, packed, N, K, scratch.ptr);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
                dense_scratch.ptr = scratch.ptr + rows_bytes;
                dense_scratch.bytes = scratch.bytes - rows_bytes;
            }
            const hipError_t e = dispatch<Pattern::Dense>(Xq, xs, rs, scratch.ptr, w_scale, M, N, K, Y, acc,
                                                          dense_scratch, stream, &dn);
            const std::string_view d(dn);
            *name = expand_names[pi][d.find("256x256") != d.npos ? 0 : d.find("128x256") != d.npos ? 1
                                     : d.find("splitk") != d.npos ? 3 : 2];
            return e;
        }
        if constexpr (P == Pattern::NM24) {
            // 2:4 on the sparse matrix cores (gemm_sparse.hip) where K allows;
            // token tile by rounds over the compute units as for the dense
            // kernel: one round costs about 4 at 256 tokens and 2 at 128
            // (1000 x 8000 x 2560: 4 / 2, measured 56 / 34 us; 2048 x 6912 x
            // 2560: 4 / 4, measured 40 / 46 us, ties take 256).  At 256 tokens
            // and more this beats the t-byte GEMM everywhere measured (512 x
            // 2560 x 6912: 41 against 75 us; 256 x 8960 x 1536: 15.7 against
            // 18.9 us).
            if (M >= 128 && K % 128 == 0) {
                auto rounds = [&](int64_t t) { return (double)((t + kCus - 1) / kCus); };
                if (4.0 * rounds(tiles(256, 256)) <= 2.0 * rounds(tiles(128, 256))) {
                    *name = "gemm_nm24_smfmac_256x256";
                    if (scratch.query) return hipSuccess;
                    return launch_gemm_nm24_sparse(Xq, xs, packed, w_scale, M, N, K, Y, acc, stream, 256);
                }
                *name = "gemm_nm24_smfmac_128x256";
                if (scratch.query) return hipSuccess;
                return launch_gemm_nm24_sparse(Xq, xs, packed, w_scale, M, N, K, Y, acc, stream, 128);
            }
        }
        if (M >= 256 && tiles(256, 256) >= 128) {
            *name = names[tb][pi][0];
            if (scratch.query) return hipSuccess;
            return launch<P, 256, 256, 2, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
        }
        // too few tiles for the chip: K split (t-byte form); measured at 32 and
        // 64 tokens, 6912 -> 2560 with 2:4: 71 us unsplit
        static const char *split_names[3][2] = {
            {"", ""}, {"gemm_nm24_splitk_128x128_tbytes", "gemm_nm24_splitk_64x128_tbytes"},
            {"gemm_nm68_splitk_128x128_tbytes", "gemm_nm68_splitk_64x128_tbytes"}};
        if (M > 64) {
            const hipError_t e = launch_tbytes_split<P, 128, 128, 2, 2>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc,
                                                                        scratch, stream);
            if (e != hipErrorNotSupported) {
                *name = split_names[pi][0];
                return e;
            }
            *name = names[tb][pi][1];
            if (scratch.query) return hipSuccess;
            return launch<P, 128, 128, 2, 2>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
        }
        const hipError_t e = launch_tbytes_split<P, 64, 128, 1, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc,
                                                                   scratch, stream);
        if (e != hipErrorNotSupported) {
            *name = split_names[pi][1];
            return e;
        }
        *name = names[tb][pi][2];
        if (scratch.query) return hipSuccess;
        return launch<P, 64, 128, 1, 4>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, stream);
    }
}

}  // namespace

// Several dense projections sharing Xq at 17-64 tokens in one launch of the
// one-wave 32 x 32 tiles, where each projection alone would take those tiles
// without a K split (K <= 4096 or N >= 8192, at least one tile per compute
// unit); hipErrorNotSupported (nothing launched) otherwise.
hipError_t launch_gemm_grouped(const int8_t *Xq, const float *xs, const int32_t *rs, FusedProjArgs args, Pattern p,
                               int64_t M, int64_t K, hipStream_t stream, const char **name, bool query)
{
    if (p != Pattern::Dense || M < 17 || M > 64 || args.nproj < 2 || args.nproj > kMaxFusedProj)
        return hipErrorNotSupported;
    constexpr int BM = 32, BN = 32, S = 8;             // launch_few_tokens<32, 32, 1, 1>'s tiles and ring
    const int64_t tiles_m = (M + BM - 1) / BM;
    int64_t blocks = 0;
    for (int i = 0; i < args.nproj; ++i) {
        const int64_t tiles_n = (args.N[i] + BN - 1) / BN;
        const bool narrow = K <= 4096 || args.N[i] >= 32 * kCus;
        if (!narrow || tiles_m * tiles_n < kCus) return hipErrorNotSupported;
        args.block_start[i] = (int32_t)blocks;
        blocks += xcd_grid(tiles_m, tiles_n);
    }
    for (int i = args.nproj; i <= kMaxFusedProj; ++i) args.block_start[i] = (int32_t)blocks;
    if (blocks > (1LL << 30)) return hipErrorNotSupported;
    *name = "gemm_dense_dma_32x32_grouped";
    if (query) return hipSuccess;
    const size_t lds = (size_t)S * (BM * 64 + BN * 16) + 8 * BM;
    hipLaunchKernelGGL((gemm_dma_grouped_kernel<BM, BN, 1, 1, S>), dim3((unsigned)blocks), dim3(64), lds, stream, Xq,
                       xs, rs, args, M, K);
    return hipGetLastError();
}

hipError_t launch_gemm(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                       const float *w_scale, Pattern p, int64_t M, int64_t N, int64_t K, float *Y,
                       int32_t *acc, Scratch &scratch, hipStream_t stream, const char **name)
{
    switch (p) {
    case Pattern::Dense:
        return dispatch<Pattern::Dense>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, scratch, stream, name);
    case Pattern::NM24:
        return dispatch<Pattern::NM24>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, scratch, stream, name);
    case Pattern::NM68:
        return dispatch<Pattern::NM68>(Xq, xs, rs, packed, w_scale, M, N, K, Y, acc, scratch, stream, name);
    }
    return hipErrorInvalidValue;
}

}  // namespace bl
