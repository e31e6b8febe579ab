/*
 * bitlinear.h -- C ABI of libbitlinear.so: the BitNet b1.58 BitLinear forward
 * pass on AMD Instinct MI355X (gfx950), with the Sparse-BitNet N:M variant.
 *
 * The operation, as the pages define it:
 *   - weights: absmean ternarisation, beta = mean|W| over the whole matrix,
 *     W_t = clamp(round(W / (beta + 1e-5)), -1, 1)
 *     ("BitNet b1.58 2B4T Technical Report 요약 설명", sec. 2 Architecture;
 *      "BitNet 논문 분석: 1-Bit LLM의 시대", section "Absmean 양자화 함수");
 *   - activations: per-token absmax quantisation to int8
 *     (same two sections);
 *   - an integer matmul of the ternary weights, four 2-bit codes per byte
 *     (2B4T summary, sec. 5.1 GPU Inference; I2_S code 00 = -1, 01 = 0,
 *      10 = +1 from "bitnet.cpp 추론 프레임워크"), with int32 accumulation,
 *     then a rescale by the weight and activation scales;
 *   - optional N:M: keep the N largest |latent weight| per group of M inputs,
 *     after ternarising with the full-matrix beta (quant-then-mask)
 *     ("Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to
 *      Semi-Structured Sparsity", review, sec. 3.2).
 *
 * Exact arithmetic contract (the readings where the pages leave room):
 *   beta    = fl32( (sum over n of (sum over k of |W[n,k]|, k ascending, in
 *             binary64), n ascending, in binary64) / (N*K) )
 *   d       = fl32(beta + 1e-5f)
 *   t[n,k]  = clamp(rne(fl32(W[n,k] / d)), -1, 1)
 *   N:M     = per row n and group [g*M, g*M+M): keep the N largest |W[n,k]|,
 *             equal magnitudes resolved towards the lower k
 *   g_m     = max_k |X[m,k]|;  if g_m == 0: Xq = 0, x_scale = 0
 *   u_m     = 2^100 if g_m < 2^-100, else 1   (exact rescaling of rows whose
 *             127 / g_m would overflow; q is unchanged wherever it does not)
 *   s_m     = fl32(127 / fl32(g_m * u_m))
 *   Xq[m,k] = clamp(rne(fl32(fl32(X[m,k] * u_m) * s_m)), -128, 127)
 *   x_scale = fl32(g_m / 127);  x_rowsum[m] = sum_k Xq[m,k]
 *   acc     = sum_k Xq[m,k] * W_eff[n,k]          (exact int32)
 *   Y[m,n]  = fl32( fl32(acc) * fl32(beta * x_scale[m]) )
 * Xq, x_scale, x_rowsum, the packed bytes, beta and acc are bit-exact with a
 * plain CPU evaluation of these formulas; Y is within 1e-5 relative of
 * acc * beta * x_scale evaluated in binary64 (and exactly 0 when acc is 0).
 *
 * Packed layout.  2-bit code c = t + 1.  A run of 16 codes j = 0..15 is one
 * little-endian 32-bit word with code j at bit 8*(j%4) + 2*(j/4), so
 * (word >> 2*i) & 0x03030303 holds codes 4i..4i+3 in its four bytes.
 *   dense: row n = K/16 words (K/4 bytes) at byte offset n*K/4.
 *   N:M (2:4 and 6:8): a values region then a masks region.
 *     values: row n holds the codes of its kept weights in increasing k,
 *             K*N_/(4*M_) bytes per row, rows back to back;
 *     masks:  K/8 bytes per row after all value rows; for M_=4 group g has a
 *             4-bit mask in byte g/2 (even g in the low nibble); for M_=8
 *             group g has byte g; bit i set = k = g*M_ + i kept.
 *   sizes: dense and 2:4 = N*K/4 bytes; 6:8 = 5*N*K/16 bytes.
 *   2:4 trit-packed (bitlinear_pack_weights_trit24): per group g of 4
 *     inputs, kept inputs i0 < i1, one 6-bit code 9*p + 3*(t[i0]+1) +
 *     (t[i1]+1), p the index of (i0, i1) in (0,1) (0,2) (0,3) (1,2) (1,3)
 *     (2,3); the 16 codes of inputs 64s..64s+63 form string s, 96 bits
 *     little-endian with group g%16 at bit 6*(g%16) (12 bytes); row n is
 *     its K/64 strings in k order at byte offset n*3*K/16: 3*N*K/16 bytes.
 *
 * Conventions for every call:
 *   - Data pointers are device pointers (hipMalloc / torch tensors) owned by
 *     the caller.  The library allocates no device memory and keeps none
 *     between calls: scratch memory comes from the caller as a workspace
 *     argument (bitlinear_pack_weights, bitlinear_forward), sized by a
 *     host-only query (bitlinear_packed_size, bitlinear_forward_workspace_size).
 *     The kernels a call launches depend on the shapes alone.  A workspace
 *     belongs to one call until that call's work has finished on its stream;
 *     calls on different streams need workspaces of their own.
 *   - Matrices are row-major and dense: W is N x K (out x in), X and Xq are
 *     M x K, Y and acc are M x N.
 *   - Work is enqueued on `stream` (NULL = the null stream); no call
 *     synchronises.  Asynchronous faults surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns a negative status and launches nothing.
 *     bitlinear_last_error() then describes the failure.
 *   - Shape limits: 64 <= K <= 1048576 with K % 64 == 0; 1 <= N <= 16777216;
 *     0 <= M <= 16777216.  M == 0 is a successful no-op, and then the
 *     M-sized buffers (X, Xq, x_scale, x_rowsum, Y, acc) may be NULL.
 *   - Alignment: W, X, Xq, packed, Y and acc must be 16-byte aligned;
 *     w_scale, x_scale and x_rowsum 4-byte aligned; the pack workspace 8-byte
 *     aligned and the forward workspace 16-byte aligned.
 *   - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same typedef as HIP's own, so this header needs no HIP include. */
typedef struct ihipStream_t *hipStream_t;

/* N:M pattern: {0,0} = dense, {2,4} = 2:4, {6,8} = 6:8.  Anything else is
 * BITLINEAR_EUNSUPPORTED. */
typedef struct {
    int32_t n;
    int32_t m;
} bitlinear_nm;

typedef enum {
    BITLINEAR_OK = 0,
    BITLINEAR_EINVAL = -1,       /* bad shape, null or misaligned pointer */
    BITLINEAR_EUNSUPPORTED = -2, /* N:M pattern not supported */
    BITLINEAR_ESIZE = -3,        /* a caller buffer is too small */
    BITLINEAR_EHIP = -4          /* a HIP launch or runtime call failed */
} bitlinear_status;

/* Host-only size query for bitlinear_pack_weights.  *packed_bytes receives
 * the packed-weight size for an N x K matrix under `nm` (2-bit codes, four per
 * byte: "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 5.1; N:M values
 * and keep masks: the layout above); *workspace_bytes the device scratch that
 * bitlinear_pack_weights needs (8*N bytes of binary64 row sums, rounded up to
 * 256).  Either output pointer may be NULL.  Launches nothing.  Errors:
 * EUNSUPPORTED for another N:M pattern, EINVAL for N or K out of range. */
bitlinear_status bitlinear_packed_size(int64_t N, int64_t K, bitlinear_nm nm,
                                       size_t *packed_bytes, size_t *workspace_bytes);

/* Pack time: absmean ternarisation ("BitNet 논문 분석: 1-Bit LLM의 시대",
 * section "Absmean 양자화 함수"; 2B4T summary, sec. 2), the optional N:M
 * mask with quant-then-mask (Sparse-BitNet review, sec. 3.2) and 2-bit
 * packing with the I2_S code map ("bitnet.cpp 추론 프레임워크").
 * W: N x K fp32 latent weights (read only).  packed: packed_bytes-byte output
 * (see the layout).  w_scale: one fp32, receives beta.  workspace: scratch of
 * at least the size bitlinear_packed_size reports; its contents on entry do
 * not matter and on exit are unspecified.  Errors: ESIZE if packed_bytes or
 * workspace_bytes is too small; EINVAL for a bad shape or a null or
 * misaligned pointer; EUNSUPPORTED for another N:M pattern. */
bitlinear_status bitlinear_pack_weights(const float *W, int64_t N, int64_t K, bitlinear_nm nm,
                                        void *packed, size_t packed_bytes, float *w_scale,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* N:M weights stored in the dense layout: the same beta, ternary values and
 * N:M mask as bitlinear_pack_weights with `nm` (quant-then-mask, the N
 * largest |W| per group of M inputs, ties to the lower k; Sparse-BitNet
 * review, sec. 3.2), with the pruned positions written as code 01 (t = 0) in
 * the dense 2-bit layout (N*K/4 bytes: fewer than the 6:8 values+masks
 * format, as many as 2:4's).  Any 1 <= N <= M with M in {4, 8, 16}: the
 * review's N:8 sweep (sec. 6.3, Table 7) as well as 2:4 and 6:8.  The result
 * feeds bitlinear_forward and the fused and grouped calls with nm = {0, 0}
 * -- the dense kernels, with no decoding of masks per call -- and for 2:4
 * and 6:8 gives the same acc, bit for bit, as their N:M format.  Errors:
 * EINVAL for {0,0}, EUNSUPPORTED for another M or N out of range, ESIZE if
 * packed_bytes < N*K/4 or the workspace (as bitlinear_pack_weights) is
 * short. */
bitlinear_status bitlinear_pack_weights_masked(const float *W, int64_t N, int64_t K, bitlinear_nm nm,
                                               void *packed, size_t packed_bytes, float *w_scale,
                                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Per-token absmax int8 quantisation of X (M x K fp32): 2B4T summary, sec. 2
 * (8-bit activations, absmax per token); "BitNet 논문 분석", section
 * "Absmean 양자화 함수" (activation_quant).  Xq: M x K int8 output.
 * x_scale: M fp32 (g_m / 127).  x_rowsum: M int32 row sums of Xq; may be NULL
 * when not wanted (bitlinear_forward needs it).  Errors: EINVAL for a bad
 * shape or a null or misaligned pointer. */
bitlinear_status bitlinear_quant_act(const float *X, int64_t M, int64_t K,
                                     int8_t *Xq, float *x_scale, int32_t *x_rowsum,
                                     hipStream_t stream);

/* Host-only size query for bitlinear_forward: *workspace_bytes receives the
 * device scratch that an M x N x K call under `nm` needs (0 for most shapes;
 * at most 32 MiB for the GEMMs that split K -- few tokens, or prefill with
 * fewer than 128 output tiles of 128 x 128 -- whose int32 partial tiles it
 * holds; for N:M weights at 65+ tokens where the 2:4 sparse MFMA does not
 * apply, N*K/4 bytes rounded up to 256 for the rows expanded to dense codes,
 * plus the partial tiles if the dense GEMM on them splits K).
 * Launches nothing.  Errors: EINVAL for a bad shape or NULL output,
 * EUNSUPPORTED for another N:M pattern. */
bitlinear_status bitlinear_forward_workspace_size(int64_t M, int64_t N, int64_t K, bitlinear_nm nm,
                                                  size_t *workspace_bytes);

/* The forward contraction and rescale: the integer matmul of the ternary
 * weights and the int8 activations with int32 accumulation, then the
 * dequantisation by beta and x_scale (2B4T summary, sec. 2 and 5.1; "BitNet
 * 논문 분석", section "Absmean 양자화 함수", BitLinear's forward; N:M:
 * Sparse-BitNet review, sec. 3.2).  Xq, x_scale, x_rowsum: as written by
 * bitlinear_quant_act (x_rowsum is required: the kernels accumulate with the
 * unsigned codes c = t + 1 and subtract the row sum).  packed, w_scale: as
 * written by bitlinear_pack_weights with the same N, K and nm.  Y: M x N fp32
 * output.  acc: optional M x N int32 output of the exact integer sums (NULL
 * to skip).  workspace: device scratch of workspace_bytes bytes, at least
 * what bitlinear_forward_workspace_size reports for the shape (NULL with 0
 * when that is 0); its contents on entry do not matter and on exit are
 * unspecified; it must not be used by other work until this call's work on
 * `stream` has finished.  The kernel is chosen from the shape: M = 1
 * (K <= 16384) packed int8 dot products; 2 <= M <= 16 (and up to 64 with few
 * weight rows, in tiles of 16 tokens) an MFMA kernel with the tokens as one
 * operand (2:4 with K % 128 == 0 and M <= 16: the sparse MFMA where it
 * measured faster); larger M the MFMA GEMM (K split over workgroups for
 * M <= 64, or past 64 with fewer than 128 tiles of 128 x 128, when the output
 * tiles alone cannot fill the GPU; 2:4 with
 * K % 128 == 0 and M >= 128 on the sparse MFMA; other N:M at M >= 65 on the
 * dense GEMM after expanding the rows to dense codes in the workspace).
 * Every path gives the same acc, bit for bit, and the same Y.
 * bitlinear_last_dispatch() names the kernel.  Errors: ESIZE when the
 * workspace is smaller than the shape needs (nothing is launched); EINVAL for
 * a bad shape or a null or misaligned pointer; EUNSUPPORTED for another N:M
 * pattern; EHIP when a launch fails. */
bitlinear_status bitlinear_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                   const void *packed, const float *w_scale, bitlinear_nm nm,
                                   int64_t M, int64_t N, int64_t K,
                                   float *Y, int32_t *acc, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* bitlinear_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels and
 * the same results, bit for bit.  Its scratch is a fixed 32 MiB array in the
 * library's device code, one copy per GPU, held until the process ends; its
 * address is looked up on the first call on each device.  Calls whose shape
 * needs more scratch than that (bitlinear_forward_workspace_size) return
 * ESIZE and launch nothing.  Every call on a GPU shares that GPU's array: such
 * calls must not overlap in time on one GPU (they race on it), whatever
 * their streams.  `stream` must belong to the current device (EINVAL
 * otherwise).  Other errors as bitlinear_forward. */
bitlinear_status bitlinear_forward_noalloc(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                           const void *packed, const float *w_scale, bitlinear_nm nm,
                                           int64_t M, int64_t N, int64_t K,
                                           float *Y, int32_t *acc, hipStream_t stream);

/* Host-only size query for bitlinear_pack_weights_trit24: *packed_bytes
 * receives 3*N*K/16 (1.5 bits per weight: the trit-packed layout above),
 * *workspace_bytes the pack's scratch (as bitlinear_packed_size).  Either
 * output pointer may be NULL.  Launches nothing.  Errors: EINVAL for N or K
 * out of range. */
bitlinear_status bitlinear_packed_size_trit24(int64_t N, int64_t K, size_t *packed_bytes,
                                              size_t *workspace_bytes);

/* 2:4 weights in the trit-packed layout: the same beta, ternary values and
 * 2:4 mask as bitlinear_pack_weights with nm = {2,4} (quant-then-mask, the
 * two largest |W| per group of 4 inputs, ties to the lower k; Sparse-BitNet
 * review, sec. 3.2), stored as one 6-bit code per group, which names the
 * kept pair and its two ternary values out of 6 x 3 x 3 = 54 (the pair index
 * over the 3 x 3 values, as bitnet.cpp's TL2 indexes a pair of ternary
 * weights by its 9 combinations: "bitnet.cpp 추론 프레임워크", section "I2_S
 * 커널의 내부 동작").  3*N*K/16 bytes: a quarter fewer than the 2:4 values +
 * masks.  Arguments and workspace as bitlinear_pack_weights.  Errors: ESIZE
 * if packed_bytes < 3*N*K/16 or the workspace is short; EINVAL for a bad
 * shape or a null or misaligned pointer. */
bitlinear_status bitlinear_pack_weights_trit24(const float *W, int64_t N, int64_t K, void *packed,
                                               size_t packed_bytes, float *w_scale, void *workspace,
                                               size_t workspace_bytes, hipStream_t stream);

/* Host-only size query for bitlinear_forward_trit24: *workspace_bytes
 * receives the device scratch of an M x N x K call (0 for one token with
 * K <= 16384; otherwise N*K/4 bytes rounded up to 256 for the rows expanded
 * to dense codes, plus what bitlinear_forward needs for the dense shape).
 * Launches nothing.  Errors: EINVAL for a bad shape or NULL output. */
bitlinear_status bitlinear_forward_trit24_workspace_size(int64_t M, int64_t N, int64_t K,
                                                         size_t *workspace_bytes);

/* The forward contraction and rescale (as bitlinear_forward: 2B4T summary,
 * sec. 2 and 5.1; Sparse-BitNet review, sec. 3.2) on weights written by
 * bitlinear_pack_weights_trit24 with the same N and K.  Arguments, outputs,
 * workspace rules and errors as bitlinear_forward with nm = {2,4}; acc and Y
 * are bit-identical to bitlinear_forward on the same weights packed by
 * bitlinear_pack_weights with nm = {2,4}.  One token with K <= 16384 runs a
 * kernel that reads the 6-bit codes and looks up their four weights in a
 * table in LDS (x_rowsum is then not read); otherwise the rows are expanded
 * to dense codes in the workspace and the dense kernels run on them.  Codes
 * 54-63, which the packer never writes, count as four zero weights. */
bitlinear_status bitlinear_forward_trit24(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                          const void *packed, const float *w_scale, int64_t M, int64_t N,
                                          int64_t K, float *Y, int32_t *acc, void *workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/* One projection of a fused decode call: packed weights and beta as written
 * by bitlinear_pack_weights (same K and nm as the call), N output features,
 * Y the M x N fp32 output, acc an optional M x N int32 output (NULL to skip). */
typedef struct {
    const void *packed;
    const float *w_scale;
    int64_t N;
    float *Y;
    int32_t *acc;
} bitlinear_proj;

/* Fused decode forward: per-token absmax int8 quantisation of X (M x K fp32,
 * exactly as bitlinear_quant_act) and the forward of `nproj` projections that
 * share X (q/k/v, or gate/up of a feed-forward block), in one launch.  The
 * outputs are bit-identical to bitlinear_quant_act followed by
 * bitlinear_forward for each projection ("BitNet b1.58 2B4T Technical Report
 * 요약 설명", sec. 2 and 5.1; "BitNet 논문 분석: 1-Bit LLM의 시대", section
 * "Absmean 양자화 함수").  `projs` is a host array of nproj entries.
 * x_scale: optional M fp32 output (g_m / 127), NULL to skip.
 * Supported: 1 <= M <= 16, 1 <= nproj <= 8, K <= 16192 (K <= 65344 when
 * M == 1); anything else returns BITLINEAR_EUNSUPPORTED and launches
 * nothing -- use the two-call path then.  Past 4 tokens the tokens run in
 * tiles of 4 along the grid, each tile quantising its own rows (for wide
 * projection groups bitlinear_quant_act then bitlinear_forward_grouped is
 * the faster form). */
bitlinear_status bitlinear_forward_fused(const float *X, int64_t M, int64_t K, bitlinear_nm nm,
                                         const bitlinear_proj *projs, int32_t nproj,
                                         float *x_scale, hipStream_t stream);

/* Forward of several projections that share one quantised input (q/k/v, or
 * gate/up of a feed-forward block) in one launch: the same contraction and
 * rescale as bitlinear_forward for each projection, bit for bit (2B4T
 * summary, sec. 2 and 5.1; "BitNet 논문 분석", section "Absmean 양자화
 * 함수"; the Sparse-BitNet review's Table 5 discussion notes that decode
 * gains are diluted by launch overhead at small batches).  Xq, x_scale,
 * x_rowsum: as written by bitlinear_quant_act for the shared input (M x K).
 * `projs`: host array of nproj entries (packed, w_scale, N, Y, acc as in
 * bitlinear_proj).  Supported: 1 <= nproj <= 8 and M <= 16, or
 * 17 <= M <= 64 while the 16-token tiles times the 16-row weight blocks of
 * all projections make at most 1024 workgroups (512 for one projection), and
 * K within the kernels' range.  Dense weights (nm = {0, 0}) with
 * 256 <= K <= 3072 over at least 6912 rows in all at 9-64 tokens, 2560 at
 * 17-64 tokens or 2048 at 33-64 tokens, run on the direct-load kernel with
 * several token tiles per workgroup (at 33-64 tokens: fewer than 13824 rows,
 * or at least 16384 with K <= 2048).  Past those, at
 * 17-64 tokens, dense weights and two or more projections, each with
 * K <= 4096 or N >= 8192 and at least 256 output tiles of 32 x 32, run as one
 * grouped launch of the few-token GEMM.  Anything else returns
 * BITLINEAR_EUNSUPPORTED and launches nothing (call bitlinear_forward per
 * projection then).  Needs no workspace. */
bitlinear_status bitlinear_forward_grouped(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                           int64_t M, int64_t K, bitlinear_nm nm, const bitlinear_proj *projs,
                                           int32_t nproj, hipStream_t stream);

/* One input of bitlinear_quant_act_multi: M x K fp32 rows X and their
 * outputs, each as in bitlinear_quant_act (x_rowsum may be NULL). */
typedef struct {
    const float *X;
    int64_t M;
    int64_t K;
    int8_t *Xq;
    float *x_scale;
    int32_t *x_rowsum;
} bitlinear_quant_group;

/* bitlinear_quant_act for several independent inputs in one launch (the
 * inputs of a block's projection groups, each then fed to
 * bitlinear_forward or bitlinear_forward_grouped): each group's outputs are
 * bit-identical to its own bitlinear_quant_act call (2B4T summary, sec. 2;
 * "BitNet 논문 분석", section "Absmean 양자화 함수").  `groups` is a host
 * array of 1 <= ngroups <= 8 entries; no group's outputs may overlap another
 * group's or any input.  One launch while every row fits the kernel's
 * registers (K <= 16384 when the groups hold at most 512 rows in all and
 * some K >= 4096, else K <= 8192); otherwise one bitlinear_quant_act launch
 * per group, with the same results.  Errors: EINVAL for a bad group (as
 * bitlinear_quant_act) or ngroups < 1, EUNSUPPORTED for ngroups > 8. */
bitlinear_status bitlinear_quant_act_multi(const bitlinear_quant_group *groups, int32_t ngroups,
                                           hipStream_t stream);

/* One quantised input of bitlinear_forward_grouped_multi: Xq, x_scale,
 * x_rowsum as written by bitlinear_quant_act (M x K), and the nproj
 * projections that read it (a host array, as for bitlinear_forward_grouped). */
typedef struct {
    const int8_t *Xq;
    const float *x_scale;
    const int32_t *x_rowsum;
    int64_t K;
    const bitlinear_proj *projs;
    int32_t nproj;
} bitlinear_act_group;

/* bitlinear_forward_grouped for several quantised inputs in one launch (the
 * projection groups of a block at a few tokens, quantised together by
 * bitlinear_quant_act_multi): each projection's acc and Y bit-identical to
 * its own bitlinear_forward (2B4T summary, sec. 2 and 5.1; "BitNet 논문
 * 분석", section "Absmean 양자화 함수"; the Sparse-BitNet review's Table 5
 * discussion: decode gains are diluted by launch overhead at small batches).
 * `groups` is a host array of 1 <= ngroups <= 4 entries; no output may
 * overlap another output or any input.  Supported: dense weights
 * (nm = {0, 0}), up to 8 projections per group, and either 5 <= M <= 8 with
 * every K in [256, 12288], or 9 <= M <= 64 with every group within the
 * direct-load token-tile kernel's rules of bitlinear_forward_grouped
 * (256 <= K <= 3072 and at least 6912 rows in the group at 9-64 tokens, 2560
 * from 17 tokens, 2048 from 33; at 33-64 tokens fewer than 13824 rows, or at
 * least 16384 with K <= 2048); anything else returns
 * BITLINEAR_EUNSUPPORTED and launches nothing (call
 * bitlinear_forward_grouped or bitlinear_forward per group then).  Needs no
 * workspace.  Errors: EINVAL for a bad group (as
 * bitlinear_forward_grouped) or ngroups < 1. */
bitlinear_status bitlinear_forward_grouped_multi(const bitlinear_act_group *groups, int32_t ngroups, int64_t M,
                                                 bitlinear_nm nm, hipStream_t stream);

/* Transform of each activation row before the absmax quantisation: the steps
 * either side of a BitNet linear, fused into the quantiser.
 *   up (ReLU^2 gate; "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 2:
 *      the feed-forward network uses squared ReLU): NULL, or M x K fp32
 *      (16-byte aligned); the row becomes h[k] = fl32(fl32(r*r) * up[k]),
 *      r = max(X[k], 0) -- X holding the gate projection's output and `up`
 *      the up projection's.  NULL: h = X.
 *   gamma, eps (RMSNorm; "BitNet 논문 분석: 1-Bit LLM의 시대", section
 *      "Absmean 양자화 함수": BitLinear_b158 applies an RMSNorm over its inputs
 *      before activation_quant; the 2B4T report, sec. 2, names subln): NULL,
 *      or K fp32 weights (16-byte aligned); eps finite and >= 0.  The row is
 *      normalised to h * rinv * gamma, rinv = 1 / sqrt(sum_k h^2 / K + eps).
 *      rinv is a positive per-row factor, so it divides out of the absmax
 *      codes: the codes are those of v[k] = fl32(h[k] * gamma[k]) (exactly
 *      the formulas above with v for X) and rinv goes into the scale:
 *      x_scale = fl32(g_m / 127 * rinv) evaluated in binary64, with the sum of
 *      squares in binary64 in an unspecified order (within one binary32 ulp of
 *      the in-order value).  NULL: no normalisation.
 * Xq and x_rowsum stay bit-exact with a plain CPU evaluation. */
typedef struct {
    const float *up;
    const float *gamma;
    float eps;
} bitlinear_act_transform;

/* bitlinear_quant_act on transformed rows.  tr: host pointer, or NULL for no
 * transform (then identical to bitlinear_quant_act). */
bitlinear_status bitlinear_quant_act_ex(const float *X, const bitlinear_act_transform *tr, int64_t M,
                                        int64_t K, int8_t *Xq, float *x_scale, int32_t *x_rowsum,
                                        hipStream_t stream);

/* bitlinear_forward_fused on transformed rows (tr as above, NULL for none):
 * for a gated feed-forward block at decode, the down projection's call takes
 * X = the gate output, tr->up = the up output and tr->gamma = the subln
 * weight, so ReLU^2, the norm, the quantisation and the projection are one
 * launch.  With a transform, supported for M == 1 and K <= 16384 (otherwise
 * BITLINEAR_EUNSUPPORTED: use bitlinear_quant_act_ex, then
 * bitlinear_forward).  x_scale receives the scale defined above. */
bitlinear_status bitlinear_forward_fused_ex(const float *X, const bitlinear_act_transform *tr, int64_t M,
                                            int64_t K, bitlinear_nm nm, const bitlinear_proj *projs,
                                            int32_t nproj, float *x_scale, hipStream_t stream);

/* One token, several input groups, one launch.  Group g is an fp32 row X
 * (1 x K, 16-byte aligned) with the nproj projections that read it (a host
 * array, as for bitlinear_forward_fused) and an optional x_scale output (one
 * fp32, NULL to skip). */
typedef struct {
    const float *X;
    int64_t K;
    const bitlinear_proj *projs;
    int32_t nproj;
    float *x_scale;
} bitlinear_input_group;

/* bitlinear_forward_fused for M = 1 over `ngroups` input groups whose inputs
 * do not depend on one another (the layers of independent sequences, several
 * experts' down projections, the projections of a step whose activations are
 * all given): per group, the per-token absmax int8 quantisation and every
 * projection's integer linear and rescale ("BitNet b1.58 2B4T Technical
 * Report 요약 설명", sec. 2 and 5.1; "BitNet 논문 분석: 1-Bit LLM의 시대",
 * section "Absmean 양자화 함수"), each group's outputs bit-identical to its
 * own bitlinear_forward_fused call.  The Sparse-BitNet review's Table 5
 * discussion notes that decode gains are diluted by launch overhead; here the
 * groups share one launch.  `groups` is a host array; no two groups' outputs
 * may overlap one another or any input.  nm applies to every group.  Dense
 * weights with every K <= 16384 and at most 16 projections in all run as one
 * launch; otherwise (N:M weights, a K past 16384, more projections) each
 * group runs as its own bitlinear_forward_fused launch, with the same
 * results.  Errors: EINVAL for a bad group (as
 * bitlinear_forward_fused) or ngroups < 1; EUNSUPPORTED for ngroups > 4 or a
 * K past 65344. */
bitlinear_status bitlinear_forward_fused_multi(const bitlinear_input_group *groups, int32_t ngroups,
                                               bitlinear_nm nm, hipStream_t stream);

/* H-BitLinear activation quantisation (the BitNet v2 summary
 * (brain.hanbit.co.kr): the activations entering a projection are
 * Hadamard-transformed online, then quantised to 4 bits).  Each row of X
 * (M x K fp32) is split into blocks of `block` inputs (a power of two,
 * 1 <= block <= 8192, dividing K); each block is multiplied by the Sylvester
 * Hadamard matrix H_block (entries +-1) with radix-2 butterflies, stage
 * h = 1, 2, 4, ..., block/2 mapping every pair (i, i + h), i & h == 0, to
 * (a + b, a - b) in binary32.  Then, with v the transformed row:
 *   g_m = max_k |v|;  u_m as above;  s_m = fl32(7 / fl32(g_m * u_m))
 *   Xq[m,k] = rne(fl32(fl32(v * u_m) * s_m))   in [-7, 7], one per int8
 *   x_scale[m] = fl32((double)g_m / 7 / sqrt(block))   (0 for a zero row)
 *   x_rowsum[m] = sum_k Xq[m,k]
 * The transform with its 1/sqrt(block) is orthonormal; that positive factor
 * divides out of the codes and is applied through x_scale.  The outputs feed
 * bitlinear_forward unchanged; the weights must be in the transformed basis
 * (the H-BitLinear's are).  All outputs are bit-exact with a plain CPU
 * evaluation of these formulas.  x_rowsum may be NULL. */
bitlinear_status bitlinear_quant_act_h4(const float *X, int64_t M, int64_t K, int64_t block, int8_t *Xq,
                                        float *x_scale, int32_t *x_rowsum, hipStream_t stream);

/* BitNet a4.8's hybrid activations ("BitNet 논문 분석: 1-Bit LLM의 시대",
 * section "BitNet a4.8: 하이브리드 양자화 전략": the largest activation
 * values are split off and kept at 8 bits, the rest is quantised to 4 bits,
 * each part with its own scale).  For each token row x of X (M x K fp32):
 *   S = the n_outliers largest |x[k]| (equal magnitudes: the lower k first);
 *   hi = x on S, 0 elsewhere;  lo = x off S, 0 on S;
 *   hi -> 8-bit codes exactly as bitlinear_quant_act (scale max|hi| / 127);
 *   lo -> 4-bit codes: g = max|lo|, s = fl32(7 / fl32(g * u)) (u the tiny-row
 *         factor above), q = rne(fl32(fl32(lo * u) * s)) in [-7, 7],
 *         scale fl32(g / 7); a zero part gives zeros and scale 0.
 * Outputs, 2M rows: Xq row 2m = token m's hi codes, row 2m + 1 its lo codes
 * (2M x K int8), x_scale and x_rowsum (2M entries; x_rowsum may be NULL).
 * The two parts share no position, so the linear of token m is the sum of
 * the linears of rows 2m and 2m + 1: run bitlinear_forward with 2M rows into
 * a 2M x N output, then bitlinear_combine_a48.  0 <= n_outliers <= K (the
 * pages give no fraction: the caller chooses it); K <= 16384
 * (BITLINEAR_EUNSUPPORTED beyond).  Bit-exact with a plain CPU evaluation. */
bitlinear_status bitlinear_quant_act_a48(const float *X, int64_t M, int64_t K, int64_t n_outliers, int8_t *Xq,
                                         float *x_scale, int32_t *x_rowsum, hipStream_t stream);

/* Y[m, n] = fl32(Y2[2m, n] + Y2[2m + 1, n]) for the 2M x N output of
 * bitlinear_forward on bitlinear_quant_act_a48's rows: token m's output is
 * beta * (x_scale_hi * acc_hi + x_scale_lo * acc_lo).  Within 1e-5 of that
 * value evaluated in binary64, relative to |hi part| + |lo part|. */
bitlinear_status bitlinear_combine_a48(const float *Y2, int64_t M, int64_t N, float *Y, hipStream_t stream);

/* Thread-local text for the last non-OK status returned on this thread (the
 * errors of a kernel path are part of what a deployment has to check: "BitNet
 * b1.58은 GPU 없이도 빠를까?", section "전용 커널은 무엇을 비교해야 하나").
 * Never NULL; the string lives until the thread's next failing call. */
const char *bitlinear_last_error(void);

/* Thread-local name of the kernel(s) the last successful call on this thread
 * launched, e.g. "decode_dot4_dense_lpr8_u5_p1" or
 * "gemm_dense_dma_256x256_w8_s4"; "none" after an M == 0 no-op.  The same
 * page, section "도입 순서는 어떻게 잡을까", warns that a runtime can drop to
 * a slow generic path without saying so; this names the path that ran.
 * Never NULL. */
const char *bitlinear_last_dispatch(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
