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
 *
 * Conventions for every call:
 *   - Data pointers are device pointers (hipMalloc / torch tensors) owned by
 *     the caller.  The one exception is internal: the first
 *     bitlinear_forward call on a device that needs scratch memory allocates
 *     a 64 MB workspace with hipMalloc, once, and keeps it until the process
 *     ends.  Two paths use it: the few-token GEMMs with K split over
 *     workgroups (M <= 64 with too few output tiles to fill the GPU; int32
 *     partial sums) and N:M weights at M >= 65 where the 2:4 sparse MFMA
 *     does not apply (the rows expanded to dense codes, N*K/4 <= 64 MB, for
 *     the dense GEMM).  That first call must not be inside HIP graph capture
 *     (a captured call that finds no workspace uses the unsplit or t-byte
 *     kernel instead, with identical results), and such calls must not
 *     overlap in time on one device (they share the workspace).
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
 *     w_scale, x_scale and x_rowsum 4-byte aligned; workspace 8-byte aligned.
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

/* Host-only size query.  *packed_bytes receives the packed-weight size for an
 * N x K matrix under `nm` (layout above); *workspace_bytes the device scratch
 * that bitlinear_pack_weights needs (8*N bytes of binary64 row sums, rounded
 * up to 256).  Either output pointer may be NULL.  Launches nothing. */
bitlinear_status bitlinear_packed_size(int64_t N, int64_t K, bitlinear_nm nm,
                                       size_t *packed_bytes, size_t *workspace_bytes);

/* Pack time (absmean ternarisation, optional N:M mask, 2-bit packing).
 * W: N x K fp32 latent weights.  packed: packed_bytes-byte output (see the
 * layout).  w_scale: one fp32, receives beta.  workspace: scratch of at least
 * the size bitlinear_packed_size reports; its contents on entry do not matter
 * and on exit are unspecified.  Returns BITLINEAR_ESIZE if packed_bytes or
 * workspace_bytes is too small. */
bitlinear_status bitlinear_pack_weights(const float *W, int64_t N, int64_t K, bitlinear_nm nm,
                                        void *packed, size_t packed_bytes, float *w_scale,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* Per-token absmax int8 quantisation of X (M x K fp32).
 * Xq: M x K int8.  x_scale: M fp32 (g_m / 127).  x_rowsum: M int32 row sums
 * of Xq; may be NULL when not wanted (bitlinear_forward needs it). */
bitlinear_status bitlinear_quant_act(const float *X, int64_t M, int64_t K,
                                     int8_t *Xq, float *x_scale, int32_t *x_rowsum,
                                     hipStream_t stream);

/* The forward contraction and rescale.  Xq, x_scale, x_rowsum: as written by
 * bitlinear_quant_act (x_rowsum is required: the kernels accumulate with the
 * unsigned codes c = t + 1 and subtract the row sum).  packed, w_scale: as
 * written by bitlinear_pack_weights with the same N, K and nm.  Y: M x N fp32
 * output.  acc: optional M x N int32 output of the exact integer sums (NULL
 * to skip).  The kernel is chosen from the shape: M = 1 (K <= 16384) packed
 * int8 dot products; 2 <= M <= 16 (and up to 64 with few weight rows, in
 * tiles of 16 tokens) an MFMA kernel with the tokens as one operand (2:4 with
 * K % 128 == 0 and M <= 16: the sparse MFMA where it measured faster);
 * larger M the MFMA GEMM (K split over workgroups for M <= 64 when the output
 * tiles alone cannot fill the GPU; 2:4 with K % 128 == 0 and M >= 128 on the
 * sparse MFMA; other N:M at M >= 65 on the dense GEMM after expanding the
 * rows to dense codes in the library's workspace).  Every path gives the
 * same acc, bit for bit, and the same Y.  bitlinear_last_dispatch() names the
 * kernel. */
bitlinear_status bitlinear_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                   const void *packed, const float *w_scale, bitlinear_nm nm,
                                   int64_t M, int64_t N, int64_t K,
                                   float *Y, int32_t *acc, hipStream_t stream);

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
 * Supported: 1 <= M <= 4, 1 <= nproj <= 8, K <= 16192 (K <= 65344 when
 * M == 1); anything else returns BITLINEAR_EUNSUPPORTED and launches
 * nothing -- use the two-call path then. */
bitlinear_status bitlinear_forward_fused(const float *X, int64_t M, int64_t K, bitlinear_nm nm,
                                         const bitlinear_proj *projs, int32_t nproj,
                                         float *x_scale, hipStream_t stream);

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

/* Thread-local text for the last non-OK status returned on this thread. */
const char *bitlinear_last_error(void);

/* Thread-local name of the kernel(s) the last successful call on this thread
 * launched, e.g. "decode_dot4_dense_lpr8_u5_p1" or
 * "gemm_dense_dma_256x256_w8_s4"; "none" after an M == 0 no-op. */
const char *bitlinear_last_dispatch(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
