/*
 * bitlinear_oracle.c -- plain, slow, obviously-correct CPU oracle for the
 * BitNet b1.58 BitLinear forward pass and its Sparse-BitNet N:M variant.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the GPU results are
 * compared against, not the product: only
 * the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * load it.  It shares no code, header, table or constant generator with the
 * HIP library; the packed byte layout is re-implemented here from its written
 * specification.
 *
 * Build: gcc -O2 -std=c99 -fno-fast-math -ffp-contract=off -fPIC -shared
 * (no FMA contraction, IEEE binary32/binary64 arithmetic, round-to-nearest-even
 * mode, which is the C default).
 *
 * Sources, cited by page and section:
 *  [2B4T]  "BitNet b1.58 2B4T Technical Report 요약 설명" (greeksharifa), sec. 2
 *          Architecture: absmean ternary weights, per-token absmax 8-bit
 *          activations; sec. 5.1 GPU Inference: four ternary weights per int8.
 *  [SURV]  "BitNet 논문 분석: 1-Bit LLM의 시대" (youngju.dev), section
 *          "Absmean 양자화 함수" (weight_quant_ternary, BitLinear_b158 with
 *          activation_quant and the integer linear + rescale), and section
 *          "bitnet.cpp 추론 프레임워크" (I2_S 2-bit code: 00 = -1, 01 = 0,
 *          10 = +1, sixteen weights per 32-bit word).
 *  [SPARSE] "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to
 *          Semi-Structured Sparsity" (manon006 review), sec. 3.2: the N:M mask
 *          keeps the N largest |master weight| per block of M, applied after
 *          ternarisation (quant-then-mask).
 *  [V2]    The BitNet v2 summary (brain.hanbit.co.kr): the H-BitLinear applies
 *          an online Hadamard transform to the activations, then quantises
 *          them to 4 bits.
 *  [A48]   [SURV], section "BitNet a4.8: 하이브리드 양자화 전략": the largest
 *          activation values are split off and kept at 8 bits, the rest is
 *          quantised to 4 bits, each part with its own scale.
 *
 * Readings where the pages are silent or disagree (each one is listed in the
 * design notes of the repository):
 *  - activation scale 127/max|x| with no epsilon, s computed once per row and
 *    multiplied in (the [SURV] listing uses 128/(max|x|+1e-5));
 *  - round half to even everywhere (torch.round semantics);
 *  - beta accumulated in binary64 as per-row sums over k ascending, then those
 *    row sums over n ascending, then divided by N*K and rounded to binary32;
 *  - d = fl32(beta + 1e-5f); the weight dequant scale is beta itself;
 *  - N:M groups run along K (the input dimension); ties keep the lower k;
 *  - a row with max|x| = 0 quantises to zeros with x_scale = 0;
 *  - the gated feed-forward input is ReLU(gate)^2 * up, in binary32;
 *  - RMSNorm: eps inside the square root, mean over the K inputs, sum of
 *    squares in binary64; its 1/rms factor is applied to the scale, not to
 *    the row before the codes are taken (it divides out of the codes);
 *  - H-BitLinear: a block-diagonal Sylvester Hadamard transform (blocks of a
 *    power of two B dividing K) in the radix-2 butterfly order, 4-bit absmax
 *    codes 7/max|v| stored in int8, 1/sqrt(B) applied to the scale;
 *  - a4.8: the caller gives the number T of outliers per token row (the
 *    page gives no fraction); they are the T largest |x| of the row, equal
 *    magnitudes resolved towards the lower k; each part gets its own
 *    per-row absmax scale (the page's per-channel scaling, read as one scale
 *    per part and token row: a scale per input channel would not factor out
 *    of the integer contraction with a per-tensor weight scale).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENONFINITE (-5)

/* ------------------------------------------------------------------------ */
/* Step 1: beta = mean |W| over the whole N x K tensor ([SURV] absmean;      */
/* [2B4T] sec. 2).  Binary64 accumulation: sum_n ( sum_k |W[n,k]| ).          */
/* ------------------------------------------------------------------------ */
int oracle_absmean(const float *W, int64_t N, int64_t K, float *beta_out)
{
    if (!W || !beta_out || N < 1 || K < 1) return OR_EINVAL;
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double row = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            float w = W[n * K + k];
            if (!isfinite(w)) return OR_ENONFINITE;
            row += fabs((double)w);
        }
        total += row;
    }
    double mean = total / (double)(N * K);
    *beta_out = (float)mean;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Steps 2-3: d = fl32(beta + 1e-5); t = clamp(round(W / d), -1, 1)          */
/* ([SURV] weight_quant_ternary).  Division and rounding in binary32.         */
/* ------------------------------------------------------------------------ */
int oracle_ternarize(const float *W, int64_t count, float beta, int8_t *t)
{
    if (!W || !t || count < 0) return OR_EINVAL;
    float d = beta + 1e-5f;
    for (int64_t i = 0; i < count; ++i) {
        float r = rintf(W[i] / d);
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        t[i] = (int8_t)r;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 4: N:M keep mask ([SPARSE] sec. 3.2).  Within each group of M        */
/* consecutive inputs of one output row, keep the N entries of largest       */
/* |W| (latent weight, not the ternary value).  Equal magnitudes: the lower  */
/* index wins.  Selection is done the plain way: N rounds, each picking the  */
/* largest not-yet-kept entry, scanning k upwards with a strict '>'.         */
/* n == m means dense (everything kept).                                     */
/* ------------------------------------------------------------------------ */
int oracle_nm_keep(const float *W, int64_t N, int64_t K, int n, int m, uint8_t *keep)
{
    if (!W || !keep || N < 0 || K < 0 || m < 1 || n < 0 || n > m || K % m) return OR_EINVAL;
    for (int64_t r = 0; r < N; ++r) {
        for (int64_t g = 0; g < K / m; ++g) {
            const float *w = W + r * K + g * m;
            uint8_t *kp = keep + r * K + g * m;
            for (int i = 0; i < m; ++i) kp[i] = 0;
            for (int round = 0; round < n; ++round) {
                int best = -1;
                float best_mag = 0.0f;
                for (int i = 0; i < m; ++i) {
                    if (kp[i]) continue;
                    float mag = fabsf(w[i]);
                    if (best < 0 || mag > best_mag) { best = i; best_mag = mag; }
                }
                kp[best] = 1;
            }
        }
    }
    return OR_OK;
}

/* W_eff = t on kept positions, 0 elsewhere (quant-then-mask, [SPARSE] 3.2). */
int oracle_apply_mask(const int8_t *t, const uint8_t *keep, int64_t count, int8_t *w_eff)
{
    if (!t || !keep || !w_eff || count < 0) return OR_EINVAL;
    for (int64_t i = 0; i < count; ++i) w_eff[i] = keep[i] ? t[i] : 0;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 5: packed byte layout.                                              */
/*                                                                          */
/* 2-bit code c = t + 1 ([SURV] I2_S: 00 -> -1, 01 -> 0, 10 -> +1), four    */
/* codes per byte ([2B4T] sec. 5.1).  A run of 16 codes j = 0..15 forms one */
/* little-endian 32-bit word with code j at bit 8*(j % 4) + 2*(j / 4).      */
/*                                                                          */
/* Dense:  row r holds its K codes (k ascending) in K/16 words, rows back   */
/*         to back: N*K/4 bytes.                                            */
/* N:M (2:4 or 6:8), two regions in one buffer:                             */
/*   values: row r holds the codes of its kept weights in increasing k,    */
/*           K*n/m codes = K*n/(4m) bytes per row, rows back to back;       */
/*   masks:  after all value rows, K/8 bytes per row.  For m = 4 each group */
/*           g has a 4-bit mask in byte g/2 (even g: low nibble, odd g:     */
/*           high nibble); for m = 8 group g has byte g.  Bit i of a mask   */
/*           set means k = g*m + i is kept.                                 */
/* ------------------------------------------------------------------------ */
static void put_code(uint8_t *words_base, int64_t code_index, unsigned code)
{
    int64_t word = code_index / 16;
    int j = (int)(code_index % 16);
    int bit = 8 * (j % 4) + 2 * (j / 4);
    /* little-endian: bit b of the word lives in byte b/8 at bit b%8 */
    words_base[word * 4 + bit / 8] |= (uint8_t)(code << (bit % 8));
}

int64_t oracle_packed_bytes(int64_t N, int64_t K, int n, int m)
{
    if (N < 1 || K < 1 || K % 64) return -1;
    if (n == 0 && m == 0) return N * K / 4;
    if (n == 2 && m == 4) return N * (K / 8) + N * (K / 8);
    if (n == 6 && m == 8) return N * (3 * K / 16) + N * (K / 8);
    return -1;
}

/* dense pack of ternary values t (N x K, row-major) */
int oracle_pack_dense(const int8_t *t, int64_t N, int64_t K, uint8_t *out)
{
    if (!t || !out || N < 1 || K < 1 || K % 64) return OR_EINVAL;
    memset(out, 0, (size_t)(N * K / 4));
    for (int64_t r = 0; r < N; ++r)
        for (int64_t k = 0; k < K; ++k) {
            int v = t[r * K + k];
            if (v < -1 || v > 1) return OR_EINVAL;
            put_code(out + r * (K / 4), k, (unsigned)(v + 1));
        }
    return OR_OK;
}

/* N:M pack of ternary values t with keep mask (exactly n kept per group) */
int oracle_pack_nm(const int8_t *t, const uint8_t *keep, int64_t N, int64_t K,
                   int n, int m, uint8_t *out)
{
    int64_t total = oracle_packed_bytes(N, K, n, m);
    if (!t || !keep || !out || total < 0 || n == 0) return OR_EINVAL;
    memset(out, 0, (size_t)total);
    int64_t vrow = K * n / m / 4;       /* value bytes per row */
    int64_t mrow = K / 8;               /* mask bytes per row  */
    uint8_t *values = out;
    uint8_t *masks = out + N * vrow;
    for (int64_t r = 0; r < N; ++r) {
        int64_t kept = 0;
        for (int64_t g = 0; g < K / m; ++g) {
            unsigned mask = 0;
            int count = 0;
            for (int i = 0; i < m; ++i) {
                int64_t k = g * m + i;
                if (!keep[r * K + k]) continue;
                int v = t[r * K + k];
                if (v < -1 || v > 1) return OR_EINVAL;
                put_code(values + r * vrow, kept, (unsigned)(v + 1));
                kept++;
                count++;
                mask |= 1u << i;
            }
            if (count != n) return OR_EINVAL;
            if (m == 4)
                masks[r * mrow + g / 2] |= (uint8_t)(mask << (4 * (g % 2)));
            else
                masks[r * mrow + g] = (uint8_t)mask;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* 2:4 trit pack: the 2:4 weights in 6 bits per group of 4 ([SPARSE] sec.  */
/* 3.2 keeps 2 of every 4; [SURV] section "I2_S 커널의 내부 동작": TL2      */
/* indexes a pair of ternary weights by its 3 x 3 = 9 combinations).  A    */
/* group keeps exactly two inputs i0 < i1; its code is                     */
/*   9 p + 3 (t[i0] + 1) + (t[i1] + 1)   (0 .. 53),                         */
/* p the index of (i0, i1) in the list (0,1) (0,2) (0,3) (1,2) (1,3) (2,3). */
/* The 16 groups of 64 consecutive inputs form one 96-bit little-endian    */
/* string, group g at bits 6 g .. 6 g + 5 (12 bytes); row r holds its      */
/* K / 64 strings in k order, rows back to back: 3 N K / 16 bytes.         */
/* ------------------------------------------------------------------------ */
static const int kPairLo[6] = {0, 0, 0, 1, 1, 2};
static const int kPairHi[6] = {1, 2, 3, 2, 3, 3};

int64_t oracle_packed_bytes_trit24(int64_t N, int64_t K)
{
    if (N < 1 || K < 1 || K % 64) return -1;
    return N * (3 * K / 16);
}

int oracle_pack_trit24(const int8_t *t, const uint8_t *keep, int64_t N, int64_t K, uint8_t *out)
{
    int64_t total = oracle_packed_bytes_trit24(N, K);
    if (!t || !keep || !out || total < 0) return OR_EINVAL;
    memset(out, 0, (size_t)total);
    for (int64_t r = 0; r < N; ++r) {
        uint8_t *row = out + r * (3 * K / 16);
        for (int64_t g = 0; g < K / 4; ++g) {
            int kept[4], nk = 0;
            for (int i = 0; i < 4; ++i)
                if (keep[r * K + 4 * g + i]) {
                    if (nk == 2) return OR_EINVAL;
                    kept[nk++] = i;
                }
            if (nk != 2) return OR_EINVAL;
            int p = -1;
            for (int j = 0; j < 6; ++j)
                if (kPairLo[j] == kept[0] && kPairHi[j] == kept[1]) p = j;
            int v0 = t[r * K + 4 * g + kept[0]], v1 = t[r * K + 4 * g + kept[1]];
            if (p < 0 || v0 < -1 || v0 > 1 || v1 < -1 || v1 > 1) return OR_EINVAL;
            unsigned code = (unsigned)(9 * p + 3 * (v0 + 1) + (v1 + 1));
            /* group g of string s = g / 16 at bit 6 (g % 16) of that string */
            int64_t bit = (g / 16) * 96 + 6 * (g % 16);
            for (int b = 0; b < 6; ++b)
                if (code & (1u << b)) row[(bit + b) / 8] |= (uint8_t)(1u << ((bit + b) % 8));
        }
    }
    return OR_OK;
}

/* The ternary matrix the trit-packed bytes hold (pruned positions 0). */
int oracle_unpack_trit24(const uint8_t *packed, int64_t N, int64_t K, int8_t *w_eff)
{
    if (!packed || !w_eff || oracle_packed_bytes_trit24(N, K) < 0) return OR_EINVAL;
    for (int64_t r = 0; r < N; ++r) {
        const uint8_t *row = packed + r * (3 * K / 16);
        for (int64_t g = 0; g < K / 4; ++g) {
            int64_t bit = (g / 16) * 96 + 6 * (g % 16);
            unsigned code = 0;
            for (int b = 0; b < 6; ++b)
                code |= (unsigned)((row[(bit + b) / 8] >> ((bit + b) % 8)) & 1u) << b;
            if (code > 53) return OR_EINVAL;
            int p = (int)code / 9, v = (int)code % 9;
            for (int i = 0; i < 4; ++i) w_eff[r * K + 4 * g + i] = 0;
            w_eff[r * K + 4 * g + kPairLo[p]] = (int8_t)(v / 3 - 1);
            w_eff[r * K + 4 * g + kPairHi[p]] = (int8_t)(v % 3 - 1);
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 6: per-token absmax int8 activation quantisation ([SURV]            */
/* activation_quant; [2B4T] sec. 2).  g = max_k |x|; s = fl32(127/g);       */
/* q = clamp(round(fl32(x*s)), -128, 127); x_scale = fl32(g/127);           */
/* rowsum = sum_k q.  variant = 1 selects the form printed in the [SURV]    */
/* listing instead: q = clamp(round(fl32(fl32(x*128) / fl32(g + 1e-5))),    */
/* -128, 127) and x_scale = g / 128 (kept only to show the difference).     */
/* ------------------------------------------------------------------------ */
int oracle_quant_act(const float *X, int64_t M, int64_t K, int variant,
                     int8_t *q, float *x_scale, int32_t *rowsum)
{
    if (!X || !q || !x_scale || M < 0 || K < 1) return OR_EINVAL;
    for (int64_t r = 0; r < M; ++r) {
        const float *x = X + r * K;
        float g = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(x[k])) return OR_ENONFINITE;
            float a = fabsf(x[k]);
            if (a > g) g = a;
        }
        int32_t sum = 0;
        if (variant == 0) {
            if (g == 0.0f) {
                for (int64_t k = 0; k < K; ++k) q[r * K + k] = 0;
                x_scale[r] = 0.0f;
            } else {
                /* A row whose max|x| is below 2^-100 is scaled by 2^100 first:
                 * fl32(127/g) overflows to +inf once g < 127/FLT_MAX, which
                 * would turn x*s into +-inf, or NaN where x = 0.  Multiplying
                 * by a power of two is exact here (|x| <= g), so q is the one
                 * the unscaled formula gives wherever its s is finite. */
                const float up = (g < 0x1p-100f) ? 0x1p100f : 1.0f;
                float s = 127.0f / (g * up);
                for (int64_t k = 0; k < K; ++k) {
                    float v = rintf((x[k] * up) * s);
                    if (v > 127.0f) v = 127.0f;
                    if (v < -128.0f) v = -128.0f;
                    q[r * K + k] = (int8_t)v;
                    sum += (int32_t)v;
                }
                x_scale[r] = g / 127.0f;
            }
        } else {
            float den = g + 1e-5f;
            for (int64_t k = 0; k < K; ++k) {
                float v = rintf((x[k] * 128.0f) / den);
                if (v > 127.0f) v = 127.0f;
                if (v < -128.0f) v = -128.0f;
                q[r * K + k] = (int8_t)v;
                sum += (int32_t)v;
            }
            x_scale[r] = g / 128.0f;
        }
        if (rowsum) rowsum[r] = sum;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 6b: the row a BitLinear quantises when its input is transformed     */
/* first (the steps either side of the linear in a BitNet block).           */
/*                                                                          */
/* ReLU^2 gate ([2B4T] sec. 2: the feed-forward network uses squared ReLU;  */
/* with separate gate and up projections the plain reading is              */
/* h = ReLU(gate)^2 * up, elementwise, in binary32):                        */
/*     h[k] = fl32( fl32(r * r) * up[k] ),   r = max(x[k], 0)               */
/* Without `up` the row is used as it is: h = x.                            */
/*                                                                          */
/* RMSNorm before the quantiser ([SURV] BitLinear_b158: the input passes    */
/* through an RMSNorm over the in-features, then activation_quant; [2B4T]   */
/* sec. 2 names subln):  xhat[k] = h[k] * rinv * gamma[k],                  */
/*     rinv = 1 / sqrt( (sum_k h[k]^2) / K + eps )                          */
/* with the sum in binary64, k ascending (each square is exact there).      */
/* The absmax codes of xhat are those of v[k] = fl32(h[k] * gamma[k]): the  */
/* positive per-row factor rinv divides out of xhat / max|xhat|.  So the    */
/* codes are quantised from v exactly as in step 6, and rinv goes into the  */
/* scale:  x_scale = fl32( (double)max|v| / 127 * rinv )  (0 for a zero     */
/* row).  Without gamma, step 6 applies to h unchanged.                     */
/* ------------------------------------------------------------------------ */
int oracle_quant_act_ex(const float *X, const float *up, const float *gamma, float eps,
                        int64_t M, int64_t K, int8_t *q, float *x_scale, int32_t *rowsum)
{
    if (!X || !q || !x_scale || M < 0 || K < 1 || !(eps >= 0.0f)) return OR_EINVAL;
    float *v = (float *)malloc((size_t)K * sizeof(float));
    if (!v) return OR_EINVAL;
    int rc = OR_OK;
    for (int64_t r = 0; r < M && rc == OR_OK; ++r) {
        const float *x = X + r * K;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(x[k]) || (up && !isfinite(up[r * K + k])) || (gamma && !isfinite(gamma[k]))) {
                rc = OR_ENONFINITE;
                break;
            }
            if (up) {
                float relu = x[k] > 0.0f ? x[k] : 0.0f;
                float sq = relu * relu;
                v[k] = sq * up[r * K + k];
            } else {
                v[k] = x[k];
            }
        }
        if (rc != OR_OK) break;
        double rinv = 1.0;
        if (gamma) {
            double ss = 0.0;
            for (int64_t k = 0; k < K; ++k) ss += (double)v[k] * (double)v[k];
            rinv = 1.0 / sqrt(ss / (double)K + (double)eps);
            for (int64_t k = 0; k < K; ++k) v[k] = v[k] * gamma[k];
        }
        rc = oracle_quant_act(v, 1, K, 0, q + r * K, x_scale + r, rowsum ? rowsum + r : NULL);
        if (rc == OR_OK && gamma) {
            float g = 0.0f;
            for (int64_t k = 0; k < K; ++k)
                if (fabsf(v[k]) > g) g = fabsf(v[k]);
            x_scale[r] = (g == 0.0f) ? 0.0f : (float)((double)g / 127.0 * rinv);
        }
    }
    free(v);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Step 6c: 4-bit activations after an online Hadamard transform            */
/* ("BitNet v2" summary (brain.hanbit.co.kr), the H-BitLinear: the          */
/* activations entering a projection are Hadamard-transformed online, then  */
/* quantised to 4 bits, then the linear runs).                              */
/*                                                                          */
/* The transform is block-diagonal: blocks of B consecutive inputs (B a    */
/* power of two dividing K), each multiplied by the Sylvester Hadamard      */
/* matrix H_B (entries +-1) and by 1/sqrt(B), which makes it orthonormal.   */
/* H_B x is formed with the radix-2 butterflies in the standard order: for  */
/* h = 1, 2, 4, ..., B/2, every pair (i, i + h) with i & h == 0 becomes     */
/* (a + b, a - b) in binary32.  Each output of a stage depends on two       */
/* inputs only, so this fixes every rounding.                               */
/* Then 4-bit absmax: g = max|v|, s = fl32(7 / g) (same tiny-row rule as    */
/* step 6), q = clamp(rne(fl32(v * s)), -8, 7).  The factor 1/sqrt(B) is    */
/* positive and common to the row, so it divides out of the codes; it goes  */
/* into the scale: x_scale = fl32( (double)g / 7 / sqrt(B) ).  The codes    */
/* are stored one per int8.                                                 */
/* ------------------------------------------------------------------------ */
int oracle_hadamard_rows(float *X, int64_t M, int64_t K, int64_t B)
{
    if (!X || M < 0 || K < 1 || B < 1 || (B & (B - 1)) || K % B) return OR_EINVAL;
    for (int64_t r = 0; r < M; ++r)
        for (int64_t b0 = 0; b0 < K; b0 += B) {
            float *v = X + r * K + b0;
            for (int64_t h = 1; h < B; h *= 2)
                for (int64_t i = 0; i < B; ++i) {
                    if (i & h) continue;
                    float a = v[i], c = v[i + h];
                    v[i] = a + c;
                    v[i + h] = a - c;
                }
        }
    return OR_OK;
}

int oracle_quant_act_h4(const float *X, int64_t M, int64_t K, int64_t B,
                        int8_t *q, float *x_scale, int32_t *rowsum)
{
    if (!X || !q || !x_scale || M < 0 || K < 1 || B < 1 || (B & (B - 1)) || K % B) return OR_EINVAL;
    float *v = (float *)malloc((size_t)K * sizeof(float));
    if (!v) return OR_EINVAL;
    int rc = OR_OK;
    for (int64_t r = 0; r < M && rc == OR_OK; ++r) {
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(X[r * K + k])) { rc = OR_ENONFINITE; break; }
            v[k] = X[r * K + k];
        }
        if (rc != OR_OK) break;
        oracle_hadamard_rows(v, 1, K, B);
        float g = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(v[k])) { rc = OR_ENONFINITE; break; }
            if (fabsf(v[k]) > g) g = fabsf(v[k]);
        }
        if (rc != OR_OK) break;
        int32_t sum = 0;
        if (g == 0.0f) {
            for (int64_t k = 0; k < K; ++k) q[r * K + k] = 0;
            x_scale[r] = 0.0f;
        } else {
            const float pre = (g < 0x1p-100f) ? 0x1p100f : 1.0f;
            float s = 7.0f / (g * pre);
            for (int64_t k = 0; k < K; ++k) {
                float c = rintf((v[k] * pre) * s);
                if (c > 7.0f) c = 7.0f;
                if (c < -8.0f) c = -8.0f;
                q[r * K + k] = (int8_t)c;
                sum += (int32_t)c;
            }
            x_scale[r] = (float)((double)g / 7.0 / sqrt((double)B));
        }
        if (rowsum) rowsum[r] = sum;
    }
    free(v);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Step 6d: BitNet a4.8's hybrid activations ([A48]: the top values of the  */
/* activation tensor are separated and handled at 8 bits, the rest is       */
/* quantised to 4 bits, each part with its own scale).                      */
/*                                                                          */
/* For each token row x (K values) and a caller-given outlier count T:      */
/*  - S = the T largest |x[k]|, found the plain way: T rounds, each taking   */
/*    the largest not-yet-taken entry, scanning k upwards with a strict '>' */
/*    (equal magnitudes: the lower k wins);                                 */
/*  - hi = x on S, 0 elsewhere; lo = x off S, 0 on S (hi + lo = x);          */
/*  - hi takes the 8-bit quantiser of step 6 (codes in [-127, 127],         */
/*    x_scale = max|hi| / 127);                                             */
/*  - lo takes the 4-bit absmax quantiser: g = max|lo|, s = fl32(7 / g)     */
/*    (same tiny-row rule as step 6), q = rne(fl32(lo * s)) in [-7, 7],      */
/*    x_scale = fl32(g / 7); a zero part quantises to zeros with scale 0.   */
/* Outputs: 2M rows, row 2m the hi codes of token m, row 2m+1 its lo codes, */
/* with their scales and row sums; sel (optional, M x K) marks S.  The      */
/* linear then runs on the 2M rows, and output m is the sum of rows 2m and  */
/* 2m+1 of the rescaled result: y = beta (x_hi acc_hi + x_lo acc_lo).        */
/* ------------------------------------------------------------------------ */
static void quant4_row(const float *v, int64_t K, int8_t *q, float *x_scale, int32_t *rowsum)
{
    float g = 0.0f;
    for (int64_t k = 0; k < K; ++k)
        if (fabsf(v[k]) > g) g = fabsf(v[k]);
    int32_t sum = 0;
    if (g == 0.0f) {
        for (int64_t k = 0; k < K; ++k) q[k] = 0;
        *x_scale = 0.0f;
    } else {
        const float pre = (g < 0x1p-100f) ? 0x1p100f : 1.0f;
        float s = 7.0f / (g * pre);
        for (int64_t k = 0; k < K; ++k) {
            float c = rintf((v[k] * pre) * s);
            if (c > 7.0f) c = 7.0f;
            if (c < -7.0f) c = -7.0f;
            q[k] = (int8_t)c;
            sum += (int32_t)c;
        }
        *x_scale = g / 7.0f;
    }
    if (rowsum) *rowsum = sum;
}

int oracle_quant_act_a48(const float *X, int64_t M, int64_t K, int64_t T, int8_t *q, float *x_scale,
                         int32_t *rowsum, uint8_t *sel)
{
    if (!X || !q || !x_scale || M < 0 || K < 1 || T < 0 || T > K) return OR_EINVAL;
    float *hi = (float *)malloc((size_t)K * sizeof(float));
    float *lo = (float *)malloc((size_t)K * sizeof(float));
    uint8_t *taken = (uint8_t *)malloc((size_t)K);
    if (!hi || !lo || !taken) {
        free(hi);
        free(lo);
        free(taken);
        return OR_EINVAL;
    }
    int rc = OR_OK;
    for (int64_t r = 0; r < M && rc == OR_OK; ++r) {
        const float *x = X + r * K;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(x[k])) { rc = OR_ENONFINITE; break; }
            taken[k] = 0;
        }
        if (rc != OR_OK) break;
        for (int64_t round = 0; round < T; ++round) {
            int64_t best = -1;
            float best_mag = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                if (taken[k]) continue;
                float mag = fabsf(x[k]);
                if (best < 0 || mag > best_mag) {
                    best = k;
                    best_mag = mag;
                }
            }
            taken[best] = 1;
        }
        for (int64_t k = 0; k < K; ++k) {
            hi[k] = taken[k] ? x[k] : 0.0f;
            lo[k] = taken[k] ? 0.0f : x[k];
            if (sel) sel[r * K + k] = taken[k];
        }
        rc = oracle_quant_act(hi, 1, K, 0, q + (2 * r) * K, x_scale + 2 * r, rowsum ? rowsum + 2 * r : NULL);
        quant4_row(lo, K, q + (2 * r + 1) * K, x_scale + 2 * r + 1, rowsum ? rowsum + 2 * r + 1 : NULL);
    }
    free(hi);
    free(lo);
    free(taken);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Steps 7-8: acc[m,n] = sum_k q[m,k] * W_eff[n,k] (exact, int64), and      */
/* Y[m,n] = acc * beta * x_scale[m] in binary64 ([SURV] BitLinear_b158      */
/* forward: integer linear, then rescale by weight and activation scales).  */
/* acc is written as int32 after checking |acc| <= 128*K.                   */
/* ------------------------------------------------------------------------ */
int oracle_forward(const int8_t *q, const float *x_scale, const int8_t *w_eff,
                   float beta, int64_t M, int64_t N, int64_t K,
                   int32_t *acc, double *Y)
{
    if (!q || !x_scale || !w_eff || M < 0 || N < 1 || K < 1) return OR_EINVAL;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)q[m * K + k] * (int64_t)w_eff[n * K + k];
            if (s > 128 * K || s < -128 * K) return OR_EINVAL;
            if (acc) acc[m * N + n] = (int32_t)s;
            if (Y) Y[m * N + n] = (double)s * (double)beta * (double)x_scale[m];
        }
    return OR_OK;
}
