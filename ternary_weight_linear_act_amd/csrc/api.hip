// C ABI of libbitlinear (include/bitlinear.h): argument validation, status
// codes, thread-local error/dispatch strings and kernel dispatch.
//
// Every check runs on the host before anything is launched, so a rejected
// call touches neither the GPU nor the HIP runtime.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "kernels.hpp"
#include "fused_impl.hpp"

namespace bl {

hipError_t launch_fused_forward(const float *X, int64_t M, int64_t K, Pattern p, FusedProjArgs args,
                                float *x_scale, hipStream_t stream, const char **name);

hipError_t launch_gemv(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                       const float *w_scale, Pattern p, int64_t M, int64_t N, int64_t K, float *Y,
                       int32_t *acc, hipStream_t stream);
hipError_t launch_gemm(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                       const float *w_scale, Pattern p, int64_t M, int64_t N, int64_t K, float *Y,
                       int32_t *acc, hipStream_t stream, const char **name);

hipError_t launch_skinny_forward(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                                 const float *w_scale, Pattern p, int64_t M, int64_t N, int64_t K, float *Y,
                                 int32_t *acc, hipStream_t stream, const char **name);

hipError_t launch_decode_dot4(const float *X, const int8_t *Xq, const float *xs, const int32_t *rs,
                              int64_t M, int64_t K, Pattern p, FusedProjArgs args, float *x_scale_out,
                              const ActTransform &tr, hipStream_t stream, const char **name);

// Largest M served by the dot4 GEMV (the fallback when the skinny MFMA kernel
// has no configuration for the shape); larger M runs on the MFMA GEMM.
constexpr int64_t kGemvMaxM = 4;

hipError_t launch_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                          const uint8_t *packed, const float *w_scale, Pattern p, int64_t M,
                          int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream,
                          const char **name)
{
    static const char *gemv_names[3] = {"gemv_dense", "gemv_nm24", "gemv_nm68"};
    const int pi = (int)p;
    if (M == 1) {
        FusedProjArgs one = {};
        one.nproj = 1;
        one.packed[0] = packed;
        one.w_scale[0] = w_scale;
        one.Y[0] = Y;
        one.acc[0] = acc;
        one.N[0] = N;
        const hipError_t e = launch_decode_dot4(nullptr, Xq, x_scale, x_rowsum, M, K, p, one, nullptr,
                                                ActTransform{nullptr, nullptr, 0.0f}, stream, name);
        if (e != hipErrorNotSupported) return e;
    }
    // 2:4 at 2-16 tokens on the sparse MFMA where it measured at least as fast
    // as the 16x16x64 kernel on dense codes: K <= 4096 (8960 x 1536, 6912 x
    // 2560: 5.6-6.7 against 5.9-6.7 us at 2-8 tokens; 1000 x 640: 3.2 against
    // 4.6-5.1 us), and any K past 8 tokens (6912 x 2560 at 16: 7.6 against
    // 10.9 us; 2560 x 6912 at 16: 9.2 against 16.4 us)
    if (p == Pattern::NM24 && M >= 2 && M <= 16 && (K <= 4096 || M > 8)) {
        const hipError_t e = launch_skinny_nm24_smfmac(Xq, x_scale, packed, w_scale, M, N, K, Y, acc, stream);
        if (e != hipErrorNotSupported) {
            *name = "skinny_smfmac_nm24";
            return e;
        }
    }
    // 17-64 tokens: the skinny kernel in tiles of 16 tokens where the tiles
    // make at most 512 workgroups (few weight rows: 2048 x 2048 at 64 tokens
    // 8.2 -> 4.2 us, 2048 x 256 9.2 -> 3.5 us); with more, the GEMM is faster
    // (2048 x 11008 at 64 tokens: 10.1 against 17.3 us)
    if (M <= 16 || (M <= kSkinnyMaxM && ((N + 15) / 16) * ((M + 15) / 16) <= 512)) {
        const hipError_t e = launch_skinny_forward(Xq, x_scale, x_rowsum, packed, w_scale, p, M, N, K, Y, acc,
                                                   stream, name);
        if (e != hipErrorNotSupported) return e;
    }
    if (M <= kGemvMaxM) {
        *name = gemv_names[pi];
        return launch_gemv(Xq, x_scale, x_rowsum, packed, w_scale, p, M, N, K, Y, acc, stream);
    }
    return launch_gemm(Xq, x_scale, x_rowsum, packed, w_scale, p, M, N, K, Y, acc, stream, name);
}

}  // namespace bl

namespace {

thread_local char g_error[512] = "";
thread_local char g_dispatch[128] = "";

constexpr int64_t kMaxK = 1048576;
constexpr int64_t kMaxN = 16777216;
constexpr int64_t kMaxM = 16777216;

bitlinear_status fail(bitlinear_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return st;
}

bitlinear_status hip_fail(const char *what, hipError_t e)
{
    return fail(BITLINEAR_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

void set_dispatch(const char *s) { snprintf(g_dispatch, sizeof g_dispatch, "%s", s); }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bitlinear_status check_nm(bitlinear_nm nm, bl::Pattern *p)
{
    if (nm.n == 0 && nm.m == 0) { *p = bl::Pattern::Dense; return BITLINEAR_OK; }
    if (nm.n == 2 && nm.m == 4) { *p = bl::Pattern::NM24; return BITLINEAR_OK; }
    if (nm.n == 6 && nm.m == 8) { *p = bl::Pattern::NM68; return BITLINEAR_OK; }
    return fail(BITLINEAR_EUNSUPPORTED, "N:M pattern %d:%d is not supported (use 0:0, 2:4 or 6:8)", nm.n, nm.m);
}

bitlinear_status check_k(int64_t K)
{
    if (K < 64 || K > kMaxK || K % 64 != 0)
        return fail(BITLINEAR_EINVAL, "K = %lld must be a multiple of 64 in [64, %lld]", (long long)K,
                    (long long)kMaxK);
    return BITLINEAR_OK;
}

bitlinear_status check_n(int64_t N)
{
    if (N < 1 || N > kMaxN) return fail(BITLINEAR_EINVAL, "N = %lld must be in [1, %lld]", (long long)N, (long long)kMaxN);
    return BITLINEAR_OK;
}

bitlinear_status check_m(int64_t M)
{
    if (M < 0 || M > kMaxM) return fail(BITLINEAR_EINVAL, "M = %lld must be in [0, %lld]", (long long)M, (long long)kMaxM);
    return BITLINEAR_OK;
}

bitlinear_status check_ptr(const void *p, uintptr_t align, const char *name)
{
    if (!p) return fail(BITLINEAR_EINVAL, "%s must not be NULL", name);
    if (!aligned(p, align)) return fail(BITLINEAR_EINVAL, "%s must be %u-byte aligned", name, (unsigned)align);
    return BITLINEAR_OK;
}

// The row transform: NULL or an all-NULL struct is none.
bitlinear_status check_transform(const bitlinear_act_transform *tr, bl::ActTransform *out)
{
    *out = bl::ActTransform{nullptr, nullptr, 0.0f};
    if (!tr) return BITLINEAR_OK;
    if (tr->up && !aligned(tr->up, 16)) return fail(BITLINEAR_EINVAL, "tr->up must be 16-byte aligned");
    if (tr->gamma) {
        if (!aligned(tr->gamma, 16)) return fail(BITLINEAR_EINVAL, "tr->gamma must be 16-byte aligned");
        if (!(tr->eps >= 0.0f) || !isfinite(tr->eps))
            return fail(BITLINEAR_EINVAL, "tr->eps must be finite and >= 0");
    }
    *out = bl::ActTransform{tr->up, tr->gamma, tr->gamma ? tr->eps : 0.0f};
    return BITLINEAR_OK;
}

size_t packed_bytes_for(int64_t N, int64_t K, bl::Pattern p)
{
    switch (p) {
    case bl::Pattern::Dense: return (size_t)(N * (K / 4));
    case bl::Pattern::NM24: return (size_t)(N * (K / 8) + N * (K / 8));
    case bl::Pattern::NM68: return (size_t)(N * (3 * K / 16) + N * (K / 8));
    }
    return 0;
}

size_t workspace_bytes_for(int64_t N) { return (size_t)((N * 8 + 255) / 256 * 256); }

#define CHECK(expr)                                   \
    do {                                              \
        bitlinear_status st_ = (expr);                \
        if (st_ != BITLINEAR_OK) return st_;          \
    } while (0)

}  // namespace

extern "C" {

bitlinear_status bitlinear_packed_size(int64_t N, int64_t K, bitlinear_nm nm, size_t *packed_bytes,
                                       size_t *workspace_bytes)
{
    bl::Pattern p;
    CHECK(check_nm(nm, &p));
    CHECK(check_n(N));
    CHECK(check_k(K));
    if (packed_bytes) *packed_bytes = packed_bytes_for(N, K, p);
    if (workspace_bytes) *workspace_bytes = workspace_bytes_for(N);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_pack_weights(const float *W, int64_t N, int64_t K, bitlinear_nm nm, void *packed,
                                        size_t packed_bytes, float *w_scale, void *workspace,
                                        size_t workspace_bytes, hipStream_t stream)
{
    bl::Pattern p;
    CHECK(check_nm(nm, &p));
    CHECK(check_n(N));
    CHECK(check_k(K));
    CHECK(check_ptr(W, 16, "W"));
    CHECK(check_ptr(packed, 16, "packed"));
    CHECK(check_ptr(w_scale, 4, "w_scale"));
    if (packed_bytes < packed_bytes_for(N, K, p))
        return fail(BITLINEAR_ESIZE, "packed buffer has %zu bytes, %zu needed", packed_bytes,
                    packed_bytes_for(N, K, p));
    if (workspace_bytes < workspace_bytes_for(N))
        return fail(BITLINEAR_ESIZE, "workspace has %zu bytes, %zu needed", workspace_bytes,
                    workspace_bytes_for(N));
    CHECK(check_ptr(workspace, 8, "workspace"));

    hipError_t e = bl::launch_absmean(W, N, K, static_cast<double *>(workspace), w_scale, stream);
    if (e != hipSuccess) return hip_fail("absmean launch", e);
    e = bl::launch_pack(W, N, K, p, w_scale, static_cast<uint8_t *>(packed), stream);
    if (e != hipSuccess) return hip_fail("pack launch", e);
    set_dispatch(p == bl::Pattern::Dense ? "absmean+pack_dense"
                 : p == bl::Pattern::NM24 ? "absmean+pack_nm24" : "absmean+pack_nm68");
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *x_scale,
                                     int32_t *x_rowsum, hipStream_t stream)
{
    return bitlinear_quant_act_ex(X, nullptr, M, K, Xq, x_scale, x_rowsum, stream);
}

bitlinear_status bitlinear_quant_act_ex(const float *X, const bitlinear_act_transform *tr, int64_t M,
                                        int64_t K, int8_t *Xq, float *x_scale, int32_t *x_rowsum,
                                        hipStream_t stream)
{
    CHECK(check_m(M));
    CHECK(check_k(K));
    bl::ActTransform t;
    CHECK(check_transform(tr, &t));
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }   // M-sized buffers may be NULL
    CHECK(check_ptr(X, 16, "X"));
    CHECK(check_ptr(Xq, 16, "Xq"));
    CHECK(check_ptr(x_scale, 4, "x_scale"));
    if (x_rowsum && !aligned(x_rowsum, 4)) return fail(BITLINEAR_EINVAL, "x_rowsum must be 4-byte aligned");
    hipError_t e = bl::launch_quant_act_ex(X, t, M, K, Xq, x_scale, x_rowsum, stream);
    if (e != hipSuccess) return hip_fail("quant_act launch", e);
    static const char *names[4] = {"quant_act", "quant_act_gate", "quant_act_norm", "quant_act_gate_norm"};
    set_dispatch(names[(t.up ? 1 : 0) | (t.gamma ? 2 : 0)]);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_quant_act_h4(const float *X, int64_t M, int64_t K, int64_t block, int8_t *Xq,
                                        float *x_scale, int32_t *x_rowsum, hipStream_t stream)
{
    CHECK(check_m(M));
    CHECK(check_k(K));
    if (block < 1 || block > 8192 || (block & (block - 1)) || K % block)
        return fail(BITLINEAR_EINVAL, "block = %lld must be a power of two in [1, 8192] dividing K = %lld",
                    (long long)block, (long long)K);
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }   // M-sized buffers may be NULL
    CHECK(check_ptr(X, 16, "X"));
    CHECK(check_ptr(Xq, 16, "Xq"));
    CHECK(check_ptr(x_scale, 4, "x_scale"));
    if (x_rowsum && !aligned(x_rowsum, 4)) return fail(BITLINEAR_EINVAL, "x_rowsum must be 4-byte aligned");
    const char *name = "";
    hipError_t e = bl::launch_quant_act_h4(X, M, K, block, Xq, x_scale, x_rowsum, stream, &name);
    if (e != hipSuccess) return hip_fail("quant_act_h4 launch", e);
    set_dispatch(name);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                   const void *packed, const float *w_scale, bitlinear_nm nm, int64_t M,
                                   int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream)
{
    bl::Pattern p;
    CHECK(check_nm(nm, &p));
    CHECK(check_m(M));
    CHECK(check_n(N));
    CHECK(check_k(K));
    CHECK(check_ptr(packed, 16, "packed"));
    CHECK(check_ptr(w_scale, 4, "w_scale"));
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }   // M-sized buffers may be NULL
    CHECK(check_ptr(Xq, 16, "Xq"));
    CHECK(check_ptr(x_scale, 4, "x_scale"));
    CHECK(check_ptr(x_rowsum, 4, "x_rowsum"));
    CHECK(check_ptr(Y, 16, "Y"));
    if (acc && !aligned(acc, 16)) return fail(BITLINEAR_EINVAL, "acc must be 16-byte aligned");
    const char *name = "";
    hipError_t e = bl::launch_forward(Xq, x_scale, x_rowsum, static_cast<const uint8_t *>(packed), w_scale, p,
                                      M, N, K, Y, acc, stream, &name);
    if (e != hipSuccess) return hip_fail("forward launch", e);
    set_dispatch(name);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_forward_fused(const float *X, int64_t M, int64_t K, bitlinear_nm nm,
                                         const bitlinear_proj *projs, int32_t nproj, float *x_scale,
                                         hipStream_t stream)
{
    return bitlinear_forward_fused_ex(X, nullptr, M, K, nm, projs, nproj, x_scale, stream);
}

bitlinear_status bitlinear_forward_fused_ex(const float *X, const bitlinear_act_transform *tr, int64_t M,
                                            int64_t K, bitlinear_nm nm, const bitlinear_proj *projs,
                                            int32_t nproj, float *x_scale, hipStream_t stream)
{
    bl::Pattern p;
    CHECK(check_nm(nm, &p));
    CHECK(check_m(M));
    CHECK(check_k(K));
    bl::ActTransform t;
    CHECK(check_transform(tr, &t));
    const bool transformed = t.up || t.gamma;
    if (!projs) return fail(BITLINEAR_EINVAL, "projs must not be NULL");
    if (nproj < 1) return fail(BITLINEAR_EINVAL, "nproj = %d must be >= 1", nproj);
    if (nproj > bl::kMaxFusedProj)
        return fail(BITLINEAR_EUNSUPPORTED, "nproj = %d: at most %d projections per fused call", nproj,
                    bl::kMaxFusedProj);
    bl::FusedProjArgs args = {};
    args.nproj = nproj;
    for (int i = 0; i < nproj; ++i) {
        CHECK(check_n(projs[i].N));
        CHECK(check_ptr(projs[i].packed, 16, "projs[i].packed"));
        CHECK(check_ptr(projs[i].w_scale, 4, "projs[i].w_scale"));
        if (M > 0) CHECK(check_ptr(projs[i].Y, 16, "projs[i].Y"));
        if (projs[i].acc && !aligned(projs[i].acc, 16)) return fail(BITLINEAR_EINVAL, "projs[i].acc must be 16-byte aligned");
        args.packed[i] = static_cast<const uint8_t *>(projs[i].packed);
        args.w_scale[i] = projs[i].w_scale;
        args.N[i] = projs[i].N;
        args.Y[i] = projs[i].Y;
        args.acc[i] = projs[i].acc;
    }
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }
    CHECK(check_ptr(X, 16, "X"));
    if (x_scale && !aligned(x_scale, 4)) return fail(BITLINEAR_EINVAL, "x_scale must be 4-byte aligned");
    const char *name = "";
    hipError_t e = bl::launch_decode_dot4(X, nullptr, nullptr, nullptr, M, K, p, args, x_scale, t, stream, &name);
    if (e == hipErrorNotSupported && transformed)
        return fail(BITLINEAR_EUNSUPPORTED, "fused decode with a row transform supports M == 1 and K <= 16384 "
                    "(M = %lld, K = %lld)", (long long)M, (long long)K);
    if (e == hipErrorNotSupported) e = bl::launch_fused_forward(X, M, K, p, args, x_scale, stream, &name);
    if (e == hipErrorNotSupported)
        return fail(BITLINEAR_EUNSUPPORTED, "fused decode supports 1 <= M <= 4 and K <= %s (M = %lld, K = %lld)",
                    M == 1 ? "65344" : "16192", (long long)M, (long long)K);
    if (e != hipSuccess) return hip_fail("fused forward launch", e);
    set_dispatch(name);
    return BITLINEAR_OK;
}

const char *bitlinear_last_error(void) { return g_error; }

const char *bitlinear_last_dispatch(void) { return g_dispatch; }

}  // extern "C"
