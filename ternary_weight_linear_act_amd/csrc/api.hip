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
                       int32_t *acc, Scratch &scratch, hipStream_t stream, const char **name);

hipError_t launch_skinny_forward(const int8_t *Xq, const float *xs, const int32_t *rs, FusedProjArgs args,
                                 Pattern p, int64_t M, int64_t K, hipStream_t stream, const char **name, bool query);

hipError_t launch_decode_dot4(const float *X, const int8_t *Xq, const float *xs, const int32_t *rs,
                              int64_t M, int64_t K, Pattern p, FusedProjArgs args, float *x_scale_out,
                              const ActTransform &tr, hipStream_t stream, const char **name, bool query);

// Largest M served by the dot4 GEMV (the fallback when the skinny MFMA kernel
// has no configuration for the shape); larger M runs on the MFMA GEMM.
constexpr int64_t kGemvMaxM = 4;

hipError_t launch_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                          const uint8_t *packed, const float *w_scale, Pattern p, int64_t M,
                          int64_t N, int64_t K, float *Y, int32_t *acc, Scratch &scratch,
                          hipStream_t stream, const char **name)
{
    const bool query = scratch.query;
    static const char *gemv_names[3] = {"gemv_dense", "gemv_nm24", "gemv_nm68"};
    const int pi = (int)p;
    FusedProjArgs one = {};
    one.nproj = 1;
    one.packed[0] = packed;
    one.w_scale[0] = w_scale;
    one.Y[0] = Y;
    one.acc[0] = acc;
    one.N[0] = N;
    if (M == 1) {
        const hipError_t e = launch_decode_dot4(nullptr, Xq, x_scale, x_rowsum, M, K, p, one, nullptr,
                                                ActTransform{nullptr, nullptr, 0.0f}, stream, name, query);
        if (e != hipErrorNotSupported) return e;
    }
    // 2:4 at 2-16 tokens on the sparse MFMA where it measured at least as fast
    // as the 16x16x64 kernel on dense codes: K <= 4096 (8960 x 1536, 6912 x
    // 2560: 5.6-6.7 against 5.9-6.7 us at 2-8 tokens; 1000 x 640: 3.2 against
    // 4.6-5.1 us), and any K past 8 tokens (6912 x 2560 at 16: 7.6 against
    // 10.9 us; 2560 x 6912 at 16: 9.2 against 16.4 us)
    if (p == Pattern::NM24 && M >= 2 && M <= 16 && (K <= 4096 || M > 8)) {
        const hipError_t e = launch_skinny_nm24_smfmac(Xq, x_scale, packed, w_scale, M, N, K, Y, acc, stream, query);
        if (e != hipErrorNotSupported) {
            *name = "skinny_smfmac_nm24";
            return e;
        }
    }
    // 9-64 tokens over wide dense projections: several token tiles per
    // workgroup on the direct-load kernel
    if (M >= 9 && M <= kSkinnyMaxM) {
        const hipError_t e = launch_skinny_direct_tiles(Xq, x_scale, x_rowsum, one, p, M, K, stream, name, query);
        if (e != hipErrorNotSupported) return e;
    }
    // 17-64 tokens: the skinny kernel in tiles of 16 tokens where the tiles
    // make at most 512 workgroups (few weight rows: 2048 x 2048 at 64 tokens
    // 8.2 -> 4.2 us, 2048 x 256 9.2 -> 3.5 us); with more, the GEMM is faster
    // (2048 x 11008 at 64 tokens: 10.1 against 17.3 us)
    if (M <= 16 || (M <= kSkinnyMaxM && ((N + 15) / 16) * ((M + 15) / 16) <= 512)) {
        const hipError_t e = launch_skinny_forward(Xq, x_scale, x_rowsum, one, p, M, K, stream, name, query);
        if (e != hipErrorNotSupported) return e;
    }
    // deep K at 9-64 tokens: the token-tile kernel with K split over the
    // workgroups
    if (M >= 9 && M <= kSkinnyMaxM) {
        const hipError_t e = launch_skinny_direct_tiles_split(Xq, x_scale, x_rowsum, packed, w_scale, p, M, N, K, Y,
                                                              acc, scratch, stream, name);
        if (e != hipErrorNotSupported) return e;
    }
    if (M <= kGemvMaxM) {
        *name = gemv_names[pi];
        if (query) return hipSuccess;
        return launch_gemv(Xq, x_scale, x_rowsum, packed, w_scale, p, M, N, K, Y, acc, stream);
    }
    return launch_gemm(Xq, x_scale, x_rowsum, packed, w_scale, p, M, N, K, Y, acc, scratch, stream, name);
}

}  // namespace bl

namespace {

thread_local char g_error[512] = "";
thread_local char g_dispatch[256] = "";

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

size_t packed_bytes_trit24(int64_t N, int64_t K) { return (size_t)(N * (3 * K / 16)); }

size_t workspace_bytes_for(int64_t N) { return (size_t)((N * 8 + 255) / 256 * 256); }

// Workspace bytes of a forward call: the dispatch run as a size query.
size_t forward_need(bl::Pattern p, int64_t M, int64_t N, int64_t K)
{
    if (M == 0) return 0;
    bl::Scratch q;
    q.query = true;
    const char *name = "";
    // a query launches nothing; its status only repeats what validation found
    (void)bl::launch_forward(nullptr, nullptr, nullptr, nullptr, nullptr, p, M, N, K, nullptr, nullptr, q, nullptr,
                             &name);
    return q.need;
}

// The forward launch on validated arguments, with the workspace in
// `scratch`; a workspace short of what the kernels for this shape use is
// BITLINEAR_ESIZE, and then nothing has been launched.
bitlinear_status run_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum, const void *packed,
                             const float *w_scale, bl::Pattern p, int64_t M, int64_t N, int64_t K, float *Y,
                             int32_t *acc, bl::Scratch &scratch, hipStream_t stream)
{
    const char *name = "";
    const hipError_t e = bl::launch_forward(Xq, x_scale, x_rowsum, static_cast<const uint8_t *>(packed), w_scale,
                                            p, M, N, K, Y, acc, scratch, stream, &name);
    if (scratch.need > scratch.bytes)
        return fail(BITLINEAR_ESIZE, "workspace has %zu bytes, %zu needed for M = %lld, N = %lld, K = %lld (%s)",
                    scratch.bytes, scratch.need, (long long)M, (long long)N, (long long)K, name);
    if (e != hipSuccess) return hip_fail("forward launch", e);
    set_dispatch(name);
    return BITLINEAR_OK;
}

#define CHECK(expr)                                   \
    do {                                              \
        bitlinear_status st_ = (expr);                \
        if (st_ != BITLINEAR_OK) return st_;          \
    } while (0)

// The projections of a fused or grouped call, checked and copied into the
// kernels' argument block.
bitlinear_status check_projs(const bitlinear_proj *projs, int32_t nproj, int64_t M, bl::FusedProjArgs *args)
{
    if (!projs) return fail(BITLINEAR_EINVAL, "projs must not be NULL");
    if (nproj < 1) return fail(BITLINEAR_EINVAL, "nproj = %d must be >= 1", nproj);
    if (nproj > bl::kMaxFusedProj)
        return fail(BITLINEAR_EUNSUPPORTED, "nproj = %d: at most %d projections per call", nproj, bl::kMaxFusedProj);
    args->nproj = nproj;
    for (int i = 0; i < nproj; ++i) {
        CHECK(check_n(projs[i].N));
        CHECK(check_ptr(projs[i].packed, 16, "projs[i].packed"));
        CHECK(check_ptr(projs[i].w_scale, 4, "projs[i].w_scale"));
        if (M > 0) CHECK(check_ptr(projs[i].Y, 16, "projs[i].Y"));
        if (projs[i].acc && !aligned(projs[i].acc, 16))
            return fail(BITLINEAR_EINVAL, "projs[i].acc must be 16-byte aligned");
        args->packed[i] = static_cast<const uint8_t *>(projs[i].packed);
        args->w_scale[i] = projs[i].w_scale;
        args->N[i] = projs[i].N;
        args->Y[i] = projs[i].Y;
        args->acc[i] = projs[i].acc;
    }
    return BITLINEAR_OK;
}

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

bitlinear_status bitlinear_pack_weights_masked(const float *W, int64_t N, int64_t K, bitlinear_nm nm, void *packed,
                                               size_t packed_bytes, float *w_scale, void *workspace,
                                               size_t workspace_bytes, hipStream_t stream)
{
    if (nm.n == 0 && nm.m == 0)
        return fail(BITLINEAR_EINVAL, "bitlinear_pack_weights_masked needs an N:M pattern");
    if (!(nm.m == 4 || nm.m == 8 || nm.m == 16) || nm.n < 1 || nm.n > nm.m)
        return fail(BITLINEAR_EUNSUPPORTED, "masked N:M pattern %d:%d: M must be 4, 8 or 16 and 1 <= N <= M", nm.n,
                    nm.m);
    CHECK(check_n(N));
    CHECK(check_k(K));
    CHECK(check_ptr(W, 16, "W"));
    CHECK(check_ptr(packed, 16, "packed"));
    CHECK(check_ptr(w_scale, 4, "w_scale"));
    const size_t need = packed_bytes_for(N, K, bl::Pattern::Dense);
    if (packed_bytes < need) return fail(BITLINEAR_ESIZE, "packed buffer has %zu bytes, %zu needed", packed_bytes, need);
    if (workspace_bytes < workspace_bytes_for(N))
        return fail(BITLINEAR_ESIZE, "workspace has %zu bytes, %zu needed", workspace_bytes, workspace_bytes_for(N));
    CHECK(check_ptr(workspace, 8, "workspace"));
    hipError_t e = bl::launch_absmean(W, N, K, static_cast<double *>(workspace), w_scale, stream);
    if (e != hipSuccess) return hip_fail("absmean launch", e);
    e = bl::launch_pack_nm_dense(W, N, K, nm.n, nm.m, w_scale, static_cast<uint8_t *>(packed), stream);
    if (e != hipSuccess) return hip_fail("pack launch", e);
    snprintf(g_dispatch, sizeof g_dispatch, "absmean+pack_nm%d%d_dense", nm.n, nm.m);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_packed_size_trit24(int64_t N, int64_t K, size_t *packed_bytes, size_t *workspace_bytes)
{
    CHECK(check_n(N));
    CHECK(check_k(K));
    if (packed_bytes) *packed_bytes = packed_bytes_trit24(N, K);
    if (workspace_bytes) *workspace_bytes = workspace_bytes_for(N);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_pack_weights_trit24(const float *W, int64_t N, int64_t K, void *packed,
                                               size_t packed_bytes, float *w_scale, void *workspace,
                                               size_t workspace_bytes, hipStream_t stream)
{
    CHECK(check_n(N));
    CHECK(check_k(K));
    CHECK(check_ptr(W, 16, "W"));
    CHECK(check_ptr(packed, 16, "packed"));
    CHECK(check_ptr(w_scale, 4, "w_scale"));
    if (packed_bytes < packed_bytes_trit24(N, K))
        return fail(BITLINEAR_ESIZE, "packed buffer has %zu bytes, %zu needed", packed_bytes,
                    packed_bytes_trit24(N, K));
    if (workspace_bytes < workspace_bytes_for(N))
        return fail(BITLINEAR_ESIZE, "workspace has %zu bytes, %zu needed", workspace_bytes, workspace_bytes_for(N));
    CHECK(check_ptr(workspace, 8, "workspace"));
    hipError_t e = bl::launch_absmean(W, N, K, static_cast<double *>(workspace), w_scale, stream);
    if (e != hipSuccess) return hip_fail("absmean launch", e);
    e = bl::launch_pack_trit24(W, N, K, w_scale, static_cast<uint8_t *>(packed), stream);
    if (e != hipSuccess) return hip_fail("pack launch", e);
    set_dispatch("absmean+pack_trit24");
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

bitlinear_status bitlinear_quant_act_multi(const bitlinear_quant_group *groups, int32_t ngroups,
                                           hipStream_t stream)
{
    if (!groups) return fail(BITLINEAR_EINVAL, "groups must not be NULL");
    if (ngroups < 1) return fail(BITLINEAR_EINVAL, "ngroups = %d must be >= 1", ngroups);
    if (ngroups > bl::kMaxQuantGroups)
        return fail(BITLINEAR_EUNSUPPORTED, "ngroups = %d: at most %d input groups per call", ngroups,
                    bl::kMaxQuantGroups);
    bl::QuantGroupArgs qa = {};
    for (int g = 0; g < ngroups; ++g) {
        const bitlinear_quant_group &q = groups[g];
        CHECK(check_m(q.M));
        CHECK(check_k(q.K));
        if (q.M > 0) {
            CHECK(check_ptr(q.X, 16, "groups[g].X"));
            CHECK(check_ptr(q.Xq, 16, "groups[g].Xq"));
            CHECK(check_ptr(q.x_scale, 4, "groups[g].x_scale"));
            if (q.x_rowsum && !aligned(q.x_rowsum, 4))
                return fail(BITLINEAR_EINVAL, "groups[g].x_rowsum must be 4-byte aligned");
        }
        qa.X[g] = q.X;
        qa.Xq[g] = q.Xq;
        qa.x_scale[g] = q.x_scale;
        qa.x_rowsum[g] = q.x_rowsum;
        qa.M[g] = q.M;
        qa.K[g] = q.K;
    }
    qa.ngroups = ngroups;
    hipError_t e = bl::launch_quant_act_multi(qa, stream);
    if (e == hipSuccess) { set_dispatch("quant_act_multi"); return BITLINEAR_OK; }
    if (e != hipErrorNotSupported) return hip_fail("quant_act_multi launch", e);
    // one launch per group
    for (int g = 0; g < ngroups; ++g) {
        if (qa.M[g] == 0) continue;
        e = bl::launch_quant_act(qa.X[g], qa.M[g], qa.K[g], qa.Xq[g], qa.x_scale[g], qa.x_rowsum[g], stream);
        if (e != hipSuccess) return hip_fail("quant_act launch", e);
    }
    set_dispatch("quant_act per group");
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

bitlinear_status bitlinear_quant_act_a48(const float *X, int64_t M, int64_t K, int64_t n_outliers, int8_t *Xq,
                                         float *x_scale, int32_t *x_rowsum, hipStream_t stream)
{
    CHECK(check_m(M));
    CHECK(check_k(K));
    if (n_outliers < 0 || n_outliers > K)
        return fail(BITLINEAR_EINVAL, "n_outliers = %lld must be in [0, K = %lld]", (long long)n_outliers,
                    (long long)K);
    if (K > 16384) return fail(BITLINEAR_EUNSUPPORTED, "a4.8 activations support K <= 16384 (K = %lld)", (long long)K);
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }
    CHECK(check_ptr(X, 16, "X"));
    CHECK(check_ptr(Xq, 16, "Xq"));
    CHECK(check_ptr(x_scale, 4, "x_scale"));
    if (x_rowsum && !aligned(x_rowsum, 4)) return fail(BITLINEAR_EINVAL, "x_rowsum must be 4-byte aligned");
    const char *name = "";
    const hipError_t e = bl::launch_quant_act_a48(X, M, K, n_outliers, Xq, x_scale, x_rowsum, stream, &name);
    if (e != hipSuccess) return hip_fail("quant_act_a48 launch", e);
    set_dispatch(name);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_combine_a48(const float *Y2, int64_t M, int64_t N, float *Y, hipStream_t stream)
{
    CHECK(check_m(M));
    CHECK(check_n(N));
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }
    CHECK(check_ptr(Y2, 4, "Y2"));
    CHECK(check_ptr(Y, 4, "Y"));
    const hipError_t e = bl::launch_a48_combine(Y2, M, N, Y, stream);
    if (e != hipSuccess) return hip_fail("combine_a48 launch", e);
    set_dispatch("a48_combine");
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_forward_workspace_size(int64_t M, int64_t N, int64_t K, bitlinear_nm nm,
                                                  size_t *workspace_bytes)
{
    bl::Pattern p;
    CHECK(check_nm(nm, &p));
    CHECK(check_m(M));
    CHECK(check_n(N));
    CHECK(check_k(K));
    if (!workspace_bytes) return fail(BITLINEAR_EINVAL, "workspace_bytes must not be NULL");
    *workspace_bytes = forward_need(p, M, N, K);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                   const void *packed, const float *w_scale, bitlinear_nm nm, int64_t M,
                                   int64_t N, int64_t K, float *Y, int32_t *acc, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream)
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
    if (workspace && !aligned(workspace, 16)) return fail(BITLINEAR_EINVAL, "workspace must be 16-byte aligned");
    bl::Scratch scratch;
    scratch.ptr = static_cast<uint8_t *>(workspace);
    scratch.bytes = workspace ? workspace_bytes : 0;
    return run_forward(Xq, x_scale, x_rowsum, packed, w_scale, p, M, N, K, Y, acc, scratch, stream);
}

bitlinear_status bitlinear_forward_trit24_workspace_size(int64_t M, int64_t N, int64_t K, size_t *workspace_bytes)
{
    CHECK(check_m(M));
    CHECK(check_n(N));
    CHECK(check_k(K));
    if (!workspace_bytes) return fail(BITLINEAR_EINVAL, "workspace_bytes must not be NULL");
    *workspace_bytes = 0;
    if (M == 0) return BITLINEAR_OK;
    bl::Scratch q;
    q.query = true;
    const char *name = "";
    // a query launches nothing; its status only repeats what validation found
    (void)bl::launch_forward_trit24(nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, nullptr, nullptr, q,
                                    nullptr, &name);
    *workspace_bytes = q.need;
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_forward_trit24(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                          const void *packed, const float *w_scale, int64_t M, int64_t N, int64_t K,
                                          float *Y, int32_t *acc, void *workspace, size_t workspace_bytes,
                                          hipStream_t stream)
{
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
    if (workspace && !aligned(workspace, 16)) return fail(BITLINEAR_EINVAL, "workspace must be 16-byte aligned");
    bl::Scratch scratch;
    scratch.ptr = static_cast<uint8_t *>(workspace);
    scratch.bytes = workspace ? workspace_bytes : 0;
    const char *name = "";
    const hipError_t e = bl::launch_forward_trit24(Xq, x_scale, x_rowsum, static_cast<const uint8_t *>(packed),
                                                   w_scale, M, N, K, Y, acc, scratch, stream, &name);
    if (scratch.need > scratch.bytes)
        return fail(BITLINEAR_ESIZE, "workspace has %zu bytes, %zu needed for M = %lld, N = %lld, K = %lld (%s)",
                    scratch.bytes, scratch.need, (long long)M, (long long)N, (long long)K, name);
    if (e != hipSuccess) return hip_fail("forward launch", e);
    set_dispatch(name);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_forward_noalloc(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
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
    const size_t need = forward_need(p, M, N, K);
    if (need > bl::kNoAllocScratchBytes)
        return fail(BITLINEAR_ESIZE, "M = %lld, N = %lld, K = %lld needs %zu bytes of scratch, more than the %zu "
                    "this entry point holds; use bitlinear_forward with a workspace", (long long)M, (long long)N,
                    (long long)K, need, bl::kNoAllocScratchBytes);
    bl::Scratch scratch;
    const hipError_t e = bl::noalloc_scratch(stream, &scratch.ptr);
    if (e == hipErrorInvalidDevice)
        return fail(BITLINEAR_EINVAL, "the stream's device must be the current device");
    if (e != hipSuccess) return hip_fail("scratch address", e);
    scratch.bytes = bl::kNoAllocScratchBytes;
    return run_forward(Xq, x_scale, x_rowsum, packed, w_scale, p, M, N, K, Y, acc, scratch, stream);
}

bitlinear_status bitlinear_forward_grouped(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                                           int64_t M, int64_t K, bitlinear_nm nm, const bitlinear_proj *projs,
                                           int32_t nproj, hipStream_t stream)
{
    bl::Pattern p;
    CHECK(check_nm(nm, &p));
    CHECK(check_m(M));
    CHECK(check_k(K));
    bl::FusedProjArgs args = {};
    CHECK(check_projs(projs, nproj, M, &args));
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }
    CHECK(check_ptr(Xq, 16, "Xq"));
    CHECK(check_ptr(x_scale, 4, "x_scale"));
    CHECK(check_ptr(x_rowsum, 4, "x_rowsum"));
    int64_t rows16 = 0;
    for (int i = 0; i < nproj; ++i) rows16 += (projs[i].N + 15) / 16;
    const char *name = "";
    hipError_t e = hipErrorNotSupported;
    if (M == 1)
        e = bl::launch_decode_dot4(nullptr, Xq, x_scale, x_rowsum, M, K, p, args, nullptr,
                                   bl::ActTransform{nullptr, nullptr, 0.0f}, stream, &name, false);
    // wide dense projections at 9-64 tokens: several token tiles per workgroup
    else if (M >= 9)
        e = bl::launch_skinny_direct_tiles(Xq, x_scale, x_rowsum, args, p, M, K, stream, &name, false);
    // 17-64 tokens in tiles of 16 while the tiles make at most 512 workgroups
    // (the rule of the single forward), 1024 for two or more projections: one
    // launch then replaces several (q, k, v of a 3B block at 64 tokens, 640
    // workgroups: 12.8 us in three launches, one grouped launch less than half)
    if (e == hipErrorNotSupported && M > 1 &&
        (M <= 16 || (M <= bl::kSkinnyMaxM && rows16 * ((M + 15) / 16) <= (nproj > 1 ? 1024 : 512))))
        e = bl::launch_skinny_forward(Xq, x_scale, x_rowsum, args, p, M, K, stream, &name, false);
    // past that, several wide projections in one launch of the few-token GEMM
    if (e == hipErrorNotSupported && M > 16)
        e = bl::launch_gemm_grouped(Xq, x_scale, x_rowsum, args, p, M, K, stream, &name, false);
    if (e == hipErrorNotSupported)
        return fail(BITLINEAR_EUNSUPPORTED, "grouped forward: no one-launch kernel for M = %lld, K = %lld and %lld "
                    "rows of 16 (call bitlinear_forward per projection)", (long long)M, (long long)K,
                    (long long)rows16);
    if (e != hipSuccess) return hip_fail("grouped forward launch", e);
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
    bl::FusedProjArgs args = {};
    CHECK(check_projs(projs, nproj, M, &args));
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }
    CHECK(check_ptr(X, 16, "X"));
    if (x_scale && !aligned(x_scale, 4)) return fail(BITLINEAR_EINVAL, "x_scale must be 4-byte aligned");
    const char *name = "";
    hipError_t e = bl::launch_decode_dot4(X, nullptr, nullptr, nullptr, M, K, p, args, x_scale, t, stream, &name,
                                          false);
    if (e == hipErrorNotSupported && transformed)
        return fail(BITLINEAR_EUNSUPPORTED, "fused decode with a row transform supports M == 1 and K <= 16384 "
                    "(M = %lld, K = %lld)", (long long)M, (long long)K);
    if (e == hipErrorNotSupported) e = bl::launch_fused_forward(X, M, K, p, args, x_scale, stream, &name);
    if (e == hipErrorNotSupported)
        return fail(BITLINEAR_EUNSUPPORTED, "fused decode supports 1 <= M <= 16 and K <= %s (M = %lld, K = %lld)",
                    M == 1 ? "65344" : "16192", (long long)M, (long long)K);
    if (e != hipSuccess) return hip_fail("fused forward launch", e);
    set_dispatch(name);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_forward_fused_multi(const bitlinear_input_group *groups, int32_t ngroups,
                                               bitlinear_nm nm, hipStream_t stream)
{
    bl::Pattern p;
    CHECK(check_nm(nm, &p));
    if (!groups) return fail(BITLINEAR_EINVAL, "groups must not be NULL");
    if (ngroups < 1) return fail(BITLINEAR_EINVAL, "ngroups = %d must be >= 1", ngroups);
    if (ngroups > bl::kMaxInputGroups)
        return fail(BITLINEAR_EUNSUPPORTED, "ngroups = %d: at most %d input groups per call", ngroups,
                    bl::kMaxInputGroups);
    bl::MultiGroupArgs mg = {};
    mg.ngroups = ngroups;
    bool one_launch = (p == bl::Pattern::Dense);
    for (int g = 0; g < ngroups; ++g) {
        CHECK(check_k(groups[g].K));
        if (groups[g].K > 65344)
            return fail(BITLINEAR_EUNSUPPORTED, "one-token fused decode supports K <= 65344 (group %d: K = %lld)", g,
                        (long long)groups[g].K);
        CHECK(check_projs(groups[g].projs, groups[g].nproj, 1, &mg.args[g]));
        CHECK(check_ptr(groups[g].X, 16, "groups[g].X"));
        if (groups[g].x_scale && !aligned(groups[g].x_scale, 4))
            return fail(BITLINEAR_EINVAL, "groups[g].x_scale must be 4-byte aligned");
        mg.X[g] = groups[g].X;
        mg.K[g] = groups[g].K;
        mg.x_scale_out[g] = groups[g].x_scale;
        if (groups[g].K > 16384) one_launch = false;
    }
    const char *name = "";
    if (one_launch) {
        const hipError_t e = bl::launch_decode_multi(mg, stream, &name, false);
        if (e == hipSuccess) { set_dispatch(name); return BITLINEAR_OK; }
        if (e != hipErrorNotSupported) return hip_fail("multi-group decode launch", e);
    }
    // one launch per group
    char names[sizeof g_dispatch] = "";
    size_t len = 0;
    for (int g = 0; g < ngroups; ++g) {
        hipError_t e = bl::launch_decode_dot4(mg.X[g], nullptr, nullptr, nullptr, 1, mg.K[g], p, mg.args[g],
                                              mg.x_scale_out[g], bl::ActTransform{nullptr, nullptr, 0.0f}, stream,
                                              &name, false);
        if (e == hipErrorNotSupported)
            e = bl::launch_fused_forward(mg.X[g], 1, mg.K[g], p, mg.args[g], mg.x_scale_out[g], stream, &name);
        if (e != hipSuccess) return hip_fail("fused forward launch", e);
        if (len < sizeof names) len += snprintf(names + len, sizeof names - len, "%s%s", g ? " + " : "", name);
    }
    set_dispatch(names);
    return BITLINEAR_OK;
}

bitlinear_status bitlinear_forward_grouped_multi(const bitlinear_act_group *groups, int32_t ngroups, int64_t M,
                                                 bitlinear_nm nm, hipStream_t stream)
{
    bl::Pattern p;
    CHECK(check_nm(nm, &p));
    CHECK(check_m(M));
    if (!groups) return fail(BITLINEAR_EINVAL, "groups must not be NULL");
    if (ngroups < 1) return fail(BITLINEAR_EINVAL, "ngroups = %d must be >= 1", ngroups);
    if (ngroups > bl::kMaxInputGroups)
        return fail(BITLINEAR_EUNSUPPORTED, "ngroups = %d: at most %d input groups per call", ngroups,
                    bl::kMaxInputGroups);
    bl::DirectMultiArgs da = {};
    da.ngroups = ngroups;
    da.M = M;
    for (int g = 0; g < ngroups; ++g) {
        const bitlinear_act_group &a = groups[g];
        CHECK(check_k(a.K));
        CHECK(check_projs(a.projs, a.nproj, M, &da.args[g]));
        if (M > 0) {
            CHECK(check_ptr(a.Xq, 16, "groups[g].Xq"));
            CHECK(check_ptr(a.x_scale, 4, "groups[g].x_scale"));
            CHECK(check_ptr(a.x_rowsum, 4, "groups[g].x_rowsum"));
        }
        da.Xq[g] = a.Xq;
        da.x_scale[g] = a.x_scale;
        da.x_rowsum[g] = a.x_rowsum;
        da.K[g] = a.K;
    }
    if (M == 0) { set_dispatch("none"); return BITLINEAR_OK; }
    if (p != bl::Pattern::Dense)
        return fail(BITLINEAR_EUNSUPPORTED, "the multi-input grouped forward takes dense weights (nm = {0, 0})");
    const char *name = "";
    const hipError_t e = M <= 8 ? bl::launch_skinny_direct_multi(da, stream, &name, false)
                                : bl::launch_skinny_direct_tiles_multi(da, stream, &name, false);
    if (e == hipErrorNotSupported)
        return fail(BITLINEAR_EUNSUPPORTED, "the multi-input grouped forward supports 5 <= M <= 8 with "
                    "256 <= K <= 12288, or 9 <= M <= 64 with every group on the token-tile kernel (M = %lld)",
                    (long long)M);
    if (e != hipSuccess) return hip_fail("multi-input grouped forward launch", e);
    set_dispatch(name);
    return BITLINEAR_OK;
}

const char *bitlinear_last_error(void) { return g_error; }

const char *bitlinear_last_dispatch(void) { return g_dispatch; }

}  // extern "C"
