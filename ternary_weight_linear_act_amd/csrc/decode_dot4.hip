// Host side of the one-token decode kernel (decode_dot4_impl.hpp): the
// configuration rule and the launch.  The row-transform variants of the fused
// form are instantiated in decode_dot4_tr.hip.
#include "decode_dot4_impl.hpp"

namespace bl {
namespace {

thread_local char g_name[64];

}  // namespace

// Lanes per row: the fewest of 8, 16, 32, 64 that keep a lane's chunks U
// <= 5, or <= 7 with the quantisation fused in (<= 4 at 64 lanes, K <= 16384).
// The fused kernel reads and quantises the whole fp32 row in every
// workgroup, so it prefers fewer, fuller workgroups: at 8 lanes per row it
// takes 8 waves (64 rows) per workgroup where 4 waves would need more than
// 320 workgroups (gate+up of a 2B FFN: 432 -> 216, 4.1 -> 4.0 us), except
// with a row transform, where 4 waves measured faster (RMSNorm on gate+up
// 5.35 -> 5.13 us).  Returns hipErrorNotSupported when M != 1 or K is too
// large.  With `query` set, launches nothing and returns hipSuccess where it
// would launch.
hipError_t launch_decode_dot4(const float *X, const int8_t *Xq, const float *xs, const int32_t *rs,
                              int64_t M, int64_t K, Pattern p, FusedProjArgs args, float *x_scale_out,
                              const ActTransform &tr, hipStream_t stream, const char **name, bool query)
{
    if (M != 1 || K > dot4::kMaxK || args.nproj < 1 || args.nproj > kMaxFusedProj) return hipErrorNotSupported;
    const int64_t C = K / 64;
    const bool fused = (X != nullptr);
    const int64_t umax = fused ? 7 : 5;
    int lpr = 8;
    while (lpr < 64 && (C + lpr - 1) / lpr > umax) lpr *= 2;
    const int u = (int)((C + lpr - 1) / lpr);
    auto count_blocks = [&](int64_t rb) {
        int64_t b = 0;
        for (int i = 0; i < args.nproj; ++i) b += (args.N[i] + rb - 1) / rb;
        return b;
    };
    const int trb = (tr.up ? kTrGate : 0) | (tr.gamma ? kTrNorm : 0);
    const bool w8 = fused && lpr == 8 && count_blocks(4 * 8) > 320 && trb == 0;
    const int64_t rb = (w8 ? 8 : 4) * (64 / lpr);
    int64_t blocks = 0;
    for (int i = 0; i < args.nproj; ++i) {
        args.block_start[i] = (int32_t)blocks;
        blocks += (args.N[i] + rb - 1) / rb;
    }
    for (int i = args.nproj; i <= kMaxFusedProj; ++i) args.block_start[i] = (int32_t)blocks;
    if (blocks > (1LL << 30)) return hipErrorNotSupported;
    if (trb && !fused) return hipErrorNotSupported;
    Fn f = nullptr;
    if (trb) f = pick_dot4_tr(p, trb, w8, lpr, u);
    else switch (p) {
    case Pattern::Dense:
        f = w8 ? pick_w8<Pattern::Dense>(u) : fused ? pick<Pattern::Dense, true>(lpr, u) : pick<Pattern::Dense, false>(lpr, u);
        break;
    case Pattern::NM24:
        f = w8 ? pick_w8<Pattern::NM24>(u) : fused ? pick<Pattern::NM24, true>(lpr, u) : pick<Pattern::NM24, false>(lpr, u);
        break;
    case Pattern::NM68:
        f = w8 ? pick_w8<Pattern::NM68>(u) : fused ? pick<Pattern::NM68, true>(lpr, u) : pick<Pattern::NM68, false>(lpr, u);
        break;
    }
    if (!f) return hipErrorNotSupported;
    static const char *trn[4] = {"", "_gate", "_norm", "_gate_norm"};
    snprintf(g_name, sizeof g_name, "%s_%s_lpr%d_u%d_p%d%s%s", fused ? "fused_decode_dot4" : "decode_dot4",
             p == Pattern::Dense ? "dense" : p == Pattern::NM24 ? "nm24" : "nm68", lpr, u, args.nproj,
             w8 ? "_w8" : "", trn[trb]);
    *name = g_name;
    if (query) return hipSuccess;
    f(dim3((unsigned)blocks), (size_t)K, stream, X, Xq, xs, rs, K, args, x_scale_out, tr);
    return hipGetLastError();
}

}  // namespace bl
