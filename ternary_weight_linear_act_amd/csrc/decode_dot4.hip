// Host side of the one-token decode kernel (decode_dot4_impl.hpp): the
// configuration rule and the launch.  The row-transform variants of the fused
// form are instantiated in decode_dot4_tr.hip.
#include "decode_dot4_impl.hpp"

namespace bl {
namespace {

thread_local char g_name[64];

}  // namespace

// The configuration comes from dot4_config (decode_dot4_impl.hpp).  Returns
// hipErrorNotSupported when M != 1 or K is too large.  With `query` set,
// launches nothing and returns hipSuccess where it would launch.
hipError_t launch_decode_dot4(const float *X, const int8_t *Xq, const float *xs, const int32_t *rs,
                              int64_t M, int64_t K, Pattern p, FusedProjArgs args, float *x_scale_out,
                              const ActTransform &tr, hipStream_t stream, const char **name, bool query)
{
    if (M != 1 || K > dot4::kMaxK || args.nproj < 1 || args.nproj > kMaxFusedProj) return hipErrorNotSupported;
    const bool fused = (X != nullptr);
    const int trb = (tr.up ? kTrGate : 0) | (tr.gamma ? kTrNorm : 0);
    const Dot4Config cfg = dot4_config(K, fused, trb, args);
    const int lpr = cfg.lpr, u = cfg.u;
    const bool w8 = cfg.w8;
    const int64_t blocks = dot4_block_starts(args, cfg.rb);
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
