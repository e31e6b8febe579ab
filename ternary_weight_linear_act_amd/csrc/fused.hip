// Host dispatch of the fused decode forward (activation quantisation + one or
// more projections sharing the activations, one launch).  Configuration rule:
// KS a power of two giving ~20 chunks per wave when there are many workgroups
// (>= 512; fewer waves per workgroup then cost less) and ~12 when there are
// few (more waves then keep more loads in flight), the smallest CMAX that
// holds a wave's range, LDS within budget.  Measured on MI355X for the
// 2B-class FFN: gate+up (864 workgroups) 5.4 us at KS = 2 against 7.0 us at
// KS = 4; down (160 workgroups) 4.9 us at KS = 8 against 6.4 us at KS = 4.
#include <math.h>
#include <stdio.h>

#include "fused_impl.hpp"

namespace bl {
namespace {

using Fn = hipError_t (*)(const float *, int64_t, int64_t, const FusedProjArgs &, int, float *, hipStream_t);

constexpr int kKS[] = {1, 2, 4, 8, 16};
constexpr int kCM[] = {4, 8, 12, 16, 20, 24, 32, 44};
constexpr int kNKS = sizeof(kKS) / sizeof(kKS[0]);
constexpr int kNCM = sizeof(kCM) / sizeof(kCM[0]);
constexpr int64_t kLds = 160 * 1024;
constexpr int64_t kMaxDynLds = 64 * 1024;

constexpr int kRows = 16;   // weight rows per workgroup

constexpr int64_t static_lds(int ks, int cmax, int mt)
{
    return (int64_t)ks * kRows * (cmax + 1) * 16 + 256 + (int64_t)mt * ks * 8 +
           (int64_t)((kRows + 15) / 16) * (ks > 1 ? ks - 1 : 1) * 64 * 16;
}

// 4 token rows with 16 waves, or with 44 chunks per wave, are never built:
// the rows' activation registers would spill to scratch (at 1024 threads a
// thread has 128 VGPRs; 44 chunks take more than 256).  8 waves of 32 chunks
// reach K = 16384, beyond the 16192 the 4-row staging allows.
template <Pattern P, int KS, int CM, int MT>
Fn get()
{
    if constexpr (MT > 1 && (KS > 8 || CM > 32)) return nullptr;
    else if constexpr (static_lds(KS, CM, MT) <= kLds - 1024) return fused::launch_fused<P, KS, CM, MT, kRows>;
    else return nullptr;
}

template <Pattern P, int MT, int KS>
Fn pick_cm(int cmi)
{
    switch (cmi) {
    case 0: return get<P, KS, 4, MT>();
    case 1: return get<P, KS, 8, MT>();
    case 2: return get<P, KS, 12, MT>();
    case 3: return get<P, KS, 16, MT>();
    case 4: return get<P, KS, 20, MT>();
    case 5: return get<P, KS, 24, MT>();
    case 6: return get<P, KS, 32, MT>();
    default: return get<P, KS, 44, MT>();
    }
}

template <Pattern P, int MT>
Fn pick(int ksi, int cmi)
{
    switch (ksi) {
    case 0: return pick_cm<P, MT, 1>(cmi);
    case 1: return pick_cm<P, MT, 2>(cmi);
    case 2: return pick_cm<P, MT, 4>(cmi);
    case 3: return pick_cm<P, MT, 8>(cmi);
    default: return pick_cm<P, MT, 16>(cmi);
    }
}

template <Pattern P>
Fn pick_p(int mt, int ksi, int cmi)
{
    return mt == 1 ? pick<P, 1>(ksi, cmi) : pick<P, 4>(ksi, cmi);
}

thread_local char g_name[64];

// Picks KS and CMAX for MT staged token rows (`chunks`: the chunks per wave
// aimed at); nullptr when none fits.
Fn choose(Pattern p, int64_t K, int mt, double chunks, int *ks_out, int *cm_out)
{
    if ((int64_t)mt * (K + 192) > kMaxDynLds) return nullptr;
    const int64_t C = K / 64;
    const double want = log2((double)C / chunks);
    int order[kNKS];
    for (int i = 0; i < kNKS; ++i) order[i] = i;
    for (int i = 0; i < kNKS; ++i)
        for (int j = i + 1; j < kNKS; ++j)
            if (fabs(log2((double)kKS[order[j]]) - want) < fabs(log2((double)kKS[order[i]]) - want)) {
                const int t = order[i];
                order[i] = order[j];
                order[j] = t;
            }
    for (int oi = 0; oi < kNKS; ++oi) {
        const int ksi = order[oi], ks = kKS[ksi];
        if (ks > C) continue;
        const int64_t need = (C + ks - 1) / ks;
        for (int cmi = 0; cmi < kNCM; ++cmi) {
            if (kCM[cmi] < need) continue;
            if (static_lds(ks, kCM[cmi], mt) + (int64_t)mt * (K + 192) > kLds) break;
            Fn f = nullptr;
            switch (p) {
            case Pattern::Dense: f = pick_p<Pattern::Dense>(mt, ksi, cmi); break;
            case Pattern::NM24: f = pick_p<Pattern::NM24>(mt, ksi, cmi); break;
            case Pattern::NM68: f = pick_p<Pattern::NM68>(mt, ksi, cmi); break;
            }
            if (f) {
                *ks_out = ks;
                *cm_out = kCM[cmi];
                return f;
            }
            break;                                     // the smallest CMAX that holds the range, or none
        }
    }
    return nullptr;
}

}  // namespace

// args.block_start is filled here.  Tokens are staged one (M = 1) or four
// at a time, more than four in tiles of 4 along the grid's y.  Chunks per
// wave aimed at: about 20 with many workgroups (>= 512), 12 with few, and 6
// for tiles (each tile quantises its own rows, so fewer chunks per wave spread
// that work: at 8 tokens, 2048 -> 2048 5.3 -> 5.0 us and 2048 -> 2560 in
// three projections 6.1 us, against 8.7 and 8.8 us with 8 staged rows and
// 16 chunks per wave).  hipErrorNotSupported: no configuration fits (M > 16,
// too many projections, or K too large for the shared row).
hipError_t launch_fused_forward(const float *X, int64_t M, int64_t K, Pattern p, FusedProjArgs args,
                                float *x_scale, hipStream_t stream, const char **name)
{
    if (M < 1 || M > 16 || args.nproj < 1 || args.nproj > kMaxFusedProj) return hipErrorNotSupported;
    int64_t blocks = 0;
    for (int i = 0; i < args.nproj; ++i) {
        args.block_start[i] = (int32_t)blocks;
        blocks += (args.N[i] + kRows - 1) / kRows;
    }
    for (int i = args.nproj; i <= kMaxFusedProj; ++i) args.block_start[i] = (int32_t)blocks;
    if (blocks > (1LL << 30)) return hipErrorNotSupported;

    const int mt = (M == 1) ? 1 : 4;
    // tiles: about 6 chunks per wave, 4 for K of 9-16 chunks (1024 x 1024 at
    // 8-16 tokens: 4 waves 4.8 -> 4.4 us against 2)
    const int64_t C = K / 64;
    const double chunks = M > 4 ? (C > 8 && C <= 16 ? 4.0 : 6.0) : blocks >= 512 ? 20.0 : 12.0;
    int ks = 0, cm = 0;
    Fn f = choose(p, K, mt, chunks, &ks, &cm);
    if (!f) return hipErrorNotSupported;
    snprintf(g_name, sizeof g_name, "fused_decode_%s_ks%d_c%d_mt%d%s_p%d",
             p == Pattern::Dense ? "dense" : p == Pattern::NM24 ? "nm24" : "nm68", ks, cm, mt, M > 4 ? "_tiles" : "",
             args.nproj);
    *name = g_name;
    return f(X, M, K, args, (int)blocks, x_scale, stream);
}

}  // namespace bl
