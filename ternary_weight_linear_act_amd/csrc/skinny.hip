// Dispatch of the skinny (1 <= M <= 16) MFMA forward: picks how many waves
// split K (KS) and the per-wave chunk capacity (CMAX) from the shape.
//
// Rule (from sweeps on MI355X over the decode shapes 2560->6912, 6912->2560,
// 1536->8960, 2048->{256,2048,11008}, 11008->2048): about 10 chunks (640
// weights) per wave, KS a power of two, the smallest CMAX that holds a wave's
// range, and the first candidate whose LDS staging fits 160 KB.  The staged
// token rows are M rounded up to 1, 4, 8 or 16: fewer rows, less LDS, more
// workgroups per compute unit and deeper K ranges that fit.
#include <math.h>
#include <stdio.h>

#include "kernels.hpp"
#include "skinny_impl.hpp"

namespace bl {
namespace {

using Fn = hipError_t (*)(const int8_t *, const float *, const int32_t *, const FusedProjArgs &, int64_t, int64_t,
                          int64_t, hipStream_t);

constexpr int kKS[] = {1, 2, 4, 8, 16};
constexpr int kCM[] = {4, 8, 12, 16, 24, 32, 44};
constexpr int kNKS = sizeof(kKS) / sizeof(kKS[0]);
constexpr int kNCM = sizeof(kCM) / sizeof(kCM[0]);

// LDS of a configuration: per-wave staging, the cross-wave partial sums and
// (2:4) the decode table
constexpr int64_t lds_bytes_c(int ks, int cmax, int mt, Pattern p)
{
    return ks * (16LL * (8 * ((cmax + 7) / 8) + 1) * 16 + (int64_t)mt * (cmax + 3) * 64 + 64) +
           (int64_t)(ks > 1 ? ks - 1 : 1) * 64 * 16 + (p == Pattern::NM24 ? 256 : 0);
}

// a configuration whose staging does not fit the 160 KB of LDS is never built
template <Pattern P, int KS, int CM, int MT>
Fn get()
{
    if constexpr (lds_bytes_c(KS, CM, MT, P) <= 160 * 1024) return skinny::launch_skinny<P, KS, CM, MT>;
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
    case 4: return get<P, KS, 24, MT>();
    case 5: return get<P, KS, 32, MT>();
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
    switch (mt) {
    case 1: return pick<P, 1>(ksi, cmi);
    case 4: return pick<P, 4>(ksi, cmi);
    case 8: return pick<P, 8>(ksi, cmi);
    default: return pick<P, 16>(ksi, cmi);
    }
}

thread_local char g_name[64];

}  // namespace

// One or more projections sharing Xq (args.block_start is filled here: 16
// weight rows per workgroup).  Returns hipErrorNotSupported (and launches
// nothing) when no configuration fits the shape; the caller then uses another
// kernel.  With `query` set, launches nothing and returns hipSuccess where it
// would launch.
hipError_t launch_skinny_forward(const int8_t *Xq, const float *xs, const int32_t *rs, FusedProjArgs args,
                                 Pattern p, int64_t M, int64_t K, hipStream_t stream, const char **name, bool query)
{
    if (M < 1 || M > kSkinnyMaxM || args.nproj < 1 || args.nproj > kMaxFusedProj) return hipErrorNotSupported;
    // the weights straight into the MFMA operand where that measured faster
    const hipError_t ed = launch_skinny_direct(Xq, xs, rs, args, p, M, K, stream, name, query);
    if (ed != hipErrorNotSupported) return ed;
    int64_t blocks = 0;
    for (int i = 0; i < args.nproj; ++i) {
        args.block_start[i] = (int32_t)blocks;
        blocks += (args.N[i] + 15) / 16;
    }
    for (int i = args.nproj; i <= kMaxFusedProj; ++i) args.block_start[i] = (int32_t)blocks;
    if (blocks > (1LL << 30)) return hipErrorNotSupported;
    // token rows staged per wave: 1, 4, 8 or 16 (rows past M read a zero
    // block); past 16 tokens, tiles of 16 along the grid's y
    const int mt = (M == 1) ? 1 : (M <= 4) ? 4 : (M <= 8) ? 8 : 16;
    const int64_t C = K / 64;
    // candidates ordered by distance (in log2) from ~10 chunks per wave
    const double want = log2((double)C / 10.0);
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
        int cmi = -1;
        for (int c = 0; c < kNCM; ++c)
            if (kCM[c] >= need) { cmi = c; break; }
        if (cmi < 0) continue;
        if (lds_bytes_c(ks, kCM[cmi], mt, p) > 160 * 1024) continue;
        Fn f = nullptr;
        switch (p) {
        case Pattern::Dense: f = pick_p<Pattern::Dense>(mt, ksi, cmi); break;
        case Pattern::NM24: f = pick_p<Pattern::NM24>(mt, ksi, cmi); break;
        case Pattern::NM68: f = pick_p<Pattern::NM68>(mt, ksi, cmi); break;
        }
        if (!f) continue;
        snprintf(g_name, sizeof g_name, "skinny_mfma_%s_ks%d_c%d_mt%d%s",
                 p == Pattern::Dense ? "dense" : p == Pattern::NM24 ? "nm24" : "nm68", ks, kCM[cmi], mt,
                 args.nproj > 1 ? "_grouped" : "");
        *name = g_name;
        if (query) return hipSuccess;
        return f(Xq, xs, rs, args, blocks, M, K, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace bl
