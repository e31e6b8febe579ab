// The fused one-token decode kernel with a row transform before the
// quantiser (ReLU^2 gate, RMSNorm, or both; common.hpp), every configuration
// the host rule in decode_dot4.hip can pick.  A translation unit of its own so
// that the two halves build in parallel.
#include "decode_dot4_impl.hpp"

namespace bl {
namespace {

// (the host rule never takes 8 waves with a transform)
template <int TR>
Dot4Fn pick_tr(Pattern p, bool w8, int lpr, int u)
{
    if (w8) return nullptr;
    switch (p) {
    case Pattern::Dense: return pick<Pattern::Dense, true, TR>(lpr, u);
    case Pattern::NM24: return pick<Pattern::NM24, true, TR>(lpr, u);
    case Pattern::NM68: return pick<Pattern::NM68, true, TR>(lpr, u);
    }
    return nullptr;
}

}  // namespace

Dot4Fn pick_dot4_tr(Pattern p, int tr_bits, bool w8, int lpr, int u)
{
    switch (tr_bits) {
    case kTrGate: return pick_tr<kTrGate>(p, w8, lpr, u);
    case kTrNorm: return pick_tr<kTrNorm>(p, w8, lpr, u);
    case kTrGate | kTrNorm: return pick_tr<kTrGate | kTrNorm>(p, w8, lpr, u);
    default: return nullptr;
    }
}

}  // namespace bl
