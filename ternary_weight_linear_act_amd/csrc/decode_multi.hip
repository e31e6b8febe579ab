// One-token decode of several input groups in one launch: each group is an
// fp32 activation row with the projections that read it (q/k/v; gate/up; a
// down projection), and the grid holds every group's workgroups.  A
// workgroup finds its group, then runs the one-token fused kernel's body
// (decode_dot4_impl.hpp) in the configuration the host rule picks for that
// group alone, so each group's outputs are bit for bit those of its own
// bitlinear_forward_fused call: per-token absmax int8 quantisation ("BitNet
// b1.58 2B4T Technical Report 요약 설명", sec. 2), the packed ternary weights
// streamed from HBM and unpacked on chip (sec. 5.1), the integer linear and
// the rescale ("BitNet 논문 분석: 1-Bit LLM의 시대", section "Absmean 양자화
// 함수").
//
// Why: at one token a launch costs a fixed ~2 us (dispatch, the first HBM
// round trip, the drain) on top of its bytes, about as much as streaming
// 8 MB.  Groups whose inputs do not depend on one another (independent
// sequences' layers, the down projections of several experts, the
// projections of a step whose activations are given) need not pay it once
// each.
//
// Workgroups are 512 threads; a group whose configuration has 4 waves runs
// them in waves 0-3 and waves 4-7 end at once.  A barrier waits only for the
// waves of the workgroup that have not ended, so the body's barriers are
// those of its own launch.
#include "decode_dot4_impl.hpp"

namespace bl {
namespace {

thread_local char g_name[160];

// The configurations of the menu, numbered: 8 waves at 8 lanes per row
// (u = 1..7), then 4 waves at 8 lanes (u = 1..7), 16 and 32 lanes (u = 4..7),
// 64 lanes (u = 4): all the dense fused ones dot4_config can pick; then
// 4 lanes per row (u = 1..8) with 4, 6 or 8 waves.
int menu_index(const Dot4Config &c, int waves)
{
    if (c.lpr == 4) {
        const int wi = waves == 4 ? 0 : waves == 6 ? 1 : waves == 8 ? 2 : -1;
        return (wi >= 0 && c.u >= 1 && c.u <= 8) ? 23 + 10 * wi + c.u - 1 : -1;
    }
    if (waves == 8) return (c.lpr == 8 && c.u >= 1 && c.u <= 7) ? c.u - 1 : -1;
    if (waves != 4) return -1;
    switch (c.lpr) {
    case 8: return (c.u >= 1 && c.u <= 7) ? 7 + c.u - 1 : -1;
    case 16: return (c.u >= 4 && c.u <= 7) ? 14 + c.u - 4 : -1;
    case 32: return (c.u >= 4 && c.u <= 7) ? 18 + c.u - 4 : -1;
    case 64: return c.u == 4 ? 22 : -1;
    default: return -1;
    }
}

// A group's configuration in the multi-input launch.  Rows of K <= 2048
// (at most 32 chunks) take 4 lanes per row (16 rows per wave) and the fewest
// of 4, 6 or 8 waves that keep the group within kMultiMaxBlocks workgroups:
// every workgroup reads and quantises its group's whole input row, so fewer,
// fuller workgroups cost less, while the chip still holds the other groups'
// workgroups beside them.  Measured, one launch of the 3B block's four
// groups: q/k/v, o, gate+up (K = 2048) on 4 lanes (40, 32, 172 workgroups)
// against 8 lanes (80, 64, 344) 8.7 -> 8.1 us.  The 2B gate+up (K = 2560,
// 10 chunks per lane on 4 lanes) measured slower that way (the step 6.8 ->
// 8.9 us), so from 33 chunks the one-input rule (dot4_config) applies.
constexpr int64_t kMultiMaxBlocks = 180;

Dot4Config multi_config(int64_t K, const FusedProjArgs &args, int *waves)
{
    const int64_t C = K / 64;
    if (C <= 32) {
        int64_t rows16 = 0;
        for (int i = 0; i < args.nproj; ++i) rows16 += (args.N[i] + 15) / 16;
        int w = 4;
        while (w < 8 && (rows16 + w - 1) / w > kMultiMaxBlocks) w += 2;
        *waves = w;
        return Dot4Config{4, (int)((C + 3) / 4), w == 8, (int64_t)w * 16};
    }
    const Dot4Config c = dot4_config(K, true, 0, args);
    *waves = c.w8 ? 8 : 4;
    return c;
}

}  // namespace

namespace dot4 {

// The kernel's argument: one record per (group, projection) pair in grid
// order, so that a workgroup finds its record with one scan of pair_start
// and has every pointer with one more load (the one-input kernel's depth).
struct MultiPair {
    const float *X;
    float *x_scale_out;          // set on the group's first pair only
    const uint8_t *packed;
    const float *w_scale;
    float *Y;
    int32_t *acc;
    int64_t K;
    int64_t N;
    int32_t cfg;
    int32_t pad;
};

// At most 16 pairs in one launch: their first blocks fill one 64-byte line
// of the argument, read by one scalar load (more pairs: one launch per
// group).
constexpr int kMultiPairs = 16;

struct MultiPairArgs {
    int32_t pair_start[kMultiPairs + 1];     // entries past the last pair: the block count
    int32_t pair_kc[kMultiPairs];            // K | configuration << 16, and the input rows, read
    const float *pair_x[kMultiPairs];        // with pair_start: the input loads wait on no second load
    MultiPair pair[kMultiPairs];
};

#define BL_MULTI_CASE(ID, LPR, U, W)                                                                            \
    case ID:                                                                                                    \
        if (wave < (W))                                                                                         \
            decode_dot4_body<Pattern::Dense, LPR, U, true, W, 0>(x, nullptr, nullptr, nullptr, k, resolve, tr); \
        return;

// The argument is read in place in the kernel-argument segment (it is the
// launch's only argument, at offset 0): indexed by the group, a by-value
// copy of it would live in scratch memory.  NP: the pairs scanned (at least
// the launch's).  Their K and row pointers are read into registers with the
// table and selected there (selecting the index first, then loading the
// entry, costs a second round trip before the input loads).
template <int NP>
__global__ __launch_bounds__(512) void decode_multi_kernel(MultiPairArgs)
{
    const MultiPairArgs &ma = *(const MultiPairArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    const int block = (int)blockIdx.x;
    int kcs[NP];
    const float *xs[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        kcs[i] = ma.pair_kc[i];
        xs[i] = ma.pair_x[i];
    }
    int q = 0, kc = kcs[0];
    const float *x = xs[0];
#pragma unroll
    for (int i = 1; i < NP; ++i)
        if (block >= ma.pair_start[i]) {
            q = i;
            kc = kcs[i];
            x = xs[i];
        }
    const int k = kc & 0xffff, cfg = kc >> 16;
    // the pair's record is read in resolve(), after the input-row loads
    const auto resolve = [&]() {
        const MultiPair &e = ma.pair[q];
        const int first = ma.pair_start[q];
        return ProjSel{ProjView{e.packed, e.w_scale, e.Y, e.acc, e.N}, (int64_t)(block - first),
                       block == first ? e.x_scale_out : nullptr};
    };
    const ActTransform tr{nullptr, nullptr, 0.0f};
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // uniform: a scalar branch
    switch (cfg) {
        BL_MULTI_CASE(0, 8, 1, 8)
        BL_MULTI_CASE(1, 8, 2, 8)
        BL_MULTI_CASE(2, 8, 3, 8)
        BL_MULTI_CASE(3, 8, 4, 8)
        BL_MULTI_CASE(4, 8, 5, 8)
        BL_MULTI_CASE(5, 8, 6, 8)
        BL_MULTI_CASE(6, 8, 7, 8)
        BL_MULTI_CASE(7, 8, 1, 4)
        BL_MULTI_CASE(8, 8, 2, 4)
        BL_MULTI_CASE(9, 8, 3, 4)
        BL_MULTI_CASE(10, 8, 4, 4)
        BL_MULTI_CASE(11, 8, 5, 4)
        BL_MULTI_CASE(12, 8, 6, 4)
        BL_MULTI_CASE(13, 8, 7, 4)
        BL_MULTI_CASE(14, 16, 4, 4)
        BL_MULTI_CASE(15, 16, 5, 4)
        BL_MULTI_CASE(16, 16, 6, 4)
        BL_MULTI_CASE(17, 16, 7, 4)
        BL_MULTI_CASE(18, 32, 4, 4)
        BL_MULTI_CASE(19, 32, 5, 4)
        BL_MULTI_CASE(20, 32, 6, 4)
        BL_MULTI_CASE(21, 32, 7, 4)
        BL_MULTI_CASE(22, 64, 4, 4)
        BL_MULTI_CASE(23, 4, 1, 4)
        BL_MULTI_CASE(24, 4, 2, 4)
        BL_MULTI_CASE(25, 4, 3, 4)
        BL_MULTI_CASE(26, 4, 4, 4)
        BL_MULTI_CASE(27, 4, 5, 4)
        BL_MULTI_CASE(28, 4, 6, 4)
        BL_MULTI_CASE(29, 4, 7, 4)
        BL_MULTI_CASE(30, 4, 8, 4)
        BL_MULTI_CASE(33, 4, 1, 6)
        BL_MULTI_CASE(34, 4, 2, 6)
        BL_MULTI_CASE(35, 4, 3, 6)
        BL_MULTI_CASE(36, 4, 4, 6)
        BL_MULTI_CASE(37, 4, 5, 6)
        BL_MULTI_CASE(38, 4, 6, 6)
        BL_MULTI_CASE(39, 4, 7, 6)
        BL_MULTI_CASE(40, 4, 8, 6)
        BL_MULTI_CASE(43, 4, 1, 8)
        BL_MULTI_CASE(44, 4, 2, 8)
        BL_MULTI_CASE(45, 4, 3, 8)
        BL_MULTI_CASE(46, 4, 4, 8)
        BL_MULTI_CASE(47, 4, 5, 8)
        BL_MULTI_CASE(48, 4, 6, 8)
        BL_MULTI_CASE(49, 4, 7, 8)
        BL_MULTI_CASE(50, 4, 8, 8)
    default: return;
    }
}

#undef BL_MULTI_CASE

}  // namespace dot4

// The groups take the grid in order of decreasing K (stable): the deepest
// rows' workgroups, which read the longest input rows, get compute units of
// their own first, and the shallower groups' workgroups fill in beside them.
// Measured against the callers' order, inputs and weights rotating through
// a 2 GiB pool: the 3B block at one token 8.7 -> 7.9 us; the 2B decode step
// (two groups) 6.85 against 6.93 us, level within the runs' spread.
void order_by_depth(MultiGroupArgs &mg)
{
    MultiGroupArgs in = mg;
    int order[kMaxInputGroups];
    for (int g = 0; g < mg.ngroups; ++g) order[g] = g;
    for (int i = 1; i < mg.ngroups; ++i)
        for (int j = i; j > 0 && in.K[order[j]] > in.K[order[j - 1]]; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    for (int g = 0; g < mg.ngroups; ++g) {
        const int o = order[g];
        mg.X[g] = in.X[o];
        mg.x_scale_out[g] = in.x_scale_out[o];
        mg.K[g] = in.K[o];
        mg.args[g] = in.args[o];
    }
}

hipError_t launch_decode_multi(MultiGroupArgs mg, hipStream_t stream, const char **name, bool query)
{
    if (mg.ngroups < 1 || mg.ngroups > kMaxInputGroups) return hipErrorNotSupported;
    order_by_depth(mg);
    int64_t blocks = 0, kmax = 0;
    int len = snprintf(g_name, sizeof g_name, "fused_decode_multi_dense");
    for (int g = 0; g < mg.ngroups; ++g) {
        FusedProjArgs &a = mg.args[g];
        if (mg.K[g] > dot4::kMaxK || a.nproj < 1 || a.nproj > kMaxFusedProj) return hipErrorNotSupported;
        int waves = 4;
        const Dot4Config c = multi_config(mg.K[g], a, &waves);
        const int id = menu_index(c, waves);
        if (id < 0) return hipErrorNotSupported;
        mg.cfg[g] = id;
        mg.group_start[g] = (int32_t)blocks;
        blocks += dot4_block_starts(a, c.rb);
        if (blocks > (1LL << 30)) return hipErrorNotSupported;
        if (mg.K[g] > kmax) kmax = mg.K[g];
        if (len < (int)sizeof g_name)
            len += snprintf(g_name + len, sizeof g_name - len, "%slpr%d_u%d_p%d%s", g ? "+" : "_", c.lpr, c.u,
                            a.nproj, waves == 4 ? "" : waves == 6 ? "_w6" : "_w8");
    }
    for (int g = mg.ngroups; g <= kMaxInputGroups; ++g) mg.group_start[g] = (int32_t)blocks;
    int pairs = 0;
    for (int g = 0; g < mg.ngroups; ++g) pairs += mg.args[g].nproj;
    if (pairs > dot4::kMultiPairs) return hipErrorNotSupported;
    dot4::MultiPairArgs ma = {};
    int q = 0;
    for (int g = 0; g < mg.ngroups; ++g)
        for (int i = 0; i < mg.args[g].nproj; ++i, ++q) {
            const FusedProjArgs &a = mg.args[g];
            ma.pair_start[q] = mg.group_start[g] + a.block_start[i];
            ma.pair_kc[q] = (int32_t)mg.K[g] | mg.cfg[g] << 16;   // K <= 16384 here
            ma.pair_x[q] = mg.X[g];
            ma.pair[q] = dot4::MultiPair{mg.X[g], i == 0 ? mg.x_scale_out[g] : nullptr, a.packed[i], a.w_scale[i],
                                         a.Y[i], a.acc[i], mg.K[g], a.N[i], mg.cfg[g], 0};
        }
    for (int i = q; i <= dot4::kMultiPairs; ++i) ma.pair_start[i] = (int32_t)blocks;
    *name = g_name;
    if (query) return hipSuccess;
    // the shortest scan that covers the launch's pairs
    void (*kern)(dot4::MultiPairArgs) = q <= 4 ? dot4::decode_multi_kernel<4>
                                      : q <= 8 ? dot4::decode_multi_kernel<8> : dot4::decode_multi_kernel<16>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(512), (size_t)kmax, stream, ma);
    return hipGetLastError();
}

}  // namespace bl
