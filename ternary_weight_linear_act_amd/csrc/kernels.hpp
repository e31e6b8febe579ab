// Host-side launchers of the HIP kernels (internal to libbitlinear).
// Shapes and pointers are validated by the C-ABI layer before these run.
#pragma once

#include "common.hpp"

namespace bl {

// Per-row absmax int8 quantisation (one workgroup per row).
hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *x_scale,
                            int32_t *x_rowsum, hipStream_t stream);

// Several independent inputs in one launch (group g: M[g] rows of K[g]
// inputs, outputs as launch_quant_act's); the launcher fills row_start.
// hipErrorNotSupported when a row does not fit the registers (K > 16384 with
// 1024 threads per row, K > 8192 with 256).
constexpr int kMaxQuantGroups = 8;

struct QuantGroupArgs {
    const float *X[kMaxQuantGroups];
    int8_t *Xq[kMaxQuantGroups];
    float *x_scale[kMaxQuantGroups];
    int32_t *x_rowsum[kMaxQuantGroups];
    int64_t M[kMaxQuantGroups];
    int64_t K[kMaxQuantGroups];
    int64_t row_start[kMaxQuantGroups + 1];
    int32_t ngroups;
};

hipError_t launch_quant_act_multi(QuantGroupArgs qa, hipStream_t stream);

// The same on rows transformed first (ReLU^2 gate and/or RMSNorm; tr.up and
// tr.gamma NULL for none).
hipError_t launch_quant_act_ex(const float *X, ActTransform tr, int64_t M, int64_t K, int8_t *Xq,
                               float *x_scale, int32_t *x_rowsum, hipStream_t stream);

// Device scratch of one forward call: the caller's workspace (int32 split-K
// partial tiles; N:M rows expanded to dense codes).  The kernel choice is a
// function of the shape alone; `take` is called by a launcher before its
// first launch with the bytes its kernels use.  In a size query nothing is
// launched and `need` collects the bytes.
struct Scratch {
    uint8_t *ptr = nullptr;   // device memory, 16-byte aligned (may be null)
    size_t bytes = 0;         // bytes at ptr
    bool query = false;       // size query: launch nothing
    size_t need = 0;          // bytes the chosen kernels use

    // Records the need; true when the launcher may go on and launch (not a
    // size query, and the workspace is large enough).
    bool take(size_t n)
    {
        if (n > need) need = n;
        return !query && n <= bytes;
    }
};

// Scratch of bitlinear_forward_noalloc: a fixed device array per GPU.
constexpr size_t kNoAllocScratchBytes = 32u << 20;

// Device address of that array on the current device (looked up once per
// device).  hipErrorInvalidDevice when `stream` belongs to another device.
hipError_t noalloc_scratch(hipStream_t stream, uint8_t **ptr);

// Largest token count of the skinny MFMA forward (tiles of 16 tokens past 16).
constexpr int64_t kSkinnyMaxM = 64;

struct FusedProjArgs;                // skinny_impl.hpp
struct MultiGroupArgs;               // skinny_impl.hpp
struct DirectMultiArgs;              // skinny_impl.hpp

// Several quantised inputs at 5-8 tokens, dense weights, in one launch of the
// direct-load skinny kernel (every group 256 <= K <= 12288);
// hipErrorNotSupported otherwise.  The host fills Xq, x_scale, x_rowsum, K,
// M, ngroups and each group's projections; the launcher fills the rest.
hipError_t launch_skinny_direct_multi(DirectMultiArgs da, hipStream_t stream, const char **name, bool query);

// The same at 9-64 tokens on the direct-load kernel with several token tiles
// per workgroup, where every group fits its single-input rule;
// hipErrorNotSupported otherwise.
hipError_t launch_skinny_direct_tiles_multi(DirectMultiArgs da, hipStream_t stream, const char **name, bool query);

// One-token fused decode of several input groups, dense weights, in one
// launch (K <= 16384 per group); hipErrorNotSupported otherwise.  The host
// fills X, x_scale_out, K, ngroups and each group's projections; the
// launcher fills the rest.
hipError_t launch_decode_multi(MultiGroupArgs mg, hipStream_t stream, const char **name, bool query);

// The skinny MFMA forward with the weights read straight into the MFMA
// operand (dense weights at 5-64 tokens, the shapes where it measured faster
// than the staged kernel); hipErrorNotSupported for every other shape.
hipError_t launch_skinny_direct(const int8_t *Xq, const float *xs, const int32_t *rs, const FusedProjArgs &args,
                                Pattern p, int64_t M, int64_t K, hipStream_t stream, const char **name, bool query);

// The direct-load skinny MFMA forward with several 16-token tiles per
// workgroup (dense weights at 9-64 tokens over at least 6912 weight rows, or
// 2560 from 17 tokens, 2048 from 33: the shapes where it measured faster);
// hipErrorNotSupported for every other shape.
hipError_t launch_skinny_direct_tiles(const int8_t *Xq, const float *xs, const int32_t *rs, const FusedProjArgs &args,
                               Pattern p, int64_t M, int64_t K, hipStream_t stream, const char **name, bool query);

// The same kernel for one dense projection with K split over the workgroups
// (9-64 tokens, 49-384 chunks of 64, 1024-4096 weight rows, 2560 past 32
// tokens): int32 partials
// in the caller's workspace, then an elementwise pass; hipErrorNotSupported
// for every other shape.
hipError_t launch_skinny_direct_tiles_split(const int8_t *Xq, const float *xs, const int32_t *rs,
                                            const uint8_t *packed, const float *w_scale, Pattern p, int64_t M,
                                            int64_t N, int64_t K, float *Y, int32_t *acc, Scratch &scratch,
                                            hipStream_t stream, const char **name);

// Several dense projections at 17-64 tokens in one launch of the few-token
// GEMM's 32 x 32 tiles (where each alone would take them unsplit);
// hipErrorNotSupported for every other shape.
hipError_t launch_gemm_grouped(const int8_t *Xq, const float *xs, const int32_t *rs, FusedProjArgs args, Pattern p,
                               int64_t M, int64_t K, hipStream_t stream, const char **name, bool query);

// 2:4 weights at 1-16 tokens on the sparse MFMA (K % 128 == 0, K <= 16384;
// hipErrorNotSupported otherwise).
hipError_t launch_skinny_nm24_smfmac(const int8_t *Xq, const float *xs, const uint8_t *packed, const float *w_scale,
                                     int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream,
                                     bool query);

// H-BitLinear activations: block Hadamard transform (block B, a power of two
// <= 8192 dividing K), then 4-bit absmax codes in int8.
hipError_t launch_quant_act_h4(const float *X, int64_t M, int64_t K, int64_t B, int8_t *Xq, float *x_scale,
                               int32_t *x_rowsum, hipStream_t stream, const char **name);

// BitNet a4.8 hybrid activations: 2M rows (hi, lo per token), K <= 16384
// (hipErrorNotSupported beyond); and the sum of each row pair of the
// rescaled result.
hipError_t launch_quant_act_a48(const float *X, int64_t M, int64_t K, int64_t T, int8_t *Xq, float *x_scale,
                                int32_t *x_rowsum, hipStream_t stream, const char **name);
hipError_t launch_a48_combine(const float *Y2, int64_t M, int64_t N, float *Y, hipStream_t stream);

// beta: per-row binary64 |W| sums into `rowsum`, then one ordered sum.
hipError_t launch_absmean(const float *W, int64_t N, int64_t K, double *rowsum, float *w_scale,
                          hipStream_t stream);

// Ternarise (with d = beta + 1e-5 read from w_scale) and pack.
hipError_t launch_pack(const float *W, int64_t N, int64_t K, Pattern p, const float *w_scale,
                       uint8_t *packed, hipStream_t stream);

// N:M-masked ternary weights (1 <= n <= m, m in {4, 8, 16}) in the dense
// 2-bit layout (pruned: code 1).
hipError_t launch_pack_nm_dense(const float *W, int64_t N, int64_t K, int n, int m, const float *w_scale,
                                uint8_t *packed, hipStream_t stream);

// 2:4 weights in the trit-packed storage (a 6-bit code per group of 4
// inputs, 16 codes in 12 bytes; trit24.hip), with d = beta + 1e-5 read from
// w_scale.
hipError_t launch_pack_trit24(const float *W, int64_t N, int64_t K, const float *w_scale, uint8_t *packed,
                              hipStream_t stream);

// Forward on the trit-packed 2:4 weights: the one-token kernel (M = 1,
// K <= 16384), else the strings expanded to dense codes in the workspace and
// the dense forward.  Workspace and query handling as launch_forward.
hipError_t launch_forward_trit24(const int8_t *Xq, const float *xs, const int32_t *rs, const uint8_t *packed,
                                 const float *w_scale, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                                 Scratch &scratch, hipStream_t stream, const char **name);

// Forward.  Returns the name of the kernel variant in *name.  With
// scratch.query set nothing is launched and scratch.need receives the
// workspace bytes; otherwise a workspace smaller than the chosen kernels need
// makes it return hipErrorOutOfMemory before anything is launched.
hipError_t launch_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                          const uint8_t *packed, const float *w_scale, Pattern p, int64_t M,
                          int64_t N, int64_t K, float *Y, int32_t *acc, Scratch &scratch,
                          hipStream_t stream, const char **name);

}  // namespace bl
