// Host-side launchers of the HIP kernels (internal to libbitlinear).
// Shapes and pointers are validated by the C-ABI layer before these run.
#pragma once

#include "common.hpp"

namespace bl {

// Per-row absmax int8 quantisation (one workgroup per row).
hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *x_scale,
                            int32_t *x_rowsum, hipStream_t stream);

// The same on rows transformed first (ReLU^2 gate and/or RMSNorm; tr.up and
// tr.gamma NULL for none).
hipError_t launch_quant_act_ex(const float *X, ActTransform tr, int64_t M, int64_t K, int8_t *Xq,
                               float *x_scale, int32_t *x_rowsum, hipStream_t stream);

// Largest token count of the skinny MFMA forward (tiles of 16 tokens past 16).
constexpr int64_t kSkinnyMaxM = 64;

// 2:4 weights at 1-16 tokens on the sparse MFMA (K % 128 == 0, K <= 16384;
// hipErrorNotSupported otherwise).
hipError_t launch_skinny_nm24_smfmac(const int8_t *Xq, const float *xs, const uint8_t *packed, const float *w_scale,
                                     int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream);

// H-BitLinear activations: block Hadamard transform (block B, a power of two
// <= 8192 dividing K), then 4-bit absmax codes in int8.
hipError_t launch_quant_act_h4(const float *X, int64_t M, int64_t K, int64_t B, int8_t *Xq, float *x_scale,
                               int32_t *x_rowsum, hipStream_t stream, const char **name);

// beta: per-row binary64 |W| sums into `rowsum`, then one ordered sum.
hipError_t launch_absmean(const float *W, int64_t N, int64_t K, double *rowsum, float *w_scale,
                          hipStream_t stream);

// Ternarise (with d = beta + 1e-5 read from w_scale) and pack.
hipError_t launch_pack(const float *W, int64_t N, int64_t K, Pattern p, const float *w_scale,
                       uint8_t *packed, hipStream_t stream);

// Forward.  Returns the name of the kernel variant in *name.
hipError_t launch_forward(const int8_t *Xq, const float *x_scale, const int32_t *x_rowsum,
                          const uint8_t *packed, const float *w_scale, Pattern p, int64_t M,
                          int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t stream,
                          const char **name);

}  // namespace bl
