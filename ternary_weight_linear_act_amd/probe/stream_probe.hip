// Streaming-read floor of one launch on this GPU: the time a kernel that only
// reads a buffer takes, to set beside the one-token decode kernels, which
// read the same number of weight bytes.  Measurement support, not part of the
// BitLinear path: libstreamprobe.so is loaded only by bench.py's
// --stream-probe leg.
//
// Each thread issues all its 16-byte loads at once (coalesced per load
// instruction across the workgroup), folds them with xor so that no load is
// dead, and writes one word.  Launch shapes: T threads per workgroup, L loads
// per thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int T, int L>
__global__ __launch_bounds__(T) void stream_read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                        uint32_t *__restrict__ out)
{
    const int64_t base = (int64_t)blockIdx.x * T * L + threadIdx.x;
    u32x4 v[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t idx = base + (int64_t)i * T;
        v[i] = src[idx < n16 ? idx : n16 - 1];
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    out[(int64_t)blockIdx.x * T + threadIdx.x] = x;
}

template <int T, int L>
static int64_t launch(const void *src, int64_t bytes, uint32_t *out, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + (int64_t)T * L - 1) / ((int64_t)T * L);
    hipLaunchKernelGGL((stream_read_kernel<T, L>), dim3((unsigned)grid), dim3(T), 0, s,
                       static_cast<const u32x4 *>(src), n16, out);
    return hipGetLastError() == hipSuccess ? grid : -1;
}

extern "C" {

// Shapes: 0: 256 threads x 7 loads, 1: 256 x 4, 2: 256 x 2, 3: 256 x 1,
// 4: 512 x 2, 5: 1024 x 1.  bytes: a multiple of 16, > 0.  out: one word per
// * thread of the grid (at least stream_probe_out_words(bytes)).  Returns the
// number of workgroups launched, or -1.
int64_t stream_probe_launch(int shape, const void *src, int64_t bytes, uint32_t *out, hipStream_t s)
{
    if (bytes < 16 || bytes % 16) return -1;
    switch (shape) {
    case 0: return launch<256, 7>(src, bytes, out, s);
    case 1: return launch<256, 4>(src, bytes, out, s);
    case 2: return launch<256, 2>(src, bytes, out, s);
    case 3: return launch<256, 1>(src, bytes, out, s);
    case 4: return launch<512, 2>(src, bytes, out, s);
    case 5: return launch<1024, 1>(src, bytes, out, s);
    default: return -1;
    }
}

// Words of `out` a launch of `bytes` writes (the largest over the shapes).
int64_t stream_probe_out_words(int64_t bytes) { return (bytes / 16 + 255) / 256 * 256; }

int stream_probe_shapes(void) { return 6; }

}  // extern "C"
