// Measurement probes, not part of the layer (built as their own library, libw4probe.so,
// declared in include/w4_probe.h):
//  - the sustained dense int8 MFMA rate of the chip: each wave keeps four independent 32x32
//    int32 accumulators busy with back-to-back v_mfma_i32_32x32x32_i8 (the shape the GEMM
//    uses) on register operands that are either pseudo-random or constant; random operands
//    toggle more of the datapath and draw more power, which is what real activation codes and
//    weights do;
//  - the HBM read rate a plain streaming kernel reaches on a buffer of a given size (the
//    practical ceiling of the HBM-bound small-M kernels, which stream ~25 MB per launch).
#include "w4_probe.h"

#include <hip/hip_runtime.h>

#include "common.h"

namespace w4 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {  // an integer hash (xorshift-multiply)
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <bool RANDOM>
__global__ void __launch_bounds__(256) k_mfma_rate(int iters, int32_t *__restrict__ sink) {
    v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t s = (uint32_t)(threadIdx.x * 977u + blockIdx.x * 131u + i * 7919u);
        if (RANDOM) {
            a[i] = v4i{(int)mix32(s), (int)mix32(s + 1), (int)mix32(s + 2), (int)mix32(s + 3)};
            b[i] = v4i{(int)mix32(s + 4), (int)mix32(s + 5), (int)mix32(s + 6), (int)mix32(s + 7)};
        } else {
            a[i] = v4i{(int)threadIdx.x, 1, 2, 3};
            b[i] = v4i{3, 2, 1, (int)blockIdx.x};
        }
    }
    v16i acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = v16i{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(i + it) & 3], b[i], acc[i], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[i][j];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Every thread reads 16-byte chunks t, t + T, t + 2T, ... of the buffer (T = threads in the
// grid, so each wave instruction reads 1 KB contiguous), 8 loads in flight per batch, and
// writes the XOR of what it read (so the loads cannot be dropped).
__global__ void __launch_bounds__(256) k_read_rate(const uint4 *__restrict__ src, int64_t chunks,
                                                   int32_t *__restrict__ sink) {
    const int64_t T = (int64_t)gridDim.x * 256;
    int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t x = 0;
    for (; c + 7 * T < chunks; c += 8 * T) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[c + u * T];
#pragma unroll
        for (int u = 0; u < 8; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; c < chunks; c += T) {
        const uint4 v = src[c];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = (int32_t)x;
}

}  // namespace
}  // namespace w4

extern "C" {

int w4_probe_mfma_rate(int64_t blocks, int iters, int random_operands, int32_t *sink, void *stream) {
    if (blocks < 1 || blocks > (int64_t)1 << 24 || iters < 1 || !sink || ((uintptr_t)sink & 15)) return 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (random_operands)
        hipLaunchKernelGGL(w4::k_mfma_rate<true>, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
    else
        hipLaunchKernelGGL(w4::k_mfma_rate<false>, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int w4_probe_read_rate(const void *src, int64_t bytes, int64_t blocks, int32_t *sink, void *stream) {
    if (!src || !sink || ((uintptr_t)src & 15) || ((uintptr_t)sink & 15) || bytes < 16 || bytes % 16 || blocks < 1 ||
        blocks > (int64_t)1 << 20)
        return 1;
    hipLaunchKernelGGL(w4::k_read_rate, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
