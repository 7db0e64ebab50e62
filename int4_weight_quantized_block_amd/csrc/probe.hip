// Measurement probe, not part of the layer: the sustained dense int8 MFMA rate of the chip.
// Each wave keeps four independent 32x32 int32 accumulators busy with back-to-back
// v_mfma_i32_32x32x32_i8 (the shape the GEMM uses) on register operands that are either
// pseudo-random or constant; random operands toggle more of the datapath and draw more
// power, which is what real activation codes and weights do.
#include "common.h"
#include "kernels.h"

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

}  // namespace

hipError_t launch_mfma_rate(int64_t blocks, int iters, bool random_operands, int32_t *sink, hipStream_t st) {
    if (random_operands) hipLaunchKernelGGL(k_mfma_rate<true>, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
    else hipLaunchKernelGGL(k_mfma_rate<false>, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
    return hipGetLastError();
}

}  // namespace w4
