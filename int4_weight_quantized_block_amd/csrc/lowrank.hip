// Low-rank down-projection t = x . l1 for the SVD / LoRA side branch, from the unrotated
// bf16 activations (ComfyUI-INT-Crush README, "Forward Pass" step 6: residual from L1/L2
// factors after the GEMM; "LoRA": residual branches live in unrotated activation space).
// t stays fp32; the linear kernels add t . l2 in their epilogue before the bias.
//
// A workgroup of 256 threads handles 4 token rows; lane j of a row's 64 lanes owns output
// column j (j < r).  x[m, k] is broadcast across the row's lanes, l1[k, :] is a contiguous
// row read by consecutive lanes.  fp32 accumulation of exact bf16 x bf16 products.
#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

__global__ void __launch_bounds__(256)
k_lowrank_down(const uint16_t *__restrict__ x, const uint16_t *__restrict__ l1, int64_t M, int K, int r,
               float *__restrict__ t) {
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int j = threadIdx.x & 63;
    if (m >= M || j >= r) return;
    const uint16_t *xr = x + m * K;
    float acc = 0.0f;
    for (int k = 0; k < K; ++k) acc = fmaf(bf16_to_f32(xr[k]), bf16_to_f32(l1[(int64_t)k * r + j]), acc);
    t[m * r + j] = acc;
}

}  // namespace

hipError_t launch_lowrank_down(const void *x, const void *l1, int64_t M, int64_t K, int r, float *t,
                               hipStream_t st) {
    if (M == 0) return hipSuccess;
    const unsigned grid = (unsigned)((M + 3) / 4);
    hipLaunchKernelGGL(k_lowrank_down, dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint16_t *>(l1), M,
                       (int)K, r, t);
    return hipGetLastError();
}

}  // namespace w4
