// Low-rank down-projection t = x . l1 for the SVD / LoRA side branch, from the unrotated
// bf16 activations (ComfyUI-INT-Crush README, "Forward Pass" step 6: residual from L1/L2
// factors after the GEMM; "LoRA": residual branches live in unrotated activation space).
// t stays fp32; the linear kernels add t . l2 in their epilogue before the bias.
//
// A skinny GEMM (r <= 64 columns) that reads x once from HBM: a workgroup of 4 waves owns 32
// token rows; wave w takes row block w & 1 and the k half w >> 1 of every 512-k chunk.  Per
// chunk the workgroup stages l1[k0 .. k0+512, 0 .. r) transposed in LDS (row q = the 512
// values of column q), so both MFMA operands are 16-byte reads: the x fragment straight from
// global memory, the l1 fragment from LDS.  v_mfma_f32_16x16x32_bf16 (exact bf16 products,
// fp32 accumulation); the two k halves are summed through LDS in a fixed order.
#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int LR_KC = 512;           // k per staged chunk
constexpr int LR_PITCH = LR_KC + 8;  // bf16 per staged row (padding spreads the banks)

template <int RQ>  // column blocks of 16 (r <= 16 * RQ)
__global__ void __launch_bounds__(256)
k_lowrank_down(const uint16_t *__restrict__ x, const uint16_t *__restrict__ l1, int64_t M, int K, int r,
               float *__restrict__ t) {
    __shared__ __attribute__((aligned(16))) uint16_t lt[16 * RQ][LR_PITCH];
    __shared__ v4f red[2][RQ][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rb = wave & 1, kh = wave >> 1;
    const int lr = lane & 15, kg = lane >> 4;
    const int64_t m = min<int64_t>((int64_t)blockIdx.x * 32 + 16 * rb + lr, M - 1);
    const uint16_t *xr = x + m * K;

    v4f acc[RQ];
#pragma unroll
    for (int cb = 0; cb < RQ; ++cb) acc[cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // rows q >= r stay zero
    for (int e = tid; e < (16 * RQ - r) * LR_KC; e += 256) lt[r + e / LR_KC][e % LR_KC] = 0;
    const bool vec = (r & 7) == 0;
    const int G = (r + 7) / 8;  // groups of 8 columns per l1 row
    for (int k0 = 0; k0 < K; k0 += LR_KC) {
        __syncthreads();  // every wave is done with the previous chunk
        // l1 rows k0 .. k0+511 -> lt[q][k - k0] (zero past K): all loads of a thread first,
        // then its LDS writes
        constexpr int IT = LR_KC * 2 * RQ / 256;  // items (k, group) per thread: 8 columns each
#pragma unroll
        for (int h = 0; h < IT; h += 8) {
            uint16_t v[8][8];
            int kk[8], g[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + 256 * (h + i);
                kk[i] = idx / G;
                g[i] = idx % G;
                const int k = k0 + kk[i];
                const bool ok = kk[i] < LR_KC && k < K;
                if (vec) {
                    const uint4 w = ok ? *reinterpret_cast<const uint4 *>(l1 + (int64_t)k * r + 8 * g[i])
                                       : make_uint4(0, 0, 0, 0);
                    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[i][2 * j] = (uint16_t)(ww[j] & 0xffffu);
                        v[i][2 * j + 1] = (uint16_t)(ww[j] >> 16);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int q = 8 * g[i] + j;
                        v[i][j] = ok && q < r ? l1[(int64_t)k * r + q] : (uint16_t)0;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (kk[i] >= LR_KC) continue;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int q = 8 * g[i] + j;
                    if (q < r) lt[q][kk[i]] = v[i][j];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < LR_KC / 2 / 32; ++ks) {
            const int kl = kh * (LR_KC / 2) + 32 * ks + 8 * kg;  // this lane's 8 k in the chunk
            const int k = k0 + kl;
            uint4 xa = make_uint4(0, 0, 0, 0);
            if (k < K) xa = *reinterpret_cast<const uint4 *>(xr + k);  // K % 8 == 0: 8 valid k
            const bf8 a = __builtin_bit_cast(bf8, xa);
#pragma unroll
            for (int cb = 0; cb < RQ; ++cb) {
                const bf8 b = __builtin_bit_cast(bf8, *reinterpret_cast<const uint4 *>(&lt[16 * cb + lr][kl]));
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[cb], 0, 0, 0);
            }
        }
    }
    // k halves: wave (rb, 1) hands its partial to wave (rb, 0); 16x16 layout: lane l,
    // register v holds token 4 (l / 16) + v of the block, column l % 16
    if (kh == 1) {
#pragma unroll
        for (int cb = 0; cb < RQ; ++cb) red[rb][cb][lane] = acc[cb];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int cb = 0; cb < RQ; ++cb) {
        const v4f s = acc[cb] + red[rb][cb][lane];
        const int q = 16 * cb + lr;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t mm = (int64_t)blockIdx.x * 32 + 16 * rb + 4 * kg + v;
            if (mm < M && q < r) t[mm * r + q] = s[v];
        }
    }
}

}  // namespace

hipError_t launch_lowrank_down(const void *x, const void *l1, int64_t M, int64_t K, int r, float *t,
                               hipStream_t st) {
    if (M == 0) return hipSuccess;
    const unsigned grid = (unsigned)((M + 31) / 32);
    const uint16_t *xp = reinterpret_cast<const uint16_t *>(x), *lp = reinterpret_cast<const uint16_t *>(l1);
    if (r <= 16) hipLaunchKernelGGL(k_lowrank_down<1>, dim3(grid), dim3(256), 0, st, xp, lp, M, (int)K, r, t);
    else if (r <= 32) hipLaunchKernelGGL(k_lowrank_down<2>, dim3(grid), dim3(256), 0, st, xp, lp, M, (int)K, r, t);
    else if (r <= 48) hipLaunchKernelGGL(k_lowrank_down<3>, dim3(grid), dim3(256), 0, st, xp, lp, M, (int)K, r, t);
    else hipLaunchKernelGGL(k_lowrank_down<4>, dim3(grid), dim3(256), 0, st, xp, lp, M, (int)K, r, t);
    return hipGetLastError();
}

}  // namespace w4
