// Low-rank down-projection t = x . l1^T for the SVD / LoRA side branch, from the unrotated
// bf16 activations (ComfyUI-INT-Crush README, "Forward Pass" step 6: residual from L1/L2
// factors after the GEMM; "LoRA": residual branches live in unrotated activation space).
// l1 is stored rank-major, [r, K] (row q = the q-th down-projection vector), so every MFMA
// operand is 16 contiguous bytes.  t stays fp32; the linear kernels add t . l2 in their
// epilogue before the bias.
//
// A skinny GEMM (r <= 64 columns) bound by reading x once from HBM.  A workgroup of 4 waves
// owns 16 token rows; wave w takes the 32-k steps w, w + 4, w + 8, ... of K.  Each wave
// streams its steps through its own LDS ring with direct global -> LDS loads (one 1 KB load
// for the 16 x 32 x-fragment, one per 16 ranks for l1), D steps ahead, and every lane reads
// back only the bytes it loaded itself, so no barrier is needed until the fixed-order sum of
// the four waves' partial tiles.  v_mfma_f32_16x16x32_bf16: exact bf16 products, fp32
// accumulation.
#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kLrWaves = 4;
constexpr int kLrSlotsBytes = 12 * 1024;  // LDS ring per wave

template <int RQ>
struct LrL {
    static constexpr int SLOT = (1 + RQ) * 1024;  // x fragment + RQ l1 fragments
    static constexpr int D = kLrSlotsBytes / SLOT;
    static constexpr int LPS = 1 + RQ;  // loads per step
    static constexpr int RING = kLrWaves * D * SLOT;
    static constexpr int RED = kLrWaves * RQ * 64 * 16;
    static constexpr int LDS = RING > RED ? RING : RED;
    static_assert(D >= 2 && (D - 1) * LPS <= 63, "low-rank ring");
};

template <int RQ>  // blocks of 16 ranks (r <= 16 RQ)
__global__ void __launch_bounds__(64 * kLrWaves) k_lowrank_down(const uint16_t *__restrict__ x,
                                                                const uint16_t *__restrict__ l1, int64_t M, int K,
                                                                int r, float *__restrict__ t) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = LrL<RQ>;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, kg = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int64_t mc = min<int64_t>(m0 + lr, M - 1) - m0;  // rows past M: clamped, never stored
    const int nks = (K + 31) / 32;
    const int nmine = (nks - wave + kLrWaves - 1) / kLrWaves;  // this wave's steps
    const uint32_t ring = lds_addr(smem) + (uint32_t)(wave * L::D * L::SLOT);
    const uint64_t xb = (uint64_t)(x + m0 * K);

    // step j of this wave (k-step wave + 4 j) into ring slot j % D; k past K reads the last 8
    // valid k (K % 8 == 0) and is masked below
    auto issue = [&](int j) __attribute__((always_inline)) {
        const uint32_t slot = ring + (uint32_t)((j % L::D) * L::SLOT);
        const int k = min((wave + kLrWaves * j) * 32 + 8 * kg, K - 8);
        gl_lds16_so(xb, (uint32_t)((mc * K + k) * 2), slot);
#pragma unroll
        for (int cb = 0; cb < RQ; ++cb) {
            const int q = min(16 * cb + lr, r - 1);  // ranks past r: clamped, never stored
            gl_lds16_so((uint64_t)l1, (uint32_t)(((int64_t)q * K + k) * 2), slot + 1024 * (1 + cb));
        }
    };

    v4f acc[RQ];
#pragma unroll
    for (int cb = 0; cb < RQ; ++cb) acc[cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < L::D; ++j)
        if (j < nmine) issue(j);
    for (int j = 0; j < nmine; ++j) {
        wait_rem<L::LPS, L::D - 1>(min(L::D - 1, nmine - 1 - j));
        const uint8_t *sl = smem + wave * L::D * L::SLOT + (j % L::D) * L::SLOT;
        uint4 xa = *reinterpret_cast<const uint4 *>(sl + 16 * lane);
        uint4 lb[RQ];
#pragma unroll
        for (int cb = 0; cb < RQ; ++cb) lb[cb] = *reinterpret_cast<const uint4 *>(sl + 1024 * (1 + cb) + 16 * lane);
        wait_lgkmcnt0();  // this lane's reads of the slot are complete before it is refilled
        if (j + L::D < nmine) issue(j + L::D);
        if ((wave + kLrWaves * j) * 32 + 8 * kg >= K) xa = make_uint4(0, 0, 0, 0);
        const bf8 a = __builtin_bit_cast(bf8, xa);
#pragma unroll
        for (int cb = 0; cb < RQ; ++cb)
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf8, lb[cb]), acc[cb], 0, 0, 0);
    }

    // fixed-order sum of the four waves' tiles; 16x16 layout: lane l, register v holds token
    // 4 (l / 16) + v of the block, rank 16 cb + l % 16
    __syncthreads();  // every wave is done with its ring
    v4f *red = reinterpret_cast<v4f *>(smem);
#pragma unroll
    for (int cb = 0; cb < RQ; ++cb) red[(wave * RQ + cb) * 64 + lane] = acc[cb];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int cb = 0; cb < RQ; ++cb) {
        v4f s = red[cb * 64 + lane];
#pragma unroll
        for (int w = 1; w < kLrWaves; ++w) s += red[(w * RQ + cb) * 64 + lane];
        const int q = 16 * cb + lr;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t mm = m0 + 4 * kg + v;
            if (mm < M && q < r) t[mm * r + q] = s[v];
        }
    }
}

template <int RQ>
hipError_t launch_rq(const uint16_t *x, const uint16_t *l1, int64_t M, int64_t K, int r, float *t, hipStream_t st) {
    using L = LrL<RQ>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_lowrank_down<RQ>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS);
    if (attr != hipSuccess) return attr;
    const unsigned grid = (unsigned)((M + 15) / 16);
    hipLaunchKernelGGL(k_lowrank_down<RQ>, dim3(grid), dim3(64 * kLrWaves), L::LDS, st, x, l1, M, (int)K, r, t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lowrank_down(const void *x, const void *l1, int64_t M, int64_t K, int r, float *t,
                               hipStream_t st) {
    if (M == 0) return hipSuccess;
    const uint16_t *xp = reinterpret_cast<const uint16_t *>(x), *lp = reinterpret_cast<const uint16_t *>(l1);
    if (r <= 16) return launch_rq<1>(xp, lp, M, K, r, t, st);
    if (r <= 32) return launch_rq<2>(xp, lp, M, K, r, t, st);
    if (r <= 48) return launch_rq<3>(xp, lp, M, K, r, t, st);
    return launch_rq<4>(xp, lp, M, K, r, t, st);
}

}  // namespace w4
