// Low-rank down-projection t = x . l1^T for the SVD / LoRA side branch, from the unrotated
// bf16 activations (ComfyUI-INT-Crush README, "Forward Pass" step 6: residual from L1/L2
// factors after the GEMM; "LoRA": residual branches live in unrotated activation space).
// l1 is stored rank-major, [r, K] (row q = the q-th down-projection vector), so every MFMA
// operand is 16 contiguous bytes.  t stays fp32; the linear kernels add t . l2 in their
// epilogue before the bias.
//
// A skinny GEMM (r <= 64 columns) bound by moving bytes: x once from HBM, and l1 once per
// workgroup from L2.  A workgroup of 4 waves owns 32 tokens, so each l1 byte it reads serves
// 32 tokens (half the l1 traffic of 16-token blocks, which moved twice as many l1 bytes as
// x bytes at r = 32).  Wave (rb, h) multiplies token block rb with the k half h of every
// 64-k step.  The step's bytes arrive in a shared LDS ring, D steps ahead, through direct
// global -> LDS loads: each wave loads its own x fragment and a share of the l1 fragments
// (which both row blocks use), and one barrier per step makes everybody's loads of the step
// visible and frees the slot of the step before.  v_mfma_f32_16x16x32_bf16: exact bf16
// products, fp32 accumulation; the two k halves are summed through LDS in a fixed order.
#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kLrD = 8;  // ring depth in 64-k steps

template <int RQ>  // blocks of 16 ranks: 1, 2 or 4 (r <= 16 RQ)
struct LrL {
    static constexpr int LB = RQ < 2 ? 1 : RQ / 2;   // l1 fragments a wave loads per step
    static constexpr int LPS = 1 + LB;                // loads per wave and step
    static constexpr int SLOT = (4 + 2 * RQ) * 1024;  // x [rb][h], l1 [cb][h]: 1 KB each
    static constexpr int LDS = kLrD * SLOT;
    static_assert((kLrD - 2) * LPS <= 63 && LDS <= 160 * 1024 && LDS >= 2 * RQ * 64 * 16, "low-rank ring");
};

template <int RQ>
__global__ void __launch_bounds__(256) k_lowrank_down(const uint16_t *__restrict__ x, const uint16_t *__restrict__ l1,
                                                      int64_t M, int K, int r, float *__restrict__ t, int64_t ldt) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = LrL<RQ>;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rb = wave & 1, h = wave >> 1;
    const int lr = lane & 15, kg = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * 32;
    const int64_t mc = min<int64_t>(m0 + 16 * rb + lr, M - 1) - m0;  // rows past M: clamped, never stored
    const int nsteps = (K + 63) / 64;
    const uint32_t base = lds_addr(smem);
    const uint64_t xb = (uint64_t)(x + m0 * K);

    // step s into ring slot s % D: this wave's x fragment (16 tokens x 32 k) and its share of
    // the l1 fragments (16 ranks x 32 k; with RQ = 1 both row blocks load the same one).  k
    // past K reads the last 8 valid k (K % 8 == 0) and the x operand is masked below.
    auto issue = [&](int s) __attribute__((always_inline)) {
        const uint32_t slot = base + (uint32_t)((s % kLrD) * L::SLOT);
        const int k = min(s * 64 + 32 * h + 8 * kg, K - 8);
        gl_lds16_so(xb, (uint32_t)((mc * K + k) * 2), slot + 1024 * (2 * rb + h));
#pragma unroll
        for (int u = 0; u < L::LB; ++u) {
            const int cb = RQ < 2 ? 0 : 2 * u + rb;
            const int q = min(16 * cb + lr, r - 1);  // ranks past r: clamped, never stored
            gl_lds16_so((uint64_t)l1, (uint32_t)(((int64_t)q * K + k) * 2), slot + 4096 + 1024 * (2 * cb + h));
        }
    };

    v4f acc[RQ];
#pragma unroll
    for (int cb = 0; cb < RQ; ++cb) acc[cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < kLrD - 1; ++s)
        if (s < nsteps) issue(s);
    for (int i = 0; i < nsteps; ++i) {
        wait_rem<L::LPS, kLrD - 2>(min(kLrD - 2, nsteps - 1 - i));  // this wave's loads of step i
        __syncthreads();  // everybody's loads of step i have landed; step i - 1 is read by all
        if (i + kLrD - 1 < nsteps) issue(i + kLrD - 1);  // into the slot of step i - 1
        const uint8_t *sl = smem + (i % kLrD) * L::SLOT;
        uint4 xa = *reinterpret_cast<const uint4 *>(sl + 1024 * (2 * rb + h) + 16 * lane);
        if (i * 64 + 32 * h + 8 * kg >= K) xa = make_uint4(0, 0, 0, 0);
        const bf8 a = __builtin_bit_cast(bf8, xa);
#pragma unroll
        for (int cb = 0; cb < RQ; ++cb) {
            const uint4 lb = *reinterpret_cast<const uint4 *>(sl + 4096 + 1024 * (2 * cb + h) + 16 * lane);
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf8, lb), acc[cb], 0, 0, 0);
        }
    }

    // k halves: wave (rb, 1) hands its tile to wave (rb, 0); 16x16 layout: lane l, register v
    // holds token 4 (l / 16) + v of the block, rank 16 cb + l % 16
    __syncthreads();  // every wave is done with the ring
    v4f *red = reinterpret_cast<v4f *>(smem);
    if (h == 1) {
#pragma unroll
        for (int cb = 0; cb < RQ; ++cb) red[(rb * RQ + cb) * 64 + lane] = acc[cb];
    }
    __syncthreads();
    if (h == 1) return;
#pragma unroll
    for (int cb = 0; cb < RQ; ++cb) {
        const v4f s = acc[cb] + red[(rb * RQ + cb) * 64 + lane];
        const int q = 16 * cb + lr;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t mm = m0 + 16 * rb + 4 * kg + v;
            if (mm < M && q < r) t[mm * ldt + q] = s[v];
        }
    }
}

template <int RQ>
hipError_t launch_rq(const uint16_t *x, const uint16_t *l1, int64_t M, int64_t K, int r, float *t, int64_t ldt,
                     hipStream_t st) {
    using L = LrL<RQ>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_lowrank_down<RQ>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS);
    if (attr != hipSuccess) return attr;
    const unsigned grid = (unsigned)((M + 31) / 32);
    hipLaunchKernelGGL(k_lowrank_down<RQ>, dim3(grid), dim3(256), L::LDS, st, x, l1, M, (int)K, r, t, ldt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lowrank_down(const void *x, const void *l1, int64_t M, int64_t K, int r, float *t,
                               hipStream_t st, int64_t ldt) {
    if (M == 0) return hipSuccess;
    if (ldt == 0) ldt = r;
    const uint16_t *xp = reinterpret_cast<const uint16_t *>(x), *lp = reinterpret_cast<const uint16_t *>(l1);
    if (r <= 16) return launch_rq<1>(xp, lp, M, K, r, t, ldt, st);
    if (r <= 32) return launch_rq<2>(xp, lp, M, K, r, t, ldt, st);
    return launch_rq<4>(xp, lp, M, K, r, t, ldt, st);  // r <= 64
}

}  // namespace w4
