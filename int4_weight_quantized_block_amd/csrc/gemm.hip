// Integer GEMM + fused dequant epilogue on the gfx950 int8 matrix cores (M > 64).
//
// ComfyUI-INT-Crush README, "Inference / INT4": unpack INT4 to INT8, INT8 GEMM with fused
// dequant (W4A8: "INT4->INT8 unpack -> dynamic-quantize activations -> fused INT8 GEMM +
// dequant"); "Forward Pass" steps 5 and 6 (GEMM, then the low-rank residual).
// stable-diffusion.cpp PR #2010, "Summary": the packed nibbles stream to the kernel as
// stored, with no load-time re-blocking, so this kernel reads the canonical [N, K/2] bytes.
//
// acc[m, n] = sum_k q[m, k] * (c[n, k] - z[n]) exactly, in int32.
//
// Unpacking.  A signed nibble moved to the high half of a byte is the int8 value 16 * c,
// so a packed dword d gives two MFMA operand dwords with one shift and two masks:
// (d << 4) & 0xF0F0F0F0 holds the even-k codes, d & 0xF0F0F0F0 the odd-k codes.
// Asymmetric (unsigned) nibbles are XORed with 8 first, which turns c into c - 8; the
// epilogue adds (8 - z[n]) * rowsum[m].  int8 activation codes are reordered into the same
// even/odd k order with v_perm when they are staged into LDS; int4 activation codes unpack
// exactly like the weights (16 * q).  The accumulator then holds 16 * acc (int8 codes) or
// 256 * acc (int4 codes), exact in int32 for K <= 65536, and is shifted back.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (2 x 2 waves of 64 x 64, i.e.
// 4 x 4 blocks of v_mfma_i32_16x16x64_i8), K staged in LDS 128 at a time, double-buffered:
// the next k-tile's global loads are in flight while the current one is multiplied.
// LDS rows are padded (144 / 80 bytes) so the 16-byte (A) and 8-byte (B) fragment reads of
// 16 consecutive rows hit distinct banks.
#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int B_STRIDE = BK / 2 + 16;  // 80 bytes per packed weight row in LDS

template <int ABITS>
struct Tile {
    static constexpr int A_ROW = ABITS == 8 ? BK : BK / 2;  // bytes of a row per k-tile
    static constexpr int A_STRIDE = A_ROW + 16;
    static constexpr int A_BYTES = BM * A_STRIDE;
    static constexpr int B_BYTES = BN * B_STRIDE;
    static constexpr int STAGE = A_BYTES + B_BYTES;
};

__device__ __forceinline__ v4i unpack16(uint32_t d0, uint32_t d1) {
    v4i r;
    r[0] = (int)nib_evens16(d0);
    r[1] = (int)nib_odds16(d0);
    r[2] = (int)nib_evens16(d1);
    r[3] = (int)nib_odds16(d1);
    return r;
}

// Global -> register part of one k-tile.  Thread layout: row = tid / 2, half = tid % 2.
template <int ABITS>
struct Loader {
    uint4 a[ABITS == 8 ? 4 : 2];
    uint4 b[2];

    __device__ __forceinline__ void load(const LinearArgs &p, int64_t m0, int64_t n0, int kt) {
        const int tid = threadIdx.x;
        const int r = tid >> 1, h = tid & 1;
        const int64_t K = p.K;
        // activation rows
        {
            const int64_t m = m0 + r;
            constexpr int NA = ABITS == 8 ? 4 : 2;
            const int64_t kb = ABITS == 8 ? (int64_t)kt * BK + h * 64 : ((int64_t)kt * BK + h * 64) / 2;
            const int64_t rowb = ABITS == 8 ? K : K / 2;
            const bool ok = m < p.M && (int64_t)kt * BK + h * 64 < K;
            const uint4 *src = reinterpret_cast<const uint4 *>(p.A + (ok ? m * rowb + kb : 0));
#pragma unroll
            for (int j = 0; j < NA; ++j) a[j] = ok ? src[j] : make_uint4(0, 0, 0, 0);
        }
        // weight rows (packed, 64 bytes per k-tile, 32 per half)
        {
            const int64_t n = n0 + r;
            const bool ok = n < p.N && (int64_t)kt * BK + h * 64 < K;
            const uint4 *src =
                reinterpret_cast<const uint4 *>(p.B + (ok ? n * (K / 2) + (int64_t)kt * (BK / 2) + h * 32 : 0));
            b[0] = ok ? src[0] : make_uint4(0, 0, 0, 0);
            b[1] = ok ? src[1] : make_uint4(0, 0, 0, 0);
        }
    }

    __device__ __forceinline__ void store(uint8_t *stage) {
        const int tid = threadIdx.x;
        const int r = tid >> 1, h = tid & 1;
        uint8_t *As = stage + r * Tile<ABITS>::A_STRIDE;
        if constexpr (ABITS == 8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 x = a[j];
                uint4 y;
                y.x = bytes_evens(x.x, x.y);
                y.y = bytes_odds(x.x, x.y);
                y.z = bytes_evens(x.z, x.w);
                y.w = bytes_odds(x.z, x.w);
                *reinterpret_cast<uint4 *>(As + h * 64 + j * 16) = y;
            }
        } else {
            *reinterpret_cast<uint4 *>(As + h * 32) = a[0];
            *reinterpret_cast<uint4 *>(As + h * 32 + 16) = a[1];
        }
        uint8_t *Bs = stage + Tile<ABITS>::A_BYTES + r * B_STRIDE;
        *reinterpret_cast<uint4 *>(Bs + h * 32) = b[0];
        *reinterpret_cast<uint4 *>(Bs + h * 32 + 16) = b[1];
    }
};

template <int ABITS>
__global__ void __launch_bounds__(kThreads) k_gemm(LinearArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using TL = Tile<ABITS>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const uint32_t bxor = p.zp ? 0x88888888u : 0u;
    const int nk = (int)((p.K + BK - 1) / BK);

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    Loader<ABITS> ld;
    ld.load(p, m0, n0, 0);
    ld.store(smem);
    __syncthreads();

    const int lr = lane & 15, kb = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
        uint8_t *cur = smem + (kt & 1) * TL::STAGE;
        if (kt + 1 < nk) ld.load(p, m0, n0, kt + 1);
#pragma unroll
        for (int s = 0; s < BK / 64; ++s) {
            v4i af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint8_t *ap = cur + (wm * 64 + i * 16 + lr) * TL::A_STRIDE;
                if constexpr (ABITS == 8) {
                    const uint4 x = *reinterpret_cast<const uint4 *>(ap + s * 64 + kb * 16);
                    af[i] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
                } else {
                    const uint2 x = *reinterpret_cast<const uint2 *>(ap + s * 32 + kb * 8);
                    af[i] = unpack16(x.x, x.y);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint8_t *bp = cur + TL::A_BYTES + (wn * 64 + j * 16 + lr) * B_STRIDE;
                const uint2 x = *reinterpret_cast<const uint2 *>(bp + s * 32 + kb * 8);
                bf[j] = unpack16(x.x ^ bxor, x.y ^ bxor);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) ld.store(smem + ((kt + 1) & 1) * TL::STAGE);
        __syncthreads();
    }

    // ---- epilogue: lane holds rows 4 * (lane / 16) + r, column lane % 16 of each block
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + j * 16 + lr;
        if (n >= p.N) continue;
        const float swn = p.sw[n];
        const int zc = p.zp ? 8 - (int)p.zp[n] : 0;
        float bn = 0.0f;
        if (p.bias) bn = p.bias_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[n])
                                     : reinterpret_cast<const float *>(p.bias)[n];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + i * 16 + kb * 4 + r;
                if (m >= p.M) continue;
                int v = acc[i][j][r] >> SHIFT;
                if (p.zp) v += zc * p.rowsum[m];
                if (p.y_i32) {
                    reinterpret_cast<int32_t *>(p.Y)[m * p.N + n] = v;
                } else {
                    float y = (float)v * p.sx[m] * swn;
                    if (p.lr_t) {
                        const float *tr = p.lr_t + m * p.lr_r;
                        float l = 0.0f;
                        for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + n]), l);
                        y += l;
                    }
                    y += bn;
                    reinterpret_cast<uint16_t *>(p.Y)[m * p.N + n] = (uint16_t)f32_to_bf16(y);
                }
            }
        }
    }
}

template <int ABITS>
hipError_t launch_t(const LinearArgs &a, hipStream_t st) {
    const size_t lds = 2 * (size_t)Tile<ABITS>::STAGE;
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL((k_gemm<ABITS>), grid, dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const LinearArgs &a, int act_bits, hipStream_t st) {
    if (a.M == 0) return hipSuccess;
    return act_bits == 8 ? launch_t<8>(a, st) : launch_t<4>(a, st);
}

}  // namespace w4
