// Small-M (M <= 64) integer GEMM + dequant epilogue for gfx950: the HBM-bound regime.
//
// ComfyUI-INT-Crush README, "Inference / INT4" (INT8 GEMM with fused dequant on unpacked
// INT4 weights); the OrbitQuant notes of the same README and the batch-size-dependent
// backend selection ("Inference") separate a small-M streaming kernel from the large-M dense
// GEMM.  stable-diffusion.cpp PR #2010, "Summary": the packed nibbles are read as stored.
//
// At M <= 64 the layer reads ~0.5 byte of weight per 2*M ops, far below the MFMA ridge, so
// the kernel is organised around streaming each packed weight byte from HBM exactly once:
//  - a workgroup owns 16 weight rows and S waves; wave s takes k-windows s, s + S, ... of
//    256 k (two 16-byte loads per lane per window, two windows in flight per wave);
//  - the weights are the MFMA "A" operand (16 rows x 64 k per v_mfma_i32_16x16x64_i8),
//    the tokens the "B" operand, so one MFMA covers 16 rows x 16 tokens;
//  - the S partial 16 x 16 int32 tiles are summed through LDS in a fixed order, so the
//    result is exact and deterministic (no atomics);
//  - the epilogue is the same as the large-M kernel's.
#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

constexpr int kMaxWaves = 8;

__device__ __forceinline__ v4i unpack16(uint32_t d0, uint32_t d1) {
    v4i r;
    r[0] = (int)nib_evens16(d0);
    r[1] = (int)nib_odds16(d0);
    r[2] = (int)nib_evens16(d1);
    r[3] = (int)nib_odds16(d1);
    return r;
}

template <int ABITS, int MB>
__device__ __forceinline__ void window_mma(const LinearArgs &p, const uint4 (&wv)[2], int64_t kw, int kb,
                                           int lr, uint32_t bxor, v4i (&acc)[MB]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t d0 = half ? wv[h].z : wv[h].x;
            const uint32_t d1 = half ? wv[h].w : wv[h].y;
            const v4i wf = unpack16(d0 ^ bxor, d1 ^ bxor);
            const int64_t k16 = kw + h * 128 + kb * 32 + half * 16;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int64_t m = mb * 16 + lr;
                const bool ok = m < p.M && k16 < p.K;
                v4i af;
                if constexpr (ABITS == 8) {
                    const uint4 x = ok ? *reinterpret_cast<const uint4 *>(p.A + m * p.K + k16)
                                       : make_uint4(0, 0, 0, 0);
                    af = v4i{(int)bytes_evens(x.x, x.y), (int)bytes_odds(x.x, x.y),
                             (int)bytes_evens(x.z, x.w), (int)bytes_odds(x.z, x.w)};
                } else {
                    const uint2 x = ok ? *reinterpret_cast<const uint2 *>(p.A + m * (p.K / 2) + k16 / 2)
                                       : make_uint2(0, 0);
                    af = unpack16(x.x, x.y);
                }
                acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf, af, acc[mb], 0, 0, 0);
            }
        }
    }
}

template <int ABITS, int MB>
__global__ void __launch_bounds__(64 * kMaxWaves) k_gemv(LinearArgs p, int S) {
    __shared__ v4i red[kMaxWaves][MB][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63, s = tid >> 6;
    const int lr = lane & 15, kb = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t nrow = n0 + lr;
    const bool nok = nrow < p.N;
    const uint32_t bxor = p.zp ? 0x88888888u : 0u;
    const int64_t K = p.K;
    const int nwin = (int)((K + 255) / 256);
    const uint8_t *wrow = p.B + (nok ? nrow : 0) * (K / 2);

    v4i acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = v4i{0, 0, 0, 0};

    for (int w = s; w < nwin; w += 2 * S) {
        uint4 wv[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t kw = (int64_t)(w + u * S) * 256;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t kst = kw + h * 128 + kb * 32;
                const bool ok = nok && (w + u * S) < nwin && kst < K;
                wv[u][h] = ok ? *reinterpret_cast<const uint4 *>(wrow + kst / 2) : make_uint4(0, 0, 0, 0);
            }
        }
        window_mma<ABITS, MB>(p, wv[0], (int64_t)w * 256, kb, lr, bxor, acc);
        if (w + S < nwin) window_mma<ABITS, MB>(p, wv[1], (int64_t)(w + S) * 256, kb, lr, bxor, acc);
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[s][mb][lane] = acc[mb];
    __syncthreads();
    if (s != 0) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        v4i t = red[0][mb][lane];
        for (int q = 1; q < S; ++q) t += red[q][mb][lane];
        acc[mb] = t;
    }

    // ---- epilogue: lane holds weight rows 4 * kb + r (r = 0..3) for token lr of block mb
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t m = mb * 16 + lr;
        if (m >= p.M) continue;
        const float sxm = p.sx[m];
        const int rsm = p.zp ? p.rowsum[m] : 0;
        uint32_t ybits[4];
        int32_t yint[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + kb * 4 + r;
            if (n >= p.N) { ybits[r] = 0; yint[r] = 0; continue; }
            int v = acc[mb][r] >> SHIFT;
            if (p.zp) v += (8 - (int)p.zp[n]) * rsm;
            yint[r] = v;
            float y = (float)v * sxm * p.sw[n];
            if (p.lr_t) {
                const float *tr = p.lr_t + m * p.lr_r;
                float l = 0.0f;
                for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + n]), l);
                y += l;
            }
            if (p.bias) y += p.bias_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[n])
                                         : reinterpret_cast<const float *>(p.bias)[n];
            ybits[r] = f32_to_bf16(y);
        }
        const int64_t nb = n0 + kb * 4;
        if (p.y_i32) {
            int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nb + r < p.N) Y[nb + r] = yint[r];
        } else {
            uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y) + m * p.N;
            if (nb + 3 < p.N && (p.N & 3) == 0) {
                *reinterpret_cast<uint2 *>(Y + nb) =
                    make_uint2(ybits[0] | (ybits[1] << 16), ybits[2] | (ybits[3] << 16));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < p.N) Y[nb + r] = (uint16_t)ybits[r];
            }
        }
    }
}

template <int ABITS, int MB>
hipError_t launch_t(const LinearArgs &a, hipStream_t st) {
    const int nwin = (int)((a.K + 255) / 256);
    int S = nwin / 2;
    if (S < 1) S = 1;
    if (S > kMaxWaves) S = kMaxWaves;
    const unsigned grid = (unsigned)((a.N + 15) / 16);
    hipLaunchKernelGGL((k_gemv<ABITS, MB>), dim3(grid), dim3(64 * S), 0, st, a, S);
    return hipGetLastError();
}

template <int ABITS>
hipError_t dispatch_mb(const LinearArgs &a, hipStream_t st) {
    const int mb = (int)((a.M + 15) / 16);
    switch (mb) {
        case 1: return launch_t<ABITS, 1>(a, st);
        case 2: return launch_t<ABITS, 2>(a, st);
        case 3: return launch_t<ABITS, 3>(a, st);
        default: return launch_t<ABITS, 4>(a, st);
    }
}

}  // namespace

hipError_t launch_gemv(const LinearArgs &a, int act_bits, hipStream_t st) {
    if (a.M == 0) return hipSuccess;
    if (a.M > 64) return hipErrorInvalidValue;
    return act_bits == 8 ? dispatch_mb<8>(a, st) : dispatch_mb<4>(a, st);
}

}  // namespace w4
