// Small-M (M <= 64) integer GEMM + dequant epilogue for gfx950: the HBM-bound regime.
//
// ComfyUI-INT-Crush README, "Inference / INT4" (INT8 GEMM with fused dequant on unpacked
// INT4 weights) and "Inference" (the backend is chosen by batch size: a small-M streaming
// kernel vs the large-M dense GEMM, as in its OrbitQuant notes); stable-diffusion.cpp PR
// #2010, "Summary": the packed nibbles are read as stored.
//
// At M <= 64 the layer reads ~0.5 byte of weight per 2*M ops, far below the MFMA ridge, so
// the kernel is organised around streaming each packed weight byte from HBM exactly once,
// with as many bytes in flight as possible:
//  - a workgroup owns 16 weight rows and 4 waves; wave s owns the contiguous quarter
//    [s*K/4, (s+1)*K/4) of K, and every lane issues all of its weight loads (16 bytes each)
//    before the first multiply, so the HBM latency is paid once per workgroup;
//  - the weights are the MFMA "A" operand (16 rows x 64 k per v_mfma_i32_16x16x64_i8), the
//    tokens the "B" operand (one MFMA per 16 tokens); token fragments come from L2 with a
//    software prefetch several k-steps ahead;
//  - the 4 partial 16 x 16 int32 tiles are summed through LDS in a fixed order (exact and
//    deterministic, no atomics); wave 0 runs the epilogue (the large-M kernel's arithmetic).
#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxChunks = 32;  // 16-byte weight chunks per lane held in registers at once

__device__ __forceinline__ v4i evod(uint32_t d0, uint32_t d1) {
    return v4i{(int)nib_evens16(d0), (int)nib_odds16(d0), (int)nib_evens16(d1), (int)nib_odds16(d1)};
}

// Loads are unconditional, from clamped (always valid) addresses, and the value is masked
// afterwards: a guarded load would become a branch with its own wait, serialising the loads.
__device__ __forceinline__ uint4 mask4(uint4 v, bool ok) {
    return ok ? v : make_uint4(0, 0, 0, 0);
}

// Token fragment of one MFMA k-step (64 k; this lane: tokens mb*16 + lr, k in [k16, k16+16)).
template <int ABITS>
__device__ __forceinline__ uint4 load_act(const LinearArgs &p, int64_t m, int64_t k16) {
    const bool ok = m < p.M && k16 < p.K;
    const int64_t mc = ok ? m : 0, kc = ok ? k16 : 0;
    if constexpr (ABITS == 8) return mask4(*reinterpret_cast<const uint4 *>(p.A + mc * p.K + kc), ok);
    const uint2 x = *reinterpret_cast<const uint2 *>(p.A + mc * (p.K / 2) + kc / 2);
    return mask4(make_uint4(x.x, x.y, 0, 0), ok);
}

template <int ABITS>
__device__ __forceinline__ v4i act_operand(const uint4 &x) {
    if constexpr (ABITS == 8)
        return v4i{(int)bytes_evens(x.x, x.y), (int)bytes_odds(x.x, x.y), (int)bytes_evens(x.z, x.w),
                   (int)bytes_odds(x.z, x.w)};
    return evod(x.x, x.y);
}

// NCH = 16-byte weight chunks per lane (each covers 32 k = two MFMA k-steps).
template <int ABITS, int MB, int NCH, bool ASYM>
__global__ void __launch_bounds__(64 * kWaves) k_gemv(LinearArgs p) {
    __shared__ v4i red[kWaves][MB][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63, s = tid >> 6;
    const int lr = lane & 15, kb = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t nrow = n0 + lr;
    const bool nok = nrow < p.N;
    const int64_t K = p.K;
    // this wave's K range, in units of 128 k (one chunk for each of the 4 lane groups kb)
    const int64_t kq = ((K + 127) / 128 + kWaves - 1) / kWaves;  // 128-k steps per wave
    const int64_t kbeg = (int64_t)s * kq * 128;
    const uint8_t *wrow = p.B + (nok ? nrow : 0) * (K / 2);

    v4i acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = v4i{0, 0, 0, 0};

    // The wave's range is processed in segments of NCH chunks (one segment up to K = 16384).
    for (int64_t seg = 0; seg < kq; seg += NCH) {
        const int64_t nseg = min<int64_t>(NCH, kq - seg);
        const int64_t kseg = kbeg + 128 * seg;
        // ---- all weight chunks of this segment, issued at once.  Chunk c covers
        //      k in [kseg + 128 c + 32 kb, +32): 16 bytes of the packed row.
        uint4 wv[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t k = kseg + 128 * c + 32 * kb;
            const bool ok = c < nseg && k < K;
            wv[c] = mask4(*reinterpret_cast<const uint4 *>(wrow + (ok ? k / 2 : 0)), ok && nok);
        }
        // ---- k-steps: step t = 2 c + h uses k in [kseg + 128 c + 32 kb + 16 h, +16) per lane
        // token-fragment prefetch distance in k-steps: deep enough that the L2 round trips of the
        // fragments overlap (fewer registers per step as the token blocks grow)
        constexpr int PF = MB == 1 ? 16 : MB == 2 ? 8 : MB == 3 ? 5 : 4;
        uint4 ab[PF][MB];
        auto kstep = [&](int t) -> int64_t { return t < 2 * nseg ? kseg + 128 * (t >> 1) + 32 * kb + 16 * (t & 1) : K; };
#pragma unroll
        for (int t = 0; t < PF; ++t)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) ab[t][mb] = load_act<ABITS>(p, mb * 16 + lr, kstep(t));
        // keep every load above issued here, before the first multiply (the compiler would
        // otherwise sink each one to its use and serialise the HBM round trips)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < 2 * NCH; ++t) {
            if (t >= 2 * nseg) break;
            const int c = t >> 1, h = t & 1;
            uint32_t d0 = h ? wv[c].z : wv[c].x, d1 = h ? wv[c].w : wv[c].y;
            if constexpr (ASYM) {
                d0 ^= 0x88888888u;
                d1 ^= 0x88888888u;
            }
            const v4i wf = evod(d0, d1);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const v4i af = act_operand<ABITS>(ab[t % PF][mb]);
                acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf, af, acc[mb], 0, 0, 0);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) ab[t % PF][mb] = load_act<ABITS>(p, mb * 16 + lr, kstep(t + PF));
        }
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[s][mb][lane] = acc[mb];
    __syncthreads();
    if (s != 0) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        v4i t = red[0][mb][lane];
#pragma unroll
        for (int q = 1; q < kWaves; ++q) t += red[q][mb][lane];
        acc[mb] = t;
    }

    // ---- epilogue: lane holds weight rows 4 * kb + r (r = 0..3) for token lr of block mb
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    const int64_t nb = n0 + kb * 4;
    float swv[4], bsv[4];
    int zcv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t n = min<int64_t>(nb + r, p.N - 1);
        swv[r] = p.sw[n];
        bsv[r] = !p.bias ? 0.0f
                         : p.bias_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[n])
                                       : reinterpret_cast<const float *>(p.bias)[n];
        zcv[r] = ASYM ? 8 - (int)p.zp[n] : 0;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t m = mb * 16 + lr;
        if (m >= p.M) continue;
        const float sxm = p.sx[m];
        const int rsm = ASYM ? p.rowsum[m] : 0;
        uint32_t ybits[4];
        int32_t yint[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int v = acc[mb][r] >> SHIFT;
            if constexpr (ASYM) v += zcv[r] * rsm;
            yint[r] = v;
            float y = fmaf((float)v, sxm * swv[r], bsv[r]);
            if (p.lr_t) {
                const int64_t n = min<int64_t>(nb + r, p.N - 1);
                const float *tr = p.lr_t + m * p.lr_r;
                float l = 0.0f;
                for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + n]), l);
                y += l;
            }
            ybits[r] = f32_to_bf16(y);
        }
        if (p.y_i32) {
            int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nb + r < p.N) Y[nb + r] = yint[r];
        } else {
            uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y) + m * p.N;
            if (nb + 3 < p.N && (p.N & 3) == 0) {
                *reinterpret_cast<uint2 *>(Y + nb) = make_uint2(ybits[0] | (ybits[1] << 16), ybits[2] | (ybits[3] << 16));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < p.N) Y[nb + r] = (uint16_t)ybits[r];
            }
        }
    }
}

template <int ABITS, int MB, int NCH>
hipError_t launch_t(const LinearArgs &a, hipStream_t st) {
    const unsigned grid = (unsigned)((a.N + 15) / 16);
    if (a.zp)
        hipLaunchKernelGGL((k_gemv<ABITS, MB, NCH, true>), dim3(grid), dim3(64 * kWaves), 0, st, a);
    else
        hipLaunchKernelGGL((k_gemv<ABITS, MB, NCH, false>), dim3(grid), dim3(64 * kWaves), 0, st, a);
    return hipGetLastError();
}

template <int ABITS, int MB>
hipError_t dispatch_k(const LinearArgs &a, hipStream_t st) {
    const int64_t kq = ((a.K + 127) / 128 + kWaves - 1) / kWaves;  // chunks per lane
    if (kq <= 4) return launch_t<ABITS, MB, 4>(a, st);
    if (kq <= 8) return launch_t<ABITS, MB, 8>(a, st);
    if (kq <= 16) return launch_t<ABITS, MB, 16>(a, st);
    return launch_t<ABITS, MB, kMaxChunks>(a, st);
}

template <int ABITS>
hipError_t dispatch_mb(const LinearArgs &a, hipStream_t st) {
    const int mb = (int)((a.M + 15) / 16);
    switch (mb) {
        case 1: return dispatch_k<ABITS, 1>(a, st);
        case 2: return dispatch_k<ABITS, 2>(a, st);
        case 3: return dispatch_k<ABITS, 3>(a, st);
        default: return dispatch_k<ABITS, 4>(a, st);
    }
}

}  // namespace

hipError_t launch_gemv(const LinearArgs &a, int act_bits, hipStream_t st) {
    if (a.M == 0) return hipSuccess;
    if (a.M > 64) return hipErrorInvalidValue;
    return act_bits == 8 ? dispatch_mb<8>(a, st) : dispatch_mb<4>(a, st);
}

}  // namespace w4
