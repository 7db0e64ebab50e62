// Offline weight step for gfx950: rotate each weight row along K in groups of g, quantize it
// per output row to int4 (symmetric, or asymmetric with a zero point) and pack two codes
// per byte along K, low nibble = even k.
//
// ComfyUI-INT-Crush README, "Weight Format" (uint8, two values per byte, scales per output
// row) and "Workflow" (the converter quantizes once, offline); stable-diffusion.cpp PR #2010,
// "Summary" (convrot_w4a4 / asym_w4a8_int8: packed nibbles plus row scales) and the
// discussion's shape report (the packed input dimension is K / 2); TINT4 README, v1.1
// section 5 (codes, scale and zero point per quantized linear).
//
// One workgroup per weight row.  The row is processed in slabs of 4096 elements staged in
// LDS as fp64: pass 1 transforms each slab and reduces max|w'| (or min/max), pass 2
// transforms it again and quantizes.  Not on the timed path, so it favours plainness: the
// division w' / s is the IEEE fp64 quotient and rint is round-half-to-even, exactly as in
// the definition.  Rotation sizes 16, 64, 256, 1024 and 4096 (ComfyUI-INT-Crush README,
// "Nodes": rot_size), and G = 1 for no rotation; every size divides the slab, so groups
// never straddle two slabs.
//
// Grouped-scale format (ComfyUI-INT-Crush README, "Weight Format": weight_scale fp16
// [out, num_groups]): symmetric codes with one fp16 scale per row and run of gw inputs,
// s = fp16(max|w'| / 7) rounded once from fp64, c = clamp(rint(w' / s), -8, 7).
#include <hip/hip_fp16.h>

#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

constexpr int kSlab = 4096;
constexpr int kThreads = 256;

template <int G, bool F32IN>
__device__ void load_rotate_slab(const void *W, int64_t n, int K, int k0, int len, double *buf) {
    const int tid = threadIdx.x;
    for (int k = tid; k < len; k += kThreads) {
        const int64_t idx = n * K + k0 + k;
        buf[k] = F32IN ? (double)reinterpret_cast<const float *>(W)[idx]
                       : (double)bf16_to_f32(reinterpret_cast<const uint16_t *>(W)[idx]);
    }
    __syncthreads();
    // butterflies for h = 1 .. G/2: pairs (i, i + h) never leave their G-aligned group
    for (int h = 1; h < G; h <<= 1) {
        for (int p = tid; p < len / 2; p += kThreads) {
            const int i = ((p & ~(h - 1)) << 1) | (p & (h - 1));
            const double a = buf[i], b = buf[i + h];
            buf[i] = a + b;
            buf[i + h] = a - b;
        }
        __syncthreads();
    }
    constexpr double INV_SQRT_G = G == 1 ? 1.0 : G == 16 ? 0.25 : G == 64 ? 0.125 : G == 256 ? 0.0625
                                  : G == 1024 ? 0.03125 : 0.015625;
    static_assert(G == 1 || G == 16 || G == 64 || G == 256 || G == 1024 || G == 4096, "rotation size");
    for (int k = tid; k < len; k += kThreads) buf[k] *= INV_SQRT_G;  // exact
    __syncthreads();
}

// Nearest fp16 of a finite non-negative double, ties to even, in one rounding: 11 significant
// bits above 2^-14, the subnormal quantum 2^-24 below it; 2^16 and above (after rounding)
// is +inf.  The rounded value is an fp16 value, so the final float -> half conversion is exact.
__device__ uint16_t f64_to_f16_rne(double v) {
    if (!(v > 0.0)) return 0;
    int e;
    frexp(v, &e);                         // v = m * 2^e, 0.5 <= m < 1
    const int E = max(e - 1, -14);
    const double quantum = ldexp(1.0, E - 10);
    const double r = rint(v / quantum) * quantum;
    if (r >= 65536.0) return 0x7c00u;
    return __half_as_ushort(__float2half((float)r));
}

__device__ double block_reduce(double v, bool is_max, double *red) {
    for (int off = 32; off >= 1; off >>= 1) {
        const double o = __shfl_xor(v, off);
        v = is_max ? fmax(v, o) : fmin(v, o);
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = is_max ? fmax(r, red[i]) : fmin(r, red[i]);
    return r;
}

template <int G, bool F32IN, bool ASYM>
__global__ void __launch_bounds__(kThreads)
k_pack(const void *__restrict__ W, int K, uint8_t *__restrict__ packed, float *__restrict__ row_scale,
       uint8_t *__restrict__ zp) {
    __shared__ double buf[kSlab];
    __shared__ double red[kThreads / 64];
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;

    // pass 1: max|w'| (symmetric) or min / max of w' (asymmetric)
    double mx = ASYM ? 0.0 : 0.0, mn = 0.0;
    for (int k0 = 0; k0 < K; k0 += kSlab) {
        const int len = min(kSlab, K - k0);
        load_rotate_slab<G, F32IN>(W, n, K, k0, len, buf);
        for (int k = tid; k < len; k += kThreads) {
            const double w = buf[k];
            if (ASYM) {
                mx = fmax(mx, w);
                mn = fmin(mn, w);
            } else {
                mx = fmax(mx, fabs(w));
            }
        }
        __syncthreads();
    }
    // mx starts at 0 and mn at 0, so hi = max(max w', 0) and lo = min(min w', 0)
    const double hi = block_reduce(mx, true, red);
    const double lo = ASYM ? block_reduce(mn, false, red) : 0.0;

    float s;
    int z = 0;
    if (ASYM) {
        s = (float)((hi - lo) / 15.0);
        if (s > 0.0f) z = min(max((int)-rint(lo / (double)s), 0), 15);
    } else {
        s = (float)(hi / 7.0);
    }
    if (tid == 0) {
        row_scale[n] = s;
        if (ASYM) zp[n] = (uint8_t)z;
    }
    const double sd = (double)s;

    // pass 2: codes, two per byte
    for (int k0 = 0; k0 < K; k0 += kSlab) {
        const int len = min(kSlab, K - k0);
        load_rotate_slab<G, F32IN>(W, n, K, k0, len, buf);
        for (int p = tid; p < len / 2; p += kThreads) {
            int c[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const double w = buf[2 * p + h];
                if (ASYM) {
                    c[h] = sd > 0.0 ? min(max((int)rint(w / sd) + z, 0), 15) : 0;
                } else {
                    c[h] = sd > 0.0 ? min(max((int)rint(w / sd), -8), 7) : 0;
                }
            }
            packed[n * (K / 2) + (k0 / 2) + p] = (uint8_t)((c[0] & 15) | ((c[1] & 15) << 4));
        }
        __syncthreads();
    }
}

// Grouped-scale pack: pass 1 per slab stores each group's fp16 scale (one thread per group,
// at most 4096 / gw <= 256 groups per slab), pass 2 quantizes with it.
template <int G, bool F32IN>
__global__ void __launch_bounds__(kThreads)
k_pack_grouped(const void *__restrict__ W, int K, int gw, uint8_t *__restrict__ packed,
               uint16_t *__restrict__ gscale) {
    __shared__ double buf[kSlab];
    __shared__ double sc[kSlab / 16];
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int ng = K / gw;
    for (int k0 = 0; k0 < K; k0 += kSlab) {
        const int len = min(kSlab, K - k0);
        load_rotate_slab<G, F32IN>(W, n, K, k0, len, buf);
        const int gs = len / gw;  // groups in this slab
        for (int j = tid; j < gs; j += kThreads) {
            double am = 0.0;
            for (int i = 0; i < gw; ++i) am = fmax(am, fabs(buf[j * gw + i]));
            const uint16_t h = f64_to_f16_rne(am / 7.0);
            gscale[n * ng + k0 / gw + j] = h;
            sc[j] = (double)__half2float(__ushort_as_half(h));
        }
        __syncthreads();
        for (int p = tid; p < len / 2; p += kThreads) {
            const double sd = sc[(2 * p) / gw];
            int c[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                c[h] = sd > 0.0 ? min(max((int)rint(buf[2 * p + h] / sd), -8), 7) : 0;
            packed[n * (K / 2) + (k0 / 2) + p] = (uint8_t)((c[0] & 15) | ((c[1] & 15) << 4));
        }
        __syncthreads();
    }
}

template <int G, bool F32IN>
hipError_t launch_grouped_t(const void *W, int64_t N, int64_t K, int gw, uint8_t *packed, uint16_t *gs,
                            hipStream_t st) {
    hipLaunchKernelGGL((k_pack_grouped<G, F32IN>), dim3((unsigned)N), dim3(kThreads), 0, st, W, (int)K, gw, packed,
                       gs);
    return hipGetLastError();
}

template <int G, bool F32IN, bool ASYM>
hipError_t launch_t(const void *W, int64_t N, int64_t K, uint8_t *packed, float *s, uint8_t *zp,
                    hipStream_t st) {
    hipLaunchKernelGGL((k_pack<G, F32IN, ASYM>), dim3((unsigned)N), dim3(kThreads), 0, st, W,
                       (int)K, packed, s, zp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const void *W, bool f32in, int64_t N, int64_t K, int g, bool asym,
                       uint8_t *packed, float *row_scale, uint8_t *zp, hipStream_t st) {
#define W4_PK(G) return f32in ? (asym ? launch_t<G, true, true>(W, N, K, packed, row_scale, zp, st)      \
                                      : launch_t<G, true, false>(W, N, K, packed, row_scale, zp, st))    \
                              : (asym ? launch_t<G, false, true>(W, N, K, packed, row_scale, zp, st)     \
                                      : launch_t<G, false, false>(W, N, K, packed, row_scale, zp, st))
    switch (g) {
        case 0: W4_PK(1);
        case 16: W4_PK(16);
        case 64: W4_PK(64);
        case 256: W4_PK(256);
        case 1024: W4_PK(1024);
        case 4096: W4_PK(4096);
        default: return hipErrorInvalidValue;
    }
#undef W4_PK
}

hipError_t launch_pack_grouped(const void *W, bool f32in, int64_t N, int64_t K, int g, int gw, uint8_t *packed,
                               uint16_t *group_scale, hipStream_t st) {
    if (gw < 16 || kSlab % gw || K % gw) return hipErrorInvalidValue;
#define W4_PG(G) return f32in ? launch_grouped_t<G, true>(W, N, K, gw, packed, group_scale, st) \
                              : launch_grouped_t<G, false>(W, N, K, gw, packed, group_scale, st)
    switch (g) {
        case 0: W4_PG(1);
        case 16: W4_PG(16);
        case 64: W4_PG(64);
        case 256: W4_PG(256);
        case 1024: W4_PG(1024);
        case 4096: W4_PG(4096);
        default: return hipErrorInvalidValue;
    }
#undef W4_PG
}

}  // namespace w4
