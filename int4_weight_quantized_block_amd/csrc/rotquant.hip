// Activation rotate + per-token quantize for gfx950.
//
// Block Hadamard rotation of each token along K in groups of g (ComfyUI-INT-Crush README,
// "Inference / INT4": Hadamard rotation fused with activation quantization), then dynamic
// per-token symmetric quantization to int8 or int4 ("Inference / INT8": dynamic per-token
// INT8 quantization; stable-diffusion.cpp PR #2010 "Summary": the W4A4 format).
//
// Work split.  A "team" of T lanes owns one token row.  Each lane holds C chunks of 16
// consecutive elements; chunk c of lane t starts at element 16 * (c * T + t), so the lanes
// of a wave read consecutive 32-byte pieces (coalesced).  A group of g elements is 16
// consecutive chunks (g = 256: an aligned 16-lane row of the wave) or 4 (g = 64: a quad).
//
// The whole row stays in registers as fp64 (C * 16 doubles per lane), so X is read from
// HBM once and the absmax needs no second pass.  fp64 makes the transform exact for bf16
// inputs (8-bit significands, 8 stages of growth fit in 53 bits), so the codes match
// rint(X' / s) of the plain definition except within ~1e-13 of a rounding tie.
//
// FWHT: 4 butterfly stages inside each 16-element chunk (bits 0-3 of the in-group index),
// then the remaining bits across lanes.  g = 64: 2 stages over the quad with DPP lane moves.
// g = 256: a 16 x 16 fp64 transpose through LDS within each 16-lane row, 4 more in-register
// stages; lane r then holds group elements r + 16 j, and the int8 codes go back to
// natural order through a 256-byte LDS transpose before the coalesced store.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

constexpr int kTrStride = 18;                 // doubles per transpose row (16 + 2 pad)
constexpr int kTrRow = 16 * kTrStride + 16;   // doubles per 16-lane row (2432 bytes)
constexpr int kMaxBlock = 512;

template <int G, int C, int BITS, bool F32IN>
__global__ void __launch_bounds__(kMaxBlock)
k_rotquant(const void *__restrict__ Xv, int64_t M, int K, int T, int R, void *__restrict__ qv,
           float *__restrict__ tok_scale, int32_t *__restrict__ tok_rowsum) {
    extern __shared__ double lds[];
    constexpr int SEG = G / 16;
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    constexpr double INV_SQRT_G = G == 64 ? 0.125 : 0.0625;

    const int tid = threadIdx.x;
    const int team = tid / T;
    const int t = tid - team * T;
    const int64_t row = (int64_t)blockIdx.x * R + team;
    const bool valid = row < M;

    double *tr = lds;                                                   // g = 256 only
    double *slot_d = lds + (G == 256 ? (int)(blockDim.x >> 4) * kTrRow : 0);
    int *slot_i = reinterpret_cast<int *>(slot_d + blockDim.x / SEG);

    double v[C][16];

    // ---- load and widen to fp64
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t e0 = ((int64_t)c * T + t) * 16;
        if (F32IN) {
            uint4 w[4] = {};
            if (valid) {
                const uint4 *p = reinterpret_cast<const uint4 *>(
                    reinterpret_cast<const float *>(Xv) + row * K + e0);
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = p[j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[c][4 * j + 0] = (double)__uint_as_float(w[j].x);
                v[c][4 * j + 1] = (double)__uint_as_float(w[j].y);
                v[c][4 * j + 2] = (double)__uint_as_float(w[j].z);
                v[c][4 * j + 3] = (double)__uint_as_float(w[j].w);
            }
        } else {
            uint4 w[2] = {};
            if (valid) {
                const uint4 *p = reinterpret_cast<const uint4 *>(
                    reinterpret_cast<const uint16_t *>(Xv) + row * K + e0);
                w[0] = p[0];
                w[1] = p[1];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                v[c][8 * j + 0] = (double)bf16_lo(w[j].x);
                v[c][8 * j + 1] = (double)bf16_hi(w[j].x);
                v[c][8 * j + 2] = (double)bf16_lo(w[j].y);
                v[c][8 * j + 3] = (double)bf16_hi(w[j].y);
                v[c][8 * j + 4] = (double)bf16_lo(w[j].z);
                v[c][8 * j + 5] = (double)bf16_hi(w[j].z);
                v[c][8 * j + 6] = (double)bf16_lo(w[j].w);
                v[c][8 * j + 7] = (double)bf16_hi(w[j].w);
            }
        }
    }

    // ---- Walsh-Hadamard transform of every group (unnormalised)
#pragma unroll
    for (int c = 0; c < C; ++c) {
        fwht16(v[c]);
        if constexpr (G == 64) {
            const double s1 = (tid & 1) ? -1.0 : 1.0;
            const double s2 = (tid & 2) ? -1.0 : 1.0;
#pragma unroll
            for (int i = 0; i < 16; ++i) v[c][i] = fma(v[c][i], s1, dpp_f64<kQuadXor1>(v[c][i]));
#pragma unroll
            for (int i = 0; i < 16; ++i) v[c][i] = fma(v[c][i], s2, dpp_f64<kQuadXor2>(v[c][i]));
        } else {
            double *buf = tr + (tid >> 4) * kTrRow;
            const int r = tid & 15;
#pragma unroll
            for (int i = 0; i < 16; ++i) buf[r * kTrStride + i] = v[c][i];
            __syncthreads();
            double u[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) u[j] = buf[j * kTrStride + r];
            __syncthreads();
            fwht16(u);
#pragma unroll
            for (int j = 0; j < 16; ++j) v[c][j] = u[j];  // group element r + 16 j
        }
    }

    // ---- per-token absmax
    double am = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmax(am, fabs(v[c][i]));
#pragma unroll
    for (int off = 1; off < SEG; off <<= 1) am = fmax(am, __shfl_xor(am, off));
    if ((tid & (SEG - 1)) == 0) slot_d[tid / SEG] = am;
    __syncthreads();
    const int nseg = T / SEG;
    double amax = 0.0;
    for (int s = 0; s < nseg; ++s) amax = fmax(amax, slot_d[team * nseg + s]);

    // s = fp32(amax' / qmax) with amax' = amax / sqrt(g) (exact power-of-two scaling)
    const float scale = (float)((amax * INV_SQRT_G) / (double)QMAX);
    const double rr = scale > 0.0f ? (1.0 / (double)scale) * INV_SQRT_G : 0.0;
    if (valid && t == 0) tok_scale[row] = scale;

    // ---- quantize, restore natural order, pack, store
    int rowsum = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        int code[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int qi = __double2loint(fma(v[c][i], rr, kRoundMagic));
            code[i] = min(max(qi, -QMAX - 1), QMAX);
        }
        uint32_t d[4];
        if constexpr (G == 256) {
            uint8_t *b = reinterpret_cast<uint8_t *>(tr + (tid >> 4) * kTrRow);
            const int r = tid & 15;
#pragma unroll
            for (int j = 0; j < 16; ++j) b[r + 16 * j] = (uint8_t)code[j];
            __syncthreads();
            const uint4 w = *reinterpret_cast<const uint4 *>(b + 16 * r);
            __syncthreads();
            d[0] = w.x; d[1] = w.y; d[2] = w.z; d[3] = w.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                d[j] = (uint32_t)(code[4 * j] & 0xff) | ((uint32_t)(code[4 * j + 1] & 0xff) << 8) |
                       ((uint32_t)(code[4 * j + 2] & 0xff) << 16) |
                       ((uint32_t)(code[4 * j + 3] & 0xff) << 24);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) rowsum = __builtin_amdgcn_sdot4((int)d[j], 0x01010101, rowsum, false);
        if (valid) {
            const int64_t e0 = ((int64_t)c * T + t) * 16;
            if constexpr (BITS == 8) {
                *reinterpret_cast<uint4 *>(reinterpret_cast<int8_t *>(qv) + row * K + e0) =
                    make_uint4(d[0], d[1], d[2], d[3]);
            } else {
                uint32_t x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = d[j] & 0x0F0F0F0Fu;
                    x[j] = lo | (lo >> 4);  // bytes 0 and 2 = (k, k+1) and (k+2, k+3) nibble pairs
                }
                const uint32_t p0 = __builtin_amdgcn_perm(x[1], x[0], 0x06040200u);
                const uint32_t p1 = __builtin_amdgcn_perm(x[3], x[2], 0x06040200u);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint8_t *>(qv) + row * (K / 2) + e0 / 2) =
                    make_uint2(p0, p1);
            }
        }
    }

    // ---- per-token code sum
#pragma unroll
    for (int off = 1; off < SEG; off <<= 1) rowsum += __shfl_xor(rowsum, off);
    if ((tid & (SEG - 1)) == 0) slot_i[tid / SEG] = rowsum;
    __syncthreads();
    if (valid && t == 0) {
        int total = 0;
        for (int s = 0; s < nseg; ++s) total += slot_i[team * nseg + s];
        tok_rowsum[row] = total;
    }
}

// ---------------------------------------------------------------------------------------------
// Streaming variant for K % 256 == 0 (every DiT / text-encoder width): no LDS transposes.
//
// A quad of lanes owns each 256-element block of a row; lane p of the quad holds the four
// 16-element chunks p, p+4, p+8, p+12 (slots c = 0..3), so a quad reads and writes 128
// contiguous bytes per slot.  Within a block, element e = 16 * (p + 4c) + i:
//   g = 256: bits 0-3 (i) and 6-7 (c) are butterflies in registers, bits 4-5 (p) use DPP quad
//            exchanges - the whole group never leaves the quad;
//   g = 64:  slot c is its own group (bits 0-3 in registers, bits 4-5 across the quad).
// Each lane's 16 codes of a chunk are contiguous in the output, so they are packed and stored
// directly.  A team of T = K / 64 lanes owns a row; a workgroup owns R rows per iteration and
// loops over row groups with the next group's input loads in flight while it transforms the
// current one (one HBM read per element, no second pass).
template <int G, int BITS, bool F32IN>
__global__ void __launch_bounds__(512)
k_rotquant_stream(const void *__restrict__ Xv, int64_t M, int K, int T, int R, int64_t ngroups,
                  void *__restrict__ qv, float *__restrict__ tok_scale, int32_t *__restrict__ tok_rowsum) {
    __shared__ double slot_d[2][128];
    __shared__ int slot_i[2][128];
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    constexpr double INV_SQRT_G = G == 64 ? 0.125 : 0.0625;
    constexpr int NW = F32IN ? 4 : 2;  // 16-byte words per 16-element chunk

    const int tid = threadIdx.x;
    const int team = tid / T;
    const int t = tid - team * T;
    const int p = tid & 3;           // position in the quad
    const int blk = t >> 2;          // 256-element block of the row
    const int nquads = T / 4;        // quads per row

    auto load = [&](int64_t rg, uint4 (&w)[4][NW]) {
        const int64_t row = rg * R + team;
        if (row < M) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t e0 = (int64_t)blk * 256 + 16 * (p + 4 * c);
                const uint4 *src = F32IN ? reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(Xv) + row * K + e0)
                                         : reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(Xv) + row * K + e0);
#pragma unroll
                for (int j = 0; j < NW; ++j) w[c][j] = src[j];
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int j = 0; j < NW; ++j) w[c][j] = make_uint4(0, 0, 0, 0);
        }
    };

    // bf16 input: the next row group's loads are issued before this one is transformed
    // (fp32 input, the small fp32 case, loads at the top of each iteration to save registers)
    uint4 nxt[4][NW];
    int64_t rg = blockIdx.x;
    if (!F32IN && rg < ngroups) load(rg, nxt);
    int par = 0;
    for (; rg < ngroups; rg += gridDim.x, par ^= 1) {
        if constexpr (F32IN) load(rg, nxt);
        double v[4][16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (F32IN) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[c][4 * j + 0] = (double)__uint_as_float(nxt[c][j].x);
                    v[c][4 * j + 1] = (double)__uint_as_float(nxt[c][j].y);
                    v[c][4 * j + 2] = (double)__uint_as_float(nxt[c][j].z);
                    v[c][4 * j + 3] = (double)__uint_as_float(nxt[c][j].w);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    v[c][8 * j + 0] = (double)bf16_lo(nxt[c][j].x);
                    v[c][8 * j + 1] = (double)bf16_hi(nxt[c][j].x);
                    v[c][8 * j + 2] = (double)bf16_lo(nxt[c][j].y);
                    v[c][8 * j + 3] = (double)bf16_hi(nxt[c][j].y);
                    v[c][8 * j + 4] = (double)bf16_lo(nxt[c][j].z);
                    v[c][8 * j + 5] = (double)bf16_hi(nxt[c][j].z);
                    v[c][8 * j + 6] = (double)bf16_lo(nxt[c][j].w);
                    v[c][8 * j + 7] = (double)bf16_hi(nxt[c][j].w);
                }
            }
        }
        const int64_t row = rg * R + team;
        if (!F32IN && rg + gridDim.x < ngroups) load(rg + gridDim.x, nxt);  // in flight during the transform

        // ---- Walsh-Hadamard butterflies (unnormalised)
#pragma unroll
        for (int c = 0; c < 4; ++c) fwht16(v[c]);
        if constexpr (G == 256) {
#pragma unroll
            for (int h = 1; h < 4; h <<= 1)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if ((c & h) == 0)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const double a = v[c][i], b = v[c + h][i];
                            v[c][i] = a + b;
                            v[c + h][i] = a - b;
                        }
        }
        {
            const double s1 = (p & 1) ? -1.0 : 1.0, s2 = (p & 2) ? -1.0 : 1.0;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 16; ++i) v[c][i] = fma(v[c][i], s1, dpp_f64<kQuadXor1>(v[c][i]));
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 16; ++i) v[c][i] = fma(v[c][i], s2, dpp_f64<kQuadXor2>(v[c][i]));
        }

        // ---- per-token absmax: quad, then the row's quads through LDS (double-buffered slots)
        double am = 0.0;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) am = fmax(am, fabs(v[c][i]));
        am = fmax(am, dpp_f64<kQuadXor1>(am));
        am = fmax(am, dpp_f64<kQuadXor2>(am));
        if (p == 0) slot_d[par][tid >> 2] = am;
        __syncthreads();
        double amax = 0.0;
        for (int s = 0; s < nquads; ++s) amax = fmax(amax, slot_d[par][team * nquads + s]);
        const float scale = (float)((amax * INV_SQRT_G) / (double)QMAX);
        const double rr = scale > 0.0f ? (1.0 / (double)scale) * INV_SQRT_G : 0.0;
        if (row < M && t == 0) tok_scale[row] = scale;

        // ---- quantize, pack, store
        int rowsum = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int q4[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = __double2loint(fma(v[c][4 * j + r], rr, kRoundMagic));
                    q4[r] = min(max(qi, -QMAX - 1), QMAX);
                }
                d[j] = (uint32_t)(q4[0] & 0xff) | ((uint32_t)(q4[1] & 0xff) << 8) | ((uint32_t)(q4[2] & 0xff) << 16) |
                       ((uint32_t)(q4[3] & 0xff) << 24);
                rowsum = __builtin_amdgcn_sdot4((int)d[j], 0x01010101, rowsum, false);
            }
            if (row < M) {
                const int64_t e0 = (int64_t)blk * 256 + 16 * (p + 4 * c);
                if constexpr (BITS == 8) {
                    *reinterpret_cast<uint4 *>(reinterpret_cast<int8_t *>(qv) + row * K + e0) = make_uint4(d[0], d[1], d[2], d[3]);
                } else {
                    uint32_t x[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = d[j] & 0x0F0F0F0Fu;
                        x[j] = lo | (lo >> 4);
                    }
                    *reinterpret_cast<uint2 *>(reinterpret_cast<uint8_t *>(qv) + row * (K / 2) + e0 / 2) =
                        make_uint2(__builtin_amdgcn_perm(x[1], x[0], 0x06040200u), __builtin_amdgcn_perm(x[3], x[2], 0x06040200u));
                }
            }
        }
        rowsum += __shfl_xor(rowsum, 1);
        rowsum += __shfl_xor(rowsum, 2);
        if (p == 0) slot_i[par][tid >> 2] = rowsum;
        __syncthreads();
        if (row < M && t == 0) {
            int total = 0;
            for (int s = 0; s < nquads; ++s) total += slot_i[par][team * nquads + s];
            tok_rowsum[row] = total;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Row-team variant for K % 1024 == 0 with K / 1024 = C * W: C <= 4 chunks of 16 per lane and
// W in {1, 2, 4, 8} waves per row, or for a few rows C = 1 and W <= 16 (3072, 4096, 6144,
// 12288, ...).  A team of W waves owns one token row at a time and walks
// the rows team, team + nteams, ... with the next row's input loads in flight while it
// transforms the current one.  Every wave carries the same amount of work, so the waves of
// a launch (two per SIMD) finish together, and W = 1 needs no workgroup barrier at all.
//
// Lane layout: a 16-lane row r16 of wave w holds C 256-element blocks, numbers
// (4 w + r16) C + c; lane l of that row holds elements 16 (l & 15) .. 16 (l & 15) + 15 of each,
// so a 16-lane row reads and writes contiguous bytes.  Within a block, element bits 0-3 are
// butterflies in registers, bits 4-5 quad DPP exchanges, and (g = 256) bits 6-7 exchanges
// with the lanes 4 and 8 apart through ds_swizzle, which runs on the LDS unit and so adds
// only the fma to the VALU's load (measured: faster than swizzling all four stages, and than
// DPP moves for these two).

// Steps of the row-team layout shared by the kernels below: a lane holds, for each of C
// 256-element blocks, the 16 elements 16 * cl .. 16 * cl + 15 (cl = lane & 15).

// Widen the raw words of C chunks (bf16: 2 x 16 bytes, fp32: 4 x 16 bytes per chunk) to fp64.
template <bool F32IN, int C>
__device__ __forceinline__ void rt_widen(const uint4 (&x)[C][F32IN ? 4 : 2], double (&v)[C][16]) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if constexpr (F32IN) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[c][4 * j + 0] = (double)__uint_as_float(x[c][j].x);
                v[c][4 * j + 1] = (double)__uint_as_float(x[c][j].y);
                v[c][4 * j + 2] = (double)__uint_as_float(x[c][j].z);
                v[c][4 * j + 3] = (double)__uint_as_float(x[c][j].w);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                v[c][8 * j + 0] = (double)bf16_lo(x[c][j].x);
                v[c][8 * j + 1] = (double)bf16_hi(x[c][j].x);
                v[c][8 * j + 2] = (double)bf16_lo(x[c][j].y);
                v[c][8 * j + 3] = (double)bf16_hi(x[c][j].y);
                v[c][8 * j + 4] = (double)bf16_lo(x[c][j].z);
                v[c][8 * j + 5] = (double)bf16_hi(x[c][j].z);
                v[c][8 * j + 6] = (double)bf16_lo(x[c][j].w);
                v[c][8 * j + 7] = (double)bf16_hi(x[c][j].w);
            }
        }
    }
}

// Walsh-Hadamard butterflies (unnormalised) of every group of G: bits 0-3 in registers, bits
// 4-5 quad DPP exchanges, and (G = 256) bits 6-7 exchanges with the lanes 4 and 8 apart
// through ds_swizzle.
template <int G, int C>
__device__ __forceinline__ void rt_fwht(double (&v)[C][16], int cl) {
#pragma unroll
    for (int c = 0; c < C; ++c) fwht16(v[c]);
    {
        const double s1 = (cl & 1) ? -1.0 : 1.0, s2 = (cl & 2) ? -1.0 : 1.0;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[c][i] = fma(v[c][i], s1, dpp_f64<kQuadXor1>(v[c][i]));
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[c][i] = fma(v[c][i], s2, dpp_f64<kQuadXor2>(v[c][i]));
    }
    if constexpr (G == 256) {
        const double s4 = (cl & 4) ? -1.0 : 1.0, s8 = (cl & 8) ? -1.0 : 1.0;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[c][i] = fma(v[c][i], s4, swz_f64<kSwzXor4>(v[c][i]));
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[c][i] = fma(v[c][i], s8, swz_f64<kSwzXor8>(v[c][i]));
    }
}

template <int C>
__device__ __forceinline__ double rt_absmax(const double (&v)[C][16]) {
    double am = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmax(am, fabs(v[c][i]));
    return am;
}

// Codes rint(v * rr) (fp64, the low word of v * rr + 1.5 * 2^52), stored as int8 or packed
// int4 (each lane's 16 codes of a block are contiguous); returns the lane's code sum.
template <int BITS, int C>
__device__ __forceinline__ int rt_quant_store(const double (&v)[C][16], double rr, void *qv, int64_t row, int K,
                                              int blk0, int cl) {
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    int rowsum = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int q4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int qi = __double2loint(fma(v[c][4 * j + r], rr, kRoundMagic));
                q4[r] = min(max(qi, -QMAX - 1), QMAX);
            }
            d[j] = (uint32_t)(q4[0] & 0xff) | ((uint32_t)(q4[1] & 0xff) << 8) | ((uint32_t)(q4[2] & 0xff) << 16) |
                   ((uint32_t)(q4[3] & 0xff) << 24);
            rowsum = __builtin_amdgcn_sdot4((int)d[j], 0x01010101, rowsum, false);
        }
        const int64_t e0 = (int64_t)(blk0 + c) * 256 + 16 * cl;
        if constexpr (BITS == 8) {
            *reinterpret_cast<uint4 *>(reinterpret_cast<int8_t *>(qv) + row * K + e0) = make_uint4(d[0], d[1], d[2], d[3]);
        } else {
            uint32_t x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = d[j] & 0x0F0F0F0Fu;
                x[j] = lo | (lo >> 4);
            }
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint8_t *>(qv) + row * (K / 2) + e0 / 2) =
                make_uint2(__builtin_amdgcn_perm(x[1], x[0], 0x06040200u), __builtin_amdgcn_perm(x[3], x[2], 0x06040200u));
        }
    }
    return rowsum;
}

template <int G, int BITS, bool F32IN, int C>
__global__ void __launch_bounds__(C == 1 ? 1024 : 512) __attribute__((amdgpu_waves_per_eu(2)))
k_rotquant_row(const void *__restrict__ Xv, int64_t M, int K, int W, int64_t nteams, void *__restrict__ qv,
               float *__restrict__ tok_scale, int32_t *__restrict__ tok_rowsum) {
    __shared__ double red_d[2][16];
    __shared__ int red_i[2][16];
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    constexpr double INV_SQRT_G = G == 64 ? 0.125 : 0.0625;
    constexpr int NW = F32IN ? 4 : 2;  // 16-byte words per 16-element chunk

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cl = lane & 15;
    const int blk0 = (w * 4 + (lane >> 4)) * C;  // this lane's first 256-element block in the row

    auto load = [&](int64_t row, uint4 (&x)[C][NW]) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t e0 = row * K + (int64_t)(blk0 + c) * 256 + 16 * cl;
            const uint4 *src = F32IN ? reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(Xv) + e0)
                                     : reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(Xv) + e0);
#pragma unroll
            for (int j = 0; j < NW; ++j) x[c][j] = src[j];
        }
    };

    uint4 nxt[C][NW];
    int64_t row = blockIdx.x;
    if (row < M) load(row, nxt);
    int par = 0;
    for (; row < M; row += nteams, par ^= 1) {
        double v[C][16];
        rt_widen<F32IN, C>(nxt, v);
        if (row + nteams < M) load(row + nteams, nxt);  // in flight during the transform
        rt_fwht<G, C>(v, cl);

        // ---- per-token absmax: the wave, then (W > 1) the team through LDS
        double am = rt_absmax<C>(v);
        am = wave_max_f64(am);
        if (W > 1) {
            if (lane == 0) red_d[par][w] = am;
            __syncthreads();
            am = red_d[par][0];
            for (int u = 1; u < W; ++u) am = fmax(am, red_d[par][u]);
        }
        const float scale = (float)((am * INV_SQRT_G) / (double)QMAX);
        const double rr = scale > 0.0f ? (1.0 / (double)scale) * INV_SQRT_G : 0.0;
        if (w == 0 && lane == 0) tok_scale[row] = scale;

        // ---- quantize, pack, store
        int rowsum = rt_quant_store<BITS, C>(v, rr, qv, row, K, blk0, cl);
        rowsum = wave_sum_i32(rowsum);
        if (W > 1) {
            if (lane == 0) red_i[par][w] = rowsum;
            __syncthreads();
            rowsum = 0;
            for (int u = 0; u < W; ++u) rowsum += red_i[par][u];
        }
        if (w == 0 && lane == 0) tok_rowsum[row] = rowsum;
    }
}

// ---------------------------------------------------------------------------------------------
// Rotate + quantize with the low-rank down-projection in the same pass (ComfyUI-INT-Crush
// README, "Forward Pass" step 6: the SVD residual from the L1 / L2 factors, on the unrotated
// activations per "LoRA"; stable-diffusion.cpp PR #2010, "Summary": the activation work is
// shared per input, so the L1 factors of every linear reading the input are stacked and
// applied once).  bf16 X, K = 1024 C W as for the row-team kernel (C chunks per lane, W waves
// per row).
//
// Workgroup b of 8 waves owns R consecutive token rows (R = ceil(M / grid) <= 16 NB, the grid
// at most one workgroup per compute unit, so there is no tail round).  Its 8 / W teams of W
// waves rotate and quantize rows team, team + 8 / W, ... of them exactly as the row-team kernel
// does (the next row's loads in flight during a row's transform; a team's absmax and code sum
// meet in LDS, and the teams step together).  Then the rows, as NB MFMA blocks of 16 tokens,
// are multiplied by l1 on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16: exact products,
// fp32 sums): wave w takes one eighth of K for every rank block, so each l1 fragment is
// loaded once per workgroup and serves all its rows; x fragments come from L2, where the
// rotation's loads of the same rows have just put them, so X is read from HBM once.  Loads
// run one 4-step batch ahead of the MFMAs (two batches per loop turn, so every buffer index
// is a constant and the buffers stay in registers).  The eight K-range partial tiles are
// added through LDS in a fixed order.
template <int G, int BITS, int C, int W, int RQ, int NB>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
k_rotquant_lr(const uint16_t *__restrict__ X, int64_t M, int K, int R, void *__restrict__ qv,
              float *__restrict__ tok_scale, int32_t *__restrict__ tok_rowsum, const uint16_t *__restrict__ l1, int r,
              float *__restrict__ t, int64_t ldt) {
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    constexpr double INV_SQRT_G = G == 64 ? 0.125 : 0.0625;
    constexpr int NT = 8 / W;  // teams
    __shared__ v4f part[8][NB * RQ][64];
    __shared__ double red_d[2][8];
    __shared__ int red_i[2][8];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int team = w / W, wt = w % W;
    const int cl = lane & 15;
    const int blk0 = (wt * 4 + (lane >> 4)) * C;
    const int64_t m0 = (int64_t)blockIdx.x * R;
    const int64_t m1 = min<int64_t>(m0 + R, M);

    // ---- rotate + quantize rows m0 + team, m0 + team + NT, ...  (every team steps R / NT times,
    // rounded up, so the teams meet at the same barriers; rows past m1 skip loads and stores)
    auto load = [&](int64_t row, uint4 (&x)[C][2]) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const uint4 *src = reinterpret_cast<const uint4 *>(X + row * K + (int64_t)(blk0 + c) * 256 + 16 * cl);
            x[c][0] = src[0];
            x[c][1] = src[1];
        }
    };
    uint4 nxt[C][2];
    const int iters = (R + NT - 1) / NT;
    int64_t row = m0 + team;
    if (row < m1) load(row, nxt);
    int par = 0;
#pragma unroll 1
    for (int it = 0; it < iters; ++it, row += NT, par ^= 1) {
        const bool valid = row < m1;
        double v[C][16];
        rt_widen<false, C>(nxt, v);
        if (row + NT < m1) load(row + NT, nxt);
        rt_fwht<G, C>(v, cl);
        double am = rt_absmax<C>(v);
        am = wave_max_f64(am);
        if constexpr (W > 1) {
            if (lane == 0) red_d[par][w] = am;
            __syncthreads();
            am = red_d[par][team * W];
            for (int u = 1; u < W; ++u) am = fmax(am, red_d[par][team * W + u]);
        }
        const float scale = (float)((am * INV_SQRT_G) / (double)QMAX);
        const double rr = scale > 0.0f ? (1.0 / (double)scale) * INV_SQRT_G : 0.0;
        int rowsum = valid ? rt_quant_store<BITS, C>(v, rr, qv, row, K, blk0, cl) : 0;
        rowsum = wave_sum_i32(rowsum);
        if constexpr (W > 1) {
            if (lane == 0) red_i[par][w] = rowsum;
            __syncthreads();
            rowsum = 0;
            for (int u = 0; u < W; ++u) rowsum += red_i[par][team * W + u];
        }
        if (valid && wt == 0 && lane == 0) {
            tok_scale[row] = scale;
            tok_rowsum[row] = rowsum;
        }
    }

    // ---- t = x . l1^T: A = 16 tokens x 32 k, B = 32 k x 16 ranks; lane l holds token (or rank)
    // l % 16 of its block and k 8 (l / 16) .. + 7 of the step.  Wave w's eighth of K is
    // 4 C W steps, taken as C W batches of 4.
    constexpr int NBAT = C * W;
    const int s0 = w * 4 * NBAT;
    const uint16_t *xa[NB];
    const uint16_t *lb[RQ];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t tok = min<int64_t>(m0 + 16 * nb + cl, m1 - 1);  // rows past the block: clamped, not stored
        xa[nb] = X + tok * K + 8 * (lane >> 4) + 32 * s0;
    }
#pragma unroll
    for (int q = 0; q < RQ; ++q) lb[q] = l1 + (int64_t)min(16 * q + cl, r - 1) * K + 8 * (lane >> 4) + 32 * s0;
    v4f acc[NB][RQ];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < RQ; ++q) acc[nb][q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    uint4 xb0[4][NB], bb0[4][RQ], xb1[4][NB], bb1[4][RQ];
    auto fetch = [&](uint4 (&xb)[4][NB], uint4 (&bb)[4][RQ], int bi) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) xb[u][nb] = *reinterpret_cast<const uint4 *>(xa[nb] + 32 * (4 * bi + u));
#pragma unroll
            for (int q = 0; q < RQ; ++q) bb[u][q] = *reinterpret_cast<const uint4 *>(lb[q] + 32 * (4 * bi + u));
        }
    };
    auto mul = [&](const uint4 (&xb)[4][NB], const uint4 (&bb)[4][RQ]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < RQ; ++q)
                    acc[nb][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xb[u][nb]),
                                                                         __builtin_bit_cast(v8bf, bb[u][q]), acc[nb][q],
                                                                         0, 0, 0);
    };
    fetch(xb0, bb0, 0);
#pragma unroll 1
    for (int bi = 0; bi + 1 < NBAT; bi += 2) {
        fetch(xb1, bb1, bi + 1);
        mul(xb0, bb0);
        if (bi + 2 < NBAT) fetch(xb0, bb0, bi + 2);
        mul(xb1, bb1);
    }
    if (NBAT & 1) mul(xb0, bb0);

    // 16x16 layout: lane l, register v holds token 4 (l / 16) + v of the block, rank l % 16
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < RQ; ++q) part[w][nb * RQ + q][lane] = acc[nb][q];
    __syncthreads();
    for (int u = w; u < NB * RQ; u += 8) {
        v4f sum = part[0][u][lane];
#pragma unroll
        for (int k = 1; k < 8; ++k) sum += part[k][u][lane];
        const int nb = u / RQ, q = 16 * (u % RQ) + cl;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t mm = m0 + 16 * nb + 4 * (lane >> 4) + v;
            if (mm < m1 && q < r) t[mm * ldt + q] = sum[v];
        }
    }
}

template <int G, int BITS, int C, int W, int NB>
hipError_t launch_lr_nb(const uint16_t *X, int64_t M, int64_t K, int R, void *q, float *s, int32_t *rs,
                        const uint16_t *l1, int r, float *t, int64_t ldt, hipStream_t st) {
    const unsigned grid = (unsigned)((M + R - 1) / R);
    if (r <= 16)
        hipLaunchKernelGGL((k_rotquant_lr<G, BITS, C, W, 1, NB>), dim3(grid), dim3(512), 0, st, X, M, (int)K, R, q, s,
                           rs, l1, r, t, ldt);
    else if (r <= 32)
        hipLaunchKernelGGL((k_rotquant_lr<G, BITS, C, W, 2, NB>), dim3(grid), dim3(512), 0, st, X, M, (int)K, R, q, s,
                           rs, l1, r, t, ldt);
    else
        hipLaunchKernelGGL((k_rotquant_lr<G, BITS, C, W, 4, NB>), dim3(grid), dim3(512), 0, st, X, M, (int)K, R, q, s,
                           rs, l1, r, t, ldt);
    return hipGetLastError();
}

// Rows per workgroup: at most one workgroup per compute unit while that keeps R <= 32 (two
// MFMA token blocks), else 32.
template <int G, int BITS, int C, int W>
hipError_t launch_lr_cw(const uint16_t *X, int64_t M, int64_t K, void *q, float *s, int32_t *rs, const uint16_t *l1,
                        int r, float *t, int64_t ldt, hipStream_t st) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const int R = (int)std::min<int64_t>(32, (M + ncu - 1) / ncu);
    if (R <= 16) return launch_lr_nb<G, BITS, C, W, 1>(X, M, K, R, q, s, rs, l1, r, t, ldt, st);
    return launch_lr_nb<G, BITS, C, W, 2>(X, M, K, R, q, s, rs, l1, r, t, ldt, st);
}

// (C, W) with K = 1024 C W: 3 or 4 chunks per lane and 1, 2, 4 or 8 waves per row
bool lr_split(int64_t K, int &C, int &W) {
    if (K <= 0 || K % 1024) return false;
    const int64_t n = K / 1024;
    for (int c : {3, 4, 2, 1}) {
        if (n % c) continue;
        const int64_t w = n / c;
        if (w == 1 || w == 2 || w == 4 || w == 8) {
            C = c;
            W = (int)w;
            return true;
        }
    }
    return false;
}

template <int G, int BITS>
hipError_t launch_lr_gb(const uint16_t *X, int64_t M, int64_t K, void *q, float *s, int32_t *rs, const uint16_t *l1,
                        int r, float *t, int64_t ldt, hipStream_t st) {
    int C = 0, W = 0;
    if (!lr_split(K, C, W)) return hipErrorInvalidValue;
#define W4_LR(CC, WW) \
    if (C == CC && W == WW) return launch_lr_cw<G, BITS, CC, WW>(X, M, K, q, s, rs, l1, r, t, ldt, st)
    W4_LR(1, 1); W4_LR(2, 1); W4_LR(3, 1); W4_LR(4, 1);
    W4_LR(3, 2); W4_LR(4, 2); W4_LR(3, 4); W4_LR(4, 4); W4_LR(3, 8); W4_LR(4, 8);
#undef W4_LR
    return hipErrorInvalidValue;
}

// (C, W) for the row-team kernel, or false.  A few rows (M <= 64) take one chunk per lane and
// up to 16 waves per row, so that they spread over many compute units and each wave's
// transform is short; more rows take 2-4 chunks per lane and 1-8 waves per row.
bool row_team_split(int64_t M, int64_t K, int &C, int &W) {
    if (K <= 0 || K % 1024) return false;
    const int64_t n = K / 1024;
    if (M <= 64 && n <= 16) {
        C = 1;
        W = (int)n;
        return true;
    }
    for (int c : {3, 4, 2, 1}) {
        if (n % c) continue;
        const int64_t w = n / c;
        if (w == 1 || w == 2 || w == 4 || w == 8) {
            C = c;
            W = (int)w;
            return true;
        }
    }
    return false;
}

template <int G, int BITS, bool F32IN, int C>
hipError_t launch_row_c(const void *X, int64_t M, int64_t K, int W, void *q, float *s, int32_t *rs, hipStream_t st) {
    // two waves per SIMD over the whole chip, one team of W waves per workgroup
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t nteams = std::min<int64_t>(M, (int64_t)ncu * 8 / W);
    hipLaunchKernelGGL((k_rotquant_row<G, BITS, F32IN, C>), dim3((unsigned)nteams), dim3(64 * W), 0, st, X, M,
                       (int)K, W, nteams, q, s, rs);
    return hipGetLastError();
}

template <int G, int BITS, bool F32IN>
hipError_t launch_row(const void *X, int64_t M, int64_t K, int C, int W, void *q, float *s, int32_t *rs,
                      hipStream_t st) {
    switch (C) {
        case 1: return launch_row_c<G, BITS, F32IN, 1>(X, M, K, W, q, s, rs, st);
        case 2: return launch_row_c<G, BITS, F32IN, 2>(X, M, K, W, q, s, rs, st);
        case 3: return launch_row_c<G, BITS, F32IN, 3>(X, M, K, W, q, s, rs, st);
        default: return launch_row_c<G, BITS, F32IN, 4>(X, M, K, W, q, s, rs, st);
    }
}

struct Split {
    int C, T, R;
};

bool choose_split(int64_t K, int g, Split &sp) {
    if (K <= 0 || K % g) return false;
    const int64_t chunks = K / 16;
    const int seg = g / 16;
    for (int C = 4; C >= 1; --C) {
        if (chunks % C) continue;
        const int64_t T = chunks / C;
        if (T % seg || T > kMaxBlock) continue;
        int R = 1;
        while (R * T < 256 && 2 * R * T <= kMaxBlock) R *= 2;
        while ((R * T) % 64 && (R + 1) * T <= kMaxBlock) ++R;
        sp = {C, (int)T, R};
        return true;
    }
    return false;
}

template <int G, int C, int BITS, bool F32IN>
hipError_t launch_t(const void *X, int64_t M, int64_t K, const Split &sp, void *q, float *s,
                    int32_t *rs, hipStream_t st) {
    const int block = sp.R * sp.T;
    const size_t lds = (G == 256 ? (size_t)(block / 16) * kTrRow * sizeof(double) : 0) +
                       (size_t)(block / (G / 16)) * (sizeof(double) + sizeof(int));
    if (lds > 65536) {
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_rotquant<G, C, BITS, F32IN>),
            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (attr != hipSuccess) return attr;
    }
    const int64_t grid = (M + sp.R - 1) / sp.R;
    hipLaunchKernelGGL((k_rotquant<G, C, BITS, F32IN>), dim3((unsigned)grid), dim3(block), lds, st,
                       X, M, (int)K, sp.T, sp.R, q, s, rs);
    return hipGetLastError();
}

template <int G, int BITS, bool F32IN>
hipError_t dispatch_c(const void *X, int64_t M, int64_t K, const Split &sp, void *q, float *s,
                      int32_t *rs, hipStream_t st) {
    switch (sp.C) {
        case 1: return launch_t<G, 1, BITS, F32IN>(X, M, K, sp, q, s, rs, st);
        case 2: return launch_t<G, 2, BITS, F32IN>(X, M, K, sp, q, s, rs, st);
        case 3: return launch_t<G, 3, BITS, F32IN>(X, M, K, sp, q, s, rs, st);
        default: return launch_t<G, 4, BITS, F32IN>(X, M, K, sp, q, s, rs, st);
    }
}

template <int G, int BITS, bool F32IN>
hipError_t launch_stream(const void *X, int64_t M, int64_t K, void *q, float *s, int32_t *rs, hipStream_t st) {
    const int T = (int)(K / 64);
    int R = 1;
    while (R * T < 256 && 2 * R * T <= 512) R *= 2;
    while ((R * T) % 64 && (R + 1) * T <= 512) ++R;
    const int block = R * T;
    const int64_t ngroups = (M + R - 1) / R;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const int waves_per_block = (block + 63) / 64;
    const int64_t resident = (int64_t)ncu * std::max(1, 8 / waves_per_block);
    const int64_t grid = std::min<int64_t>(ngroups, resident);
    hipLaunchKernelGGL((k_rotquant_stream<G, BITS, F32IN>), dim3((unsigned)grid), dim3(block), 0, st, X, M, (int)K,
                       T, R, ngroups, q, s, rs);
    return hipGetLastError();
}

bool stream_ok(int64_t K) { return K % 256 == 0 && K / 64 <= 512; }

// ---------------------------------------------------------------------------------------------
// Any rotation size (ComfyUI-INT-Crush README, "Nodes": rot_size 16 / 64 / 256 / 1024 / 4096):
// one workgroup per token row, the row in slabs of 4096 elements staged in LDS as fp64.
// Pass 1 transforms each slab with in-place butterflies and reduces max|x'|; pass 2 reads
// and transforms it again (from L2) and quantizes with the IEEE quotient x' / s.  It serves
// the sizes the register kernels above do not (16, 1024, 4096); every size divides the slab,
// so no group straddles two slabs.
constexpr int kGenSlab = 4096;
constexpr int kGenThreads = 256;

template <int G, bool F32IN>
__device__ void gen_load_rotate(const void *X, int64_t row, int K, int k0, int len, double *buf) {
    const int tid = threadIdx.x;
    for (int k = tid; k < len; k += kGenThreads) {
        const int64_t idx = row * K + k0 + k;
        buf[k] = F32IN ? (double)reinterpret_cast<const float *>(X)[idx]
                       : (double)bf16_to_f32(reinterpret_cast<const uint16_t *>(X)[idx]);
    }
    __syncthreads();
    for (int h = 1; h < G; h <<= 1) {
        for (int p = tid; p < len / 2; p += kGenThreads) {
            const int i = ((p & ~(h - 1)) << 1) | (p & (h - 1));
            const double a = buf[i], b = buf[i + h];
            buf[i] = a + b;
            buf[i + h] = a - b;
        }
        __syncthreads();
    }
}

template <int G, int BITS, bool F32IN>
__global__ void __launch_bounds__(kGenThreads)
k_rotquant_gen(const void *__restrict__ Xv, int K, void *__restrict__ qv, float *__restrict__ tok_scale,
               int32_t *__restrict__ tok_rowsum) {
    __shared__ double buf[kGenSlab];
    __shared__ double red_d[kGenThreads / 64];
    __shared__ int red_i[kGenThreads / 64];
    constexpr int QMAX = BITS == 8 ? 127 : 7;
    constexpr double INV_SQRT_G = G == 16 ? 0.25 : G == 64 ? 0.125 : G == 256 ? 0.0625 : G == 1024 ? 0.03125
                                                                                                  : 0.015625;
    static_assert(G == 16 || G == 64 || G == 256 || G == 1024 || G == 4096, "rotation size");
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

    double am = 0.0;
    for (int k0 = 0; k0 < K; k0 += kGenSlab) {
        const int len = min(kGenSlab, K - k0);
        gen_load_rotate<G, F32IN>(Xv, row, K, k0, len, buf);
        for (int k = tid; k < len; k += kGenThreads) am = fmax(am, fabs(buf[k]));
        __syncthreads();
    }
    for (int off = 32; off >= 1; off >>= 1) am = fmax(am, __shfl_xor(am, off));
    if (lane == 0) red_d[w] = am;
    __syncthreads();
    am = red_d[0];
    for (int i = 1; i < kGenThreads / 64; ++i) am = fmax(am, red_d[i]);
    const float scale = (float)((am * INV_SQRT_G) / (double)QMAX);  // amax / sqrt(g): exact scaling
    const double sd = (double)scale;
    if (tid == 0) tok_scale[row] = scale;

    int rowsum = 0;
    for (int k0 = 0; k0 < K; k0 += kGenSlab) {
        const int len = min(kGenSlab, K - k0);
        gen_load_rotate<G, F32IN>(Xv, row, K, k0, len, buf);
        for (int p = tid; p < len / 2; p += kGenThreads) {
            int c[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                c[h] = sd > 0.0 ? min(max((int)rint((buf[2 * p + h] * INV_SQRT_G) / sd), -QMAX - 1), QMAX) : 0;
                rowsum += c[h];
            }
            if constexpr (BITS == 8) {
                int8_t *q = reinterpret_cast<int8_t *>(qv) + row * K + k0 + 2 * p;
                q[0] = (int8_t)c[0];
                q[1] = (int8_t)c[1];
            } else {
                reinterpret_cast<uint8_t *>(qv)[row * (K / 2) + k0 / 2 + p] =
                    (uint8_t)((c[0] & 15) | ((c[1] & 15) << 4));
            }
        }
        __syncthreads();
    }
    for (int off = 32; off >= 1; off >>= 1) rowsum += __shfl_xor(rowsum, off);
    if (lane == 0) red_i[w] = rowsum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
        for (int i = 0; i < kGenThreads / 64; ++i) total += red_i[i];
        tok_rowsum[row] = total;
    }
}

template <int G, int BITS, bool F32IN>
hipError_t launch_gen_t(const void *X, int64_t M, int64_t K, void *q, float *s, int32_t *rs, hipStream_t st) {
    hipLaunchKernelGGL((k_rotquant_gen<G, BITS, F32IN>), dim3((unsigned)M), dim3(kGenThreads), 0, st, X, (int)K, q,
                       s, rs);
    return hipGetLastError();
}

template <int G>
hipError_t launch_gen(const void *X, bool f32in, int64_t M, int64_t K, int bits, void *q, float *s, int32_t *rs,
                      hipStream_t st) {
    if (bits == 8) return f32in ? launch_gen_t<G, 8, true>(X, M, K, q, s, rs, st)
                                : launch_gen_t<G, 8, false>(X, M, K, q, s, rs, st);
    return f32in ? launch_gen_t<G, 4, true>(X, M, K, q, s, rs, st) : launch_gen_t<G, 4, false>(X, M, K, q, s, rs, st);
}

}  // namespace

bool rotquant_lr_fusable(int64_t K, int g) {
    int C = 0, W = 0;
    return (g == 64 || g == 256) && lr_split(K, C, W);
}

hipError_t launch_rotquant_lr(const void *X, int64_t M, int64_t K, int g, int bits, void *q, float *tok_scale,
                              int32_t *tok_rowsum, const void *l1, int r, float *t, int64_t ldt, hipStream_t st) {
    if (M == 0) return hipSuccess;
    if (!rotquant_lr_fusable(K, g) || r < 1 || r > 64) return hipErrorInvalidValue;
    const uint16_t *x = static_cast<const uint16_t *>(X), *l = static_cast<const uint16_t *>(l1);
    if (g == 64)
        return bits == 8 ? launch_lr_gb<64, 8>(x, M, K, q, tok_scale, tok_rowsum, l, r, t, ldt, st)
                         : launch_lr_gb<64, 4>(x, M, K, q, tok_scale, tok_rowsum, l, r, t, ldt, st);
    return bits == 8 ? launch_lr_gb<256, 8>(x, M, K, q, tok_scale, tok_rowsum, l, r, t, ldt, st)
                     : launch_lr_gb<256, 4>(x, M, K, q, tok_scale, tok_rowsum, l, r, t, ldt, st);
}

bool rotquant_supported(int64_t K, int g) {
    if (g == 16 || g == 1024 || g == 4096) return K > 0 && K % g == 0;
    Split sp;
    return stream_ok(K) || choose_split(K, g, sp);
}

hipError_t launch_rotquant(const void *X, bool f32in, int64_t M, int64_t K, int g, int bits,
                           void *q, float *tok_scale, int32_t *tok_rowsum, hipStream_t st) {
    if (M == 0) return hipSuccess;
    if (g == 16) return launch_gen<16>(X, f32in, M, K, bits, q, tok_scale, tok_rowsum, st);
    if (g == 1024) return launch_gen<1024>(X, f32in, M, K, bits, q, tok_scale, tok_rowsum, st);
    if (g == 4096) return launch_gen<4096>(X, f32in, M, K, bits, q, tok_scale, tok_rowsum, st);
    if (g != 64 && g != 256) return hipErrorInvalidValue;
    int C = 0, W = 0;
    if (row_team_split(M, K, C, W)) {
#define W4_RT(G, B, F) return launch_row<G, B, F>(X, M, K, C, W, q, tok_scale, tok_rowsum, st)
        if (g == 64) {
            if (bits == 8) { if (f32in) W4_RT(64, 8, true); else W4_RT(64, 8, false); }
            else { if (f32in) W4_RT(64, 4, true); else W4_RT(64, 4, false); }
        } else {
            if (bits == 8) { if (f32in) W4_RT(256, 8, true); else W4_RT(256, 8, false); }
            else { if (f32in) W4_RT(256, 4, true); else W4_RT(256, 4, false); }
        }
#undef W4_RT
    }
    if (stream_ok(K)) {
#define W4_RS(G, B, F) return launch_stream<G, B, F>(X, M, K, q, tok_scale, tok_rowsum, st)
        if (g == 64) {
            if (bits == 8) { if (f32in) W4_RS(64, 8, true); else W4_RS(64, 8, false); }
            else { if (f32in) W4_RS(64, 4, true); else W4_RS(64, 4, false); }
        } else {
            if (bits == 8) { if (f32in) W4_RS(256, 8, true); else W4_RS(256, 8, false); }
            else { if (f32in) W4_RS(256, 4, true); else W4_RS(256, 4, false); }
        }
#undef W4_RS
    }
    Split sp;
    if (!choose_split(K, g, sp)) return hipErrorInvalidValue;
#define W4_RQ(G, B, F) return dispatch_c<G, B, F>(X, M, K, sp, q, tok_scale, tok_rowsum, st)
    if (g == 64) {
        if (bits == 8) { if (f32in) W4_RQ(64, 8, true); else W4_RQ(64, 8, false); }
        else { if (f32in) W4_RQ(64, 4, true); else W4_RQ(64, 4, false); }
    } else {
        if (bits == 8) { if (f32in) W4_RQ(256, 8, true); else W4_RQ(256, 8, false); }
        else { if (f32in) W4_RQ(256, 4, true); else W4_RQ(256, 4, false); }
    }
#undef W4_RQ
}

}  // namespace w4
