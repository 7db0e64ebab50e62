// GEMM + dequant for the grouped-scale weight format on gfx950 (large and small M).
//
// ComfyUI-INT-Crush README, "Weight Format": INT4 weights are two nibbles per byte plus
// weight_scale fp16 [out, num_groups]; "Inference / INT4": W4A8 = unpack INT4 to INT8,
// dynamic activation quantization, INT8 GEMM with fused dequant; W4A16 (rot_size 0) =
// unpack INT4 to a float matrix and a float GEMM.
//
//   W4A8 / W4A4:  y[m, n] = s_x[m] * sum_j s_w[n, j] * acc_j[m, n] + lr[m, n] + bias[n]
//                 acc_j = sum over group j (gw consecutive k) of q[m, k] * c[n, k]   (int32)
//   W4A16:        y[m, n] = sum_j s_w[n, j] * sum_{k in j} x[m, k] * c[n, k] + lr + bias
//
// Weight codes are signed (symmetric) nibbles.  Group partial sums are exact: int32 on the
// int8 matrix cores, and on the bf16 ones every product of a bf16 activation and a small
// integer code is exact with fp32 accumulation.  At the end of each group the lane's
// accumulators are scaled by the group's fp16 scale into fp32 running sums and restarted.
//
// Operands.  Weights are the MFMA A operand (rows = output features), activations the B
// operand (columns = tokens); a lane ends up holding 4 consecutive features of one token per
// register group.  A signed nibble moved into the high half of a byte is the int8 value
// 16 * c; the factor 16 (256 for int4 x int4) goes into the final scale, exactly.  For the
// bf16 path the same int8 values are converted to bf16 (exact).  k order inside a step is
// natural (int8 x int8, bf16) or even/odd on both sides (int4 x int4).
//
// Tiles.  4 waves, WM x WN of them, each FM x FN blocks of 32 x 32.  Large M: 2 x 2 waves of
// 2 x 2 blocks (128 x 128 tile), an LDS ring of 64-k stages.  Small M (<= 64): 1 x 4
// waves of FM x 1 blocks (32 or 64 tokens x 128 features), and K split over
// several workgroups whose partial sums (fp32, or int32 for the raw output) go to the
// caller's workspace and are added in a fixed order by k_grp_reduce, which applies the
// epilogue.  Each stage (activations, weights, and the stage's weight scales, one dword per
// feature) arrives by direct global -> LDS loads spread evenly over the waves.
#include <algorithm>
#include <type_traits>

#include <hip/hip_fp16.h>

#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

constexpr int BK = 64;

enum { kOutBf16 = 0, kOutI32 = 1, kPartF32 = 2, kPartI32 = 3 };

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float fl16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

template <int AT, int FM, int FN, int WM, int WN, int STAGES>
struct Cfg {
    static_assert(WM * WN == 4, "four waves");
    static constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
    static constexpr int AROW = AT == 8 ? BK : AT == 4 ? BK / 2 : 2 * BK;  // activation bytes per row
    static constexpr int ACT = BM * AROW;
    static constexpr int WROW = BK / 2;                                     // 32 packed weight bytes
    static constexpr int WB = BN * WROW;
    static constexpr int SC = BN * 4;                                       // one dword per feature
    static constexpr int STAGE = ACT + WB + SC;
    static constexpr int CA = ACT / 16 / 4;                                 // activation chunks per wave
    static constexpr int CW = WB / 16 / 4;                                  // weight chunks per wave
    static constexpr int AI = (CA + 63) / 64;                               // instructions
    static constexpr int WI = (CW + 63) / 64;
    static constexpr int LOADS = AI + WI + 1;                               // per wave and stage
    static constexpr int LDS = STAGES * STAGE;
    static_assert(BN / 4 <= 64, "one scale instruction per wave");
    static_assert((STAGES - 1) * LOADS <= 63, "vmcnt range");
};

// physical 16-byte chunk of logical chunk c in row r (involutions)
template <int ROWBYTES>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (ROWBYTES == 128) return c ^ (r & 7);
    else if constexpr (ROWBYTES == 64) return c ^ ((r >> 1) & 3);
    else return c ^ ((r >> 3) & 1);  // 32-byte rows: rows r and r + 8 of a 16-lane read differ
}

struct GrpArgs {
    const uint8_t *A;        // int8 [M, K], packed int4 [M, K/2], or bf16 [M, K]
    const float *sx;         // [M] (integer activations)
    const uint8_t *B;        // packed weights [N, K/2]
    const uint16_t *gs;      // fp16 [N, K / gw]
    int gw;
    const void *bias;
    int bias_bf16;
    const float *lr_t;       // [M, r] (row stride lr_ldt) or null
    const uint16_t *lr_l2;   // bf16 [r, N]
    int lr_r;
    int64_t lr_ldt;
    void *Y;
    int64_t M, N, K;
    int S;                   // K ranges
    void *part;              // [S, M, N] partial sums (split)
};

// Per-lane byte offsets of one stage's direct loads, relative to the stage's uniform base
// addresses (computed once: rows clamped to the last valid row, chunks swizzled), and the
// number of lanes of the last activation instruction that carry a chunk.
template <int AT, int FM, int FN, int WM, int WN, int STAGES>
struct StageOffsets {
    using C = Cfg<AT, FM, FN, WM, WN, STAGES>;
    uint32_t a[C::AI], w[C::WI], s;
};

template <int AT, int FM, int FN, int WM, int WN, int STAGES>
__device__ __forceinline__ StageOffsets<AT, FM, FN, WM, WN, STAGES> stage_offsets(const GrpArgs &p, int64_t m0,
                                                                                 int64_t n0, int wave, int lane) {
    using C = Cfg<AT, FM, FN, WM, WN, STAGES>;
    StageOffsets<AT, FM, FN, WM, WN, STAGES> o;
    const int ebits = AT == 8 ? 8 : AT == 4 ? 4 : 16;
    const int64_t krow = (p.K * ebits) / 8;  // activation row bytes
#pragma unroll
    for (int i = 0; i < C::AI; ++i) {
        const int ci = min(wave * C::CA + i * 64 + lane, (wave + 1) * C::CA - 1);
        const int r = (ci * 16) / C::AROW, pc = ci % (C::AROW / 16);
        const int64_t rr = min<int64_t>(m0 + r, p.M - 1) - m0;
        o.a[i] = (uint32_t)(rr * krow + 16 * swz<C::AROW>(r, pc));
    }
#pragma unroll
    for (int i = 0; i < C::WI; ++i) {
        const int ci = min(wave * C::CW + i * 64 + lane, (wave + 1) * C::CW - 1);
        const int n = ci / 2, pc = ci % 2;
        const int64_t nn = min<int64_t>(n0 + n, p.N - 1) - n0;
        o.w[i] = (uint32_t)(nn * (p.K / 2) + 16 * swz<32>(n, pc));
    }
    {
        const int nf = C::BN / 4;
        const int n = wave * nf + min(lane, nf - 1);
        const int64_t nn = min<int64_t>(n0 + n, p.N - 1) - n0;
        o.s = (uint32_t)(nn * (p.K / p.gw) * 2);
    }
    return o;
}

// Issue the loads of one stage (global k0 .. k0 + 63) into LDS slot `slot`.  Lanes past a
// wave's share issue nothing (their offsets are clamped only to stay in range); every
// instruction keeps at least one active lane, so each counts once in vmcnt.
template <int AT, int FM, int FN, int WM, int WN, int STAGES>
__device__ __forceinline__ void issue_stage(const GrpArgs &p, const StageOffsets<AT, FM, FN, WM, WN, STAGES> &o,
                                            uint8_t *smem, int slot, int64_t m0, int64_t n0, int64_t k0, int wave,
                                            int lane) {
    using C = Cfg<AT, FM, FN, WM, WN, STAGES>;
    const uint32_t base = lds_addr(smem) + slot * C::STAGE;
    const int ebits = AT == 8 ? 8 : AT == 4 ? 4 : 16;
    const int64_t krow = (p.K * ebits) / 8;
    const uint64_t ga = (uint64_t)(p.A + m0 * krow + (k0 * ebits) / 8);
#pragma unroll
    for (int i = 0; i < C::AI; ++i)
        if (C::CA % 64 == 0 || i * 64 + lane < C::CA) gl_lds16_so(ga, o.a[i], base + (wave * C::CA + i * 64) * 16);
    const uint64_t gb = (uint64_t)(p.B + n0 * (p.K / 2) + k0 / 2);
#pragma unroll
    for (int i = 0; i < C::WI; ++i)
        if (C::CW % 64 == 0 || i * 64 + lane < C::CW) gl_lds16_so(gb, o.w[i], base + C::ACT + (wave * C::CW + i * 64) * 16);
    // scales of this stage: one dword per feature (gw = 32: the stage's two groups; else the
    // group holding the stage, zero-extended)
    const int nf = C::BN / 4;
    const uint64_t gs = (uint64_t)(p.gs + n0 * (p.K / p.gw) + k0 / p.gw);
    const uint32_t lb = base + C::ACT + C::WB + wave * nf * 4;
    if (lane < nf) {
        if (p.gw == 32) gl_lds4_so(gs, o.s, lb);
        else gl_lds2_so(gs, o.s, lb);
    }
}

__device__ __forceinline__ v4i nat16(uint32_t d0, uint32_t d1) {
    uint32_t a, b, c, d;
    unpack_nat(d0, a, b);
    unpack_nat(d1, c, d);
    return v4i{(int)a, (int)b, (int)c, (int)d};
}

// 8 codes of one packed dword (k .. k+7) as bf16 values 16 * c in natural order
__device__ __forceinline__ bf8 bf16_codes(uint32_t d) {
    const uint32_t e = nib_evens16(d), o = nib_odds16(d);
    bf8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = (__bf16)(float)(int)(int8_t)(e >> (8 * i));
        r[2 * i + 1] = (__bf16)(float)(int)(int8_t)(o >> (8 * i));
    }
    return r;
}

// Byte offset of the epilogue's bf16 staging rows: past the staged l2 rows (r x BN bf16).
__host__ __device__ constexpr int grp_stg_off(int r, int bn) { return (2 * r * bn + 15) / 16 * 16; }

// Two waves per SIMD (at most 256 registers per lane): one wave's group scaling and operand
// unpacking then runs beside the other's MFMAs.
template <int AT, int FM, int FN, int WM, int WN, int STAGES, int EPI>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) k_gemm_grp(GrpArgs p, int tiles_m,
                                                                                           int tiles_n) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using C = Cfg<AT, FM, FN, WM, WN, STAGES>;
    constexpr bool INT = AT != 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, h = lane >> 5;

    // tile and K range: the blocks are dealt to the 8 XCDs round-robin; XCD x takes one of
    // 4 x 2 rectangular regions of the tile grid (when the grid divides so), walking M inside
    // each column of its region, so the A and B panels it streams are a quarter of M and half
    // of N; otherwise a contiguous run of column-major tiles
    const int ntiles = tiles_m * tiles_n;
    int b = (int)blockIdx.x;
    const int kp = b / ntiles;
    b -= kp * ntiles;
    int tm, tn;
    if (tiles_m % 4 == 0 && tiles_n % 2 == 0) {
        const int x = b % 8, j = b / 8;                    // XCD, index inside its region
        const int rm = tiles_m / 4, rn = tiles_n / 2;      // region size
        tm = (x % 4) * rm + j % rm;
        tn = (x / 4) * rn + j / rm;
    } else {
        if (ntiles % 8 == 0) b = (b % 8) * (ntiles / 8) + b / 8;
        tm = b % tiles_m;
        tn = b / tiles_m;
    }
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int64_t KS = p.K / p.S;
    const int64_t kbeg = kp * KS;
    const int nk = (int)(KS / BK);

    // groups end after this many 32-k (int) or 16-k (bf16) steps
    constexpr int KSTEP = INT ? 32 : 16;
    constexpr int NSTEP = BK / KSTEP;
    const int steps_per_group = p.gw / KSTEP;

    typedef typename std::conditional<INT, v16i, fl16>::type AccT;
    AccT acc[FM][FN];
    fl16 accf[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc[i][j][v] = 0;
                accf[i][j][v] = 0.0f;
            }
        }

    const StageOffsets<AT, FM, FN, WM, WN, STAGES> so = stage_offsets<AT, FM, FN, WM, WN, STAGES>(p, m0, n0, wave, lane);
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue_stage<AT, FM, FN, WM, WN, STAGES>(p, so, smem, s, m0, n0, kbeg + s * BK, wave, lane);

    int gstep = 0;  // steps into the current group
    for (int kt = 0; kt < nk; ++kt) {
        const int slot = kt % STAGES;
        // stage kt has landed once at most (stages issued after it) * LOADS remain
        const int after = min(nk - 1 - kt, STAGES - 2);
        wait_rem<C::LOADS, STAGES - 2>(after);
        // publish: every wave's share of stage kt is in LDS and every wave is done with stage
        // kt - 1, whose slot the loads issued next overwrite (a bare s_barrier: the waits above
        // are the only ones wanted, not a drain of every stage in flight)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + STAGES - 1 < nk)
            issue_stage<AT, FM, FN, WM, WN, STAGES>(p, so, smem, (kt + STAGES - 1) % STAGES, m0, n0,
                                                    kbeg + (int64_t)(kt + STAGES - 1) * BK, wave, lane);
        const uint8_t *st = smem + slot * C::STAGE;
        const uint8_t *wst = st + C::ACT;
        const uint32_t *sct = reinterpret_cast<const uint32_t *>(st + C::ACT + C::WB);
#pragma unroll
        for (int ks = 0; ks < NSTEP; ++ks) {
            if constexpr (INT) {
                v4i wf[FN], xf[FM];
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = wn * FN * 32 + j * 32 + l32;
                    const uint2 d = *reinterpret_cast<const uint2 *>(wst + n * 32 + 16 * swz<32>(n, ks) + 8 * h);
                    wf[j] = AT == 8 ? nat16(d.x, d.y) : evod(d.x, d.y);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = wm * FM * 32 + i * 32 + l32;
                    if constexpr (AT == 8) {
                        const uint4 x = *reinterpret_cast<const uint4 *>(st + r * C::AROW + 16 * swz<64>(r, 2 * ks + h));
                        xf[i] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
                    } else {
                        const uint2 x = *reinterpret_cast<const uint2 *>(st + r * C::AROW + 16 * swz<32>(r, ks) + 8 * h);
                        xf[i] = evod(x.x, x.y);
                    }
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[j], xf[i], acc[i][j], 0, 0, 0);
            } else {
                bf8 wf[FN], xf[FM];
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = wn * FN * 32 + j * 32 + l32;
                    // codes k = 16 ks + 8 h .. + 7: byte 8 ks + 4 h of the 32-byte stage row
                    const uint32_t d = *reinterpret_cast<const uint32_t *>(
                        wst + n * 32 + 16 * swz<32>(n, ks >> 1) + 8 * (ks & 1) + 4 * h);
                    wf[j] = bf16_codes(d);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = wm * FM * 32 + i * 32 + l32;
                    xf[i] = *reinterpret_cast<const bf8 *>(st + r * C::AROW + 16 * swz<128>(r, 2 * ks + h));
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
            }
            if constexpr (EPI == kOutBf16 || EPI == kPartF32) {
                if (++gstep == steps_per_group) {
                    gstep = 0;
                    // group scale of the lane's features: for gw = 32 the stage holds two
                    // groups, the first in the low half of the feature's dword
                    const int sh = (p.gw == 32 && (ks * KSTEP) / 32 == 1) ? 16 : 0;
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        float sv[16];
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int nl = wn * FN * 32 + j * 32 + 8 * g + 4 * h;
                            const uint4 s4 = *reinterpret_cast<const uint4 *>(sct + nl);
                            const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                sv[4 * g + u] = __half2float(__ushort_as_half((uint16_t)(sw[u] >> sh)));
                        }
#pragma unroll
                        for (int i = 0; i < FM; ++i) {
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                accf[i][j][v] = fmaf((float)acc[i][j][v], sv[v], accf[i][j][v]);
                                acc[i][j][v] = 0;
                            }
                        }
                    }
                }
            }
        }
    }

    // ---- output.  Block (i, j), lane l, register v: feature n = 8 (v / 4) + 4 h + v % 4 of the
    // block, token m = l % 32 of the block.
    constexpr float UNSCALE = AT == 4 ? 1.0f / 256 : 1.0f / 16;
    constexpr int SHIFT = AT == 4 ? 8 : 4;
    if constexpr (EPI == kPartF32 || EPI == kPartI32) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t m = m0 + wm * FM * 32 + i * 32 + l32;
            if (m >= p.M) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t n = n0 + wn * FN * 32 + j * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                    if (n >= p.N) continue;
                    const int64_t o = ((int64_t)kp * p.M + m) * p.N + n;
                    if constexpr (EPI == kPartF32) reinterpret_cast<float *>(p.part)[o] = accf[i][j][v];
                    else reinterpret_cast<int32_t *>(p.part)[o] = acc[i][j][v];
                }
        }
        return;
    }
    if constexpr (EPI == kOutI32) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t m = m0 + wm * FM * 32 + i * 32 + l32;
            if (m >= p.M) continue;
            int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t n = n0 + wn * FN * 32 + j * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                    if (n < p.N) Y[n] = acc[i][j][v] >> SHIFT;
                }
        }
        return;
    }
    // bf16 output: stage the tile's l2 rows in LDS (the ring is free once every wave is past it)
    const int r = p.lr_t ? p.lr_r : 0;
    uint16_t *l2s = reinterpret_cast<uint16_t *>(smem);
    __syncthreads();  // every wave is past the ring
    if (r) {
        for (int e = tid; e < r * C::BN; e += 256) {
            const int q = e / C::BN, nl = e % C::BN;
            const int64_t n = min<int64_t>(n0 + nl, p.N - 1);
            l2s[e] = p.lr_l2[(int64_t)q * p.N + n];
        }
        __syncthreads();
    }
    // Each wave converts 32 tokens at a time into its own bf16 staging rows (past the l2 rows)
    // and stores them as 16-byte row chunks: stores of 8-byte pieces straight from the
    // accumulator layout (one per token row and lane half) cost far more.
    constexpr int WF = 32 * FN;                  // features per wave
    constexpr int SROW = 2 * WF + 16;            // staged row bytes (padded)
    constexpr int CPR = 2 * WF / 16;             // 16-byte chunks per row
    uint8_t *stg = smem + grp_stg_off(r, C::BN) + wave * 32 * SROW;
    const bool tile_in = m0 + C::BM <= p.M && n0 + C::BN <= p.N && (p.N & 7) == 0;
    uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = min<int64_t>(m0 + wm * FM * 32 + i * 32 + l32, p.M - 1);  // rows past M: staged, not stored
        const float xs = INT ? p.sx[m] * UNSCALE : UNSCALE;
        const float *tr = r ? p.lr_t + m * p.lr_ldt : nullptr;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * FN * 32 + j * 32 + 8 * g + 4 * h;
                const int64_t n = n0 + nl;
                float y[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) y[u] = accf[i][j][4 * g + u] * xs;
                if (r) {
                    for (int q = 0; q < r; ++q) {
                        const float t = tr[q];
#pragma unroll
                        for (int u = 0; u < 4; ++u) y[u] = fmaf(t, bf16_to_f32(l2s[q * C::BN + nl + u]), y[u]);
                    }
                }
                if (p.bias) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int64_t nb = min<int64_t>(n + u, p.N - 1);
                        y[u] += p.bias_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[nb])
                                            : reinterpret_cast<const float *>(p.bias)[nb];
                    }
                }
                *reinterpret_cast<uint2 *>(stg + l32 * SROW + (j * 32 + 8 * g + 4 * h) * 2) =
                    make_uint2(f32_to_bf16(y[0]) | (f32_to_bf16(y[1]) << 16), f32_to_bf16(y[2]) | (f32_to_bf16(y[3]) << 16));
            }
        // the block's rows: LDS operations of one wave complete in order, so these reads see
        // the writes above and the next block's writes follow them
        const int64_t mrow0 = m0 + wm * FM * 32 + i * 32;
        const int64_t ncol0 = n0 + wn * WF;
        constexpr int NCH = 32 * CPR / 64;
        uint4 v[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int c = lane + 64 * k;
            v[k] = *reinterpret_cast<const uint4 *>(stg + (c / CPR) * SROW + (c % CPR) * 16);
        }
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int c = lane + 64 * k;
            const int64_t mm = mrow0 + c / CPR, nn = ncol0 + (c % CPR) * 8;
            if (tile_in) {
                *reinterpret_cast<uint4 *>(Y + mm * p.N + nn) = v[k];
            } else if (mm < p.M) {
                const uint16_t *hv = reinterpret_cast<const uint16_t *>(&v[k]);
                for (int u = 0; u < 8; ++u)
                    if (nn + u < p.N) Y[mm * p.N + nn + u] = hv[u];
            }
        }
    }
}

// Fixed-order sum of the S partial sums and the epilogue (one thread per output).
template <int AT, bool I32>
__global__ void __launch_bounds__(256) k_grp_reduce(GrpArgs p) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= p.M * p.N) return;
    const int64_t m = e / p.N, n = e % p.N;
    const int64_t MN = p.M * p.N;
    if constexpr (I32) {
        constexpr int SHIFT = AT == 4 ? 8 : 4;
        const int32_t *part = reinterpret_cast<const int32_t *>(p.part);
        int32_t s = 0;
        for (int k = 0; k < p.S; ++k) s += part[k * MN + e];
        reinterpret_cast<int32_t *>(p.Y)[e] = s >> SHIFT;
    } else {
        constexpr float UNSCALE = AT == 4 ? 1.0f / 256 : 1.0f / 16;
        const float *part = reinterpret_cast<const float *>(p.part);
        float s = 0.0f;
        for (int k = 0; k < p.S; ++k) s += part[k * MN + e];
        float y = s * (AT != 16 ? p.sx[m] * UNSCALE : UNSCALE);
        if (p.lr_t)
            for (int q = 0; q < p.lr_r; ++q) y = fmaf(p.lr_t[m * p.lr_ldt + q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + n]), y);
        if (p.bias)
            y += p.bias_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[n])
                             : reinterpret_cast<const float *>(p.bias)[n];
        reinterpret_cast<uint16_t *>(p.Y)[e] = (uint16_t)f32_to_bf16(y);
    }
}

template <int AT, int FM, int FN, int WM, int WN, int STAGES, int EPI>
hipError_t launch_cfg(const GrpArgs &a, hipStream_t st) {
    using C = Cfg<AT, FM, FN, WM, WN, STAGES>;
    // the ring, or (bf16 output) the staged l2 rows and the four waves' staging rows
    const size_t lds = std::max<size_t>(C::LDS, (size_t)grp_stg_off(a.lr_r, C::BN) + 4 * 32 * (64 * FN + 16));
    auto kern = k_gemm_grp<AT, FM, FN, WM, WN, STAGES, EPI>;
    if (lds > 65536) {
        static const hipError_t attr =
            hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024);
        if (attr != hipSuccess) return attr;
    }
    const int tiles_m = (int)((a.M + C::BM - 1) / C::BM), tiles_n = (int)((a.N + C::BN - 1) / C::BN);
    hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n * a.S)), dim3(256), lds, st, a, tiles_m, tiles_n);
    return hipGetLastError();
}

// K ranges for a small-M grid: about three workgroups per compute unit, each range a whole
// number of stages and of groups and at least 4 stages long.
int plan_s(int64_t M, int64_t N, int64_t K, int gw) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t tiles = (N + 127) / 128;
    int S = 1;
    while (S < 32 && tiles * S < 3 * ncu && K % (2 * S * std::max(gw, BK)) == 0 && K / (2 * S) >= 4 * BK)
        S *= 2;
    return S;
}

// Ring depths (measured at 4096 x 3072 x 3072 and at 1 and 16 tokens x 4096 -> 12288, two waves
// per SIMD): large M, 3 stages for int8 and bf16 activations, 4 for int4; small M, 4 stages
// with K split over about three workgroups per CU.
template <int AT, int EPI>
hipError_t launch_at(const GrpArgs &a, hipStream_t st) {
    if (a.M > 64) return AT == 4 ? launch_cfg<AT, 2, 2, 2, 2, 4, EPI>(a, st) : launch_cfg<AT, 2, 2, 2, 2, 3, EPI>(a, st);
    if (a.M > 32) return launch_cfg<AT, 2, 1, 1, 4, 4, EPI>(a, st);
    return launch_cfg<AT, 1, 1, 1, 4, 4, EPI>(a, st);
}

// ---------------------------------------------------------------------------------------------
// Streaming form for M <= 16 (the HBM-bound regime): no workgroup barrier in the main loop and
// no K split.  A workgroup of NW waves owns R = 16 RB weight rows; in each stage of 256 NW k,
// wave w takes k in [256 w, 256 w + 256) and streams, through its own LDS ring of D stages,
// its slice of every staged token, its 128-byte piece of each of the R rows and those rows'
// scales of the groups in its slice (direct global -> LDS loads), multiplying a stage as soon
// as its own loads have landed.  Output layout of the 16 x 16 MFMA: lane l, register r holds
// weight row 4 (l / 16) + r of token l % 16.  The k order inside an MFMA is chosen so that each
// MFMA covers whole groups: integer activations, v_mfma_i32_16x16x64_i8 over 64 consecutive k
// (lane group kb the 16 k at 16 kb); bf16 activations, v_mfma_f32_16x16x32_bf16 over 32
// consecutive k (lane group kb the 8 k at 8 kb).  After each group the lane's four int32 (or
// fp32) sums are scaled by their rows' group scales into fp32 running sums; the waves' sums
// are added through LDS in a fixed order at the end.
constexpr int kGsDepth = 2;  // stages in flight per wave

template <int AT, int TM, int RB, int NW, int GW>
struct GSL {
    static constexpr int KS = 256 * NW;                                  // k per stage
    static constexpr int R = 16 * RB;
    static constexpr int TB = AT == 8 ? 256 : AT == 4 ? 128 : 512;       // token bytes per wave and stage
    static constexpr int CPT = TB / 16;                                  // 16-byte chunks per token slice
    static constexpr int ACT = TM * TB < 1024 ? 1024 : TM * TB;          // whole 1 KB loads
    static constexpr int WB = R * 128;                                   // weight bytes per wave and stage
    static constexpr int SB = 512 / GW;                                  // scale bytes per row and wave-stage
    static constexpr int SCL = GW == 256 ? 1 : (R * SB / 4 + 63) / 64;   // scale loads (dwords per lane)
    static constexpr int SCB = SCL * 256;
    static constexpr int SLOT = ACT + WB + SCB;
    static constexpr int D = kGsDepth;
    static constexpr int LA = ACT / 1024, LB = WB / 1024;
    static constexpr int LPS = LA + LB + SCL;                            // loads per stage
    static constexpr int RED = NW * RB * 1024;                           // fp32 tiles of the waves
    static constexpr int RING = NW * D * SLOT > RED ? NW * D * SLOT : RED;
    static constexpr int C_SX = RING, C_BIAS = C_SX + 256;
    static constexpr int LDS = C_BIAS + 256;
    static constexpr int NG = 256 / GW;                                  // groups per wave-stage
    static_assert(R <= 64 && (D - 1) * LPS <= 63 && LDS <= 160 * 1024, "grouped streaming layout");
};

template <int AT, int TM, int RB, int NW, int GW, bool I32>
__global__ void __launch_bounds__(64 * NW) k_grp_stream(GrpArgs p) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = GSL<AT, TM, RB, NW, GW>;
    constexpr int R = L::R;
    constexpr uint32_t ASTEP = L::KS * (AT == 16 ? 2 : AT == 8 ? 1 : 0) + (AT == 4 ? L::KS / 2 : 0);
    constexpr uint32_t BSTEP = L::KS / 2;
    constexpr bool INT = AT != 16;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kb = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * R;
    const int64_t K = p.K, M = p.M;
    const int nst = (int)(K / L::KS);
    const int64_t rowA = (K * AT) / 8;
    const int64_t rowB = K / 2;
    const int64_t ng = K / GW;  // scale groups per row
    const uint32_t smem_base = lds_addr(smem);
    const int ring = wave * L::D * L::SLOT;

    // per-lane load offsets at stage 0: LDS position (t, c) of a token slice holds global
    // chunk c ^ (t & (CPT - 1)); position (r, c) of a weight row holds chunk c ^ (r & 7)
    uint32_t arow[L::LA], ain[L::LA], brow[L::LB], bin[L::LB], srow[L::SCL], sin_[L::SCL];
#pragma unroll
    for (int j = 0; j < L::LA; ++j) {
        const int f = min(j * 64 + lane, TM * L::CPT - 1);
        const int t = f / L::CPT, c = f % L::CPT;
        arow[j] = (uint32_t)(min<int64_t>(t, M - 1) * rowA);
        ain[j] = (uint32_t)(wave * L::TB + 16 * (c ^ (t & (L::CPT - 1))));
    }
#pragma unroll
    for (int j = 0; j < L::LB; ++j) {
        const int r = 8 * j + lane / 8;
        brow[j] = (uint32_t)((min<int64_t>(n0 + r, p.N - 1) - n0) * rowB);
        bin[j] = (uint32_t)(128 * wave + 16 * ((lane & 7) ^ (r & 7)));
    }
    // scales: GW = 256, one fp16 per row (lane = row); GW = 128, one dword (two groups) per
    // row; GW = 64, two dwords per row (lane = 2 row + half)
#pragma unroll
    for (int j = 0; j < L::SCL; ++j) {
        const int f = j * 64 + lane;
        const int r = GW == 64 ? min(f / 2, R - 1) : min(f, R - 1);
        const int h = GW == 64 ? f % 2 : 0;
        srow[j] = (uint32_t)((min<int64_t>(n0 + r, p.N - 1) - n0) * ng * 2);
        sin_[j] = (uint32_t)(((int64_t)256 * wave / GW) * 2 + 4 * h);
    }
    const uint64_t abase = (uint64_t)p.A;
    const uint64_t bbase = (uint64_t)(p.B + n0 * rowB);
    const uint64_t sbase = (uint64_t)(p.gs + n0 * ng);
    auto issue = [&](int i) __attribute__((always_inline)) {
        const uint32_t slot = smem_base + (uint32_t)(ring + (i % L::D) * L::SLOT);
#pragma unroll
        for (int j = 0; j < L::LA; ++j) gl_lds16_so(abase, arow[j] + ain[j] + (uint32_t)i * ASTEP, slot + 1024 * j);
#pragma unroll
        for (int j = 0; j < L::LB; ++j) gl_lds16_so(bbase, brow[j] + bin[j] + (uint32_t)i * BSTEP, slot + L::ACT + 1024 * j);
        const uint32_t soff = (uint32_t)i * (uint32_t)(L::KS / GW * 2);
#pragma unroll
        for (int j = 0; j < L::SCL; ++j) {
            if constexpr (GW == 256) gl_lds2_so(sbase, srow[j] + sin_[j] + soff, slot + L::ACT + L::WB + 256 * j);
            else gl_lds4_so(sbase, srow[j] + sin_[j] + soff, slot + L::ACT + L::WB + 256 * j);
        }
    };

    // constants first (wave 0): token scales and biases, one dword each (oldest loads, so the
    // stage waits below need not count them)
    if (wave == 0) {
        const uint32_t t = (uint32_t)min<int64_t>(lane, M - 1);
        if (INT) gl_lds4_so((uint64_t)p.sx, 4 * t, smem_base + L::C_SX);
        const uint32_t c = (uint32_t)(min<int64_t>(n0 + min(lane, R - 1), p.N - 1) - n0);
        if (p.bias && p.bias_bf16) gl_lds2_so((uint64_t)((const uint16_t *)p.bias + n0), 2 * c, smem_base + L::C_BIAS);
        else if (p.bias) gl_lds4_so((uint64_t)((const float *)p.bias + n0), 4 * c, smem_base + L::C_BIAS);
    }
    for (int i = 0; i < L::D; ++i)
        if (i < nst) issue(i);

    typedef typename std::conditional<INT, v4i, v4f>::type Acc;
    Acc acc[RB];
    v4f accf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        acc[rb] = Acc{0, 0, 0, 0};
        accf[rb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int tt = min(lr, (int)M - 1);

    // The stage's scales of the lane's rows 16 rb + 4 kb + 0..3, read from the slot into
    // registers with the operands (the slot is refilled before the MFMAs): per row one dword
    // (GW = 256: the group's fp16 zero-extended; GW = 128: the two groups) or two (GW = 64).
    constexpr int SCW = GW == 64 ? 2 : 1;
    uint4 scv[RB][SCW];
    auto read_scales = [&](const uint8_t *sc) __attribute__((always_inline)) {
        if constexpr (!I32) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int r0 = 16 * rb + 4 * kb;
#pragma unroll
                for (int h = 0; h < SCW; ++h) scv[rb][h] = *reinterpret_cast<const uint4 *>(sc + 4 * SCW * r0 + 16 * h);
            }
        }
    };
    // scale group g (0 .. NG - 1) into the running sums
    auto flush = [&](int g) __attribute__((always_inline)) {
        if constexpr (!I32) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                uint32_t w[4];
                if constexpr (GW == 64) {
                    const uint32_t d[8] = {scv[rb][0].x, scv[rb][0].y, scv[rb][0].z, scv[rb][0].w,
                                           scv[rb][1].x, scv[rb][1].y, scv[rb][1].z, scv[rb][1].w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) w[r] = d[2 * r + g / 2] >> (16 * (g & 1));
                } else {
                    const uint32_t d[4] = {scv[rb][0].x, scv[rb][0].y, scv[rb][0].z, scv[rb][0].w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) w[r] = d[r] >> (16 * g);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sv = __half2float(__ushort_as_half((uint16_t)w[r]));
                    accf[rb][r] = fmaf((float)acc[rb][r], sv, accf[rb][r]);
                    acc[rb][r] = 0;
                }
            }
        }
    };

    for (int i = 0; i < nst; ++i) {
        wait_rem<L::LPS, L::D - 1>(min(L::D - 1, nst - 1 - i));
        const uint8_t *sl = smem + ring + (i % L::D) * L::SLOT;
        const uint8_t *ws_ = sl + L::ACT;
        const uint8_t *sc = sl + L::ACT + L::WB;
        const uint8_t *ta = sl + tt * L::TB;
        if constexpr (INT) {
            // two 64-k MFMAs per 128-k half u; 16 k per lane group
            uint4 xa[4];
            uint2 wv[4][RB];
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // q = 2 u + h: k in [64 q, 64 q + 64)
                if constexpr (AT == 8) {
                    const int g = 4 * q + kb;  // global chunk of the token slice
                    xa[q] = *reinterpret_cast<const uint4 *>(ta + 16 * (g ^ (tt & (L::CPT - 1))));
                } else {
                    const int g = 2 * q + (kb >> 1);
                    const uint2 x2 = *reinterpret_cast<const uint2 *>(ta + 16 * (g ^ (tt & (L::CPT - 1))) + 8 * (kb & 1));
                    xa[q] = make_uint4(x2.x, x2.y, 0, 0);
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int r = 16 * rb + lr;
                    const int g = 2 * q + (kb >> 1);
                    wv[q][rb] = *reinterpret_cast<const uint2 *>(ws_ + r * 128 + 16 * (g ^ (r & 7)) + 8 * (kb & 1));
                }
            }
            read_scales(sc);
            wait_lgkmcnt0();
            if (i + L::D < nst) issue(i + L::D);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v4i a;
                if constexpr (AT == 8) a = __builtin_bit_cast(v4i, xa[q]);
                else a = evod(xa[q].x, xa[q].y);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    v4i w;
                    if constexpr (AT == 8) {
                        uint32_t lo0, hi0, lo1, hi1;
                        unpack_nat(wv[q][rb].x, lo0, hi0);
                        unpack_nat(wv[q][rb].y, lo1, hi1);
                        w = v4i{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
                    } else {
                        w = evod(wv[q][rb].x, wv[q][rb].y);
                    }
                    acc[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a, acc[rb], 0, 0, 0);
                }
                if constexpr (GW == 64) flush(q);
                else if constexpr (GW == 128) {
                    if (q & 1) flush(q >> 1);
                }
            }
            if constexpr (GW == 256) flush(0);
        } else {
            // four 32-k MFMAs per 128-k half u; 8 k per lane group
            bf8 xa[8];
            uint32_t wv[8][RB];
#pragma unroll
            for (int q = 0; q < 8; ++q) {  // k in [32 q, 32 q + 32)
                const int g = 4 * q + kb;
                xa[q] = *reinterpret_cast<const bf8 *>(ta + 16 * (g ^ (tt & (L::CPT - 1))));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int r = 16 * rb + lr;
                    wv[q][rb] = *reinterpret_cast<const uint32_t *>(ws_ + r * 128 + 16 * (q ^ (r & 7)) + 4 * kb);
                }
            }
            read_scales(sc);
            wait_lgkmcnt0();
            if (i + L::D < nst) issue(i + L::D);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf16_codes(wv[q][rb]), xa[q], acc[rb], 0, 0, 0);
                if constexpr (GW == 64) {
                    if (q & 1) flush(q >> 1);
                } else if constexpr (GW == 128) {
                    if ((q & 3) == 3) flush(q >> 2);
                }
            }
            if constexpr (GW == 256) flush(0);
        }
    }

    // ---- reduction of the NW waves' tiles in a fixed order, then the epilogue
    wait_vmcnt<0>();
    __syncthreads();
    v4f *red = reinterpret_cast<v4f *>(smem);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        v4f v;
        if constexpr (I32) v = __builtin_bit_cast(v4f, acc[rb]);
        else v = accf[rb];
        red[(wave * RB + rb) * 64 + lane] = v;
    }
    __syncthreads();
    constexpr float UNSCALE = AT == 4 ? 1.0f / 256 : 1.0f / 16;
    constexpr int SHIFT = AT == 4 ? 8 : 4;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        if (rb % NW != wave) continue;
        const int64_t m = lr;
        if (m >= M) continue;
        const int rl = 16 * rb + 4 * kb;
        const int64_t nb = n0 + rl;
        if constexpr (I32) {
            v4i t = __builtin_bit_cast(v4i, red[rb * 64 + lane]);
#pragma unroll
            for (int q = 1; q < NW; ++q) t += __builtin_bit_cast(v4i, red[(q * RB + rb) * 64 + lane]);
            int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nb + r < p.N) Y[nb + r] = t[r] >> SHIFT;
        } else {
            v4f t = red[rb * 64 + lane];
#pragma unroll
            for (int q = 1; q < NW; ++q) t += red[(q * RB + rb) * 64 + lane];
            const float xs = INT ? *reinterpret_cast<const float *>(smem + L::C_SX + 4 * m) * UNSCALE : UNSCALE;
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = t[r] * xs;
            if (p.lr_t) {
                const float *tr = p.lr_t + m * p.lr_ldt;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t nc = min<int64_t>(nb + r, p.N - 1);
                    float l = y[r];
                    for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + nc]), l);
                    y[r] = l;
                }
            }
            if (p.bias) {
                const uint4 b4 = *reinterpret_cast<const uint4 *>(smem + L::C_BIAS + 4 * rl);
                const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) y[r] += __uint_as_float(p.bias_bf16 ? bw[r] << 16 : bw[r]);
            }
            uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y) + m * p.N;
            if (nb + 3 < p.N && (p.N & 3) == 0) {
                *reinterpret_cast<uint2 *>(Y + nb) =
                    make_uint2(f32_to_bf16(y[0]) | (f32_to_bf16(y[1]) << 16), f32_to_bf16(y[2]) | (f32_to_bf16(y[3]) << 16));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < p.N) Y[nb + r] = (uint16_t)f32_to_bf16(y[r]);
            }
        }
    }
}

template <int AT, int TM, int RB, int NW, int GW, bool I32>
hipError_t launch_gs_k(const GrpArgs &a, hipStream_t st) {
    using L = GSL<AT, TM, RB, NW, GW>;
    auto kern = k_grp_stream<AT, TM, RB, NW, GW, I32>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS);
    if (attr != hipSuccess) return attr;
    const unsigned grid = (unsigned)((a.N + L::R - 1) / L::R);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), L::LDS, st, a);
    return hipGetLastError();
}

int num_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu;
}

// Waves per workgroup of the grouped streaming launch: 8 (two per SIMD) when 16-row
// workgroups give about one per CU and K holds whole 2048-k stages, else 4 (K % 1024 == 0).
int gs_waves(int64_t M, int64_t N, int64_t K) {
    if (M <= 8 && (N + 15) / 16 <= num_cus() && K % 2048 == 0) return 8;
    return K % 1024 == 0 ? 4 : 0;
}

template <int AT, int TM, int GW, bool I32>
hipError_t gs_shape(const GrpArgs &a, hipStream_t st) {
    if constexpr (TM <= 8) {
        if (gs_waves(a.M, a.N, a.K) == 8) return launch_gs_k<AT, TM, 1, 8, GW, I32>(a, st);
        return launch_gs_k<AT, TM, 1, 4, GW, I32>(a, st);
    } else {
        const int64_t rb = (a.N + 16 * 256 - 1) / (16 * 256);
        if (rb <= 1) return launch_gs_k<AT, TM, 1, 4, GW, I32>(a, st);
        if (rb <= 2) return launch_gs_k<AT, TM, 2, 4, GW, I32>(a, st);
        if (rb <= 3) return launch_gs_k<AT, TM, 3, 4, GW, I32>(a, st);
        return launch_gs_k<AT, TM, 4, 4, GW, I32>(a, st);
    }
}

template <int AT, int GW, bool I32>
hipError_t gs_tm(const GrpArgs &a, hipStream_t st) {
    if (a.M <= 1) return gs_shape<AT, 1, GW, I32>(a, st);
    if (a.M <= 2) return gs_shape<AT, 2, GW, I32>(a, st);
    if (a.M <= 4) return gs_shape<AT, 4, GW, I32>(a, st);
    if (a.M <= 8) return gs_shape<AT, 8, GW, I32>(a, st);
    return gs_shape<AT, 16, GW, I32>(a, st);
}

// The streaming form takes M <= 16, gw >= 64 and K a whole number of 1024-k stages.
bool gs_ok(const GrpArgs &a) { return a.M <= 16 && a.gw >= 64 && gs_waves(a.M, a.N, a.K) != 0; }

template <int AT, bool I32>
hipError_t launch_gs(const GrpArgs &a, hipStream_t st) {
    switch (a.gw) {
        case 64: return gs_tm<AT, 64, I32>(a, st);
        case 128: return gs_tm<AT, 128, I32>(a, st);
        default: return gs_tm<AT, 256, I32>(a, st);
    }
}

template <int AT, bool I32>
hipError_t launch_grp(GrpArgs a, void *ws, size_t ws_bytes, hipStream_t st) {
    a.S = 1;
    a.part = nullptr;
    if (gs_ok(a)) return launch_gs<AT, I32>(a, st);
    if (a.M <= 64) {
        const int S = plan_s(a.M, a.N, a.K, a.gw);
        const size_t need = (size_t)S * a.M * a.N * 4;
        if (S > 1 && ws && ws_bytes >= need) {
            a.S = S;
            a.part = ws;
            hipError_t e = launch_at<AT, I32 ? kPartI32 : kPartF32>(a, st);
            if (e != hipSuccess) return e;
            const int64_t n = a.M * a.N;
            hipLaunchKernelGGL((k_grp_reduce<AT, I32>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
            return hipGetLastError();
        }
    }
    return launch_at<AT, I32 ? kOutI32 : kOutBf16>(a, st);
}

}  // namespace

size_t grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int gw) {
    if (M <= 0 || M > 64) return 0;
    const int S = plan_s(M, N, K, gw);
    return S > 1 ? (size_t)S * M * N * 4 : 0;
}

hipError_t launch_gemm_grouped(const GroupedArgs &g, int act_bits, void *ws, size_t ws_bytes, hipStream_t st) {
    if (g.M == 0) return hipSuccess;
    GrpArgs a{};
    a.A = static_cast<const uint8_t *>(g.A);
    a.sx = g.sx;
    a.B = g.B;
    a.gs = g.gs;
    a.gw = g.gw;
    a.bias = g.bias;
    a.bias_bf16 = g.bias_bf16;
    a.lr_t = g.lr_t;
    a.lr_l2 = g.lr_l2;
    a.lr_r = g.lr_t ? g.lr_r : 0;
    a.lr_ldt = g.lr_ldt;
    a.Y = g.Y;
    a.M = g.M;
    a.N = g.N;
    a.K = g.K;
    if (act_bits == 16 && g.y_i32) return hipErrorInvalidValue;
    switch (act_bits) {
        case 8: return g.y_i32 ? launch_grp<8, true>(a, ws, ws_bytes, st) : launch_grp<8, false>(a, ws, ws_bytes, st);
        case 4: return g.y_i32 ? launch_grp<4, true>(a, ws, ws_bytes, st) : launch_grp<4, false>(a, ws, ws_bytes, st);
        case 16: return launch_grp<16, false>(a, ws, ws_bytes, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4
