// Small-M (M <= 64) integer GEMM + dequant epilogue for gfx950: the HBM-bound regime.
//
// ComfyUI-INT-Crush README, "Inference / INT4" (INT8 GEMM with fused dequant on unpacked
// INT4 weights) and "Inference / OrbitQuant" (the kernel is chosen by batch size: a
// small-M kernel next to the large-M dense GEMM); stable-diffusion.cpp PR #2010, "Summary":
// the packed nibbles are read as stored.
//
// At M <= 64 the layer reads ~0.5 byte of weight per 2 * M integer ops, far below the MFMA
// ridge, so the kernel is organised around streaming the packed weights from HBM once, with
// many bytes in flight and in long contiguous runs:
//  - a workgroup (4 waves) owns R = 16 * RB consecutive weight rows; their bytes for one
//    stage of 512 k (R rows x 256 bytes) and the token codes of that stage (16 * MB tokens x
//    512 or 256 bytes, from L2) go straight from global memory into an LDS ring with 16-byte
//    global->LDS loads (every wave-instruction reads 1 KB of consecutive bytes), issued up to
//    STAGES - 1 stages ahead without holding any register;
//  - within a stage, wave w takes k in [128 w, 128 w + 128): per 16 weight rows and 16
//    tokens, two v_mfma_i32_16x16x64_i8 (weights the "A" operand, tokens the "B" operand);
//  - the 4 per-wave partial tiles are summed through LDS in a fixed order (exact and
//    deterministic), then the epilogue (the large-M kernel's arithmetic) stores 4 consecutive
//    features of a token per lane.
// Unpacking follows the large-M kernel: nibble -> 16 * code bytes, natural k order against
// int8 token codes, even/odd order on both sides against int4 token codes.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int KC = 512;             // k per stage
constexpr int KW = KC / kWaves;     // 128 k per wave and stage: one pair of MFMA k-steps
constexpr int kLdsBudget = 144 * 1024;

template <int ABITS, int MB, int RB>
struct GL {
    static constexpr int R = 16 * RB;                          // weight rows per workgroup
    static constexpr int T = 16 * MB;                          // token rows staged
    static constexpr int A_ROW = ABITS == 8 ? KC : KC / 2;     // token bytes per stage: 512 / 256
    static constexpr int A_CHUNKS = A_ROW / 16;                // 32 / 16
    static constexpr int A_BYTES = T * A_ROW;
    static constexpr int B_ROW = KC / 2;                       // 256 packed weight bytes per row
    static constexpr int B_BYTES = R * B_ROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int STAGES = kLdsBudget / STAGE < 12 ? kLdsBudget / STAGE : 12;
    static constexpr int DEPTH = STAGES - 1;                   // stages in flight ahead
    static constexpr int A_INSTR = A_BYTES / 1024;             // 1 KB wave-instructions per stage
    static constexpr int B_INSTR = B_BYTES / 1024;
    static constexpr int LW = (A_INSTR + B_INSTR) / kWaves;    // per wave and stage
    static constexpr int RED = kWaves * RB * MB * 1024;        // reduction buffer
    static constexpr int RING = STAGES * STAGE > RED ? STAGES * STAGE : RED;
    static constexpr int C_SW = RING, C_BIAS = C_SW + 256, C_ZP = C_BIAS + 256, C_SX = C_ZP + 256,
                         C_RS = C_SX + 256;
    static constexpr int LDS = C_RS + 256;
    static_assert((A_INSTR + B_INSTR) % kWaves == 0, "whole loads per wave");
    static_assert(STAGES >= 2 && DEPTH * LW <= 63, "vmcnt range");
};

// LDS chunk swizzle (an involution inside a row): the 16 rows / tokens read by one MFMA
// operand land on distinct banks.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 15); }

// Wait until at most s stages of this wave's loads are still in flight (s <= S).
template <int LW, int S>
__device__ __forceinline__ void wait_stages(int s) {
    if constexpr (S == 0) {
        wait_vmcnt<0>();
    } else {
        if (s >= S) wait_vmcnt<S * LW>();
        else wait_stages<LW, S - 1>(s);
    }
}

template <int ABITS, int MB, int RB, bool ASYM>
__global__ void __launch_bounds__(kThreads) k_gemv_ring(LinearArgs p) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = GL<ABITS, MB, RB>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kb = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * L::R;
    const int64_t K = p.K;
    const int nk = (int)((K + KC - 1) / KC);
    const int64_t rowA = ABITS == 8 ? K : K / 2;  // bytes per token row of the codes
    const int64_t rowB = K / 2;

    // ---- per-row constants (scale, bias, zero point) and per-token constants (scale,
    // rowsum) go to LDS past the ring with 4/2/1-byte direct loads issued ahead of the ring's
    // loads (so every wait of the pipeline also covers them); one dword per entry.
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    constexpr float kUnscale = ABITS == 8 ? 1.0f / 16 : 1.0f / 256;
    const uint32_t smem_base = lds_addr(smem);
    if (wave == 0) {
        const uint32_t c = (uint32_t)(min<int64_t>(n0 + min(lane, L::R - 1), p.N - 1) - n0);
        const uint32_t t = (uint32_t)min<int64_t>(lane, p.M - 1);
        gl_lds4_so((uint64_t)(p.sw + n0), 4 * c, smem_base + L::C_SW);
        if (p.bias) {
            if (p.bias_bf16) gl_lds2_so((uint64_t)((const uint16_t *)p.bias + n0), 2 * c, smem_base + L::C_BIAS);
            else gl_lds4_so((uint64_t)((const float *)p.bias + n0), 4 * c, smem_base + L::C_BIAS);
        }
        if constexpr (ASYM) {
            gl_lds1_so((uint64_t)(p.zp + n0), c, smem_base + L::C_ZP);
            gl_lds4_so((uint64_t)p.rowsum, 4 * t, smem_base + L::C_RS);
        }
        gl_lds4_so((uint64_t)p.sx, 4 * t, smem_base + L::C_SX);
    }

    // ---- global->LDS loads.  Load j of a stage (j = wave + 4 i) is 1 KB: token codes for
    // j < A_INSTR (1024 / A_ROW tokens), else 4 weight rows.  Lane l writes LDS bytes
    // [16 l, 16 l + 16) of the load and reads the matching global chunk of the swizzled row.
    // Rows past M / N are clamped to the last valid one (their outputs are never stored), and
    // chunks past K to the last valid chunk of the row (those k are masked to zero codes).
    auto load = [&](int kt, int slot, int i) __attribute__((always_inline)) {
        const int j = wave + kWaves * i;
        const uint32_t dst = smem_base + (uint32_t)(slot * L::STAGE + j * 1024);
        if (j < L::A_INSTR) {
            constexpr int TPI = 1024 / L::A_ROW;
            const int t = j * TPI + lane / L::A_CHUNKS;
            const int c = swz(t, lane % L::A_CHUNKS);
            const int64_t tc = min<int64_t>(t, p.M - 1);
            const int64_t off = min<int64_t>((int64_t)kt * L::A_ROW + 16 * c, rowA - 16);
            gl_lds16_so((uint64_t)p.A, (uint32_t)(tc * rowA + off), dst);
        } else {
            const int r = (j - L::A_INSTR) * 4 + lane / 16;
            const int c = swz(r, lane % 16);
            const int64_t rc = min<int64_t>(n0 + r, p.N - 1) - n0;
            const int64_t off = min<int64_t>((int64_t)kt * L::B_ROW + 16 * c, rowB - 16);
            gl_lds16_so((uint64_t)(p.B + n0 * rowB), (uint32_t)(rc * rowB + off), dst);
        }
    };
    auto issue = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < L::LW; ++i) load(kt, kt % L::STAGES, i);
    };

    v4i acc[RB][MB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = v4i{0, 0, 0, 0};

    for (int s = 0; s < L::DEPTH; ++s)
        if (s < nk) issue(s);

    for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed for every wave; every wave is done with stage kt - 1, whose
        // slot takes stage kt + DEPTH
        wait_stages<L::LW, L::DEPTH - 1>(min(L::DEPTH - 1, nk - 1 - kt));
        __builtin_amdgcn_s_barrier();
        if (kt + L::DEPTH < nk) issue(kt + L::DEPTH);
        const uint8_t *st = smem + (kt % L::STAGES) * L::STAGE;
        // this lane's 32 k: [kt * 512 + 128 * wave + 32 * kb, + 32)
        const bool kvalid = (int64_t)kt * KC + KW * wave + 32 * kb < K;
        v4i a0[MB], a1[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int t = 16 * mb + lr;
            const uint8_t *row = st + t * L::A_ROW;
            if constexpr (ABITS == 8) {
                const int c = 8 * wave + 2 * kb;
                uint4 x0 = *reinterpret_cast<const uint4 *>(row + 16 * swz(t, c));
                uint4 x1 = *reinterpret_cast<const uint4 *>(row + 16 * swz(t, c + 1));
                if (!kvalid) x0 = x1 = make_uint4(0, 0, 0, 0);
                a0[mb] = __builtin_bit_cast(v4i, x0);
                a1[mb] = __builtin_bit_cast(v4i, x1);
            } else {
                uint4 x = *reinterpret_cast<const uint4 *>(row + 16 * swz(t, 4 * wave + kb));
                if (!kvalid) x = make_uint4(0, 0, 0, 0);
                a0[mb] = evod(x.x, x.y);
                a1[mb] = evod(x.z, x.w);
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = 16 * rb + lr;
            uint4 w = *reinterpret_cast<const uint4 *>(st + L::A_BYTES + r * L::B_ROW + 16 * swz(r, 4 * wave + kb));
            if constexpr (ASYM) {
                w.x ^= 0x88888888u; w.y ^= 0x88888888u; w.z ^= 0x88888888u; w.w ^= 0x88888888u;
            }
            v4i w0, w1;
            if constexpr (ABITS == 8) {
                uint32_t q[8];
                unpack_nat(w.x, q[0], q[1]);
                unpack_nat(w.y, q[2], q[3]);
                unpack_nat(w.z, q[4], q[5]);
                unpack_nat(w.w, q[6], q[7]);
                w0 = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
                w1 = v4i{(int)q[4], (int)q[5], (int)q[6], (int)q[7]};
            } else {
                w0 = evod(w.x, w.y);
                w1 = evod(w.z, w.w);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                acc[rb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w0, a0[mb], acc[rb][mb], 0, 0, 0);
                acc[rb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w1, a1[mb], acc[rb][mb], 0, 0, 0);
            }
        }
    }

    // ---- reduce the 4 waves' partial tiles (fixed order), then the epilogue: wave w takes
    // the (row block, token block) pairs p with p % 4 == w.  16x16 layout: lane l, register r
    // holds weight row 4 (l / 16) + r of token l % 16.
    __syncthreads();  // every wave is past its last read of the ring
    v4i *red = reinterpret_cast<v4i *>(smem);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) red[((wave * RB + rb) * MB + mb) * 64 + lane] = acc[rb][mb];
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if ((rb * MB + mb) % kWaves != wave) continue;
            v4i t = red[((0 * RB + rb) * MB + mb) * 64 + lane];
#pragma unroll
            for (int q = 1; q < kWaves; ++q) t += red[((q * RB + rb) * MB + mb) * 64 + lane];
            const int64_t m = 16 * mb + lr;
            if (m >= p.M) continue;
            const int64_t nb = n0 + 16 * rb + 4 * kb;
            const int rl = 16 * rb + 4 * kb;  // row within the workgroup
            const float4 sw4 = *reinterpret_cast<const float4 *>(smem + L::C_SW + 4 * rl);
            const float sw[4] = {sw4.x * kUnscale, sw4.y * kUnscale, sw4.z * kUnscale, sw4.w * kUnscale};
            const float sxm = *reinterpret_cast<const float *>(smem + L::C_SX + 4 * lr + 64 * mb);
            int a[4];
            if constexpr (ASYM) {
                const uint4 z4 = *reinterpret_cast<const uint4 *>(smem + L::C_ZP + 4 * rl);
                const int rsm = *reinterpret_cast<const int *>(smem + L::C_RS + 4 * lr + 64 * mb);
                const uint32_t z[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] = t[r] + ((8 - (int)z[r]) << SHIFT) * rsm;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] = t[r];
            }
            float bs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (p.bias) {
                const uint4 b4 = *reinterpret_cast<const uint4 *>(smem + L::C_BIAS + 4 * rl);
                const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) bs[r] = __uint_as_float(p.bias_bf16 ? bw[r] << 16 : bw[r]);
            }
            if (p.y_i32) {
                int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < p.N) Y[nb + r] = a[r] >> SHIFT;
                continue;
            }
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = fmaf((float)a[r], sxm * sw[r], bs[r]);
            if (p.lr_t) {
                const float *tr = p.lr_t + m * p.lr_ldt;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t nc = min<int64_t>(nb + r, p.N - 1);
                    float l = 0.0f;
                    for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + nc]), l);
                    y[r] += l;
                }
            }
            uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y) + m * p.N;
            const uint32_t b0 = f32_to_bf16(y[0]), b1 = f32_to_bf16(y[1]), b2 = f32_to_bf16(y[2]),
                           b3 = f32_to_bf16(y[3]);
            if (nb + 3 < p.N && (p.N & 3) == 0) {
                *reinterpret_cast<uint2 *>(Y + nb) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
            } else {
                const uint32_t bb[4] = {b0, b1, b2, b3};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < p.N) Y[nb + r] = (uint16_t)bb[r];
            }
        }
    }
}

template <int ABITS, int MB, int RB>
hipError_t launch_ring_t(const LinearArgs &a, hipStream_t st) {
    using L = GL<ABITS, MB, RB>;
    const unsigned grid = (unsigned)((a.N + L::R - 1) / L::R);
    if (a.zp) {
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_gemv_ring<ABITS, MB, RB, true>), hipFuncAttributeMaxDynamicSharedMemorySize,
            L::LDS);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL((k_gemv_ring<ABITS, MB, RB, true>), dim3(grid), dim3(kThreads), L::LDS, st, a);
    } else {
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_gemv_ring<ABITS, MB, RB, false>), hipFuncAttributeMaxDynamicSharedMemorySize,
            L::LDS);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL((k_gemv_ring<ABITS, MB, RB, false>), dim3(grid), dim3(kThreads), L::LDS, st, a);
    }
    return hipGetLastError();
}

// Rows per workgroup: enough 16-row blocks that about 256 workgroups (one per CU) cover N.
template <int ABITS, int MB>
hipError_t dispatch_rb(const LinearArgs &a, hipStream_t st) {
    const int64_t rb = (a.N + 16 * 256 - 1) / (16 * 256);
    if (rb <= 1) return launch_ring_t<ABITS, MB, 1>(a, st);
    if (rb <= 2) return launch_ring_t<ABITS, MB, 2>(a, st);
    if (rb <= 3) return launch_ring_t<ABITS, MB, 3>(a, st);
    return launch_ring_t<ABITS, MB, 4>(a, st);
}

template <int ABITS>
hipError_t dispatch_mb(const LinearArgs &a, hipStream_t st) {
    switch ((a.M + 15) / 16) {
        case 1: return dispatch_rb<ABITS, 1>(a, st);
        case 2: return dispatch_rb<ABITS, 2>(a, st);
        case 3: return dispatch_rb<ABITS, 3>(a, st);
        default: return dispatch_rb<ABITS, 4>(a, st);
    }
}


// ---------------------------------------------------------------------------------------
// Split path (used when the caller's workspace holds the partial sums): a workgroup owns R
// rows and one of S equal K ranges.  All of its bytes are requested at once, token codes
// first (at most 48 KB, from L2), then the weights stage by stage (about 96 KB, in 1 KB runs)
// into LDS; the waves compute each 512-k stage as soon as it has landed (the loads complete
// in issue order), so the whole HBM stream is in flight from the start.  With S > 1 each
// workgroup writes its int32 partial tile and k_gemv_reduce sums the S partials in a fixed
// order and runs the epilogue; with S = 1 the workgroup runs the epilogue itself.
constexpr int kSplitActMax = 48 * 1024;
constexpr int kSplitWeightMax = 96 * 1024;
constexpr int KCS = 2048;           // k per stage of the split kernel: 1 KB of each weight row

struct SplitPlan {
    int S, KS, RB, MB, nst;
    int64_t act_bytes;  // LDS bytes of one wave's token codes
    int cbase;  // LDS offset of the per-row / per-token constants (past everything else)
    int lds;
    unsigned grid;
};

// Choose S (K ranges) and RB (16-row blocks per workgroup) so that about 256 workgroups
// cover the layer, the token codes of a K range fit kSplitActMax and the weights of a
// workgroup fit kSplitWeightMax.  Returns S = 0 when no split fits (the ring kernel runs).
SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int act_bits) {
    if (M < 1 || M > 64) return SplitPlan{};
    for (int S = 1; S <= 8; S *= 2) {
        if (K % (64 * S)) continue;
        const int64_t KS = K / S;
        SplitPlan pl{};
        pl.nst = (int)((KS + KCS - 1) / KCS);
        // per wave: nst stages x M tokens x 512 (int8) or 256 (int4) bytes, whole 1 KB loads
        const int64_t actw = ((int64_t)pl.nst * M * (act_bits == 8 ? 512 : 256) + 1023) / 1024 * 1024;
        if (kWaves * actw > kSplitActMax) continue;
        int64_t rb = (N * S + 4095) / 4096;
        const int64_t rbmax = kSplitWeightMax / (16 * (int64_t)pl.nst * (KCS / 2));
        rb = std::min<int64_t>(std::min<int64_t>(rb, rbmax), 8);
        if (rb < 1) continue;
        pl.S = S;
        pl.KS = (int)KS;
        pl.RB = (int)rb;
        pl.MB = (int)((M + 15) / 16);
        pl.act_bytes = actw;  // per wave
        const int64_t wbytes = (int64_t)pl.nst * 16 * rb * (KCS / 2);
        const int64_t red = (int64_t)kWaves * rb * pl.MB * 1024;
        pl.cbase = (int)std::max<int64_t>(kWaves * actw + wbytes, red);
        pl.lds = pl.cbase + 3 * 4 * (int)((16 * rb + 63) / 64 * 64) + 512;
        if (pl.lds > 160 * 1024) continue;
        // loads a wave keeps in flight (weights, token codes, constants) within vmcnt's range
        if (4 * rb * pl.nst + actw / 1024 + 7 > 63) continue;
        pl.grid = (unsigned)(((N + 16 * rb - 1) / (16 * rb)) * S);
        return pl;
    }
    return SplitPlan{};
}

// Per-wave layout: within each 2048-k stage wave w takes k in [512 w, 512 w + 512) and loads
// exactly the bytes it multiplies (its token-code slices and its 256-byte piece of every
// weight row) into its own LDS region, so the waves never wait for each other until the
// final reduction.  Token codes: [stage][token][512 or 256 bytes]; weights: [stage][row][256
// bytes]; 16-byte chunks swizzled by row / token inside groups of 16.
template <int ABITS, int MB, int RB>
__global__ void __launch_bounds__(kThreads) k_gemv_split(LinearArgs p, int S, int KS, int nst, int actw,
                                                         int cbase, int32_t *part, int asym) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr int R = 16 * RB;
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    constexpr float kUnscale = ABITS == 8 ? 1.0f / 16 : 1.0f / 256;
    constexpr int SLB = ABITS == 8 ? 512 : 256;  // token-code bytes per wave, stage and token
    constexpr int SLC = SLB / 16;
    constexpr int NACC = RB * MB <= 4 ? 2 : 1;   // independent accumulator chains
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kb = lane >> 4;
    const int blk = blockIdx.x / S, sp = blockIdx.x % S;
    const int64_t n0 = (int64_t)blk * R, k0 = (int64_t)sp * KS;
    const int64_t K = p.K, M = p.M;
    const int Mi = (int)M;
    const int64_t rowA = ABITS == 8 ? K : K / 2;
    const int64_t rowB = K / 2;
    const int abase = wave * actw;                              // this wave's token codes
    const int wbase = kWaves * actw + wave * nst * R * 256;     // this wave's weights
    const uint32_t smem_base = lds_addr(smem);
    const uint32_t xr = asym ? 0x88888888u : 0u;

    // ---- requests: constants (wave 0), this wave's token codes, its weights stage by stage.
    // Constants: row scales, biases, zero points (one dword per row, RP rows each), token
    // scales and rowsums (one dword per token).
    constexpr int RP = (R + 63) / 64 * 64;
    const int c_sw = cbase, c_bias = c_sw + 4 * RP, c_zp = c_bias + 4 * RP, c_sx = c_zp + 4 * RP, c_rs = c_sx + 256;
    if (wave == 0) {
#pragma unroll
        for (int h = 0; h < RP / 64; ++h) {
            const uint32_t c = (uint32_t)(min<int64_t>(n0 + min(64 * h + lane, R - 1), p.N - 1) - n0);
            gl_lds4_so((uint64_t)(p.sw + n0), 4 * c, smem_base + c_sw + 256 * h);
            if (p.bias) {
                if (p.bias_bf16) gl_lds2_so((uint64_t)((const uint16_t *)p.bias + n0), 2 * c, smem_base + c_bias + 256 * h);
                else gl_lds4_so((uint64_t)((const float *)p.bias + n0), 4 * c, smem_base + c_bias + 256 * h);
            }
            if (asym) gl_lds1_so((uint64_t)(p.zp + n0), c, smem_base + c_zp + 256 * h);
        }
        const uint32_t t = (uint32_t)min<int64_t>(lane, M - 1);
        if (asym) gl_lds4_so((uint64_t)p.rowsum, 4 * t, smem_base + c_rs);
        gl_lds4_so((uint64_t)p.sx, 4 * t, smem_base + c_sx);
    }
    {
        const int total = nst * Mi * SLC;  // 16-byte chunks of this wave's token codes
        const int ninstr = (total + 63) / 64;
        for (int j = 0; j < ninstr; ++j) {
            const int f = min(j * 64 + lane, total - 1);
            const int c = f % SLC, it = f / SLC;
            const int t = it % Mi, i = it / Mi;
            const int64_t kbyte = (k0 + (int64_t)i * KCS + 512 * wave) * ABITS / 8 + 16 * (c ^ (t & 15));
            gl_lds16_so((uint64_t)p.A, (uint32_t)(t * rowA + min<int64_t>(kbyte, rowA - 16)),
                        smem_base + (uint32_t)(abase + 1024 * j));
        }
    }
    for (int i = 0; i < nst; ++i) {
#pragma unroll
        for (int q = 0; q < 4 * RB; ++q) {  // 4 rows x 256 bytes per load
            const int r = 4 * q + lane / 16;
            const int64_t rc = min<int64_t>(n0 + r, p.N - 1) - n0;
            const int64_t off = min<int64_t>(k0 / 2 + (int64_t)i * (KCS / 2) + 256 * wave + 16 * swz(r, lane & 15),
                                             rowB - 16);
            gl_lds16_so((uint64_t)(p.B + n0 * rowB), (uint32_t)(rc * rowB + off),
                        smem_base + (uint32_t)(wbase + i * R * 256 + 1024 * q));
        }
    }

    v4i acc[NACC][RB][MB];
#pragma unroll
    for (int h = 0; h < NACC; ++h)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[h][rb][mb] = v4i{0, 0, 0, 0};

    for (int i = 0; i < nst; ++i) {
        wait_rem<4 * RB, 7>(nst - 1 - i);  // this wave's data up to stage i has landed
        // fragments of the stage's 4 steps of 128 k (k within the range: kl + 32 kb)
        uint4 xa[4][MB][ABITS == 8 ? 2 : 1], wv[4][RB];
        bool kv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kl = i * KCS + 512 * wave + 128 * u + 32 * kb;
            kv[u] = kl < KS;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int t = min(16 * mb + lr, Mi - 1);
                const uint8_t *sl = smem + abase + (i * Mi + t) * SLB;
                if constexpr (ABITS == 8) {
                    const int c0 = 8 * u + 2 * kb;
                    xa[u][mb][0] = *reinterpret_cast<const uint4 *>(sl + 16 * (c0 ^ (t & 15)));
                    xa[u][mb][1] = *reinterpret_cast<const uint4 *>(sl + 16 * ((c0 + 1) ^ (t & 15)));
                } else {
                    xa[u][mb][0] = *reinterpret_cast<const uint4 *>(sl + 16 * ((4 * u + kb) ^ (t & 15)));
                }
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int r = 16 * rb + lr;
                wv[u][rb] = *reinterpret_cast<const uint4 *>(smem + wbase + i * R * 256 + r * 256 +
                                                             16 * swz(r, 4 * u + kb));
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v4i a0[MB], a1[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if constexpr (ABITS == 8) {
                    a0[mb] = kv[u] ? __builtin_bit_cast(v4i, xa[u][mb][0]) : v4i{0, 0, 0, 0};
                    a1[mb] = kv[u] ? __builtin_bit_cast(v4i, xa[u][mb][1]) : v4i{0, 0, 0, 0};
                } else {
                    const uint4 x = xa[u][mb][0];
                    a0[mb] = kv[u] ? evod(x.x, x.y) : v4i{0, 0, 0, 0};
                    a1[mb] = kv[u] ? evod(x.z, x.w) : v4i{0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                uint4 w = wv[u][rb];
                w.x ^= xr; w.y ^= xr; w.z ^= xr; w.w ^= xr;
                v4i w0, w1;
                if constexpr (ABITS == 8) {
                    uint32_t q[8];
                    unpack_nat(w.x, q[0], q[1]);
                    unpack_nat(w.y, q[2], q[3]);
                    unpack_nat(w.z, q[4], q[5]);
                    unpack_nat(w.w, q[6], q[7]);
                    w0 = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
                    w1 = v4i{(int)q[4], (int)q[5], (int)q[6], (int)q[7]};
                } else {
                    w0 = evod(w.x, w.y);
                    w1 = evod(w.z, w.w);
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    v4i &c = acc[u % NACC][rb][mb];
                    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(w0, a0[mb], c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(w1, a1[mb], c, 0, 0, 0);
                }
            }
        }
    }
#pragma unroll
    for (int h = 1; h < NACC; ++h)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[0][rb][mb] += acc[h][rb][mb];

    // ---- fixed-order reduction of the 4 waves' tiles, then partials or the epilogue
    __syncthreads();
    v4i *red = reinterpret_cast<v4i *>(smem);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) red[((wave * RB + rb) * MB + mb) * 64 + lane] = acc[0][rb][mb];
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if ((rb * MB + mb) % kWaves != wave) continue;
            v4i t = red[((0 * RB + rb) * MB + mb) * 64 + lane];
#pragma unroll
            for (int q = 1; q < kWaves; ++q) t += red[((q * RB + rb) * MB + mb) * 64 + lane];
            const int64_t m = 16 * mb + lr;
            if (m >= M) continue;
            const int64_t nb = n0 + 16 * rb + 4 * kb;
            if (part) {  // raw partial sums of this K range (2^SHIFT * acc)
                int32_t *P = part + ((int64_t)sp * M + m) * p.N;
                if (nb + 3 < p.N && (p.N & 3) == 0) {
                    *reinterpret_cast<int4 *>(P + nb) = make_int4(t[0], t[1], t[2], t[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (nb + r < p.N) P[nb + r] = t[r];
                }
                continue;
            }
            const int rl = 16 * rb + 4 * kb;
            const float4 sw4 = *reinterpret_cast<const float4 *>(smem + c_sw + 4 * rl);
            const float sw[4] = {sw4.x * kUnscale, sw4.y * kUnscale, sw4.z * kUnscale, sw4.w * kUnscale};
            const float sxm = *reinterpret_cast<const float *>(smem + c_sx + 4 * m);
            int a[4] = {t[0], t[1], t[2], t[3]};
            if (asym) {
                const uint4 z4 = *reinterpret_cast<const uint4 *>(smem + c_zp + 4 * rl);
                const int rsm = *reinterpret_cast<const int *>(smem + c_rs + 4 * m);
                const uint32_t z[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] += ((8 - (int)z[r]) << SHIFT) * rsm;
            }
            if (p.y_i32) {
                int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < p.N) Y[nb + r] = a[r] >> SHIFT;
                continue;
            }
            float bs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (p.bias) {
                const uint4 b4 = *reinterpret_cast<const uint4 *>(smem + c_bias + 4 * rl);
                const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) bs[r] = __uint_as_float(p.bias_bf16 ? bw[r] << 16 : bw[r]);
            }
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = fmaf((float)a[r], sxm * sw[r], bs[r]);
            if (p.lr_t) {
                const float *tr = p.lr_t + m * p.lr_ldt;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t nc = min<int64_t>(nb + r, p.N - 1);
                    float l = 0.0f;
                    for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + nc]), l);
                    y[r] += l;
                }
            }
            uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y) + m * p.N;
            const uint32_t b0 = f32_to_bf16(y[0]), b1 = f32_to_bf16(y[1]), b2 = f32_to_bf16(y[2]),
                           b3 = f32_to_bf16(y[3]);
            if (nb + 3 < p.N && (p.N & 3) == 0) {
                *reinterpret_cast<uint2 *>(Y + nb) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
            } else {
                const uint32_t bb[4] = {b0, b1, b2, b3};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < p.N) Y[nb + r] = (uint16_t)bb[r];
            }
        }
    }
}

// Sum of the S partial sums in a fixed order (exact), then the epilogue.  One thread per
// token and 4 consecutive output features.
template <int ABITS>
__global__ void __launch_bounds__(256) k_gemv_reduce(LinearArgs p, int S, const int32_t *part, int asym) {
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    constexpr float kUnscale = ABITS == 8 ? 1.0f / 16 : 1.0f / 256;
    const int64_t nq = (p.N + 3) / 4;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= p.M * nq) return;
    const int64_t m = id / nq, nb = (id % nq) * 4;
    const bool vec = (p.N & 3) == 0;  // 16-byte rows: whole quads of partials and constants
    int a[4] = {0, 0, 0, 0};
    float swv[4], bsv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int zv[4] = {8, 8, 8, 8};
    if (vec) {
        for (int s = 0; s < S; ++s) {
            const int4 v = *reinterpret_cast<const int4 *>(part + ((int64_t)s * p.M + m) * p.N + nb);
            a[0] += v.x; a[1] += v.y; a[2] += v.z; a[3] += v.w;
        }
        const float4 w4v = *reinterpret_cast<const float4 *>(p.sw + nb);
        swv[0] = w4v.x; swv[1] = w4v.y; swv[2] = w4v.z; swv[3] = w4v.w;
        if (p.bias) {
            if (p.bias_bf16) {
                const uint2 b = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p.bias) + nb);
                bsv[0] = __uint_as_float(b.x << 16); bsv[1] = __uint_as_float(b.x & 0xffff0000u);
                bsv[2] = __uint_as_float(b.y << 16); bsv[3] = __uint_as_float(b.y & 0xffff0000u);
            } else {
                const float4 b = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p.bias) + nb);
                bsv[0] = b.x; bsv[1] = b.y; bsv[2] = b.z; bsv[3] = b.w;
            }
        }
        if (asym) {
            const uint32_t z = *reinterpret_cast<const uint32_t *>(p.zp + nb);
#pragma unroll
            for (int r = 0; r < 4; ++r) zv[r] = (int)((z >> (8 * r)) & 0xffu);
        }
    } else {
        for (int s = 0; s < S; ++s) {
            const int32_t *P = part + ((int64_t)s * p.M + m) * p.N;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nb + r < p.N) a[r] += P[nb + r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = min<int64_t>(nb + r, p.N - 1);
            swv[r] = p.sw[n];
            if (p.bias)
                bsv[r] = p.bias_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[n])
                                     : reinterpret_cast<const float *>(p.bias)[n];
            if (asym) zv[r] = p.zp[n];
        }
    }
    const float sxm = p.sx[m];
    const int rsm = asym ? p.rowsum[m] : 0;
    float y[4];
    uint32_t yb[4];
    int32_t yi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t n = min<int64_t>(nb + r, p.N - 1);
        int v = a[r] + (asym ? ((8 - zv[r]) << SHIFT) * rsm : 0);
        yi[r] = v >> SHIFT;
        y[r] = fmaf((float)v, sxm * (swv[r] * kUnscale), bsv[r]);
        if (p.lr_t) {
            const float *tr = p.lr_t + m * p.lr_ldt;
            float l = 0.0f;
            for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + n]), l);
            y[r] += l;
        }
        yb[r] = f32_to_bf16(y[r]);
    }
    if (p.y_i32) {
        int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (nb + r < p.N) Y[nb + r] = yi[r];
        return;
    }
    uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y) + m * p.N;
    if (nb + 3 < p.N && (p.N & 3) == 0) {
        *reinterpret_cast<uint2 *>(Y + nb) = make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (nb + r < p.N) Y[nb + r] = (uint16_t)yb[r];
    }
}

template <int ABITS, int MB, int RB>
hipError_t launch_split_t(const LinearArgs &a, const SplitPlan &pl, int32_t *part, hipStream_t st) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemv_split<ABITS, MB, RB>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_gemv_split<ABITS, MB, RB>), dim3(pl.grid), dim3(kThreads), pl.lds, st, a, pl.S, pl.KS,
                       pl.nst, (int)pl.act_bytes, pl.cbase, pl.S > 1 ? part : nullptr, a.zp ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.S == 1) return e;
    const int64_t threads = a.M * ((a.N + 3) / 4);
    hipLaunchKernelGGL((k_gemv_reduce<ABITS>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a, pl.S,
                       part, a.zp ? 1 : 0);
    return hipGetLastError();
}

template <int ABITS, int MB>
hipError_t split_rb(const LinearArgs &a, const SplitPlan &pl, int32_t *part, hipStream_t st) {
    switch (pl.RB) {
        case 1: return launch_split_t<ABITS, MB, 1>(a, pl, part, st);
        case 2: return launch_split_t<ABITS, MB, 2>(a, pl, part, st);
        case 3: return launch_split_t<ABITS, MB, 3>(a, pl, part, st);
        case 4: return launch_split_t<ABITS, MB, 4>(a, pl, part, st);
        case 5: return launch_split_t<ABITS, MB, 5>(a, pl, part, st);
        case 6: return launch_split_t<ABITS, MB, 6>(a, pl, part, st);
        case 7: return launch_split_t<ABITS, MB, 7>(a, pl, part, st);
        default: return launch_split_t<ABITS, MB, 8>(a, pl, part, st);
    }
}

template <int ABITS>
hipError_t split_mb(const LinearArgs &a, const SplitPlan &pl, int32_t *part, hipStream_t st) {
    switch (pl.MB) {
        case 1: return split_rb<ABITS, 1>(a, pl, part, st);
        case 2: return split_rb<ABITS, 2>(a, pl, part, st);
        case 3: return split_rb<ABITS, 3>(a, pl, part, st);
        default: return split_rb<ABITS, 4>(a, pl, part, st);
    }
}


// ---------------------------------------------------------------------------------------
// Streaming K-split path for 16 < M <= 64 (with a workspace).  A workgroup of 4 waves owns
// R = 16 RB weight rows and one of S equal K ranges; in each stage of 512 k, wave w takes
// k in [128 w, 128 w + 128) and streams its 128-k slice of every one of the (up to 64) tokens
// and its 64-byte piece of each of the R rows through its own 2-stage LDS ring (direct
// global -> LDS loads), multiplying a stage as soon as its own loads have landed.  Per 64 k,
// one v_mfma_i32_16x16x64_i8 per (16-token block, 16-row block), lane group kb taking the
// 16 k at 16 kb in both operands.  The 4 waves' partial tiles are summed through LDS in a
// fixed order and stored as int32 partials [S, M, N]; k_gemv_reduce adds the S ranges in
// a fixed order and applies the epilogue.  Workgroup b takes K range b % S, so the blocks
// dealt round-robin to one XCD share a K range and its token slices stay in that XCD's L2.
constexpr int kSkWaves = 4;
constexpr int kSkStage = 128 * kSkWaves;  // k per stage

template <int ABITS, int MB, int RB>
struct SKL {
    static constexpr int T = 16 * MB, R = 16 * RB;
    static constexpr int TB = ABITS == 8 ? 128 : 64;            // token bytes per wave and stage
    static constexpr int CPT = TB / 16;                          // 8 or 4 chunks
    static constexpr int ACT = T * TB < 1024 ? 1024 : T * TB;    // whole 1 KB loads
    static constexpr int WB = R * 64;                            // weight bytes per wave and stage
    static constexpr int SLOT = ACT + WB;
    static constexpr int D = 2;
    static constexpr int LA = ACT / 1024, LB = WB / 1024;
    static constexpr int LPS = LA + LB;
    static constexpr int RED = kSkWaves * RB * MB * 1024;        // v4i tiles of the waves
    static constexpr int RING = kSkWaves * D * SLOT > RED ? kSkWaves * D * SLOT : RED;
    static constexpr int LDS = RING;
    static_assert(WB % 1024 == 0 && (D - 1) * LPS <= 63 && LDS <= 160 * 1024, "split stream layout");
};

template <int ABITS, int MB, int RB>
__global__ void __launch_bounds__(64 * kSkWaves) k_gemv_sk(LinearArgs p, int S, int32_t *__restrict__ part, int asym) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = SKL<ABITS, MB, RB>;
    constexpr int R = L::R, CPT = L::CPT;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kb = lane >> 4;
    const int sp = (int)blockIdx.x % S, tile = (int)blockIdx.x / S;
    const int64_t n0 = (int64_t)tile * R;
    const int64_t K = p.K, M = p.M;
    const int64_t KS = K / S;
    const int nst = (int)(KS / kSkStage);
    const int64_t rowA = ABITS == 8 ? K : K / 2;
    const int64_t rowB = K / 2;
    const uint32_t smem_base = lds_addr(smem);
    const uint32_t xr = asym ? 0x88888888u : 0u;
    const int ring = wave * L::D * L::SLOT;
    constexpr uint32_t ASTEP = kSkStage * ABITS / 8, BSTEP = kSkStage / 2;

    // LDS position (t, c) of a token slice holds global chunk c ^ (t & (CPT - 1)); position
    // (r, c) of a 64-byte weight piece holds chunk c ^ ((r >> 1) & 3)
    uint32_t arow[L::LA], ain[L::LA], brow[L::LB], bin[L::LB];
#pragma unroll
    for (int j = 0; j < L::LA; ++j) {
        const int f = min(j * 64 + lane, L::T * CPT - 1);
        const int t = f / CPT, c = f % CPT;
        arow[j] = (uint32_t)(min<int64_t>(t, M - 1) * rowA);
        ain[j] = (uint32_t)(KS * sp * ABITS / 8 + wave * L::TB + 16 * (c ^ (t & (CPT - 1))));
    }
#pragma unroll
    for (int j = 0; j < L::LB; ++j) {
        const int r = 16 * j + lane / 4;
        brow[j] = (uint32_t)((min<int64_t>(n0 + r, p.N - 1) - n0) * rowB);
        bin[j] = (uint32_t)(KS * sp / 2 + 64 * wave + 16 * ((lane & 3) ^ ((r >> 1) & 3)));
    }
    const uint64_t bbase = (uint64_t)(p.B + n0 * rowB);
    auto issue = [&](int i) __attribute__((always_inline)) {
        const uint32_t slot = smem_base + (uint32_t)(ring + (i % L::D) * L::SLOT);
#pragma unroll
        for (int j = 0; j < L::LA; ++j) gl_lds16_so((uint64_t)p.A, arow[j] + ain[j] + (uint32_t)i * ASTEP, slot + 1024 * j);
#pragma unroll
        for (int j = 0; j < L::LB; ++j) gl_lds16_so(bbase, brow[j] + bin[j] + (uint32_t)i * BSTEP, slot + L::ACT + 1024 * j);
    };
    for (int i = 0; i < L::D; ++i)
        if (i < nst) issue(i);

    v4i acc[MB][RB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[mb][rb] = v4i{0, 0, 0, 0};

    for (int i = 0; i < nst; ++i) {
        wait_rem<L::LPS, L::D - 1>(min(L::D - 1, nst - 1 - i));
        const uint8_t *sl = smem + ring + (i % L::D) * L::SLOT;
        uint4 xa[2][MB];
        uint2 wv[2][RB];
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // k in [64 h, 64 h + 64) of the wave's slice
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int t = min(16 * mb + lr, (int)M - 1);
                const uint8_t *ta = sl + (16 * mb + lr) * L::TB;
                if constexpr (ABITS == 8) {
                    xa[h][mb] = *reinterpret_cast<const uint4 *>(ta + 16 * ((4 * h + kb) ^ (t & (CPT - 1))));
                } else {
                    const uint2 x2 = *reinterpret_cast<const uint2 *>(ta + 16 * ((2 * h + (kb >> 1)) ^ (t & (CPT - 1))) +
                                                                      8 * (kb & 1));
                    xa[h][mb] = make_uint4(x2.x, x2.y, 0, 0);
                }
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int r = 16 * rb + lr;
                wv[h][rb] = *reinterpret_cast<const uint2 *>(sl + L::ACT + r * 64 + 16 * ((2 * h + (kb >> 1)) ^ ((r >> 1) & 3)) +
                                                             8 * (kb & 1));
            }
        }
        wait_lgkmcnt0();  // this wave's reads of the slot are complete before it is refilled
        if (i + L::D < nst) issue(i + L::D);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4i w[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const uint32_t d0 = wv[h][rb].x ^ xr, d1 = wv[h][rb].y ^ xr;
                if constexpr (ABITS == 8) {
                    uint32_t lo0, hi0, lo1, hi1;
                    unpack_nat(d0, lo0, hi0);
                    unpack_nat(d1, lo1, hi1);
                    w[rb] = v4i{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
                } else {
                    w[rb] = evod(d0, d1);
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                v4i a;
                if constexpr (ABITS == 8) a = __builtin_bit_cast(v4i, xa[h][mb]);
                else a = evod(xa[h][mb].x, xa[h][mb].y);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) acc[mb][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[rb], a, acc[mb][rb], 0, 0, 0);
            }
        }
    }

    // fixed-order sum of the 4 waves' tiles, then int32 partials: 16x16 layout, lane l,
    // register r holds row 4 (l / 16) + r of token l % 16
    wait_vmcnt<0>();
    __syncthreads();
    v4i *red = reinterpret_cast<v4i *>(smem);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) red[((wave * MB + mb) * RB + rb) * 64 + lane] = acc[mb][rb];
    __syncthreads();
    for (int b = wave; b < MB * RB; b += kSkWaves) {
        const int mb = b / RB, rb = b % RB;
        v4i t = red[(mb * RB + rb) * 64 + lane];
#pragma unroll
        for (int q = 1; q < kSkWaves; ++q) t += red[((q * MB + mb) * RB + rb) * 64 + lane];
        const int64_t m = 16 * mb + lr;
        const int64_t nb = n0 + 16 * rb + 4 * kb;
        if (m >= M) continue;
        int32_t *P = part + ((int64_t)sp * M + m) * p.N;
        if (nb + 3 < p.N && (p.N & 3) == 0) {
            *reinterpret_cast<int4 *>(P + nb) = make_int4(t[0], t[1], t[2], t[3]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nb + r < p.N) P[nb + r] = t[r];
        }
    }
}

// Plan of the split stream: 32, 48 or 64 rows per workgroup and S K ranges (whole 512-k
// stages, at least 2 per range), minimising the per-CU bytes of the busiest round: weight
// bytes (HBM), token bytes (re-read from L2, weighted 0.3) and the partials written and read
// back.  S = 0: no plan.
struct SkPlan {
    int RB, S;
    unsigned grid;
};

// Used where it measured faster than the split and ring kernels (M = 24 ... 64 at K = 4096 and
// 12288): a plan with several K ranges, or up to 32 tokens; one K range at 48-64 tokens (at
// K = 4096, N = 12288) lost to the ring kernel.
SkPlan plan_sk(int64_t M, int64_t N, int64_t K, int act_bits);
bool sk_used(const SkPlan &pl, int64_t M) { return pl.S >= 2 || (pl.S == 1 && M <= 32); }

SkPlan plan_sk(int64_t M, int64_t N, int64_t K, int act_bits) {
    SkPlan best{0, 0, 0};
    if (M <= 16 || M > 64 || K % kSkStage) return best;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    double bestv = 1e30;
    for (int rb = 4; rb >= 2; --rb) {
        const int64_t tiles = (N + 16 * rb - 1) / (16 * rb);
        for (int S = 1; S <= 8; S *= 2) {
            if (K % ((int64_t)S * kSkStage) || K / S < 2 * kSkStage) continue;
            const int64_t wg = tiles * S, rounds = (wg + ncu - 1) / ncu, KS = K / S;
            const double v = (double)rounds * (16.0 * rb * KS / 2 + 0.3 * (double)M * KS * act_bits / 8) +
                             2.0 * S * (double)M * N * 4 / ncu;
            if (v < bestv) {
                bestv = v;
                best = SkPlan{rb, S, (unsigned)wg};
            }
        }
    }
    return best;
}

template <int ABITS, int MB, int RB>
hipError_t launch_sk_t(const LinearArgs &a, const SkPlan &pl, int32_t *part, hipStream_t st) {
    using L = SKL<ABITS, MB, RB>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemv_sk<ABITS, MB, RB>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((k_gemv_sk<ABITS, MB, RB>), dim3(pl.grid), dim3(64 * kSkWaves), L::LDS, st, a, pl.S, part,
                       a.zp ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = a.M * ((a.N + 3) / 4);
    hipLaunchKernelGGL((k_gemv_reduce<ABITS>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a, pl.S,
                       part, a.zp ? 1 : 0);
    return hipGetLastError();
}

template <int ABITS, int MB>
hipError_t sk_rb(const LinearArgs &a, const SkPlan &pl, int32_t *part, hipStream_t st) {
    switch (pl.RB) {
        case 2: return launch_sk_t<ABITS, MB, 2>(a, pl, part, st);
        case 3: return launch_sk_t<ABITS, MB, 3>(a, pl, part, st);
        default: return launch_sk_t<ABITS, MB, 4>(a, pl, part, st);
    }
}

template <int ABITS>
hipError_t sk_mb(const LinearArgs &a, const SkPlan &pl, int32_t *part, hipStream_t st) {
    if (a.M <= 32) return sk_rb<ABITS, 2>(a, pl, part, st);
    if (a.M <= 48) return sk_rb<ABITS, 3>(a, pl, part, st);
    return sk_rb<ABITS, 4>(a, pl, part, st);
}

// ---------------------------------------------------------------------------------------
// Streaming path for M <= 16 (no workspace, one pass over K): every wave streams its own
// slices through its own LDS ring.  A workgroup of NW waves owns R = 16 RB weight rows; in
// each stage of 256 NW k, wave w takes k in [256 w, 256 w + 256): it loads its 256-byte
// (int8) or 128-byte (int4) slice of each staged token and its 128-byte piece of each of the
// R rows (8 rows x 128 bytes per 1 KB load), D stages ahead, and multiplies a stage as soon
// as its own loads have landed; no workgroup barrier until the final reduction.
//
// With one workgroup per CU a SIMD runs NW / 4 waves, so little hides a wave's own latency.
// The loop is kept short (measured): load offsets advance by a fixed stride per stage, and
// when K is a whole number of stages (KFULL) there is no clamping of chunks past K and no
// masking of their codes.  Deeper rings, and issuing a stage before waiting for the oldest
// one, measured slower.
constexpr int kStreamLds = 144 * 1024;
constexpr int kStreamDepth = 2;   // stages in flight per wave (2 to 4 measured: deeper only
                                  // lengthens the start, as every wave waits for its first stage)
constexpr int kNC = 5;            // constant loads of wave 0

template <int ABITS, int TM, int RB, int NW>
struct SL {
    static constexpr int KS = 256 * NW;                               // k per stage
    static constexpr int R = 16 * RB;
    static constexpr int TB = ABITS == 8 ? 256 : 128;                 // token bytes per wave and stage
    static constexpr int ACT = TM * TB < 1024 ? 1024 : TM * TB;       // whole 1 KB loads
    static constexpr int WB = R * 128;                                // weight bytes per wave and stage
    static constexpr int SLOT = ACT + WB;
    static constexpr int D0 = kStreamLds / NW / SLOT;
    static constexpr int D = D0 > kStreamDepth ? kStreamDepth : D0;   // stages per wave ring
    static constexpr int LA = ACT / 1024, LB = WB / 1024;             // loads per stage
    static constexpr int LPS = LA + LB;
    static constexpr int RED = NW * RB * 1024;
    static constexpr int RING = NW * D * SLOT > RED ? NW * D * SLOT : RED;
    static constexpr int RP = (R + 63) / 64 * 64;
    static constexpr int C_SW = RING, C_BIAS = C_SW + 4 * RP, C_ZP = C_BIAS + 4 * RP, C_SX = C_ZP + 4 * RP,
                         C_RS = C_SX + 256;
    static constexpr int LDS = C_RS + 256;
    static_assert(D >= 2 && (D - 1) * LPS + kNC <= 63 && LDS <= 160 * 1024 && RP == 64, "streaming ring");
};

__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }

// Fixed-order reduction of the NW waves' tiles through LDS (from offset 0), then the dequant
// epilogue: wave rb % NW takes row block rb.  16x16 layout: lane l, register r holds weight
// row 4 (l / 16) + r of token l % 16.  The per-row and per-token constants sit in LDS at the
// given offsets, one dword per entry.
template <int ABITS, int RB, int NW>
__device__ __forceinline__ void stream_epilogue(const LinearArgs &p, uint8_t *smem, const v4i (&acc)[2][RB], int64_t n0,
                                                int asym, int c_sw, int c_bias, int c_zp, int c_sx, int c_rs) {
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    constexpr float kUnscale = ABITS == 8 ? 1.0f / 16 : 1.0f / 256;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, kb = lane >> 4;
    const int64_t M = p.M;
    __syncthreads();
    v4i *red = reinterpret_cast<v4i *>(smem);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) red[(wave * RB + rb) * 64 + lane] = acc[0][rb] + acc[1][rb];
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        if (rb % NW != wave) continue;
        v4i tt = red[rb * 64 + lane];
#pragma unroll
        for (int q = 1; q < NW; ++q) tt += red[(q * RB + rb) * 64 + lane];
        const int64_t m = lr;
        if (m >= M) continue;
        const int64_t nb = n0 + 16 * rb + 4 * kb;
        const int rl = 16 * rb + 4 * kb;
        const float4 sw4 = *reinterpret_cast<const float4 *>(smem + c_sw + 4 * rl);
        const float sw[4] = {sw4.x * kUnscale, sw4.y * kUnscale, sw4.z * kUnscale, sw4.w * kUnscale};
        const float sxm = *reinterpret_cast<const float *>(smem + c_sx + 4 * m);
        int a[4] = {tt[0], tt[1], tt[2], tt[3]};
        if (asym) {
            const uint4 z4 = *reinterpret_cast<const uint4 *>(smem + c_zp + 4 * rl);
            const int rsm = *reinterpret_cast<const int *>(smem + c_rs + 4 * m);
            const uint32_t z[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] += ((8 - (int)z[r]) << SHIFT) * rsm;
        }
        if (p.y_i32) {
            int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nb + r < p.N) Y[nb + r] = a[r] >> SHIFT;
            continue;
        }
        float bs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (p.bias) {
            const uint4 b4 = *reinterpret_cast<const uint4 *>(smem + c_bias + 4 * rl);
            const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) bs[r] = __uint_as_float(p.bias_bf16 ? bw[r] << 16 : bw[r]);
        }
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = fmaf((float)a[r], sxm * sw[r], bs[r]);
        if (p.lr_t) {
            const float *tr = p.lr_t + m * p.lr_ldt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t nc = min<int64_t>(nb + r, p.N - 1);
                float l = 0.0f;
                for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + nc]), l);
                y[r] += l;
            }
        }
        uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y) + m * p.N;
        const uint32_t b0 = f32_to_bf16(y[0]), b1 = f32_to_bf16(y[1]), b2 = f32_to_bf16(y[2]),
                       b3 = f32_to_bf16(y[3]);
        if (nb + 3 < p.N && (p.N & 3) == 0) {
            *reinterpret_cast<uint2 *>(Y + nb) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
            const uint32_t bb[4] = {b0, b1, b2, b3};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (nb + r < p.N) Y[nb + r] = (uint16_t)bb[r];
        }
    }
}

template <int ABITS, int TM, int RB, int NW, bool KFULL>
__global__ void __launch_bounds__(64 * NW) k_gemv_stream(LinearArgs p, int asym) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = SL<ABITS, TM, RB, NW>;
    constexpr int KST = L::KS;
    constexpr int R = L::R;
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    constexpr float kUnscale = ABITS == 8 ? 1.0f / 16 : 1.0f / 256;
    constexpr int CPT = L::TB / 16;                  // 16-byte chunks per token slice
    constexpr uint32_t ASTEP = KST * ABITS / 8;      // token bytes per stage
    constexpr uint32_t BSTEP = KST / 2;              // weight bytes per stage
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kb = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * R;
    const int64_t K = p.K, M = p.M;
    const int nst = (int)((K + KST - 1) / KST);
    const int64_t rowA = ABITS == 8 ? K : K / 2;
    const int64_t rowB = K / 2;
    const uint32_t smem_base = lds_addr(smem);
    const uint32_t xr = asym ? 0x88888888u : 0u;
    const int ring = wave * L::D * L::SLOT;  // this wave's ring

    // Stage i of this wave goes into ring slot i % D.  Token slice chunk c of token t sits at
    // position c ^ (t & (CPT - 1)); weight chunk c of row r at position swz8(r, c).  Per lane
    // and load: the byte offset of the row (token rows clamped to M - 1, weight rows to N - 1:
    // their outputs are never stored) and the offset inside it at stage 0.  Without KFULL,
    // chunks past K read the last valid chunk of the row and their codes are masked to zero.
    uint32_t arow[L::LA], ain[L::LA], brow[L::LB], bin[L::LB];
#pragma unroll
    for (int j = 0; j < L::LA; ++j) {
        const int f = min(j * 64 + lane, TM * CPT - 1);
        const int t = f / CPT, c = f % CPT;
        arow[j] = (uint32_t)(min<int64_t>(t, M - 1) * rowA);
        ain[j] = (uint32_t)(256 * wave * ABITS / 8 + 16 * (c ^ (t & (CPT - 1))));
    }
#pragma unroll
    for (int j = 0; j < L::LB; ++j) {
        const int r = 8 * j + lane / 8;
        brow[j] = (uint32_t)((min<int64_t>(n0 + r, p.N - 1) - n0) * rowB);
        bin[j] = (uint32_t)(128 * wave + 16 * swz8(r, lane & 7));
    }
    const uint64_t bbase = (uint64_t)(p.B + n0 * rowB);
    auto issue = [&](int i) __attribute__((always_inline)) {
        const uint32_t slot = smem_base + (uint32_t)(ring + (i % L::D) * L::SLOT);
#pragma unroll
        for (int j = 0; j < L::LA; ++j) {
            uint32_t in = ain[j] + (uint32_t)i * ASTEP;
            if constexpr (!KFULL) in = min(in, (uint32_t)(rowA - 16));
            gl_lds16_so((uint64_t)p.A, arow[j] + in, slot + 1024 * j);
        }
#pragma unroll
        for (int j = 0; j < L::LB; ++j) {
            uint32_t in = bin[j] + (uint32_t)i * BSTEP;
            if constexpr (!KFULL) in = min(in, (uint32_t)(rowB - 16));
            gl_lds16_so(bbase, brow[j] + in, slot + L::ACT + 1024 * j);
        }
    };

    v4i acc[2][RB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[h][rb] = v4i{0, 0, 0, 0};

    for (int i = 0; i < L::D; ++i)
        if (i < nst) issue(i);
    // Constants (wave 0): row scales, biases, zero points, token scales and rowsums, one dword
    // per row and per token, always kNC loads (a missing bias, zero point or rowsum loads the
    // row scales or token scales into its unused slot).  They are issued after the first D
    // stages so that the weight stream starts at once; wave 0's waits for those stages allow
    // for them.
    if (wave == 0) {
        const uint32_t c = (uint32_t)(min<int64_t>(n0 + min(lane, R - 1), p.N - 1) - n0);
        const uint64_t sw = (uint64_t)(p.sw + n0);
        gl_lds4_so(sw, 4 * c, smem_base + L::C_SW);
        if (p.bias && p.bias_bf16) gl_lds2_so((uint64_t)((const uint16_t *)p.bias + n0), 2 * c, smem_base + L::C_BIAS);
        else if (p.bias) gl_lds4_so((uint64_t)((const float *)p.bias + n0), 4 * c, smem_base + L::C_BIAS);
        else gl_lds4_so(sw, 4 * c, smem_base + L::C_BIAS);
        if (asym) gl_lds1_so((uint64_t)(p.zp + n0), c, smem_base + L::C_ZP);
        else gl_lds4_so(sw, 4 * c, smem_base + L::C_ZP);
        const uint32_t t = (uint32_t)min<int64_t>(lane, M - 1);
        gl_lds4_so(asym ? (uint64_t)p.rowsum : (uint64_t)p.sx, 4 * t, smem_base + L::C_RS);
        gl_lds4_so((uint64_t)p.sx, 4 * t, smem_base + L::C_SX);
    }
    const int tt = min(lr, (int)M - 1);
    for (int i = 0; i < nst; ++i) {
        if (wave == 0 && i < L::D) wait_rem<L::LPS, L::D - 1, kNC>(min(L::D - 1, nst - 1 - i));
        else wait_rem<L::LPS, L::D - 1>(min(L::D - 1, nst - 1 - i));
        const uint8_t *sl = smem + ring + (i % L::D) * L::SLOT;
        uint4 xa[2][ABITS == 8 ? 2 : 1], wv[2][RB];
        bool kv[2] = {true, true};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if constexpr (!KFULL) kv[u] = (int64_t)i * KST + 256 * wave + 128 * u + 32 * kb < K;
            if constexpr (ABITS == 8) {  // 16 chunks per token slice
                const int c0 = 8 * u + 2 * kb;
                xa[u][0] = *reinterpret_cast<const uint4 *>(sl + tt * L::TB + 16 * (c0 ^ (tt & 15)));
                xa[u][1] = *reinterpret_cast<const uint4 *>(sl + tt * L::TB + 16 * ((c0 + 1) ^ (tt & 15)));
            } else {  // 8 chunks per token slice
                xa[u][0] = *reinterpret_cast<const uint4 *>(sl + tt * L::TB + 16 * ((4 * u + kb) ^ (tt & 7)));
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int r = 16 * rb + lr;
                wv[u][rb] = *reinterpret_cast<const uint4 *>(sl + L::ACT + r * 128 + 16 * swz8(r, 4 * u + kb));
            }
        }
        // this wave's reads of the slot are complete before the slot is refilled
        wait_lgkmcnt0();
        if (i + L::D < nst) issue(i + L::D);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            v4i a0, a1;
            if constexpr (ABITS == 8) {
                a0 = __builtin_bit_cast(v4i, xa[u][0]);
                a1 = __builtin_bit_cast(v4i, xa[u][1]);
            } else {
                a0 = evod(xa[u][0].x, xa[u][0].y);
                a1 = evod(xa[u][0].z, xa[u][0].w);
            }
            if constexpr (!KFULL) {
                if (!kv[u]) a0 = a1 = v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                uint4 w = wv[u][rb];
                w.x ^= xr; w.y ^= xr; w.z ^= xr; w.w ^= xr;
                v4i w0, w1;
                if constexpr (ABITS == 8) {
                    uint32_t q[8];
                    unpack_nat(w.x, q[0], q[1]);
                    unpack_nat(w.y, q[2], q[3]);
                    unpack_nat(w.z, q[4], q[5]);
                    unpack_nat(w.w, q[6], q[7]);
                    w0 = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
                    w1 = v4i{(int)q[4], (int)q[5], (int)q[6], (int)q[7]};
                } else {
                    w0 = evod(w.x, w.y);
                    w1 = evod(w.z, w.w);
                }
                acc[u][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w0, a0, acc[u][rb], 0, 0, 0);
                acc[u][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w1, a1, acc[u][rb], 0, 0, 0);
            }
        }
    }

    // wave 0's constants were issued after the first D stages; with nst <= D no wait of the
    // loop covered them, so drain every load before the epilogue reads them
    wait_vmcnt<0>();
    stream_epilogue<ABITS, RB, NW>(p, smem, acc, n0, asym, L::C_SW, L::C_BIAS, L::C_ZP, L::C_SX, L::C_RS);
}

template <int ABITS, int TM, int RB, int NW, bool KFULL>
hipError_t launch_stream_k(const LinearArgs &a, hipStream_t st) {
    using L = SL<ABITS, TM, RB, NW>;
    const void *fn = reinterpret_cast<const void *>(&k_gemv_stream<ABITS, TM, RB, NW, KFULL>);
    static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS);
    if (attr != hipSuccess) return attr;
    const unsigned grid = (unsigned)((a.N + L::R - 1) / L::R);
    hipLaunchKernelGGL((k_gemv_stream<ABITS, TM, RB, NW, KFULL>), dim3(grid), dim3(64 * NW), L::LDS, st, a,
                       a.zp ? 1 : 0);
    return hipGetLastError();
}

template <int ABITS, int TM, int RB, int NW>
hipError_t launch_stream_t(const LinearArgs &a, hipStream_t st) {
    return a.K % (256 * NW) == 0 ? launch_stream_k<ABITS, TM, RB, NW, true>(a, st)
                                 : launch_stream_k<ABITS, TM, RB, NW, false>(a, st);
}

// Shape of the streaming launch (measured at M = 1 to 16, K = 3072 to 12288, N = 3072 to
// 12288).  Up to 8 tokens the staged token slices are small, so 16 rows per workgroup (the
// most workgroups): 8 waves when that gives about one workgroup per CU (two waves per SIMD
// to overlap one wave's stage turnaround with another's), else 4.  At 16 tokens every
// workgroup re-reads 4 KB of token codes per wave and stage from L2, so rows per workgroup
// grow with N to keep the grid near one workgroup per CU.
template <int ABITS, int TM>
hipError_t stream_rb(const LinearArgs &a, hipStream_t st) {
    if constexpr (TM <= 8) {
        int dev = 0, ncu = 256;
        if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if ((a.N + 15) / 16 <= ncu) return launch_stream_t<ABITS, TM, 1, 8>(a, st);
        return launch_stream_t<ABITS, TM, 1, 4>(a, st);
    } else {
        const int64_t rb = (a.N + 16 * 256 - 1) / (16 * 256);
        if (rb <= 1) return launch_stream_t<ABITS, TM, 1, 4>(a, st);
        if (rb <= 2) return launch_stream_t<ABITS, TM, 2, 4>(a, st);
        if (rb <= 3) return launch_stream_t<ABITS, TM, 3, 4>(a, st);
        return launch_stream_t<ABITS, TM, 4, 4>(a, st);
    }
}

template <int ABITS>
hipError_t launch_stream(const LinearArgs &a, hipStream_t st) {
    if (a.M <= 1) return stream_rb<ABITS, 1>(a, st);
    if (a.M <= 2) return stream_rb<ABITS, 2>(a, st);
    if (a.M <= 4) return stream_rb<ABITS, 4>(a, st);
    if (a.M <= 8) return stream_rb<ABITS, 8>(a, st);
    return stream_rb<ABITS, 16>(a, st);
}

// ---------------------------------------------------------------------------------------
// Fused path for one token (K <= 16384, bf16 X, K a whole number of stages; the kernel takes
// up to 4 tokens): rotation, quantization and the streaming GEMM in one launch, the single-kernel
// ConvRot path of the INT4 README ("Inference / INT4").  Every workgroup rotates and
// quantizes the whole token block itself (at most 16384 elements; the fp64 work overlaps the
// first weight stages in flight) and keeps the codes in LDS for the whole K, so the stream
// carries weights only and the separate rotate launch, with its gap, disappears.
//   1. direct loads: X (M K bf16 in 1 KB pieces), the first 2 weight stages, the constants
//      (as in the streaming kernel);
//   2. each 16-lane group takes 256-element blocks (token t, block j), lane c elements
//      16 c .. 16 c + 15, in fp64 with the row rotate-quant kernel's butterflies, amax, scale
//      and rounding, so codes, scales and rowsums are the same bit for bit;
//   3. per-token amax and rowsum through LDS across the workgroup; the int8 (or packed int4)
//      codes go to LDS over X, in the streaming kernel's token layout (window of 256 k,
//      16-byte chunk c of token t at position c ^ (t & (chunks - 1)));
//   4. the streaming loop over the weights, token fragments from the resident codes, and the
//      streaming epilogue with the token scales and rowsums of step 3.
// Waves per workgroup (one workgroup per CU): 12 when K is a multiple of 3072 up to 12288
// (each 16-lane group then rotates one 256-element block), else 8 (up to 16384 elements,
// two blocks per group); 12 measured 4.5% faster at 12288 -> 4096.
constexpr int fuse_max_elems(int nw) { return nw == 12 ? 12288 : 16384; }  // M K per workgroup
constexpr int kFuseDMax = 2;          // weight stages in flight per wave (deeper rings measured
                                      // slower: the rotation then trails the stream)
constexpr int fuse_pmax(int nw) { return fuse_max_elems(nw) / (4 * nw * 256); }  // blocks per 16-lane group

template <int ABITS, int TM, int G, int RB, int NWV>
struct FL {
    static constexpr int NW = NWV;
    static constexpr int MAXE = fuse_max_elems(NW), PMAX = fuse_pmax(NW);
    static constexpr int D = kFuseDMax;
    static constexpr int LB = 2 * RB;    // weight loads per stage: 16 RB rows x 128 bytes
    static constexpr int WB = LB * 1024;
    static constexpr int RING = NW * D * WB;
    static constexpr int XOFF = RING;    // X (bf16), then the codes over it
    static constexpr int C_SW = XOFF + MAXE * 2, C_BIAS = C_SW + 256, C_ZP = C_BIAS + 256,
                         C_DUMMY = C_ZP + 256, C_SX = C_DUMMY + 512, C_RS = C_SX + 64, C_RD = C_RS + 64,
                         C_RI = C_RD + 8 * NW * TM;
    static constexpr int LDS = C_RI + 4 * NW * TM;
    static_assert(TM <= 4 && LDS <= 160 * 1024 && D * LB + kNC + MAXE * 2 / 1024 / NW <= 63 &&
                      4 * NW * PMAX * 256 == MAXE && RING >= NW * 1024,
                  "fused layout");
};

template <int ABITS, int TM, int G, int RB, int NWV>
__global__ void __launch_bounds__(64 * NWV) k_gemv_fused(LinearArgs p, const uint16_t *__restrict__ X, int asym) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using F = FL<ABITS, TM, G, RB, NWV>;
    constexpr int kFusePMax = F::PMAX;
    constexpr int NW = F::NW;
    constexpr int R = 16 * RB;
    constexpr int DM = F::D, LB = F::LB;
    constexpr int KST = 256 * NW;
    constexpr int QMAX = ABITS == 8 ? 127 : 7;
    constexpr double INV_SQRT_G = G == 64 ? 0.125 : 0.0625;
    constexpr int TB = ABITS == 8 ? 256 : 128;  // code bytes per token and 256-k window
    constexpr int CPT = TB / 16;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kb = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * R;
    const int K = (int)p.K, M = (int)p.M;
    const int nst = K / KST;
    const int64_t rowB = K / 2;
    const int CB = K * ABITS / 8;  // code bytes per token
    const uint32_t smem_base = lds_addr(smem);
    const uint32_t xr = asym ? 0x88888888u : 0u;
    const int D = min(nst, DM);  // stages in flight
    const int ring = wave * DM * F::WB;

    // ---- 1. loads: X, the first D weight stages, the constants
    const int nx = M * K * 2 / 1024;
    for (int q = wave; q < nx; q += NW)
        gl_lds16_so((uint64_t)X, (uint32_t)(1024 * q + 16 * lane), smem_base + F::XOFF + 1024 * q);
    uint32_t brow[LB], bin[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int r = 8 * j + lane / 8;
        brow[j] = (uint32_t)((min<int64_t>(n0 + r, p.N - 1) - n0) * rowB);
        bin[j] = (uint32_t)(128 * wave + 16 * swz8(r, lane & 7));
    }
    const uint64_t bbase = (uint64_t)(p.B + n0 * rowB);
    auto issue = [&](int i) __attribute__((always_inline)) {
        const uint32_t slot = smem_base + (uint32_t)(ring + (i % D) * F::WB);
#pragma unroll
        for (int j = 0; j < LB; ++j) gl_lds16_so(bbase, brow[j] + bin[j] + (uint32_t)i * (KST / 2), slot + 1024 * j);
    };
    for (int i = 0; i < D; ++i) issue(i);
    if (wave == 0) {  // kNC loads like the streaming kernel; token scales and rowsums come from step 3
        const uint32_t c = (uint32_t)(min<int64_t>(n0 + min(lane, R - 1), p.N - 1) - n0);
        const uint64_t sw = (uint64_t)(p.sw + n0);
        gl_lds4_so(sw, 4 * c, smem_base + F::C_SW);
        if (p.bias && p.bias_bf16) gl_lds2_so((uint64_t)((const uint16_t *)p.bias + n0), 2 * c, smem_base + F::C_BIAS);
        else if (p.bias) gl_lds4_so((uint64_t)((const float *)p.bias + n0), 4 * c, smem_base + F::C_BIAS);
        else gl_lds4_so(sw, 4 * c, smem_base + F::C_BIAS);
        if (asym) gl_lds1_so((uint64_t)(p.zp + n0), c, smem_base + F::C_ZP);
        else gl_lds4_so(sw, 4 * c, smem_base + F::C_ZP);
        gl_lds4_so(sw, 4 * c, smem_base + F::C_DUMMY);
        gl_lds4_so(sw, 4 * c, smem_base + F::C_DUMMY + 256);
    }
    // this wave's X pieces have landed; the stages and constants issued after them may still
    // be in flight, so the weight stream runs on while the tokens are rotated
    if (wave == 0) wait_rem<LB, DM, kNC>(D);
    else wait_rem<LB, DM>(D);
    __syncthreads();  // every wave's X pieces

    // ---- 2. rotate: 16-lane group lg takes blocks u = lg + 4 NW pp (pp < P, uniform)
    const int lg = tid >> 4, cl = tid & 15;
    const int nblk = K / 256, U = M * nblk, P = (U + 4 * NW - 1) / (4 * NW);
    double v[kFusePMax][16];
    double am[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) am[t] = 0.0;
#pragma unroll
    for (int pp = 0; pp < kFusePMax; ++pp) {
        if (pp >= P) break;
        const int u = lg + 4 * NW * pp;
        const bool ok = u < U;
        const int t = ok ? u / nblk : 0, j = ok ? u - t * nblk : 0;
        uint4 w0 = make_uint4(0, 0, 0, 0), w1 = w0;
        if (ok) {
            const uint8_t *src = smem + F::XOFF + 2 * (t * K + 256 * j + 16 * cl);
            w0 = *reinterpret_cast<const uint4 *>(src);
            w1 = *reinterpret_cast<const uint4 *>(src + 16);
        }
        const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[pp][2 * e] = (double)bf16_lo(wd[e]);
            v[pp][2 * e + 1] = (double)bf16_hi(wd[e]);
        }
        fwht16(v[pp]);
        // lane exchanges stay inside the 16-lane group (quads; lanes 4 and 8 apart)
        const double s1 = (cl & 1) ? -1.0 : 1.0, s2 = (cl & 2) ? -1.0 : 1.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[pp][i] = fma(v[pp][i], s1, dpp_f64<kQuadXor1>(v[pp][i]));
#pragma unroll
        for (int i = 0; i < 16; ++i) v[pp][i] = fma(v[pp][i], s2, dpp_f64<kQuadXor2>(v[pp][i]));
        if constexpr (G == 256) {
            const double s4 = (cl & 4) ? -1.0 : 1.0, s8 = (cl & 8) ? -1.0 : 1.0;
#pragma unroll
            for (int i = 0; i < 16; ++i) v[pp][i] = fma(v[pp][i], s4, swz_f64<kSwzXor4>(v[pp][i]));
#pragma unroll
            for (int i = 0; i < 16; ++i) v[pp][i] = fma(v[pp][i], s8, swz_f64<kSwzXor8>(v[pp][i]));
        }
        double mx = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmax(mx, fabs(v[pp][i]));
        if (ok) {
#pragma unroll
            for (int tt = 0; tt < TM; ++tt)
                if (tt == t) am[tt] = fmax(am[tt], mx);
        }
    }

    // ---- 3. per-token amax across the workgroup, scales, codes, rowsums
    double *rd = reinterpret_cast<double *>(smem + F::C_RD);
    int *ri = reinterpret_cast<int *>(smem + F::C_RI);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        am[t] = wave_max_f64(am[t]);
        if (lane == 0) rd[wave * TM + t] = am[t];
    }
    __syncthreads();  // also: every lane is past its reads of X
    double rr[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        double a = rd[t];
#pragma unroll
        for (int w = 1; w < NW; ++w) a = fmax(a, rd[w * TM + t]);
        const float scale = (float)((a * INV_SQRT_G) / (double)QMAX);
        rr[t] = scale > 0.0f ? (1.0 / (double)scale) * INV_SQRT_G : 0.0;
        if (tid == 0) *reinterpret_cast<float *>(smem + F::C_SX + 4 * t) = scale;
    }
    int rsum[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) rsum[t] = 0;
#pragma unroll
    for (int pp = 0; pp < kFusePMax; ++pp) {
        if (pp >= P) break;
        const int u = lg + 4 * NW * pp;
        if (u < U) {
            const int t = u / nblk, j = u - t * nblk;
            double rt = 0.0;
#pragma unroll
            for (int tt = 0; tt < TM; ++tt)
                if (tt == t) rt = rr[tt];
            uint32_t d[4];
            int rs = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int q4[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = __double2loint(fma(v[pp][4 * q + r], rt, kRoundMagic));
                    q4[r] = min(max(qi, -QMAX - 1), QMAX);
                }
                d[q] = (uint32_t)(q4[0] & 0xff) | ((uint32_t)(q4[1] & 0xff) << 8) | ((uint32_t)(q4[2] & 0xff) << 16) |
                       ((uint32_t)(q4[3] & 0xff) << 24);
                rs = __builtin_amdgcn_sdot4((int)d[q], 0x01010101, rs, false);
            }
#pragma unroll
            for (int tt = 0; tt < TM; ++tt)
                if (tt == t) rsum[tt] += rs;
            uint8_t *dst = smem + F::XOFF + t * CB + j * TB;
            if constexpr (ABITS == 8) {
                *reinterpret_cast<uint4 *>(dst + 16 * (cl ^ (t & 15))) = make_uint4(d[0], d[1], d[2], d[3]);
            } else {
                uint32_t x[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = d[q] & 0x0F0F0F0Fu;
                    x[q] = lo | (lo >> 4);
                }
                *reinterpret_cast<uint2 *>(dst + 16 * ((cl >> 1) ^ (t & 7)) + 8 * (cl & 1)) =
                    make_uint2(__builtin_amdgcn_perm(x[1], x[0], 0x06040200u), __builtin_amdgcn_perm(x[3], x[2], 0x06040200u));
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        rsum[t] = wave_sum_i32(rsum[t]);
        if (lane == 0) ri[wave * TM + t] = rsum[t];
    }
    __syncthreads();  // codes and per-wave rowsums
    if (tid < TM) {
        int a = 0;
        for (int w = 0; w < NW; ++w) a += ri[w * TM + tid];
        *reinterpret_cast<int *>(smem + F::C_RS + 4 * tid) = a;
    }

    // ---- 4. the streaming loop over the weights
    v4i acc[2][RB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[h][rb] = v4i{0, 0, 0, 0};
    const int tt = min(lr, M - 1);
    const uint8_t *codes = smem + F::XOFF + tt * CB;
    for (int i = 0; i < nst; ++i) {
        if (wave == 0 && i < D) wait_rem<LB, DM - 1, kNC>(min(D - 1, nst - 1 - i));
        else wait_rem<LB, DM - 1>(min(D - 1, nst - 1 - i));
        const uint8_t *sl = smem + ring + (i % D) * F::WB;
        const uint8_t *cw = codes + (i * NW + wave) * TB;  // this wave's 256-k window
        uint4 xa[2][ABITS == 8 ? 2 : 1], wv[2][RB];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if constexpr (ABITS == 8) {
                const int c0 = 8 * u + 2 * kb;
                xa[u][0] = *reinterpret_cast<const uint4 *>(cw + 16 * (c0 ^ (tt & 15)));
                xa[u][1] = *reinterpret_cast<const uint4 *>(cw + 16 * ((c0 + 1) ^ (tt & 15)));
            } else {
                xa[u][0] = *reinterpret_cast<const uint4 *>(cw + 16 * ((4 * u + kb) ^ (tt & 7)));
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int r = 16 * rb + lr;
                wv[u][rb] = *reinterpret_cast<const uint4 *>(sl + r * 128 + 16 * swz8(r, 4 * u + kb));
            }
        }
        wait_lgkmcnt0();
        if (i + D < nst) issue(i + D);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            v4i a0, a1;
            if constexpr (ABITS == 8) {
                a0 = __builtin_bit_cast(v4i, xa[u][0]);
                a1 = __builtin_bit_cast(v4i, xa[u][1]);
            } else {
                a0 = evod(xa[u][0].x, xa[u][0].y);
                a1 = evod(xa[u][0].z, xa[u][0].w);
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                uint4 w = wv[u][rb];
                w.x ^= xr; w.y ^= xr; w.z ^= xr; w.w ^= xr;
                v4i w0, w1;
                if constexpr (ABITS == 8) {
                    uint32_t q[8];
                    unpack_nat(w.x, q[0], q[1]);
                    unpack_nat(w.y, q[2], q[3]);
                    unpack_nat(w.z, q[4], q[5]);
                    unpack_nat(w.w, q[6], q[7]);
                    w0 = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
                    w1 = v4i{(int)q[4], (int)q[5], (int)q[6], (int)q[7]};
                } else {
                    w0 = evod(w.x, w.y);
                    w1 = evod(w.z, w.w);
                }
                acc[u][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w0, a0, acc[u][rb], 0, 0, 0);
                acc[u][rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w1, a1, acc[u][rb], 0, 0, 0);
            }
        }
    }
    // as in the streaming kernel: with nst <= D no wait of the loop covered the constants
    wait_vmcnt<0>();
    stream_epilogue<ABITS, RB, NW>(p, smem, acc, n0, asym, F::C_SW, F::C_BIAS, F::C_ZP, F::C_SX, F::C_RS);
}

template <int ABITS, int TM, int G, int RB, int NW>
hipError_t launch_fused_t(const LinearArgs &a, const void *X, hipStream_t st) {
    using F = FL<ABITS, TM, G, RB, NW>;
    const void *fn = reinterpret_cast<const void *>(&k_gemv_fused<ABITS, TM, G, RB, NW>);
    static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, F::LDS);
    if (attr != hipSuccess) return attr;
    const unsigned grid = (unsigned)((a.N + 16 * RB - 1) / (16 * RB));
    hipLaunchKernelGGL((k_gemv_fused<ABITS, TM, G, RB, NW>), dim3(grid), dim3(64 * NW), F::LDS, st, a,
                       static_cast<const uint16_t *>(X), a.zp ? 1 : 0);
    return hipGetLastError();
}

// Waves per workgroup of the fused launch for this K (0: K is not a whole number of stages).
int fused_waves(int64_t K) {
    if (K % 3072 == 0 && K <= fuse_max_elems(12)) return 12;
    if (K % 2048 == 0 && K <= fuse_max_elems(8)) return 8;
    return 0;
}

// Rows per workgroup of the fused launch: enough 16-row blocks that the grid stays within
// one workgroup per CU (each workgroup repeats the rotation); at most 2 by gemv_fusable.
int fused_row_blocks(int64_t N) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return (int)((N + 16 * (int64_t)ncu - 1) / (16 * (int64_t)ncu));
}

template <int ABITS, int G>
hipError_t fused_tm(const LinearArgs &a, const void *X, hipStream_t st) {
    const bool w12 = fused_waves(a.K) == 12;
    if (fused_row_blocks(a.N) <= 1)
        return w12 ? launch_fused_t<ABITS, 1, G, 1, 12>(a, X, st) : launch_fused_t<ABITS, 1, G, 1, 8>(a, X, st);
    return w12 ? launch_fused_t<ABITS, 1, G, 2, 12>(a, X, st) : launch_fused_t<ABITS, 1, G, 2, 8>(a, X, st);
}

}  // namespace

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits) {
    if (M <= 16) return 0;  // the streaming kernel needs none
    const SkPlan sk = plan_sk(M, N, K, act_bits);
    if (sk_used(sk, M)) return (size_t)sk.S * (size_t)M * (size_t)N * sizeof(int32_t);
    const SplitPlan pl = plan_split(M, N, K, act_bits);
    return pl.S > 1 ? (size_t)pl.S * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

hipError_t launch_gemv(const LinearArgs &a, int act_bits, void *ws, size_t ws_bytes, hipStream_t st) {
    if (a.M == 0) return hipSuccess;
    if (a.M > 64) return hipErrorInvalidValue;
    if (a.M <= 16) return act_bits == 8 ? launch_stream<8>(a, st) : launch_stream<4>(a, st);
    {
        const SkPlan sk = plan_sk(a.M, a.N, a.K, act_bits);
        if (sk_used(sk, a.M) && ws && ws_bytes >= (size_t)sk.S * (size_t)a.M * (size_t)a.N * sizeof(int32_t)) {
            int32_t *part = static_cast<int32_t *>(ws);
            return act_bits == 8 ? sk_mb<8>(a, sk, part, st) : sk_mb<4>(a, sk, part, st);
        }
    }
    const SplitPlan pl = plan_split(a.M, a.N, a.K, act_bits);
    const size_t need = pl.S > 1 ? (size_t)pl.S * (size_t)a.M * (size_t)a.N * sizeof(int32_t) : 0;
    if (pl.S >= 1 && (need == 0 || (ws && ws_bytes >= need))) {
        int32_t *part = static_cast<int32_t *>(ws);
        return act_bits == 8 ? split_mb<8>(a, pl, part, st) : split_mb<4>(a, pl, part, st);
    }
    return act_bits == 8 ? dispatch_mb<8>(a, st) : dispatch_mb<4>(a, st);
}

// Fused where it measured faster than the two launches: one token (at 2 to 4 tokens the
// rotation outlasts the weight stages in flight), at most one workgroup per CU with up to 32
// rows each (more workgroups would repeat the rotation on each CU; 48 rows measured level
// with the two launches), whole stages.  The kernel itself takes up to 4 tokens.
bool gemv_fusable(int64_t M, int64_t N, int64_t K, int g, int act_bits, bool f32in) {
    const int nw = fused_waves(K);
    if (f32in || M != 1 || nw == 0 || M * K > fuse_max_elems(nw) || (g != 64 && g != 256) ||
        (act_bits != 8 && act_bits != 4))
        return false;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return (N + 31) / 32 <= ncu;
}

hipError_t launch_gemv_fused(const LinearArgs &a, const void *X, int g, int act_bits, hipStream_t st) {
    if (!gemv_fusable(a.M, a.N, a.K, g, act_bits, false)) return hipErrorInvalidValue;
    if (act_bits == 8) return g == 64 ? fused_tm<8, 64>(a, X, st) : fused_tm<8, 256>(a, X, st);
    return g == 64 ? fused_tm<4, 64>(a, X, st) : fused_tm<4, 256>(a, X, st);
}

}  // namespace w4
