// Integer GEMM + fused dequant epilogue on the gfx950 int8 matrix cores (M > 64).
//
// ComfyUI-INT-Crush README, "Inference / INT4": unpack INT4 to INT8, INT8 GEMM with fused
// dequant (W4A8: unpack, dynamic activation quantization, fused INT8 GEMM + dequant);
// "Forward Pass" steps 5 and 6 (GEMM, then the low-rank residual).
// stable-diffusion.cpp PR #2010, "Summary": the packed nibbles stream to the kernel as
// stored, with no load-time re-blocking, so this kernel reads the canonical [N, K/2] bytes.
//
// acc[m, n] = sum_k q[m, k] * (c[n, k] - z[n]) exactly, in int32.
//
// Unpacking.  A signed nibble moved to the high half of a byte is the int8 value 16 * c, so
// a packed dword d (codes k..k+7) gives (d << 4) & 0xF0F0F0F0 = even-k codes and
// d & 0xF0F0F0F0 = odd-k codes.  Asymmetric (unsigned) nibbles are XORed with 8 first
// (c -> c - 8); the epilogue adds (8 - z[n]) * rowsum[m].  Against int8 activation codes the
// two halves are interleaved back to natural k order with two v_perm; against int4
// activation codes both operands keep the even/odd order (only the pairing of k between A
// and B matters).  The accumulator holds 16 * acc (int8 codes) or 256 * acc (int4 codes),
// exact in int32 for K <= 65536, and is shifted back in the epilogue.
//
// Tiling.  One workgroup of 8 waves (two per SIMD) computes a BM x BN = 256 x 192 output tile;
// each wave owns 64 tokens x 96 output features = 2 x 3 blocks of v_mfma_i32_32x32x32_i8 (the
// int8 MFMA shape that runs at the full rate on gfx950).  The weights are the MFMA "A" operand
// and the tokens the "B" operand, so a lane ends up holding 4 consecutive output features of
// one token: the epilogue packs them into one 8-byte bf16 store.  K advances 128 per stage
// through a 3-deep LDS ring filled by direct global->LDS 16-byte loads (no register staging).
// Each stage is read in two halves; the barrier sits between them, so the fragment reads of
// the next stage are issued while the MFMAs of the current one run, and each stage's loads
// are issued three stages ahead.  Within a row the 16-byte chunks are XOR-swizzled so the
// fragment reads of 16 consecutive rows hit distinct banks.  256 x 192 tiles give exactly one
// tile per CU for a 4096 x 3072 output.
//
// The block -> tile map keeps each XCD (blocks are dealt to the 8 XCDs round-robin) on a
// compact group of tiles so the A row panels and B column panels it streams stay in its L2.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 192, BK = 128;
constexpr int WAVES_M = 4, WAVES_N = 2;
constexpr int kThreads = 64 * WAVES_M * WAVES_N;  // 512
constexpr int WTM = BM / WAVES_M;                 // 64 tokens per wave
constexpr int WTN = BN / WAVES_N;                 // 96 output features per wave
constexpr int FM = WTM / 32, FN = WTN / 32;       // 2 x 3 MFMA blocks per wave
constexpr int STAGES = 3;
constexpr int kOutStride = BN * 2 + 16;        // bytes per staged output row (padded)
constexpr int kOutBytes = BM * kOutStride;
constexpr int kEpiBytes = kOutBytes + 3 * BN * 4;  // plus per-feature scale, bias, zero-point term

template <int ABITS>
struct Lay {
    static constexpr int A_ROW = ABITS == 8 ? BK : BK / 2;  // activation bytes per row per stage
    static constexpr int A_CHUNKS = A_ROW / 16;              // 8 or 4
    static constexpr int A_BYTES = BM * A_ROW;
    static constexpr int A_INSTR = A_BYTES / (1024 * (kThreads / 64));  // per wave: 4 or 2
    static constexpr int B_ROW = BK / 2;                     // 64 packed weight bytes per row
    static constexpr int B_BYTES = BN * B_ROW;               // 12 KB = 16 loads of 48 lanes
    static constexpr int B_INSTR = 2;                        // per wave, 12 rows each
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LOADS = A_INSTR + B_INSTR;          // per wave and stage
};

// physical chunk of logical chunk c in row r (an involution)
__device__ __forceinline__ int swz_a8(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int swz_4(int r, int c) { return c ^ ((r >> 2) & 3); }

// One 16-byte global -> LDS load per active lane: lane l's bytes land at lds_base + 16 * l
// (lds_base is wave-uniform and goes through M0).  Issued through inline asm so that the
// compiler does not add its own conservative vmcnt(0) waits in front of every LDS read of the
// other stages: the kernel waits for its own loads explicitly (s_waitcnt vmcnt(n) +
// s_barrier).  The instruction writes no VGPR, so no register is left pending when the asm
// returns.  M0 is written inside the asm; no other code in these kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void gl_lds16(const void *g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base) : "memory", "m0");
}
// Same, addressed as a wave-uniform 64-bit base (SGPRs) plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void gl_lds16_so(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void unpack_nat(uint32_t d, uint32_t &lo, uint32_t &hi) {
    const uint32_t e = nib_evens16(d), o = nib_odds16(d);
    lo = __builtin_amdgcn_perm(o, e, 0x05010400u);  // codes k, k+1, k+2, k+3
    hi = __builtin_amdgcn_perm(o, e, 0x07030602u);  // codes k+4 .. k+7
}

__device__ __forceinline__ v4i evod(uint32_t d0, uint32_t d1) {
    return v4i{(int)nib_evens16(d0), (int)nib_odds16(d0), (int)nib_evens16(d1), (int)nib_odds16(d1)};
}

// Fragments of one half stage (64 k): per lane the 32 k values [32 * kb, 32 * kb + 32) of
// that half, used as two MFMA k-steps of 16.
template <int ABITS>
struct Frags {
    uint4 w[FN];                        // packed weights, one 16-byte chunk per n-block
    uint4 x[FM][ABITS == 8 ? 2 : 1];    // activation codes per m-block
};

template <int ABITS>
__device__ __forceinline__ void read_half(Frags<ABITS> &f, const uint8_t *stage, int t, int wm, int wn, int lr,
                                          int kb) {
    using L = Lay<ABITS>;
    const uint8_t *As = stage;
    const uint8_t *Bs = stage + L::A_BYTES;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = wn * WTN + j * 32 + lr;
        f.w[j] = *reinterpret_cast<const uint4 *>(Bs + n * L::B_ROW + 16 * swz_4(n, 2 * t + kb));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 32 + lr;
        if constexpr (ABITS == 8) {
            const uint8_t *row = As + r * L::A_ROW;
            f.x[i][0] = *reinterpret_cast<const uint4 *>(row + 16 * swz_a8(r, 4 * t + 2 * kb));
            f.x[i][1] = *reinterpret_cast<const uint4 *>(row + 16 * swz_a8(r, 4 * t + 2 * kb + 1));
        } else {
            f.x[i][0] = *reinterpret_cast<const uint4 *>(As + r * L::A_ROW + 16 * swz_4(r, 2 * t + kb));
        }
    }
}

// Unpacked weight operands of one half stage: two MFMA k-steps per n-block.
struct WOps {
    v4i w0[FN], w1[FN];
};

template <int ABITS, bool ASYM>
__device__ __forceinline__ void unpack_w(const Frags<ABITS> &f, WOps &o) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        uint4 x = f.w[j];
        if constexpr (ASYM) {
            x.x ^= 0x88888888u; x.y ^= 0x88888888u; x.z ^= 0x88888888u; x.w ^= 0x88888888u;
        }
        if constexpr (ABITS == 8) {
            uint32_t q[8];
            unpack_nat(x.x, q[0], q[1]);
            unpack_nat(x.y, q[2], q[3]);
            unpack_nat(x.z, q[4], q[5]);
            unpack_nat(x.w, q[6], q[7]);
            o.w0[j] = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
            o.w1[j] = v4i{(int)q[4], (int)q[5], (int)q[6], (int)q[7]};
        } else {
            o.w0[j] = evod(x.x, x.y);
            o.w1[j] = evod(x.z, x.w);
        }
    }
}

template <int ABITS>
__device__ __forceinline__ void mma_half(const Frags<ABITS> &f, const WOps &o, v16i (&acc)[FN][FM]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        v4i a0, a1;
        if constexpr (ABITS == 8) {
            a0 = __builtin_bit_cast(v4i, f.x[i][0]);
            a1 = __builtin_bit_cast(v4i, f.x[i][1]);
        } else {
            a0 = evod(f.x[i][0].x, f.x[i][0].y);
            a1 = evod(f.x[i][0].z, f.x[i][0].w);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.w0[j], a0, acc[j][i], 0, 0, 0);
            acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.w1[j], a1, acc[j][i], 0, 0, 0);
        }
    }
}

template <int ABITS, bool ASYM>
__global__ void __launch_bounds__(kThreads) k_gemm(LinearArgs p, int tiles_m, int tiles_n) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = Lay<ABITS>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int lr = lane & 31, kb = lane >> 5;

    // ---- XCD-aware tile order: XCD x = blockIdx % 8 gets a contiguous run of tile ids, and
    // tile ids walk M within groups of 4 column tiles.
    const int ntiles = tiles_m * tiles_n;
    int tile = blockIdx.x;
    if (ntiles % 8 == 0) tile = (blockIdx.x % 8) * (ntiles / 8) + blockIdx.x / 8;
    constexpr int GN = 4;
    int tm, tn;
    {
        const int gsize = GN * tiles_m;
        const int grp = tile / gsize;
        const int first_n = grp * GN;
        const int gn = min(GN, tiles_n - first_n);
        const int in = tile - grp * gsize;
        tm = in / gn;
        tn = first_n + in % gn;
    }
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t K = p.K;
    const int nk = (int)((K + BK - 1) / BK);
    const bool ktail = (K % BK) != 0;  // last stage holds only 64 valid k

    // ---- per-lane DMA byte offsets relative to the tile's row panel (rows clamped: rows >= M
    // or >= N are computed on valid data and never stored), and LDS destinations per stage.
    // The panel base advances by one stage of k per k-tile in scalar registers.
    uint32_t offA[L::A_INSTR];
    int chA[L::A_INSTR];
    const int64_t rowbA = ABITS == 8 ? K : K / 2;
    {
        constexpr int ROWS = 1024 / L::A_ROW;  // rows per wave-instruction: 8 or 16
#pragma unroll
        for (int i = 0; i < L::A_INSTR; ++i) {
            const int j = wave * L::A_INSTR + i;
            const int r = j * ROWS + lane / L::A_CHUNKS;
            const int c = ABITS == 8 ? swz_a8(r, lane % L::A_CHUNKS) : swz_4(r, lane % L::A_CHUNKS);
            const int64_t rc = min<int64_t>(m0 + r, p.M - 1) - m0;
            chA[i] = c;
            offA[i] = (uint32_t)(rc * rowbA + 16 * c);
        }
    }
    uint32_t offB[L::B_INSTR];
    int chB[L::B_INSTR];
    const bool bact = lane < 48;  // B loads use 48 lanes: 12 rows of 64 bytes
#pragma unroll
    for (int i = 0; i < L::B_INSTR; ++i) {
        const int j = wave * L::B_INSTR + i;  // 12 rows per wave-instruction
        const int r = j * 12 + (bact ? lane / 4 : 0);
        const int c = swz_4(r, lane % 4);
        const int64_t rc = min<int64_t>(n0 + r, p.N - 1) - n0;
        chB[i] = c;
        offB[i] = (uint32_t)(rc * (K / 2) + 16 * c);
    }
    const uint8_t *panelA = p.A + m0 * rowbA;
    const uint8_t *panelB = p.B + n0 * (K / 2);
    const uint32_t smem_base = lds_addr(smem);
    // A stage's loads; in a 64-wide last stage the chunks past K re-read chunk 0 of the same
    // row and stage (in bounds; that half is never multiplied).
    auto issue = [&](int kt) {
        const uint32_t sb = smem_base + (uint32_t)((kt % STAGES) * L::STAGE);
        const uint8_t *ba = panelA + (int64_t)kt * L::A_ROW;
        const uint8_t *bb = panelB + (int64_t)kt * L::B_ROW;
        const bool tail = ktail && kt == nk - 1;
#pragma unroll
        for (int i = 0; i < L::A_INSTR; ++i) {
            const uint32_t o = tail && chA[i] >= L::A_CHUNKS / 2 ? offA[i] - 16 * chA[i] : offA[i];
            gl_lds16_so((uint64_t)ba, o, sb + (uint32_t)(wave * L::A_INSTR + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < L::B_INSTR; ++i) {
            const uint32_t o = tail && chB[i] >= 2 ? offB[i] - 16 * chB[i] : offB[i];
            if (bact) gl_lds16_so((uint64_t)bb, o, sb + (uint32_t)(L::A_BYTES + (wave * L::B_INSTR + i) * 768));
        }
    };

    v16i acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = v16i{};

    // ---- prologue: three stages in flight, wait for the first
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 2) issue(2);
    if (nk > 2) wait_vmcnt<2 * L::LOADS>();
    else if (nk > 1) wait_vmcnt<L::LOADS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    // Per stage: the second half's reads go out before the first half's MFMAs; the barrier
    // sits between the halves; the next stage's first-half reads go out before the second
    // half's MFMAs.  Operands are unpacked right before the MFMAs that use them.
    Frags<ABITS> f0, f1;
    WOps o;
    read_half<ABITS>(f0, smem, 0, wm, wn, lr, kb);
    for (int kt = 0; kt < nk; ++kt) {
        const uint8_t *stage = smem + (kt % STAGES) * L::STAGE;
        const bool second = !(ktail && kt == nk - 1);
        unpack_w<ABITS, ASYM>(f0, o);
        if (second) read_half<ABITS>(f1, stage, 1, wm, wn, lr, kb);
        mma_half<ABITS>(f0, o, acc);
        // this wave has read all of stage kt; wait for stage kt+1 and for every wave
        if (kt + 1 < nk) {
            if (kt + 2 < nk) wait_vmcnt<L::LOADS>();
            else wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();
        if (kt + 3 < nk) issue(kt + 3);
        if (second) {
            unpack_w<ABITS, ASYM>(f1, o);
            if (kt + 1 < nk) read_half<ABITS>(f0, smem + ((kt + 1) % STAGES) * L::STAGE, 0, wm, wn, lr, kb);
            mma_half<ABITS>(f1, o, acc);
        } else if (kt + 1 < nk) {
            read_half<ABITS>(f0, smem + ((kt + 1) % STAGES) * L::STAGE, 0, wm, wn, lr, kb);
        }
    }

    // ---- epilogue.  32x32 block layout: lane l, register v holds output feature
    // n = 8 * (v / 4) + 4 * (l / 32) + v % 4 of token m = l % 32, so registers 4g .. 4g+3 are
    // four consecutive features of one token.  bf16 results go through LDS (the pipeline
    // buffers are free once every wave is past its last MFMA) so that the tile leaves in
    // full, 16-byte-vector rows; the raw int32 accumulator output (a test path) is stored
    // directly.
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    // staged output tile rows, then the tile's per-feature constants
    float *c_sw = reinterpret_cast<float *>(smem + kOutBytes);
    float *c_bias = c_sw + BN;
    int *c_zc = reinterpret_cast<int *>(c_bias + BN);
    __syncthreads();  // every wave is past its last LDS read of the pipeline
    for (int t = tid; t < BN; t += kThreads) {
        const int64_t n = min<int64_t>(n0 + t, p.N - 1);
        c_sw[t] = p.sw[n];
        c_bias[t] = !p.bias ? 0.0f
                            : p.bias_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[n])
                                          : reinterpret_cast<const float *>(p.bias)[n];
        c_zc[t] = ASYM ? 8 - (int)p.zp[n] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int ml = wm * WTM + i * 32 + lr;  // token within the tile
        const int64_t m = m0 + ml;
        const bool mok = m < p.M;
        const int64_t mc = mok ? m : p.M - 1;
        const float sxm = p.sx[mc];
        const int rsm = ASYM ? p.rowsum[mc] : 0;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * WTN + j * 32 + 8 * g + 4 * kb;  // feature within the tile
                const int64_t n = n0 + nl;
                const float4 sw = *reinterpret_cast<const float4 *>(c_sw + nl);
                int a[4] = {acc[j][i][4 * g] >> SHIFT, acc[j][i][4 * g + 1] >> SHIFT, acc[j][i][4 * g + 2] >> SHIFT,
                            acc[j][i][4 * g + 3] >> SHIFT};
                if constexpr (ASYM) {
                    const int4 zc = *reinterpret_cast<const int4 *>(c_zc + nl);
                    a[0] += zc.x * rsm; a[1] += zc.y * rsm; a[2] += zc.z * rsm; a[3] += zc.w * rsm;
                }
                if (p.y_i32) {
                    if (!mok) continue;
                    int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < p.N) Y[n + r] = a[r];
                    continue;
                }
                const float4 bs = *reinterpret_cast<const float4 *>(c_bias + nl);
                float y[4] = {fmaf((float)a[0], sxm * sw.x, bs.x), fmaf((float)a[1], sxm * sw.y, bs.y),
                              fmaf((float)a[2], sxm * sw.z, bs.z), fmaf((float)a[3], sxm * sw.w, bs.w)};
                if (p.lr_t) {
                    const float *tr = p.lr_t + mc * p.lr_r;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t nc = min<int64_t>(n + r, p.N - 1);
                        float l = 0.0f;
                        for (int q = 0; q < p.lr_r; ++q) l = fmaf(tr[q], bf16_to_f32(p.lr_l2[(int64_t)q * p.N + nc]), l);
                        y[r] += l;
                    }
                }
                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                typedef float fl2 __attribute__((ext_vector_type(2)));
                const fl2 f01 = {y[0], y[1]}, f23 = {y[2], y[3]};
                const bf2 h0 = __builtin_convertvector(f01, bf2);
                const bf2 h1 = __builtin_convertvector(f23, bf2);
                *reinterpret_cast<uint2 *>(smem + ml * kOutStride + nl * 2) =
                    make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
            }
        }
    }
    if (p.y_i32) return;
    __syncthreads();
    // the whole 256 x 192 tile, 24 chunks of 16 bytes per row
    constexpr int CPR = BN * 2 / 16;
    const bool full_n = (p.N & 7) == 0;  // 16-byte aligned rows
    uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y);
#pragma unroll 4
    for (int c = tid; c < BM * CPR; c += kThreads) {
        const int row = c / CPR, ch = c % CPR;
        const int64_t m = m0 + row, n = n0 + ch * 8;
        if (m >= p.M || n >= p.N) continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(smem + row * kOutStride + ch * 16);
        if (full_n && n + 7 < p.N) {
            *reinterpret_cast<uint4 *>(Y + m * p.N + n) = v;
        } else {
            const uint16_t *h = reinterpret_cast<const uint16_t *>(&v);
            for (int r = 0; r < 8 && n + r < p.N; ++r) Y[m * p.N + n + r] = h[r];
        }
    }
}

template <int ABITS, bool ASYM>
hipError_t launch_t(const LinearArgs &a, hipStream_t st) {
    // the pipeline ring, reused at the end to stage the bf16 output tile
    const size_t lds = std::max((size_t)STAGES * Lay<ABITS>::STAGE, (size_t)kEpiBytes);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm<ABITS, ASYM>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    const int tm = (int)((a.M + BM - 1) / BM), tn = (int)((a.N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm<ABITS, ASYM>), dim3((unsigned)(tm * tn)), dim3(kThreads), lds, st, a, tm, tn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const LinearArgs &a, int act_bits, hipStream_t st) {
    if (a.M == 0) return hipSuccess;
    if (act_bits == 8) return a.zp ? launch_t<8, true>(a, st) : launch_t<8, false>(a, st);
    return a.zp ? launch_t<4, true>(a, st) : launch_t<4, false>(a, st);
}

}  // namespace w4
