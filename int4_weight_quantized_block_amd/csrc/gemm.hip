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
// exact in int32 for K <= 65536.  The epilogue converts it to float as is and folds the
// power-of-two factor into the row scale (exact: float(2^s * a) = 2^s * float(a)).
//
// Tiling.  One workgroup of 4 waves (one per SIMD) computes a BM x BN = 256 x 192 output
// tile; each wave owns 128 tokens x 96 output features = 4 x 3 blocks of
// v_mfma_i32_32x32x32_i8 (the int8 MFMA shape that runs at the full rate on gfx950), so each
// unpacked weight operand feeds 4 MFMAs.  The weights are the MFMA "A" operand and the
// tokens the "B" operand, so a lane ends up holding 4 consecutive output features of one
// token.  K advances 128 per stage through a 3-deep LDS ring filled by direct global->LDS
// 16-byte loads (no register staging), issued three stages ahead.  Within a row the 16-byte
// chunks are XOR-swizzled so the fragment reads of 16 consecutive rows hit distinct banks.
//
// Schedule.  With one wave per SIMD every instruction of the wave takes an issue slot, and
// the matrix core only stays busy if the wave's other work (LDS fragment reads, weight
// unpacking, the global->LDS loads of a later stage) sits in the shadow of its own MFMAs.
// Each half stage (64 k, 24 MFMAs) is therefore emitted in a fixed order: MFMA, then a
// fragment read of the next half, an unpacking unit of the next half, or one global->LDS
// load, spread over the 24 MFMA slots (sched_barrier pins the order).
//
// The block -> tile map keeps each XCD (blocks are dealt to the 8 XCDs round-robin) on a
// compact group of tiles so the A row panels and B column panels it streams stay in its L2.
//
// Low-rank branch (stable-diffusion.cpp PR #2010, "Summary"; ComfyUI-INT-Crush README,
// "Forward Pass" step 6): T . L2 runs in the epilogue on the bf16 matrix cores, from t rows
// and a transposed l2 tile staged in LDS (r <= 32) or from t read per token block (r <= 64).
// Two linears that read the same codes can share one launch (GemmPair): the grid holds the
// tiles of both, so neither leaves its last round of tiles partly idle.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace w4 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 192, BK = 128;
constexpr int WAVES_M = 2, WAVES_N = 2;
constexpr int kWaves = WAVES_M * WAVES_N;
constexpr int kThreads = 64 * kWaves;             // 256: one wave per SIMD
constexpr int WTM = BM / WAVES_M;                 // 128 tokens per wave
constexpr int WTN = BN / WAVES_N;                 // 96 output features per wave
constexpr int FM = WTM / 32, FN = WTN / 32;       // 4 x 3 MFMA blocks per wave
constexpr int STAGES = 3;

template <int ABITS>
struct Lay {
    static constexpr int A_ROW = ABITS == 8 ? BK : BK / 2;    // activation bytes per row per stage
    static constexpr int A_CHUNKS = A_ROW / 16;                // 8 or 4
    static constexpr int A_BYTES = BM * A_ROW;
    static constexpr int A_INSTR = A_BYTES / (1024 * kWaves);  // per wave: 8 or 4
    static constexpr int B_ROW = BK / 2;                       // 64 packed weight bytes per row
    static constexpr int B_BYTES = BN * B_ROW;                 // 12 KB
    static constexpr int B_INSTR = B_BYTES / (1024 * kWaves);  // per wave: 3 (16 rows each)
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LOADS = A_INSTR + B_INSTR;            // per wave and stage
    static constexpr int XW = ABITS == 8 ? 2 : 1;              // 16-byte activation chunks per half
    static constexpr int READS = FN + FM * XW;                 // ds_read_b128 per wave and half
    // the per-feature constants of the tile (raw row scales, bias, zero points) sit past the
    // ring
    static constexpr int CONST_OFF = STAGES * STAGE;
    // (one dword per feature each: f32 scale, f32 or zero-extended bf16 bias, zero-extended
    // zero point)
    static constexpr int C_SW = CONST_OFF, C_BIAS = C_SW + BN * 4, C_ZP = C_BIAS + BN * 4;
    static constexpr int LDS_BYTES = C_ZP + BN * 4;
};

constexpr int SROW = WTN * 2 + 16;            // epilogue staging row: 96 bf16 + pad
constexpr int STG_BYTES = kWaves * 32 * SROW;  // one block of 32 tokens per wave

// LDS placement of the low-rank operands for ranks r <= 16 * LRK (r % 4 == 0): the tile's
// rows of t (fp32, RP ranks + 16 pad bytes per row, so that the 16-byte reads of 8
// consecutive lanes hit distinct banks) and l2 transposed to [feature][rank] (bf16, same
// padding), so that every MFMA operand is one 16-byte LDS read.  Each goes into a ring slot
// that is free by the epilogue when it fits (t: the slot of stage nk - 3; l2T: past the
// output staging in the slot of stage nk - 2), else past the l2 tile.
template <int ABITS, int LRK>
struct LrLay {
    static constexpr int RP = 16 * LRK;
    static constexpr int T_PITCH = RP * 4 + 16;
    static constexpr int T_CPR = T_PITCH / 16;                 // 16-byte chunks per row (last: pad)
    static constexpr int T_BYTES = BM * T_PITCH;
    static constexpr int T_INS = BM * T_CPR / 64 / kWaves;     // direct loads per wave
    static constexpr int L2T_PITCH = RP * 2 + 16;
    static constexpr int L2T_BYTES = BN * L2T_PITCH;
    static constexpr int L2_BYTES = 6 * 1024 * LRK;            // the [r, BN] l2 tile (whole 1 KB loads)
    static constexpr bool T_IN_SLOT = T_BYTES <= Lay<ABITS>::STAGE;
    static constexpr bool L2T_IN_SLOT = STG_BYTES + L2T_BYTES <= Lay<ABITS>::STAGE;
    static constexpr int DED = Lay<ABITS>::LDS_BYTES + L2_BYTES;  // dedicated room past the l2 tile
    static constexpr int T_DED = DED, L2T_DED = DED + (T_IN_SLOT ? 0 : T_BYTES);
    static constexpr int LDS_TOTAL = L2T_DED + (L2T_IN_SLOT ? 0 : L2T_BYTES);
    static_assert(BM * T_CPR % (64 * kWaves) == 0, "t staging loads");
    static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget");
};

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float fl8 __attribute__((ext_vector_type(8)));
typedef float fl16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// physical chunk of logical chunk c in row r (an involution)
__device__ __forceinline__ int swz_a8(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int swz_4(int r, int c) { return c ^ ((r >> 2) & 3); }

// Fragments of one half stage (64 k): per lane the 32 k values [32 * kb, 32 * kb + 32) of
// that half, used as two MFMA k-steps of 16.
template <int ABITS>
struct Frags {
    uint4 w[FN];                    // packed weights, one 16-byte chunk per n-block
    uint4 x[FM][Lay<ABITS>::XW];    // activation codes per m-block
};

// Fragment read number idx of a half: the FN weight chunks first (their unpacking waits only
// for them), then the activation chunks.
template <int ABITS>
__device__ __forceinline__ void read_one(Frags<ABITS> &f, const uint8_t *stage, int t, int wm, int wn, int lr,
                                         int kb, int idx) {
    using L = Lay<ABITS>;
    if (idx < FN) {
        const int n = wn * WTN + idx * 32 + lr;
        f.w[idx] = *reinterpret_cast<const uint4 *>(stage + L::A_BYTES + n * L::B_ROW + 16 * swz_4(n, 2 * t + kb));
    } else if constexpr (ABITS == 8) {
        const int i = (idx - FN) / 2, c = (idx - FN) % 2;
        const int r = wm * WTM + i * 32 + lr;
        f.x[i][c] = *reinterpret_cast<const uint4 *>(stage + r * L::A_ROW + 16 * swz_a8(r, 4 * t + 2 * kb + c));
    } else {
        const int i = idx - FN;
        const int r = wm * WTM + i * 32 + lr;
        f.x[i][0] = *reinterpret_cast<const uint4 *>(stage + r * L::A_ROW + 16 * swz_4(r, 2 * t + kb));
    }
}

// Unpacked operands of one half stage (two MFMA k-steps): weights per n-block, and for int4
// activations the unpacked token codes per m-block (int8 codes are used as read).
struct Ops {
    v4i w[2][FN];
    v4i x[2][FM];
};

// Keeps the unpacked operands computed where they are written: without it the compiler sinks
// the unpacking into the half that consumes it, out of the half whose MFMAs should hide it.
template <int ABITS>
__device__ __forceinline__ void pin(Ops &o) {
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(o.w[0][j]), "+v"(o.w[1][j]));
    if constexpr (ABITS == 4) {
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(o.x[0][i]), "+v"(o.x[1][i]));
    }
}

// Unpacking work of one half, cut into units of a few VALU instructions so that it can be
// spread between MFMAs.  int8 activations: 12 units (one packed weight dword -> 8 codes in k
// order, 5 instructions).  int4 activations: 6 weight units + 8 activation units (two packed
// dwords -> 16 codes in even/odd order, 6 instructions each).
template <int ABITS>
constexpr int kUnits = ABITS == 8 ? 4 * FN : 2 * FN + 2 * FM;

template <int ABITS, bool ASYM>
__device__ __forceinline__ void unit(const Frags<ABITS> &f, Ops &o, int u) {
    if constexpr (ABITS == 8) {
        const int j = u / 4, d = u % 4;  // dword d of chunk j: codes 8d .. 8d+7 of the lane's 32
        uint32_t x = d == 0 ? f.w[j].x : d == 1 ? f.w[j].y : d == 2 ? f.w[j].z : f.w[j].w;
        if constexpr (ASYM) x ^= 0x88888888u;
        uint32_t lo, hi;
        unpack_nat(x, lo, hi);
        o.w[d / 2][j][2 * (d % 2)] = (int)lo;
        o.w[d / 2][j][2 * (d % 2) + 1] = (int)hi;
    } else if (u < 2 * FN) {
        const int j = u / 2, h = u % 2;
        uint32_t x0 = h ? f.w[j].z : f.w[j].x, x1 = h ? f.w[j].w : f.w[j].y;
        if constexpr (ASYM) {
            x0 ^= 0x88888888u;
            x1 ^= 0x88888888u;
        }
        o.w[h][j] = evod(x0, x1);
    } else {
        const int i = (u - 2 * FN) / 2, h = (u - 2 * FN) % 2;
        const uint4 &x = f.x[i][0];
        o.x[h][i] = h ? evod(x.z, x.w) : evod(x.x, x.y);
    }
}

// MFMA number `step` of a half: k-step s = step / 12, then m-block, then n-block (an
// accumulator is reused only 12 MFMAs later).
template <int ABITS>
__device__ __forceinline__ void mma_step(const Frags<ABITS> &f, const Ops &o, v16i (&acc)[FN][FM], int step) {
    const int s = step / (FM * FN), i = (step % (FM * FN)) / FN, j = step % FN;
    v4i a;
    if constexpr (ABITS == 8) a = __builtin_bit_cast(v4i, f.x[i][s]);
    else a = o.x[s][i];
    acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.w[s][j], a, acc[j][i], 0, 0, 0);
}

// Slot positions inside a half: fragment reads of the next half at MFMA slots 0..; in a half
// without global->LDS loads the unpacking starts at slot 5 (once the weight chunks have had
// time to arrive); in a half with loads, the loads take slots 0.. and the unpacking the last
// slots, so that no slot carries much more than an MFMA's worth of other instructions.
template <int ABITS, bool LOAD>
constexpr int kUnitAt = LOAD ? 2 * FM * FN - kUnits<ABITS> - 1 : 5;
constexpr int kLoadAt = 0;

// One half stage: the 24 MFMAs of the current half (fragments fc, operands oc), with the next
// half's reads and unpacking (into fn, on) and, with LOAD, the global->LDS loads of stage
// lkt into ring slot lslot, spread over them in a fixed order.
template <int ABITS, bool ASYM, bool NEXT, bool LOAD, class LoadFn>
__device__ __forceinline__ void half_stage(const Frags<ABITS> &fc, const Ops &oc, Frags<ABITS> &fn, Ops &on,
                                           const uint8_t *nstage, int nt, int wm, int wn, int lr, int kb,
                                           v16i (&acc)[FN][FM], LoadFn &load, int lkt, int lslot) {
    using L = Lay<ABITS>;
    constexpr int NM = 2 * FM * FN;
    constexpr int UA = kUnitAt<ABITS, LOAD>;
    static_assert(UA + kUnits<ABITS> <= NM && kLoadAt + L::LOADS <= NM, "half-stage slots");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int step = 0; step < NM; ++step) {
        mma_step<ABITS>(fc, oc, acc, step);
        if constexpr (NEXT) {
            if (step < L::READS) read_one<ABITS>(fn, nstage, nt, wm, wn, lr, kb, step);
            if (step >= UA && step - UA < kUnits<ABITS>) unit<ABITS, ASYM>(fn, on, step - UA);
        }
        if constexpr (LOAD) {
            if (step >= kLoadAt && step - kLoadAt < L::LOADS) load(lkt, lslot, step - kLoadAt);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) pin<ABITS>(on);
}

// Output forms, one kernel each (the epilogue is straight-line code run once per tile, so
// leaving out what a launch does not need keeps it short)
// kEpiPartial: raw int32 partial tiles of one K range (the split tail, summed by k_gemm_tail)
enum Epi { kEpiBf16 = 0, kEpiLowRank = 1, kEpiI32 = 2, kEpiPartial = 3, kEpiLowRank16 = 4, kEpiLowRank32 = 5 };
// bf16 output with the low-rank branch, by rank: r <= 16, r <= 32 or r <= 64 (1, 2, 4 k-steps
// of 16 ranks on the bf16 MFMA)
constexpr bool epi_lr(int e) { return e == kEpiLowRank || e == kEpiLowRank16 || e == kEpiLowRank32; }
constexpr int epi_lrk(int e) { return e == kEpiLowRank16 ? 1 : e == kEpiLowRank32 ? 2 : 4; }
// r <= 16 / 32 with r % 4 == 0, 16-byte aligned t rows and N % 8 == 0: t and l2 staged in LDS
// (LrLay); kEpiLowRank (any r <= 64) reads t from global memory per token block
constexpr bool epi_lr_lds(int e) { return e == kEpiLowRank16 || e == kEpiLowRank32; }
constexpr int epi_lds_k(int e) { return epi_lr_lds(e) ? epi_lrk(e) : 1; }  // LrLay's LRK

// The tiles one launch covers: ids [base, base + count); with kEpiPartial each tile is split
// into kparts equal K ranges (one workgroup each) whose partial tiles go to part.
struct TileRange {
    int base, count, kparts;
    int32_t *part;
};

// Tile id -> (tile row, tile column): ids walk M within groups of GN column tiles, so the
// workgroups that share A and B panels run close together.  GN = 8: an XCD's 32 tiles of a
// round then cover 4 row panels x 8 column panels (at 4096 tokens x 3072 features, 3.1 MB of
// int8 codes + 2.4 MB of packed weights, the least of the 32-tile rectangles).
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, int &tm, int &tn) {
    constexpr int GN = 8;
    const int gsize = GN * tiles_m;
    const int grp = tile / gsize;
    const int first_n = grp * GN;
    const int gn = min(GN, tiles_n - first_n);
    const int in = tile - grp * gsize;
    tm = in / gn;
    tn = first_n + in % gn;
}

// One or two linears launched as one grid: tile ids [0, n0) are the first's, the rest the
// second's.  Two linears that read the same activation codes (same M, K and code width, the
// same weight mode and epilogue form) fill the compute units together, where each alone would
// leave its last round partly idle.
struct GemmPair {
    LinearArgs p[2];
    int tiles_m[2], tiles_n[2];
    int n0;
};

template <int ABITS, bool ASYM, bool KTAIL, int EPI, bool PAIR>
__global__ void __launch_bounds__(kThreads) k_gemm(GemmPair gp, int l2_dma, TileRange tr) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = Lay<ABITS>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int lr = lane & 31, kb = lane >> 5;

    // ---- XCD-aware tile order: XCD x = blockIdx % 8 gets a contiguous run of tile ids
    // (a split tail: consecutive workgroups are the K ranges of one tile)
    int tile, kpart = 0;
    if constexpr (EPI == kEpiPartial) {
        tile = tr.base + (int)blockIdx.x / tr.kparts;
        kpart = (int)blockIdx.x % tr.kparts;
    } else {
        tile = blockIdx.x;
        if (tr.count % 8 == 0) tile = (blockIdx.x % 8) * (tr.count / 8) + blockIdx.x / 8;
        tile += tr.base;
    }
    // (a single linear reads p[0] at fixed offsets: selecting the problem per workgroup
    // costs registers and time that only a pair needs)
    const int pi = PAIR && tile >= gp.n0 ? 1 : 0;
    const LinearArgs &p = gp.p[PAIR ? pi : 0];
    int tm, tn;
    tile_coords(tile - pi * gp.n0, gp.tiles_m[pi], gp.tiles_n[pi], tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t K = p.K;
    // stages of this workgroup (the last holds 64 valid k when KTAIL); a K range of a split
    // tail starts ks0 stages in (K % BK == 0 there)
    const int nk = EPI == kEpiPartial ? (int)(K / BK) / tr.kparts : (int)((K + BK - 1) / BK);
    const int ks0 = EPI == kEpiPartial ? kpart * nk : 0;

    // ---- the tile's per-feature constants go to LDS with the same direct loads (ahead of the
    // pipeline's loads, so the first stage's wait covers them); per-lane token constants go to
    // registers and are first used in the epilogue.
    if (EPI != kEpiPartial && wave == 0) {
        const uint32_t cb = lds_addr(smem);
#pragma unroll
        for (int q = 0; q < BN / 64; ++q) {
            const uint32_t c = (uint32_t)(min<int64_t>(n0 + q * 64 + lane, p.N - 1) - n0);  // clamped column
            gl_lds4_so((uint64_t)(p.sw + n0), 4 * c, cb + L::C_SW + q * 256);
            if (p.bias) {
                if (p.bias_bf16) gl_lds2_so((uint64_t)((const uint16_t *)p.bias + n0), 2 * c, cb + L::C_BIAS + q * 256);
                else gl_lds4_so((uint64_t)((const float *)p.bias + n0), 4 * c, cb + L::C_BIAS + q * 256);
            }
            if constexpr (ASYM) gl_lds1_so((uint64_t)(p.zp + n0), c, cb + L::C_ZP + q * 256);
        }
    }
    // The low-rank l2 tile [r, BN] (bf16 rows of the tile's features; columns past N hold
    // clamped copies, never used) goes past the constants: with the same direct loads, spread
    // over the waves, when its rows are 16-byte aligned (N % 8 == 0), else element by element
    // through registers (a one-off wait, ragged N only).  The prologue's wait and barrier
    // make it visible to every wave.
    if constexpr (epi_lr(EPI)) {
        if (epi_lr_lds(EPI) || l2_dma) {
            constexpr int CPR = BN * 2 / 16;  // 24 chunks of 16 bytes per row
            const int nins = (CPR * p.lr_r + 63) / 64;
            const uint32_t lb = lds_addr(smem) + L::LDS_BYTES;
            for (int ins = wave; ins < nins; ins += kWaves) {
                const int c = ins * 64 + lane;
                const int q = min(c / CPR, p.lr_r - 1);  // whole 1 KB blocks: the tail repeats row r-1
                const int64_t nn = min<int64_t>(n0 + 8 * (c % CPR), p.N - 8) - n0;
                gl_lds16_so((uint64_t)(p.lr_l2 + n0), (uint32_t)((int64_t)q * p.N * 2 + nn * 2), lb + ins * 1024);
            }
        } else if constexpr (!epi_lr_lds(EPI)) {
            uint16_t *lt = reinterpret_cast<uint16_t *>(smem + L::LDS_BYTES);
            const int tot = p.lr_r * BN;
            for (int e0 = tid; e0 < tot; e0 += 8 * kThreads) {
                uint16_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + u * kThreads;
                    const int64_t nc = min<int64_t>(n0 + e % BN, p.N - 1);
                    v[u] = e < tot ? p.lr_l2[(int64_t)(e / BN) * p.N + nc] : (uint16_t)0;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (e0 + u * kThreads < tot) lt[e0 + u * kThreads] = v[u];
            }
            wait_vmcnt<0>();
            wait_lgkmcnt0();
        }
    }
    float sxv[FM];
    int rsv[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = min<int64_t>(m0 + wm * WTM + i * 32 + lr, p.M - 1);
        sxv[i] = EPI == kEpiPartial ? 0.0f : p.sx[m];
        rsv[i] = ASYM && EPI != kEpiPartial ? p.rowsum[m] : 0;
    }

    // ---- per-lane DMA byte offsets relative to the tile's row panel (rows clamped: rows >= M
    // or >= N are computed on valid data and never stored), and LDS destinations per stage.
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
#pragma unroll
    for (int i = 0; i < L::B_INSTR; ++i) {
        const int j = wave * L::B_INSTR + i;  // 16 rows per wave-instruction
        const int r = j * 16 + lane / 4;
        const int c = swz_4(r, lane % 4);
        const int64_t rc = min<int64_t>(n0 + r, p.N - 1) - n0;
        chB[i] = c;
        offB[i] = (uint32_t)(rc * (K / 2) + 16 * c);
    }
    const uint8_t *panelA = p.A + m0 * rowbA + (int64_t)ks0 * L::A_ROW;
    const uint8_t *panelB = p.B + n0 * (K / 2) + (int64_t)ks0 * L::B_ROW;
    const uint32_t smem_base = lds_addr(smem);
    // Load number idx of stage kt (into ring slot `slot`); in a 64-wide last stage the chunks
    // past K re-read chunk 0 of the same row and stage (in bounds; that half is never
    // multiplied).
    auto load_one = [&](int kt, int slot, int idx) __attribute__((always_inline)) {
        const uint32_t sb = smem_base + (uint32_t)(slot * L::STAGE);
        const bool tail = KTAIL && kt == nk - 1;
        if (idx < L::A_INSTR) {
            const int i = idx;
            const uint32_t o = tail && chA[i] >= L::A_CHUNKS / 2 ? offA[i] - 16 * chA[i] : offA[i];
            gl_lds16_so((uint64_t)(panelA + (int64_t)kt * L::A_ROW), o, sb + (uint32_t)(wave * L::A_INSTR + i) * 1024);
        } else {
            const int i = idx - L::A_INSTR;
            const uint32_t o = tail && chB[i] >= 2 ? offB[i] - 16 * chB[i] : offB[i];
            gl_lds16_so((uint64_t)(panelB + (int64_t)kt * L::B_ROW), o,
                        sb + (uint32_t)(L::A_BYTES + (wave * L::B_INSTR + i) * 1024));
        }
    };

    // Low-rank forms with staged operands: the tile's t rows go to LDS by direct loads, issued
    // once the slot of stage nk - 3 is free (or at the epilogue when nk < 3), so their latency
    // hides under the last stages.  Chunk c of a staged row holds ranks 4c .. 4c+3; the padding
    // chunk and chunks past r re-read the row's last chunk (finite values that meet zero ranks
    // of l2T); rows past M repeat row M - 1 (computed, never stored).
    using LL = LrLay<ABITS, epi_lds_k(EPI)>;
    constexpr int TW = epi_lr_lds(EPI) ? LL::T_INS : 0;
    const uint32_t t_lds = smem_base + (uint32_t)(LL::T_IN_SLOT ? (nk % STAGES) * L::STAGE : LL::T_DED);
    auto issue_t = [&]() __attribute__((always_inline)) {
        const int last = (p.lr_r >> 2) - 1;
#pragma unroll
        for (int u = 0; u < LL::T_INS; ++u) {
            const int ins = wave * LL::T_INS + u;
            const int c = ins * 64 + lane;
            const int row = c / LL::T_CPR, cc = min(c % LL::T_CPR, last);
            const int64_t rr = min<int64_t>(m0 + row, p.M - 1) - m0;
            gl_lds16_so((uint64_t)(p.lr_t + m0 * p.lr_ldt), (uint32_t)((rr * p.lr_ldt + 4 * cc) * 4),
                        t_lds + (uint32_t)ins * 1024);
        }
    };

    v16i acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = v16i{};

    // ---- prologue: three stages in flight, wait for the first (and the constants)
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
        if (s < nk)
#pragma unroll
            for (int q = 0; q < L::LOADS; ++q) load_one(s, s, q);
    if (nk > 2) wait_vmcnt<2 * L::LOADS>();
    else if (nk > 1) wait_vmcnt<L::LOADS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    // ---- main loop.  Software pipeline over half stages: while the MFMAs of half h run, the
    // fragments of half h+1 are read from LDS and unpacked.  Between the halves of stage kt:
    // wait for stage kt+1's loads, barrier (every wave has read all of stage kt), then the
    // second half issues stage kt+3's loads into stage kt's slot.
    Frags<ABITS> fa, fb;  // fa: first half of a stage, fb: second half
    Ops oa, ob;
#pragma unroll
    for (int q = 0; q < L::READS; ++q) read_one<ABITS>(fa, smem, 0, wm, wn, lr, kb, q);
#pragma unroll
    for (int u = 0; u < kUnits<ABITS>; ++u) unit<ABITS, ASYM>(fa, oa, u);
    int slot = 0;  // kt % STAGES
    int kt = 0;
    // steady state: stage kt+3 exists, its loads ride in the second half
    for (; kt < nk - 3; ++kt) {
        const int nslot = slot == STAGES - 1 ? 0 : slot + 1;
        half_stage<ABITS, ASYM, true, false>(fa, oa, fb, ob, smem + slot * L::STAGE, 1, wm, wn, lr, kb, acc, load_one,
                                             0, 0);
        wait_vmcnt<L::LOADS>();
        wait_lgkmcnt0();  // this wave's reads of stage kt have completed
        __builtin_amdgcn_s_barrier();
        half_stage<ABITS, ASYM, true, true>(fb, ob, fa, oa, smem + nslot * L::STAGE, 0, wm, wn, lr, kb, acc, load_one,
                                            kt + 3, slot);
        slot = nslot;
    }
    // the last two stages before the final one: nothing left to load
    for (; kt < nk - 1; ++kt) {
        const int nslot = slot == STAGES - 1 ? 0 : slot + 1;
        half_stage<ABITS, ASYM, true, false>(fa, oa, fb, ob, smem + slot * L::STAGE, 1, wm, wn, lr, kb, acc, load_one,
                                             0, 0);
        if (kt + 2 < nk) wait_vmcnt<L::LOADS>();
        else if (epi_lr_lds(EPI) && nk >= 3) wait_vmcnt<TW>();  // the staged t may still be in flight
        else wait_vmcnt<0>();
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        // every wave has read stage kt: with kt = nk - 3 its slot is the t slot
        if constexpr (epi_lr_lds(EPI)) {
            if (kt == nk - 3) issue_t();
        }
        half_stage<ABITS, ASYM, true, false>(fb, ob, fa, oa, smem + nslot * L::STAGE, 0, wm, wn, lr, kb, acc, load_one,
                                             0, 0);
        slot = nslot;
    }
    // last stage (64 k only when K % 128 == 64)
    if constexpr (!KTAIL) {
        half_stage<ABITS, ASYM, true, false>(fa, oa, fb, ob, smem + slot * L::STAGE, 1, wm, wn, lr, kb, acc, load_one, 0,
                                             0);
        half_stage<ABITS, ASYM, false, false>(fb, ob, fa, oa, nullptr, 0, wm, wn, lr, kb, acc, load_one, 0, 0);
    } else {
        half_stage<ABITS, ASYM, false, false>(fa, oa, fb, ob, nullptr, 0, wm, wn, lr, kb, acc, load_one, 0, 0);
    }

    if constexpr (EPI == kEpiPartial) {
        // raw accumulators of this K range: lane l holds features 4 consecutive n of token
        // l % 32 per register group (the layout described below), stored as 16-byte pieces
        int32_t *P = tr.part + ((int64_t)(tile - tr.base) * tr.kparts + kpart) * (BM * BN);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ml = wm * WTM + i * 32 + lr, nl = wn * WTN + j * 32 + 8 * g + 4 * kb;
                    *reinterpret_cast<int4 *>(P + ml * BN + nl) =
                        make_int4(acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]);
                }
        return;
    }
    // ---- epilogue.  32x32 block layout: lane l, register v holds output feature
    // n = 8 * (v / 4) + 4 * (l / 32) + v % 4 of token m = l % 32, so registers 4g .. 4g+3 are
    // four consecutive features of one token.  Each wave finishes on its own (no workgroup
    // barrier): per block of 32 tokens it converts its 32 x 96 outputs, stages them as bf16
    // rows in its own piece of a ring slot that no wave reads any more (the slot of stage
    // nk-2, or one never filled), and stores full 16-byte row chunks, so the stores of one
    // block drain while the next one is converted.  The raw int32 accumulator output (a test
    // path) is stored directly.
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    constexpr float kUnscale = ABITS == 8 ? 1.0f / 16 : 1.0f / 256;
    const float *c_sw = reinterpret_cast<const float *>(smem + L::C_SW);
    const uint8_t *c_bias = smem + L::C_BIAS;
    const uint8_t *c_zp = smem + L::C_ZP;
    // per-feature constants of a group of 4 features (row scale with the code factor, bias,
    // (8 - z) * 2^SHIFT), read from LDS where they are used: holding all 12 groups in
    // registers through the epilogue made the low-rank form spill, and each reload's vmcnt(0)
    // then also waited for the output stores of the previous token block
    auto consts_lds = [&](int j, int g, float (&sw)[4], float (&bs)[4], int (&zc)[4]) __attribute__((always_inline)) {
        const int nl = wn * WTN + j * 32 + 8 * g + 4 * kb;  // feature within the tile
        const float4 sw4 = *reinterpret_cast<const float4 *>(c_sw + nl);
        sw[0] = sw4.x * kUnscale; sw[1] = sw4.y * kUnscale; sw[2] = sw4.z * kUnscale; sw[3] = sw4.w * kUnscale;
        const uint4 b4 = p.bias ? *reinterpret_cast<const uint4 *>(c_bias + 4 * nl) : make_uint4(0, 0, 0, 0);
        const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) bs[r] = __uint_as_float(p.bias_bf16 ? bw[r] << 16 : bw[r]);
        if constexpr (ASYM) {
            const uint4 z4 = *reinterpret_cast<const uint4 *>(c_zp + 4 * nl);
            zc[0] = (8 - (int)z4.x) << SHIFT; zc[1] = (8 - (int)z4.y) << SHIFT;
            zc[2] = (8 - (int)z4.z) << SHIFT; zc[3] = (8 - (int)z4.w) << SHIFT;
        } else {
            zc[0] = zc[1] = zc[2] = zc[3] = 0;
        }
    };
    // Forms with registers to spare (bf16 without the low-rank branch, raw int32, and the
    // symmetric low-rank form with staged operands) read all 12 groups once, with one wait,
    // before the first token block: per-use reads put an LDS round trip, and its wait behind
    // the staging traffic, into every group of every block (4096 x 3072 -> 3072: 38 us per
    // launch with the constants held, 47 us without).  The other low-rank forms would spill, and
    // the paired launch's low-rank form spends those registers on the check-free store path
    // below instead (twenty double blocks: 15.2 -> 15.0 ms).
    constexpr bool HOLD = !epi_lr(EPI) || (epi_lr_lds(EPI) && !ASYM && !PAIR);
    float swv[HOLD ? FN : 1][4][4], bsv[HOLD ? FN : 1][4][4];
    int zcv[HOLD ? FN : 1][4][4];
    if constexpr (HOLD) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) consts_lds(j, g, swv[j][g], bsv[j][g], zcv[j][g]);
    }
    auto consts = [&](int j, int g, float (&sw)[4], float (&bs)[4], int (&zc)[4]) __attribute__((always_inline)) {
        if constexpr (HOLD) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sw[r] = swv[j][g][r];
                bs[r] = bsv[j][g][r];
                zc[r] = zcv[j][g][r];
            }
        } else {
            consts_lds(j, g, sw, bs, zc);
        }
    };
    if constexpr (EPI == kEpiI32) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t m = m0 + wm * WTM + i * 32 + lr;
            if (m >= p.M) continue;
            int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t n = n0 + wn * WTN + j * 32 + 8 * g + 4 * kb;
                    float sw[4], bs[4];
                    int zc[4];
                    consts(j, g, sw, bs, zc);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < p.N) Y[n + r] = (acc[j][i][4 * g + r] + (ASYM ? zc[r] * rsv[i] : 0)) >> SHIFT;
                }
        }
        return;
    }
    uint8_t *stg = smem + ((nk + 1) % STAGES) * L::STAGE + wave * 32 * SROW;
    uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y);
    const bool full_n = (p.N & 7) == 0;  // 16-byte aligned rows
    // Tiles inside the output with 16-byte aligned rows take a path without per-store checks:
    // each lane's 6 chunk offsets (row * N + column, 32-bit) are computed once per tile in a
    // single linear, and at each store in the paired launch (fewer registers).
    constexpr int CPR = WTN * 2 / 16;      // 16-byte chunks per staged row
    constexpr int NCH = 32 * CPR / 64;     // stores per lane and block
    const bool tile_in = full_n && m0 + BM <= p.M && n0 + BN <= p.N && p.N < (1 << 26);
    uint32_t soff[PAIR ? 1 : NCH];
    if constexpr (!PAIR) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int c = lane + 64 * k;
            soff[k] = (uint32_t)(c / CPR) * (uint32_t)p.N + (uint32_t)(c % CPR) * 8;
        }
    }
    // stores of a staged block: 32 rows x 12 chunks of 16 bytes; LDS operations of one wave
    // complete in order, so the reads see this block's writes and the next block's writes
    // follow these reads
    auto store_block = [&](int64_t mrow0) __attribute__((always_inline)) {
        if (tile_in) {
            uint16_t *yb = Y + mrow0 * p.N + n0 + wn * WTN;
            // all of the block's staged chunks are read before the first store, so the stores
            // wait for one LDS round trip instead of one each
            u32x4 v[NCH];
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const int c = lane + 64 * k;
                v[k] = *reinterpret_cast<const u32x4 *>(stg + (c / CPR) * SROW + (c % CPR) * 16);
            }
#pragma unroll
            for (int k = 0; k < NCH; ++k) {  // streaming stores: the output is not read again here
                const int c = lane + 64 * k;
                const uint32_t off = PAIR ? (uint32_t)(c / CPR) * (uint32_t)p.N + (uint32_t)(c % CPR) * 8 : soff[PAIR ? 0 : k];
                __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4 *>(yb + off));
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int c = lane + 64 * k;
            const int row = c / CPR, ch = c % CPR;
            const int64_t m = mrow0 + row, n = n0 + wn * WTN + ch * 8;
            const uint4 v = *reinterpret_cast<const uint4 *>(stg + row * SROW + ch * 16);
            if (m >= p.M || n >= p.N) continue;
            if (full_n && n + 7 < p.N) {
                // streaming store: the output is not read again by this kernel
                __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(Y + m * p.N + n));
            } else {
                const uint16_t *h = reinterpret_cast<const uint16_t *>(&v);
                for (int r = 0; r < 8 && n + r < p.N; ++r) Y[m * p.N + n + r] = h[r];
            }
        }
    };
    // a block's outputs as bf16 into this wave's staging rows (y: 4 consecutive features of
    // token lr per register group g)
    auto stage_bf16 = [&](int j, const float (&y)[16]) __attribute__((always_inline)) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
        typedef float fl2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const fl2 f01 = {y[4 * g], y[4 * g + 1]}, f23 = {y[4 * g + 2], y[4 * g + 3]};
            const bf2 h0 = __builtin_convertvector(f01, bf2);
            const bf2 h1 = __builtin_convertvector(f23, bf2);
            *reinterpret_cast<uint2 *>(stg + lr * SROW + (j * 32 + 8 * g + 4 * kb) * 2) =
                make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
        }
    };

    if constexpr (epi_lr_lds(EPI)) {
        // Low-rank branch from LDS: lr[n][m] = sum_q l2[q][n] t[m][q] on the bf16 MFMA with l2
        // transposed as the A operand (rows = features) and t as the B operand (columns =
        // tokens), so the product lands in the accumulators' 32x32 layout; it is accumulated
        // onto the dequantized output (the MFMA's C operand).  t (f32) goes in as a bf16 high
        // part plus a bf16 remainder (about 16 significant bits per product); l2 is bf16.
        constexpr int LRK = epi_lrk(EPI);
        const int lrr = p.lr_r;
        if (nk < 3) issue_t();
        // l2 [q][BN] -> l2T [BN][RP] (ranks past r zero), by all waves, while t lands
        const uint16_t *l2s = reinterpret_cast<const uint16_t *>(smem + L::LDS_BYTES);
        uint8_t *l2t = LL::L2T_IN_SLOT ? smem + ((nk + 1) % STAGES) * L::STAGE + STG_BYTES : smem + LL::L2T_DED;
        for (int e = tid; e < BN * (LL::RP / 8); e += kThreads) {
            const int n = e % BN, q8 = e / BN;
            uint32_t h[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) h[u] = 8 * q8 + u < lrr ? l2s[(8 * q8 + u) * BN + n] : 0u;
            *reinterpret_cast<uint4 *>(l2t + n * LL::L2T_PITCH + 16 * q8) =
                make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
        }
        wait_vmcnt<0>();  // this wave's t loads (no stores are in flight yet)
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        const uint8_t *ts = smem + (LL::T_IN_SLOT ? (nk % STAGES) * L::STAGE : LL::T_DED);
        bf8 la[FN][LRK];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int ks = 0; ks < LRK; ++ks)
                la[j][ks] = *reinterpret_cast<const bf8 *>(l2t + (wn * WTN + j * 32 + lr) * LL::L2T_PITCH +
                                                           (16 * ks + 8 * kb) * 2);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WTM + i * 32 + lr;
            bf8 th[LRK], tl[LRK];
#pragma unroll
            for (int ks = 0; ks < LRK; ++ks) {
                const uint8_t *tp = ts + row * LL::T_PITCH + (16 * ks + 8 * kb) * 4;
                const float4 u = *reinterpret_cast<const float4 *>(tp);
                const float4 w = *reinterpret_cast<const float4 *>(tp + 16);
                const fl8 tv = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
                th[ks] = __builtin_convertvector(tv, bf8);
                tl[ks] = __builtin_convertvector(tv - __builtin_convertvector(th[ks], fl8), bf8);
            }
            fl16 y[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float sw[4], bs[4];
                    int zc[4];
                    consts(j, g, sw, bs, zc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int a = acc[j][i][4 * g + r] + (ASYM ? zc[r] * rsv[i] : 0);
                        y[j][4 * g + r] = fmaf((float)a, sxv[i] * sw[r], bs[r]);
                    }
                }
#pragma unroll
            for (int ks = 0; ks < LRK; ++ks)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    y[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[j][ks], th[ks], y[j], 0, 0, 0);
                    y[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[j][ks], tl[ks], y[j], 0, 0, 0);
                }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                float yv[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) yv[v] = y[j][v];
                stage_bf16(j, yv);
            }
            store_block(m0 + wm * WTM + i * 32);
        }
        return;
    }

    // Low-rank branch on the bf16 MFMA: lr[n][m] = sum_q l2[q][n] t[m][q] comes out in the
    // accumulators' 32x32 layout when l2 transposed is the A operand (rows = features) and t
    // the B operand (columns = tokens).  Each lane holds the same 8 consecutive ranks q of
    // both operands (k-steps of 16, ranks past r zero).  t (f32) goes in as a bf16 high part
    // plus a bf16 remainder, so its products keep about 16 significant bits; l2 is bf16.
    constexpr int LRK = epi_lrk(EPI);
    const int lrr = epi_lr(EPI) ? p.lr_r : 0;
    const uint16_t *l2t = reinterpret_cast<const uint16_t *>(smem + L::LDS_BYTES);
    // t of token block i (8 consecutive ranks per k-step per lane), as raw floats: each block's
    // loads are issued before the previous block's output stores, since a wait for a load
    // issued after stores (vmcnt counts both) would also wait for those stores to drain.  One
    // block at a time keeps the epilogue's registers low; the scheduling barriers keep the
    // unrolled blocks from overlapping (the register ceiling would otherwise push the main
    // loop's values into AGPRs).
    fl8 tv[LRK];
    auto load_t = [&](int i) __attribute__((always_inline)) {
        const float *tr = p.lr_t + min<int64_t>(m0 + wm * WTM + i * 32 + lr, p.M - 1) * p.lr_ldt;
#pragma unroll
        for (int ks = 0; ks < LRK; ++ks) {
            const int q0 = 16 * ks + 8 * kb;
            // 16-byte aligned rows: whole quads valid or not
            if ((lrr & 3) == 0 && (p.lr_ldt & 3) == 0 && ((uintptr_t)p.lr_t & 15) == 0) {
                const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                const float4 u = q0 < lrr ? *reinterpret_cast<const float4 *>(tr + q0) : z;
                const float4 w = q0 + 4 < lrr ? *reinterpret_cast<const float4 *>(tr + q0 + 4) : z;
                tv[ks] = fl8{u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) tv[ks][e] = q0 + e < lrr ? tr[q0 + e] : 0.0f;
            }
        }
    };
    if constexpr (epi_lr(EPI)) load_t(0);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if constexpr (epi_lr(EPI)) __builtin_amdgcn_sched_barrier(0);
        const int64_t mrow0 = m0 + wm * WTM + i * 32;
        bf8 th[LRK], tl[LRK];
        if constexpr (epi_lr(EPI)) {
#pragma unroll
            for (int ks = 0; ks < LRK; ++ks) {
                th[ks] = __builtin_convertvector(tv[ks], bf8);
                tl[ks] = __builtin_convertvector(tv[ks] - __builtin_convertvector(th[ks], fl8), bf8);
            }
            if (i + 1 < FM) load_t(i + 1);  // before this block's stores
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (epi_lr(EPI)) __builtin_amdgcn_sched_barrier(0);
            fl16 lacc = {};
            const int nl = wn * WTN + j * 32 + lr;  // feature within the tile
            if constexpr (epi_lr(EPI)) {
#pragma unroll
                for (int ks = 0; ks < LRK; ++ks) {
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int q = 16 * ks + 8 * kb + e;
                        h[e] = q < lrr ? l2t[q * BN + nl] : 0u;
                    }
                    const bf8 la = __builtin_bit_cast(bf8, make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16,
                                                                      h[4] | h[5] << 16, h[6] | h[7] << 16));
                    lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la, th[ks], lacc, 0, 0, 0);
                    lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la, tl[ks], lacc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float y[4], sw[4], bs[4];
                int zc[4];
                consts(j, g, sw, bs, zc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int a = acc[j][i][4 * g + r] + (ASYM ? zc[r] * rsv[i] : 0);
                    y[r] = fmaf((float)a, sxv[i] * sw[r], bs[r]);
                    if constexpr (epi_lr(EPI)) y[r] += lacc[4 * g + r];
                }
                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                typedef float fl2 __attribute__((ext_vector_type(2)));
                const fl2 f01 = {y[0], y[1]}, f23 = {y[2], y[3]};
                const bf2 h0 = __builtin_convertvector(f01, bf2);
                const bf2 h1 = __builtin_convertvector(f23, bf2);
                *reinterpret_cast<uint2 *>(stg + lr * SROW + (j * 32 + 8 * g + 4 * kb) * 2) =
                    make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
            }
        }
        store_block(mrow0);
    }
}

// ---- split tail: the last partial round of tiles (fewer tiles than compute units) runs as
// S K ranges per tile, and this kernel sums the S int32 partials (exact, fixed order) and
// applies the epilogue of k_gemm (the same arithmetic; the low-rank term on the VALU).
// One thread per 4 consecutive outputs of a tile.
template <int ABITS, bool ASYM>
__global__ void __launch_bounds__(256) k_gemm_tail(LinearArgs p, int tiles_m, int tiles_n, TileRange tr) {
    constexpr int SHIFT = ABITS == 8 ? 4 : 8;
    constexpr float kUnscale = ABITS == 8 ? 1.0f / 16 : 1.0f / 256;
    constexpr int PER_TILE = BM * BN / 4 / 256;  // workgroups per tile
    constexpr int TROWS = 8;                     // tile rows one workgroup touches (at most 7)
    // low-rank operands of the workgroup: the tile's l2 columns [r, BN] and its t rows
    __shared__ __attribute__((aligned(16))) uint16_t l2s[64 * BN];
    __shared__ float ts[TROWS * 64];
    const int t = (int)blockIdx.x / PER_TILE;
    const int idx = ((int)blockIdx.x % PER_TILE) * 256 + (int)threadIdx.x;
    const int ml = idx / (BN / 4), nl = 4 * (idx % (BN / 4));
    const int ml0 = ((int)blockIdx.x % PER_TILE) * 256 / (BN / 4);
    int tm, tn;
    tile_coords(tr.base + t, tiles_m, tiles_n, tm, tn);
    const int64_t m = (int64_t)tm * BM + ml, n = (int64_t)tn * BN + nl;
    const bool lr = p.lr_t && !p.y_i32;
    if (lr) {
        const int64_t n0 = (int64_t)tn * BN;
        const int r = p.lr_r;
        if ((p.N & 7) == 0 && ((uintptr_t)p.lr_l2 & 15) == 0) {  // 16-byte rows; chunks all in [0, N) or all past it
            for (int c = threadIdx.x; c < r * (BN / 8); c += 256) {
                const int q = c / (BN / 8), cn = 8 * (c % (BN / 8));
                const int64_t col = min<int64_t>(n0 + cn, p.N - 8);  // past N: unused columns
                *reinterpret_cast<uint4 *>(l2s + q * BN + cn) =
                    *reinterpret_cast<const uint4 *>(p.lr_l2 + (int64_t)q * p.N + col);
            }
        } else {
            for (int c = threadIdx.x; c < r * BN; c += 256)
                l2s[c] = p.lr_l2[(int64_t)(c / BN) * p.N + min<int64_t>(n0 + c % BN, p.N - 1)];
        }
        for (int c = threadIdx.x; c < TROWS * r; c += 256) {
            const int row = c / r, q = c % r;
            const int64_t mm = min<int64_t>((int64_t)tm * BM + ml0 + row, p.M - 1);
            ts[row * 64 + q] = p.lr_t[mm * p.lr_ldt + q];
        }
        __syncthreads();
    }
    if (m >= p.M || n >= p.N) return;
    const int32_t *P = tr.part + (int64_t)t * tr.kparts * (BM * BN) + ml * BN + nl;
    int4 s = *reinterpret_cast<const int4 *>(P);
    for (int q = 1; q < tr.kparts; ++q) {
        const int4 v = *reinterpret_cast<const int4 *>(P + (int64_t)q * (BM * BN));
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    int a[4] = {s.x, s.y, s.z, s.w};
    const int nv = (int)min<int64_t>(4, p.N - n);
    if constexpr (ASYM) {
        const int rs = p.rowsum[m];
        for (int r = 0; r < nv; ++r) a[r] += ((8 - (int)p.zp[n + r]) << SHIFT) * rs;
    }
    if (p.y_i32) {
        int32_t *Y = reinterpret_cast<int32_t *>(p.Y) + m * p.N + n;
        for (int r = 0; r < nv; ++r) Y[r] = a[r] >> SHIFT;
        return;
    }
    // low-rank term of the 4 outputs from the staged operands (columns past N hold copies,
    // never stored)
    float lw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (lr) {
        const float *tq = ts + (ml - ml0) * 64;
#pragma unroll 8
        for (int q = 0; q < p.lr_r; ++q) {
            const uint2 w = *reinterpret_cast<const uint2 *>(l2s + q * BN + nl);
            lw[0] = fmaf(tq[q], bf16_lo(w.x), lw[0]);
            lw[1] = fmaf(tq[q], bf16_hi(w.x), lw[1]);
            lw[2] = fmaf(tq[q], bf16_lo(w.y), lw[2]);
            lw[3] = fmaf(tq[q], bf16_hi(w.y), lw[3]);
        }
    }
    const float sx = p.sx[m];
    uint32_t h[4] = {0, 0, 0, 0};
    for (int r = 0; r < nv; ++r) {
        const float sw = p.sw[n + r] * kUnscale;
        const float b = !p.bias ? 0.0f
                        : p.bias_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[n + r])
                                      : reinterpret_cast<const float *>(p.bias)[n + r];
        h[r] = f32_to_bf16(fmaf((float)a[r], sx * sw, b) + lw[r]);
    }
    uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y) + m * p.N + n;
    if (nv == 4 && (p.N & 3) == 0) {
        *reinterpret_cast<uint2 *>(Y) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    } else {
        for (int r = 0; r < nv; ++r) Y[r] = (uint16_t)h[r];
    }
}

// Tiles in whole rounds over the compute units (tmain) and the tail split into S K ranges,
// S the largest of 8 .. 4 that divides the stage count with ttail * S <= units; S = 1: no
// split (at most one round, K % BK != 0, or a tail of more than a quarter round: there the
// partial sums' extra traffic and the summing launch cost more than the idle units; measured
// on the 20-block workload: a tail of 32 tiles gains, tails of 96 and 128 lose).
struct TailPlan {
    int tmain, ttail, S;
};

TailPlan tail_plan(int64_t M, int64_t N, int64_t K) {
    const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    TailPlan pl{tiles, 0, 1};
    if (K % BK || tiles <= ncu) return pl;
    const int tmain = tiles / ncu * ncu, ttail = tiles - tmain, nk = (int)(K / BK);
    if (ttail == 0) return pl;
    for (int S = std::min(8, ncu / ttail); S >= 4; --S) {
        if (nk % S == 0) return TailPlan{tmain, ttail, S};
    }
    return pl;
}

GemmPair single(const LinearArgs &a) {
    const int tm = (int)((a.M + BM - 1) / BM), tn = (int)((a.N + BN - 1) / BN);
    return GemmPair{{a, a}, {tm, tm}, {tn, tn}, tm * tn};
}

bool l2_rows_aligned(const LinearArgs &a) { return a.N % 8 == 0 && ((uintptr_t)a.lr_l2 & 15) == 0; }

// The epilogue form of a linear (the k_gemm instantiation its tiles need)
int epi_kind(const LinearArgs &a) {
    if (a.y_i32) return kEpiI32;
    if (!a.lr_t) return kEpiBf16;
    const bool staged = l2_rows_aligned(a) && a.lr_r % 4 == 0 && a.lr_ldt % 4 == 0 && ((uintptr_t)a.lr_t & 15) == 0;
    if (staged && a.lr_r <= 16) return kEpiLowRank16;
    if (staged && a.lr_r <= 32) return kEpiLowRank32;
    return kEpiLowRank;
}

template <int ABITS, bool ASYM, bool KTAIL, int EPI, bool PAIR = false>
hipError_t launch_t(const GemmPair &gp, const TileRange &tr, unsigned grid, hipStream_t st) {
    // LDS: ring + constants, plus the low-rank l2 tile (whole 1 KB direct-load blocks of
    // 24 * r 16-byte chunks, at most 24 KB for r <= 64), plus the staged t and l2T where they
    // do not fit in free ring slots
    constexpr size_t base = Lay<ABITS>::LDS_BYTES, maxl2 = 24 * 1024;
    constexpr size_t maxlds = epi_lr_lds(EPI) ? (size_t)LrLay<ABITS, epi_lds_k(EPI)>::LDS_TOTAL : base + maxl2;
    static_assert(maxlds <= 160 * 1024, "LDS budget");
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm<ABITS, ASYM, KTAIL, EPI, PAIR>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)maxlds);
    if (attr != hipSuccess) return attr;
    const LinearArgs &a = gp.p[0], &b = gp.p[1];
    const int l2_dma = l2_rows_aligned(a) && l2_rows_aligned(b);
    const int rmax = std::max(a.lr_r, b.lr_r);
    const size_t lds = epi_lr_lds(EPI) ? maxlds : base + (epi_lr(EPI) ? (size_t)((24 * rmax + 63) / 64) * 1024 : 0);
    hipLaunchKernelGGL((k_gemm<ABITS, ASYM, KTAIL, EPI, PAIR>), dim3(grid), dim3(kThreads), lds, st, gp, l2_dma, tr);
    return hipGetLastError();
}

template <int ABITS, bool ASYM, bool KTAIL, bool PAIR = false>
hipError_t launch_epi(const GemmPair &gp, const TileRange &tr, hipStream_t st) {
    const unsigned grid = (unsigned)tr.count;
    switch (epi_kind(gp.p[0])) {
        case kEpiI32: return launch_t<ABITS, ASYM, KTAIL, kEpiI32, PAIR>(gp, tr, grid, st);
        case kEpiLowRank16: return launch_t<ABITS, ASYM, KTAIL, kEpiLowRank16, PAIR>(gp, tr, grid, st);
        case kEpiLowRank32: return launch_t<ABITS, ASYM, KTAIL, kEpiLowRank32, PAIR>(gp, tr, grid, st);
        case kEpiLowRank: return launch_t<ABITS, ASYM, KTAIL, kEpiLowRank, PAIR>(gp, tr, grid, st);
        default: return launch_t<ABITS, ASYM, KTAIL, kEpiBf16, PAIR>(gp, tr, grid, st);
    }
}

template <int ABITS, bool ASYM>
hipError_t launch_k(const LinearArgs &a, void *ws, size_t ws_bytes, hipStream_t st) {
    const TailPlan pl = tail_plan(a.M, a.N, a.K);
    const int tiles = pl.tmain + pl.ttail;
    const size_t need = (size_t)pl.ttail * pl.S * BM * BN * sizeof(int32_t);
    const TileRange all{0, tiles, 1, nullptr};
    const GemmPair gp = single(a);
    if (a.K % BK) return launch_epi<ABITS, ASYM, true>(gp, all, st);
    if (pl.S < 2 || !ws || ws_bytes < need) return launch_epi<ABITS, ASYM, false>(gp, all, st);
    // whole rounds, then the tail's K ranges, then their sum and epilogue
    hipError_t e = launch_epi<ABITS, ASYM, false>(gp, TileRange{0, pl.tmain, 1, nullptr}, st);
    if (e != hipSuccess) return e;
    const TileRange tail{pl.tmain, pl.ttail, pl.S, static_cast<int32_t *>(ws)};
    e = launch_t<ABITS, ASYM, false, kEpiPartial>(gp, tail, (unsigned)(pl.ttail * pl.S), st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_tail<ABITS, ASYM>), dim3((unsigned)(pl.ttail * (BM * BN / 4 / 256))), dim3(256), 0, st,
                       a, gp.tiles_m[0], gp.tiles_n[0], tail);
    return hipGetLastError();
}

template <int ABITS, bool ASYM>
hipError_t launch_pair_t(const LinearArgs &a, const LinearArgs &b, hipStream_t st) {
    GemmPair gp = single(a);
    const GemmPair gb = single(b);
    gp.p[1] = b;
    gp.tiles_m[1] = gb.tiles_m[0];
    gp.tiles_n[1] = gb.tiles_n[0];
    const TileRange all{0, gp.n0 + gb.n0, 1, nullptr};
    return a.K % BK ? launch_epi<ABITS, ASYM, true, true>(gp, all, st) : launch_epi<ABITS, ASYM, false, true>(gp, all, st);
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 64 || N <= 0 || K <= 0) return 0;
    const TailPlan pl = tail_plan(M, N, K);
    return pl.S > 1 ? (size_t)pl.ttail * pl.S * BM * BN * sizeof(int32_t) : 0;
}

bool gemm_pairable(const LinearArgs &a, const LinearArgs &b) {
    if (a.M <= 64 || a.M != b.M || a.K != b.K || !a.zp != !b.zp || a.y_i32 != b.y_i32) return false;
    if (epi_kind(a) != epi_kind(b)) return false;
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN + (b.N + BN - 1) / BN);
    return tiles < ((int64_t)1 << 31);
}

hipError_t launch_gemm_pair(const LinearArgs &a, const LinearArgs &b, int act_bits, hipStream_t st) {
    if (!gemm_pairable(a, b)) return hipErrorInvalidValue;
    if (act_bits == 8) return a.zp ? launch_pair_t<8, true>(a, b, st) : launch_pair_t<8, false>(a, b, st);
    return a.zp ? launch_pair_t<4, true>(a, b, st) : launch_pair_t<4, false>(a, b, st);
}

hipError_t launch_gemm(const LinearArgs &a, int act_bits, void *ws, size_t ws_bytes, hipStream_t st) {
    if (a.M == 0) return hipSuccess;
    if (act_bits == 8) return a.zp ? launch_k<8, true>(a, ws, ws_bytes, st) : launch_k<8, false>(a, ws, ws_bytes, st);
    return a.zp ? launch_k<4, true>(a, ws, ws_bytes, st) : launch_k<4, false>(a, ws, ws_bytes, st);
}

}  // namespace w4
