// Device helpers shared by the gfx950 kernels of the W4 linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// 1.5 * 2^52: adding it to a double |y| < 2^31 leaves rint(y) (ties to even, the default
// rounding mode) in the low 32 bits of the sum, as two's complement.
constexpr double kRoundMagic = 6755399441055744.0;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// One packed dword holds 8 signed nibbles (k .. k+7, low nibble = even k).  Placing each
// nibble in the high half of a byte gives the int8 value 16 * code, so no sign extension is
// needed: evens = codes k, k+2, k+4, k+6; odds = codes k+1, k+3, k+5, k+7.
__device__ __forceinline__ uint32_t nib_evens16(uint32_t d) { return (d << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_odds16(uint32_t d) { return d & 0xF0F0F0F0u; }

// Reorder 8 int8 codes (a0: k..k+3, a1: k+4..k+7) into the same even/odd order as above.
__device__ __forceinline__ uint32_t bytes_evens(uint32_t a0, uint32_t a1) {
    return __builtin_amdgcn_perm(a1, a0, 0x06040200u);
}
__device__ __forceinline__ uint32_t bytes_odds(uint32_t a0, uint32_t a1) {
    return __builtin_amdgcn_perm(a1, a0, 0x07050301u);
}

// Lane exchange inside a quad for a double (two 32-bit DPP moves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    int lo = __double2loint(x), hi = __double2hiint(x);
    lo = __builtin_amdgcn_mov_dpp(lo, CTRL, 0xF, 0xF, false);
    hi = __builtin_amdgcn_mov_dpp(hi, CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kRowMirror = 0x140;      // lane l of a 16-lane row takes lane 15 - l
constexpr int kRowHalfMirror = 0x141;  // lane l of an 8-lane half row takes lane 7 - l

// Wave-wide max of non-negative doubles and sum of ints, in registers: the two quad exchanges
// and the half-row and row mirrors leave each 16-lane row's result in every lane of the row
// (every step pairs lanes whose partial results cover disjoint lane sets), and four readlanes
// combine the rows.  Every lane of the wave must be active.  A max is exact in any order and
// an int sum is exact, so the result equals the butterfly over __shfl_xor, without its chain
// of LDS round trips.
__device__ __forceinline__ double wave_max_f64(double x) {
    x = fmax(x, dpp_f64<kQuadXor1>(x));
    x = fmax(x, dpp_f64<kQuadXor2>(x));
    x = fmax(x, dpp_f64<kRowHalfMirror>(x));
    x = fmax(x, dpp_f64<kRowMirror>(x));
    const int lo = __double2loint(x), hi = __double2hiint(x);
    double r = __hiloint2double(__builtin_amdgcn_readlane(hi, 0), __builtin_amdgcn_readlane(lo, 0));
    r = fmax(r, __hiloint2double(__builtin_amdgcn_readlane(hi, 16), __builtin_amdgcn_readlane(lo, 16)));
    r = fmax(r, __hiloint2double(__builtin_amdgcn_readlane(hi, 32), __builtin_amdgcn_readlane(lo, 32)));
    return fmax(r, __hiloint2double(__builtin_amdgcn_readlane(hi, 48), __builtin_amdgcn_readlane(lo, 48)));
}
__device__ __forceinline__ int wave_sum_i32(int x) {
    x += __builtin_amdgcn_mov_dpp(x, kQuadXor1, 0xF, 0xF, false);
    x += __builtin_amdgcn_mov_dpp(x, kQuadXor2, 0xF, 0xF, false);
    x += __builtin_amdgcn_mov_dpp(x, kRowHalfMirror, 0xF, 0xF, false);
    x += __builtin_amdgcn_mov_dpp(x, kRowMirror, 0xF, 0xF, false);
    return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
           __builtin_amdgcn_readlane(x, 48);
}

// Lane exchange for a double through ds_swizzle (bit-mask mode), for lanes 4 and 8 apart.
template <int PAT>
__device__ __forceinline__ double swz_f64(double x) {
    const int lo = __builtin_amdgcn_ds_swizzle(__double2loint(x), PAT);
    const int hi = __builtin_amdgcn_ds_swizzle(__double2hiint(x), PAT);
    return __hiloint2double(hi, lo);
}
constexpr int kSwzXor4 = 0x101F;  // and 0x1f, or 0, xor 4
constexpr int kSwzXor8 = 0x201F;  // xor 8

// In-register Walsh-Hadamard butterflies over 16 values (Sylvester order, unnormalised):
// after the call v[i] = sum_j (-1)^popcount(i & j) * v_in[j].
__device__ __forceinline__ void fwht16(double (&v)[16]) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                double a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}


// Global -> LDS loads (16 or 4 bytes per lane), addressed as a wave-uniform 64-bit base
// (SGPRs) plus a per-lane 32-bit byte offset: lane l's bytes land at lds_base + size * l
// (lds_base is wave-uniform and goes through M0; one wait state separates the M0 write from
// the load that reads it).  Issued through inline asm so that the compiler does not add its
// own conservative vmcnt(0) waits in front of every LDS read of the other stages: the kernel
// waits for its own loads explicitly (s_waitcnt vmcnt(n) + s_barrier).  The instruction
// writes no VGPR, so no register is left pending when the asm returns.  M0 is written inside
// the asm; no other code in these kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void gl_lds16_so(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);  // keep both in SGPRs
    sbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32)) << 32) |
            (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sbase);  // (no sign extension)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(lds_base)
                 : "memory", "m0");
}
__device__ __forceinline__ void gl_lds4_so(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);  // keep both in SGPRs
    sbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32)) << 32) |
            (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sbase);  // (no sign extension)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(lds_base)
                 : "memory", "m0");
}
// 2- and 1-byte forms: each lane's value lands zero-extended in its own dword at
// lds_base + 4 * l.
__device__ __forceinline__ void gl_lds2_so(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);  // keep both in SGPRs
    sbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32)) << 32) |
            (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sbase);  // (no sign extension)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ushort %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(lds_base)
                 : "memory", "m0");
}
__device__ __forceinline__ void gl_lds1_so(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);  // keep both in SGPRs
    sbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32)) << 32) |
            (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sbase);  // (no sign extension)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(lds_base)
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
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wait until at most r * PER + EXTRA of this wave's loads are in flight (0 <= r <= RMAX).
template <int PER, int RMAX, int EXTRA = 0>
__device__ __forceinline__ void wait_rem(int r) {
    if constexpr (RMAX == 0) {
        wait_vmcnt<EXTRA>();
    } else {
        if (r >= RMAX) wait_vmcnt<(RMAX * PER + EXTRA < 63 ? RMAX * PER + EXTRA : 63)>();
        else wait_rem<PER, RMAX - 1, EXTRA>(r);
    }
}

// Unpack one packed dword (codes k .. k+7) to int8 values 16 * code in natural k order.
__device__ __forceinline__ void unpack_nat(uint32_t d, uint32_t &lo, uint32_t &hi) {
    const uint32_t e = nib_evens16(d), o = nib_odds16(d);
    lo = __builtin_amdgcn_perm(o, e, 0x05010400u);  // codes k, k+1, k+2, k+3
    hi = __builtin_amdgcn_perm(o, e, 0x07030602u);  // codes k+4 .. k+7
}

// 16 packed codes (two dwords) -> int8 values 16 * code in even/odd order.
__device__ __forceinline__ v4i evod(uint32_t d0, uint32_t d1) {
    return v4i{(int)nib_evens16(d0), (int)nib_odds16(d0), (int)nib_evens16(d1), (int)nib_odds16(d1)};
}

}  // namespace w4
