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

}  // namespace w4
