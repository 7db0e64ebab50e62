// Internal launchers of the gfx950 kernels (C++ linkage, not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

// Activation rotate + per-token quantize.  Returns hipSuccess or the launch error;
// returns hipErrorInvalidValue when K has no supported (C, T) split.
bool rotquant_supported(int64_t K, int g);
hipError_t launch_rotquant(const void *X, bool f32in, int64_t M, int64_t K, int g, int bits,
                           void *q, float *tok_scale, int32_t *tok_rowsum, hipStream_t st);

// Rotate + quantize bf16 X and t = X . l1^T (l1 bf16 [r, K], r <= 64; t rows ldt floats apart)
// in one pass; for g in {64, 256} and K in {1024, 2048, 3072, 4096} (rotquant_lr_fusable).
bool rotquant_lr_fusable(int64_t K, int g);
hipError_t launch_rotquant_lr(const void *X, int64_t M, int64_t K, int g, int bits, void *q, float *tok_scale,
                              int32_t *tok_rowsum, const void *l1, int r, float *t, int64_t ldt, hipStream_t st);

// Offline weight rotate + per-row quantize + nibble pack (g in {0 = none, 16, 64, 256, 1024,
// 4096}).
hipError_t launch_pack(const void *W, bool f32in, int64_t N, int64_t K, int g, bool asym,
                       uint8_t *packed, float *row_scale, uint8_t *zp, hipStream_t st);
// The same with symmetric codes and fp16 scales per (row, run of gw inputs) [N, K/gw];
// gw divides 4096 and K.
hipError_t launch_pack_grouped(const void *W, bool f32in, int64_t N, int64_t K, int g, int gw, uint8_t *packed,
                               uint16_t *group_scale, hipStream_t st);

struct LinearArgs {
    const uint8_t *A;      // activation codes: int8 [M, K] or packed int4 [M, K/2]
    const float *sx;       // [M]
    const int32_t *rowsum; // [M]
    const uint8_t *B;      // packed weights [N, K/2]
    const float *sw;       // [N]
    const uint8_t *zp;     // [N] or null (symmetric)
    const void *bias;      // [N] or null
    int bias_bf16;
    const float *lr_t;        // [M, lr_r] (row stride lr_ldt floats) or null
    const uint16_t *lr_l2;    // bf16 [lr_r, N]
    int lr_r;
    int64_t lr_ldt;
    void *Y;               // bf16 or int32 [M, N]
    int y_i32;
    int64_t M, N, K;
};

// Large-M path (M > 64).  With a workspace of gemm_workspace_bytes() bytes (0 when the tiles
// fill whole rounds of the compute units) the last partial round is split along K.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const LinearArgs &a, int act_bits, void *ws, size_t ws_bytes, hipStream_t st);
// Two large-M linears on the same activation codes as one launch (no K split), when they have
// the same M > 64, K, weight mode, output kind and epilogue form (gemm_pairable); each output
// equals launch_gemm's without a workspace bit for bit.  hipErrorInvalidValue otherwise.
bool gemm_pairable(const LinearArgs &a, const LinearArgs &b);
hipError_t launch_gemm_pair(const LinearArgs &a, const LinearArgs &b, int act_bits, hipStream_t st);
// Small-M path (M <= 64).  With a workspace of gemv_workspace_bytes() bytes (0 when none is
// needed) the K-split kernel runs; without one, the LDS-ring kernel.
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits);
hipError_t launch_gemv(const LinearArgs &a, int act_bits, void *ws, size_t ws_bytes, hipStream_t st);
// Fused rotate + quantize + small-M GEMM from bf16 X [M, K] (a.A, a.sx and a.rowsum unused),
// for the shapes gemv_fusable() accepts (one token); the result equals launch_rotquant +
// launch_gemv bit for bit.
bool gemv_fusable(int64_t M, int64_t N, int64_t K, int g, int act_bits, bool f32in);
hipError_t launch_gemv_fused(const LinearArgs &a, const void *X, int g, int act_bits, hipStream_t st);

// Grouped-scale format: signed codes [N, K/2] with fp16 scales [N, K/gw] (gw in 32, 64, 128,
// 256), against int8 / packed int4 activation codes with token scales (act_bits 8 / 4) or
// bf16 activations (act_bits 16).  K % 64 == 0 and K % gw == 0.  For M <= 64, a workspace of
// grouped_workspace_bytes() bytes splits K over several workgroups.
struct GroupedArgs {
    const void *A;            // int8 [M, K], packed int4 [M, K/2] or bf16 [M, K]
    const float *sx;          // [M] (act_bits 8 / 4)
    const uint8_t *B;         // [N, K/2]
    const uint16_t *gs;       // fp16 [N, K / gw]
    int gw;
    const void *bias;         // [N] or null
    int bias_bf16;
    const float *lr_t;        // [M, lr_r] (row stride lr_ldt floats) or null
    const uint16_t *lr_l2;    // bf16 [lr_r, N]
    int lr_r;
    int64_t lr_ldt;
    void *Y;                  // bf16 [M, N], or int32 (act_bits 8 / 4: sum_k q c, no scales)
    int y_i32;
    int64_t M, N, K;
};
size_t grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int gw);
hipError_t launch_gemm_grouped(const GroupedArgs &a, int act_bits, void *ws, size_t ws_bytes, hipStream_t st);

hipError_t launch_lowrank_down(const void *x, const void *l1, int64_t M, int64_t K, int r,
                               float *t, hipStream_t st, int64_t ldt = 0);

}  // namespace w4
