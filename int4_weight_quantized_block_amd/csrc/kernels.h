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

// Offline weight rotate + per-row quantize + nibble pack.
hipError_t launch_pack(const void *W, bool f32in, int64_t N, int64_t K, int g, bool asym,
                       uint8_t *packed, float *row_scale, uint8_t *zp, hipStream_t st);

struct LinearArgs {
    const uint8_t *A;      // activation codes: int8 [M, K] or packed int4 [M, K/2]
    const float *sx;       // [M]
    const int32_t *rowsum; // [M]
    const uint8_t *B;      // packed weights [N, K/2]
    const float *sw;       // [N]
    const uint8_t *zp;     // [N] or null (symmetric)
    const void *bias;      // [N] or null
    int bias_bf16;
    const float *lr_t;        // [M, lr_r] or null
    const uint16_t *lr_l2;    // bf16 [lr_r, N]
    int lr_r;
    void *Y;               // bf16 or int32 [M, N]
    int y_i32;
    int64_t M, N, K;
};

// Large-M path (M > 64).  With a workspace of gemm_workspace_bytes() bytes (0 when the tiles
// fill whole rounds of the compute units) the last partial round is split along K.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const LinearArgs &a, int act_bits, void *ws, size_t ws_bytes, hipStream_t st);
// Small-M path (M <= 64).  With a workspace of gemv_workspace_bytes() bytes (0 when none is
// needed) the K-split kernel runs; without one, the LDS-ring kernel.
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits);
hipError_t launch_gemv(const LinearArgs &a, int act_bits, void *ws, size_t ws_bytes, hipStream_t st);
// Fused rotate + quantize + small-M GEMM from bf16 X [M, K] (a.A, a.sx and a.rowsum unused),
// for the shapes gemv_fusable() accepts (one token); the result equals launch_rotquant +
// launch_gemv bit for bit.
bool gemv_fusable(int64_t M, int64_t N, int64_t K, int g, int act_bits, bool f32in);
hipError_t launch_gemv_fused(const LinearArgs &a, const void *X, int g, int act_bits, hipStream_t st);

// Measurement probe: blocks workgroups of 4 waves, each wave iters rounds of 4 int8 MFMAs.
hipError_t launch_mfma_rate(int64_t blocks, int iters, bool random_operands, int32_t *sink, hipStream_t st);

hipError_t launch_lowrank_down(const void *x, const void *l1, int64_t M, int64_t K, int r,
                               float *t, hipStream_t st);

}  // namespace w4
