/* w4.h - C ABI of the MI355X (gfx950) ConvRot INT4 weight-quantized linear layer.
 *
 * The layer (ComfyUI-INT-Crush README, "Inference / INT4" and "Forward Pass";
 * stable-diffusion.cpp PR #2010 "feat: packed int4 convrot model loading and
 * dispatch", "Summary"):
 *
 *   X' = X . blockdiag(H_g / sqrt(g))            block Hadamard rotation along K
 *   q  = rint(X' / s_x),  s_x = fp32(max|X'| / qmax) per token      (qmax 127 or 7)
 *   W' = W . blockdiag(H_g / sqrt(g)),  c = packed int4 codes per output row
 *   acc[m, n] = sum_k q[m, k] * (c[n, k] - z[n])                     int32, exact
 *   Y  = bf16( acc * s_x[m] * s_w[n] + (X . L1) . L2 + bias[n] )
 *
 * H_g is the Sylvester-ordered Hadamard matrix, g in {16, 64, 256, 1024, 4096}, groups
 * are contiguous blocks of g along K.  rint is round-half-to-even.  Two 4-bit codes
 * per byte along K, low nibble = even k.  Symmetric weights: signed codes in
 * [-8, 7] (two's complement nibbles), z = 0, s_w = fp32(max|W'| / 7).
 * Asymmetric weights: unsigned codes in [0, 15] with a zero point z[n] in [0, 15],
 * s_w = fp32((max(W', 0) - min(W', 0)) / 15), z = clamp(-rint(min(W', 0) / s_w)).
 * Codes are rounded first and the zero point added after.
 *
 * Conventions for every call:
 *  - Every pointer is a DEVICE pointer unless stated otherwise; the caller owns
 *    and allocates every buffer.  The library never allocates, never frees and
 *    never synchronizes; work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream) and is complete when that stream is.
 *  - Matrices are row-major and dense (row stride = number of columns).
 *  - Device pointers must be 16-byte aligned.
 *  - Return value: W4_OK (0) or a positive W4_ERR_* code.  Arguments are checked
 *    before anything is launched, so an error leaves every output untouched
 *    (except W4_ERR_HIP, a launch failure).  w4_last_error() gives a message
 *    for the calling thread's last error.  Faults during execution surface at
 *    the caller's next synchronization, as for any HIP work.
 *  - M == 0 is a valid no-op.  N >= 1 and K >= g are required.
 *  - Thread-safe: no global state besides the per-thread error message and the
 *    per-device scratch array of w4_linear_noalloc (see there).
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define W4_OK 0
#define W4_ERR_INVALID_ARG 1 /* null pointer, unknown enum value */
#define W4_ERR_SHAPE 2       /* negative or zero size, K % g != 0, K out of range */
#define W4_ERR_UNSUPPORTED 3 /* g, gw or act_bits not supported, K not tileable */
#define W4_ERR_ALIGN 4       /* a device pointer is not 16-byte aligned */
#define W4_ERR_HIP 5         /* a HIP launch failed (message from hipGetErrorString) */
#define W4_ERR_WORKSPACE 6   /* workspace missing or smaller than w4_workspace_bytes() */

/* element types of floating-point inputs */
#define W4_F32 0
#define W4_BF16 1

/* weight quantization modes */
#define W4_SYM 0  /* signed codes, no zero point */
#define W4_ASYM 1 /* unsigned codes with a per-row zero point */

/* output kinds of the linear calls */
#define W4_OUT_BF16 0 /* Y bf16 [M, N]: the dequantized layer output */
#define W4_OUT_I32 1  /* Y int32 [M, N]: the raw exact accumulator acc[m, n] (no epilogue) */

/* Largest K the library accepts.  The int32 accumulation of 16 * q * c would stay exact up to
 * K = 65536; the activation kernel keeps a whole token row in registers and stops at 32768. */
#define W4_MAX_K 32768

/* Low-rank side branch added before the bias: lr = (X . L1) . L2 with the UNROTATED
 * activations (ComfyUI-INT-Crush README, "Forward Pass" step 6 and "LoRA").
 *  x  : bf16 [M, K] unrotated layer input; read only when t == NULL
 *  l1 : bf16 [r, K], rank-major: row q holds the q-th down-projection vector over the K
 *       inputs (L1 transposed; a LoRA down weight is stored this way); read only when
 *       t == NULL
 *  t  : optional f32 [M, r] = x . L1 computed earlier (e.g. by w4_lowrank_down, and
 *       shared by linears that read the same input); NULL -> computed into the workspace
 *  l2 : bf16 [r, N], rank-major: row q holds the q-th up-projection vector over the N
 *       outputs
 *  r  : rank, 1 <= r <= 64
 *  ldt: row stride of a supplied t in floats (0 means r; otherwise >= r).  With a stride, t
 *       can be a column range of a wider t computed once for several linears that read the
 *       same input (w4_rotate_quant_act_lowrank with their L1 factors stacked); a multiple of
 *       4 (and a 16-byte aligned t) keeps the kernels' vector loads. */
typedef struct w4_lowrank {
    const void *x;
    const void *l1;
    const float *t;
    const void *l2;
    int r;
    int ldt;
} w4_lowrank;

/* w4_pack_weights - offline weight step: rotate every row of W along K in groups of g,
 * quantize it per row to int4 and pack two codes per byte.
 * (ComfyUI-INT-Crush README, "Weight Format" and "Workflow" step 1 (converter);
 *  stable-diffusion.cpp PR #2010, "Summary": packed nibbles + row scales, and the
 *  discussion's shape report: the packed input dimension is K / 2.)
 *  W        : [N, K] of w_dtype (W4_F32 or W4_BF16)
 *  wmode    : W4_SYM or W4_ASYM
 *  packed   : out uint8 [N, K/2]
 *  row_scale: out f32 [N]
 *  zp       : out uint8 [N] zero points; required for W4_ASYM, must be NULL for W4_SYM
 * Requires K % g == 0, g in {16, 64, 256, 1024, 4096}, K <= W4_MAX_K.  Rotation, scales and
 * quotients are computed in fp64 with IEEE division, exactly as in the definition above. */
int w4_pack_weights(const void *W, int w_dtype, int64_t N, int64_t K, int g, int wmode,
                    uint8_t *packed, float *row_scale, uint8_t *zp, void *stream);

/* w4_rotate_quant_act - activation step: rotate each token (row of X) along K in groups
 * of g and quantize it per token to act_bits.
 * (ComfyUI-INT-Crush README, "Inference / INT4": Hadamard rotation + dynamic activation
 *  quantization; "Inference / INT8": dynamic per-token quantization;
 *  stable-diffusion.cpp PR #2010, "Summary": this result is what gets shared and cached
 *  per (input, group size).)
 *  X         : [M, K] of x_dtype
 *  q         : out, act_bits == 8: int8 [M, K]; act_bits == 4: uint8 [M, K/2] packed like
 *              the weights (low nibble = even k, two's complement)
 *  tok_scale : out f32 [M]
 *  tok_rowsum: out int32 [M] = sum_k q[m, k] (used by the asymmetric-weight correction)
 * The rotation runs in fp64 (exact for bf16 inputs); codes equal rint(X'/s_x) up to the
 * last fp64 bit of the quotient.  Requires K % g == 0; for g = 64 or 256 also one of:
 * K % 256 == 0 with K <= 32768 (K % 1024 == 0 takes the row-team kernel), or K/16 = C * T for
 * some C in 1..4 and T a multiple of g/16 with T <= 512 (every K used by DiT / text-encoder
 * linears qualifies); else W4_ERR_UNSUPPORTED.  g = 16, 1024 and 4096 run a general kernel
 * (one workgroup per token, two passes over the row) that takes any K % g == 0. */
int w4_rotate_quant_act(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits,
                        void *q, float *tok_scale, int32_t *tok_rowsum, void *stream);

/* w4_linear_cached_rot - integer GEMM + fused dequant epilogue on already rotated and
 * quantized activations (the cached half of the layer).
 * (ComfyUI-INT-Crush README, "Inference / INT4" (INT8 GEMM with fused dequant; W4A8 and
 *  fused ConvRot paths) and "Forward Pass" steps 5-6; stable-diffusion.cpp PR #2010,
 *  "Summary": packed weights stream to the kernel unconverted.)
 *  q, tok_scale, tok_rowsum, act_bits : as produced by w4_rotate_quant_act
 *  packed, row_scale, zp              : as produced by w4_pack_weights (zp NULL = symmetric)
 *  bias      : NULL or [N] of bias_dtype (W4_F32 or W4_BF16)
 *  lr        : NULL or the low-rank branch (host pointer to the struct; its fields are
 *              device pointers)
 *  Y         : out [M, N], bf16 for W4_OUT_BF16, int32 for W4_OUT_I32 (bias and lr unused)
 *  ws        : workspace, w4_workspace_bytes(M, N, K, act_bits, r_needed) bytes where
 *              r_needed = lr->r when lr && !lr->t, else 0.  It holds the low-rank t (first,
 *              required when r_needed > 0) and then int32 partial sums: for M <= 64 those of
 *              the K-split small-M kernel, for larger M those of the last partial round of
 *              GEMM tiles when it is split along K (both optional: with less room, or
 *              ws == NULL, the kernels run without splitting K; the results are the same,
 *              bit for bit without a low-rank branch).  Contents are scratch; nothing
 *              persists.
 * M <= 64 runs the HBM-streaming small-M kernels, larger M the MFMA GEMM. */
int w4_linear_cached_rot(const void *q, const float *tok_scale, const int32_t *tok_rowsum,
                         int act_bits, const uint8_t *packed, const float *row_scale,
                         const uint8_t *zp, const void *bias, int bias_dtype,
                         const w4_lowrank *lr, int64_t M, int64_t N, int64_t K, void *Y,
                         int y_kind, void *ws, size_t ws_bytes, void *stream);

/* One linear of w4_linear_cached_rot_multi: the arguments of w4_linear_cached_rot that differ
 * between linears reading the same activation codes.  lr, when not NULL, must supply t. */
typedef struct w4_linear_out {
    const uint8_t *packed;
    const float *row_scale;
    const uint8_t *zp;
    const void *bias;
    int bias_dtype;
    const w4_lowrank *lr;
    int64_t N;
    void *Y;
    int y_kind;
} w4_linear_out;

/* w4_linear_cached_rot_multi - count linears on the same rotated and quantized activations
 * (stable-diffusion.cpp PR #2010, "Summary": the activation work of one input is shared by
 * every linear that reads it, e.g. the fused QKV and the MLP up-projection of a block with
 * parallel attention and MLP).
 *  q, tok_scale, tok_rowsum, act_bits, M, K : as for w4_linear_cached_rot, shared
 *  outs[i]   : host array of count (1..8) linears; output i is written to outs[i].Y
 *  ws        : serves the linears that run on their own, as in w4_linear_cached_rot
 * For M > 64, consecutive linears i, i + 1 with the same weight mode (zp NULL or not), output
 * kind and low-rank form run as ONE launch, so the tiles of both fill the compute units
 * together instead of each leaving its last round partly idle; each such output equals
 * w4_linear_cached_rot's without a workspace bit for bit.  The other linears run exactly as
 * w4_linear_cached_rot.  Every argument is checked before anything is launched. */
#define W4_MULTI_MAX 8
int w4_linear_cached_rot_multi(const void *q, const float *tok_scale, const int32_t *tok_rowsum,
                               int act_bits, int64_t M, int64_t K, int count,
                               const w4_linear_out *outs, void *ws, size_t ws_bytes, void *stream);

/* w4_linear - the whole layer: w4_rotate_quant_act into the workspace, then
 * w4_linear_cached_rot.  Arguments as above; ws must hold at least
 * w4_workspace_bytes(M, N, K, act_bits, r) + room for the activation codes, i.e.
 * w4_linear_workspace_bytes(M, N, K, act_bits, r_needed).  For one bf16 token (M = 1,
 * N <= 32 x the compute units, K a multiple of 3072 up to 12288 or of 2048 up to 16384) a
 * single kernel rotates, quantizes and multiplies, the fused ConvRot path of the INT4 README
 * ("Inference / INT4");
 * Y is the same bit for bit, and the workspace then holds no codes (its contents are
 * scratch either way). */
int w4_linear(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits,
              const uint8_t *packed, const float *row_scale, const uint8_t *zp, const void *bias,
              int bias_dtype, const w4_lowrank *lr, int64_t N, void *Y, int y_kind, void *ws,
              size_t ws_bytes, void *stream);

/* w4_linear_noalloc - w4_linear for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc.  Same arguments
 * as w4_linear minus the workspace; same kernels and the same result (bit for bit, except
 * that with a low-rank branch a shape whose K-split partials do not fit the scratch runs
 * unsplit, within the usual bf16 bar of the split result).  Instead of a caller workspace it
 * uses a file-scope device array of w4_noalloc_scratch_bytes() = 64 MiB that every GPU the
 * library runs on holds until the process ends.  The codes, token scales and row sums (plus
 * the low-rank t when computed here) must fit it: M * K (A8) or M * K / 2 (A4) bytes plus
 * 8 * M plus 4 * M * r, each rounded up to 256 bytes; larger calls fail with
 * W4_ERR_WORKSPACE before anything is launched.  K-split partial sums use whatever room is
 * left.  The stream must belong to the current device.  Calls never allocate or free
 * anything; calls that overlap on one GPU (concurrent streams or threads) share that GPU's
 * array and race, so the caller orders them.  Nothing in the array has to start at zero. */
int w4_linear_noalloc(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits,
                      const uint8_t *packed, const float *row_scale, const uint8_t *zp,
                      const void *bias, int bias_dtype, const w4_lowrank *lr, int64_t N, void *Y,
                      int y_kind, void *stream);

/* Size in bytes of the per-device scratch array w4_linear_noalloc uses (host-only query). */
size_t w4_noalloc_scratch_bytes(void);

/* ---- Grouped-scale weight format ----------------------------------------------------------
 * (ComfyUI-INT-Crush README, "Weight Format": INT4 weights are uint8, two values per byte, with
 *  weight_scale fp16 [out, num_groups]; "Nodes": rot_size 0/16/64/256/1024/4096;
 *  "Inference / INT4", Triton backend: W4A8 for rot_size > 0, W4A16 for rot_size 0.)
 * Symmetric signed codes packed as above, [N, K/2], and one fp16 scale per output row and run
 * of gw consecutive inputs: group_scale [N, K/gw] (row-major, raw fp16 bits),
 *   s[n, j] = fp16(max over the group of |W'| / 7)   (one rounding from fp64)
 *   c[n, k] = clamp(rint(W'[n, k] / s[n, k / gw]), -8, 7)      (a zero scale gives codes 0)
 * gw in {32, 64, 128, 256}; K a multiple of 64 and of gw.  The layer:
 *   W4A8 / W4A4 (act_bits 8 / 4, g > 0): y = s_x[m] * sum_j s[n, j] * acc_j[m, n] + lr + bias,
 *     acc_j the exact integer sum of q * c over group j;
 *   W4A16 (act_bits 16, g = 0, bf16 X): y = sum_k X[m, k] * s[n, k / gw] * c[n, k] + lr + bias,
 *     group partial sums exact in fp32 (bf16 times small integers), scaled per group.
 * Y is bf16; W4_OUT_I32 (integer activations only) gives sum_k q * c with no scales. */

/* w4_pack_weights_grouped - offline: rotate each row of W along K in groups of g (g = 0: no
 * rotation; else g in {16, 64, 256, 1024, 4096}), quantize per (row, run of gw inputs) and pack.
 *  W           : [N, K] of w_dtype
 *  packed      : out uint8 [N, K/2]
 *  group_scale : out fp16 bits [N, K/gw]
 * A group scale that overflows fp16 (max |W'| > 7 * 65504) is not detected. */
int w4_pack_weights_grouped(const void *W, int w_dtype, int64_t N, int64_t K, int g, int gw,
                            uint8_t *packed, uint16_t *group_scale, void *stream);

/* w4_linear_cached_rot_grouped - the GEMM half on codes from w4_rotate_quant_act (act_bits 8 or
 * 4; tok_rowsum is not needed with symmetric codes).  bias, lr, Y, y_kind as for
 * w4_linear_cached_rot.  ws: w4_grouped_workspace_bytes(M, N, K, act_bits, gw, r_needed) bytes
 * (the low-rank t when computed here, then, for M <= 64, optional partial sums of a split of K
 * over several workgroups; with less room K is not split). */
int w4_linear_cached_rot_grouped(const void *q, const float *tok_scale, int act_bits,
                                 const uint8_t *packed, const uint16_t *group_scale, int gw,
                                 const void *bias, int bias_dtype, const w4_lowrank *lr, int64_t M,
                                 int64_t N, int64_t K, void *Y, int y_kind, void *ws,
                                 size_t ws_bytes, void *stream);

/* w4_linear_grouped - the whole layer on the grouped format.  act_bits 8 / 4: rotate and quantize
 * X (g in {16, 64, 256, 1024, 4096}) into the workspace, then as above.  act_bits 16: g must be
 * 0 and X bf16; X feeds the bf16 matrix cores directly.  ws: at least
 * w4_linear_grouped_workspace_bytes(M, N, K, act_bits, gw, r_needed). */
int w4_linear_grouped(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits,
                      const uint8_t *packed, const uint16_t *group_scale, int gw, const void *bias,
                      int bias_dtype, const w4_lowrank *lr, int64_t N, void *Y, int y_kind,
                      void *ws, size_t ws_bytes, void *stream);

size_t w4_grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits, int gw, int r);
size_t w4_linear_grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits, int gw, int r);

/* w4_rotate_quant_act_lowrank - w4_rotate_quant_act plus the low-rank down-projection
 * t = X . L1 of the same bf16 input in the same pass (ComfyUI-INT-Crush README, "Forward Pass"
 * step 6 and "LoRA": the residual from L1 / L2 on the unrotated activations;
 * stable-diffusion.cpp PR #2010, "Summary": the work on an input is shared by the linears that
 * read it, so their L1 factors are stacked into one l1 and applied once).
 *  X, x_dtype (W4_BF16 only), M, K, g, act_bits, q, tok_scale, tok_rowsum: as for
 *              w4_rotate_quant_act; the outputs are the same bit for bit
 *  l1        : bf16 [r, K], rank-major (stacked rows of every consumer's L1 transposed)
 *  r         : 1 <= r <= 64
 *  t         : out f32 [M, r] with rows ldt floats apart (ldt = 0 means r), X . L1 with exact
 *              bf16 products and fp32 sums
 * For g in {64, 256} and K in {1024, 2048, 3072, 4096} one kernel does both and reads X from
 * HBM once (w4_rotate_quant_act_lowrank_fused reports it); other shapes run the two steps as
 * two launches.  K % 8 == 0. */
int w4_rotate_quant_act_lowrank(const void *X, int x_dtype, int64_t M, int64_t K, int g,
                                int act_bits, void *q, float *tok_scale, int32_t *tok_rowsum,
                                const void *l1, int r, float *t, int64_t ldt, void *stream);
/* 1 when w4_rotate_quant_act_lowrank runs as one kernel for (K, g), else 0 (host-only query). */
int w4_rotate_quant_act_lowrank_fused(int64_t K, int g);

/* w4_lowrank_down - t = x . L1, f32 [M, r], from bf16 x [M, K] and bf16 l1 = L1 transposed,
 * [r, K] rank-major (ComfyUI-INT-Crush README, "Forward Pass" step 6: the first factor of
 * the low-rank residual).  Lets linears that read the same input share t.  1 <= r <= 64;
 * K a multiple of 8 (W4_ERR_SHAPE otherwise); x, l1 and t 16-byte aligned.  Exact bf16
 * products, fp32 accumulation. */
int w4_lowrank_down(const void *x, const void *l1, int64_t M, int64_t K, int r, float *t,
                    void *stream);

/* Workspace sizes in bytes (0 when nothing is needed).
 * w4_workspace_bytes: for w4_linear_cached_rot (the low-rank t when not supplied, and the
 * K-split partial sums when the kernels split K for this shape: for M <= 64, S * M * N int32
 * with S in {2, 4, 8}; for larger M, when the 256 x 192 output tiles fill whole rounds of the
 * compute units plus a tail of at most a quarter round, tail * S * 256 * 192 int32 with S in
 * 4..8).
 * w4_linear_workspace_bytes: for w4_linear (activation codes, token scales and row sums,
 * plus the above).  Each piece is 256-byte aligned inside the workspace. */
size_t w4_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits, int r);
size_t w4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits, int r);

/* 1 when w4_linear on this shape runs as the single fused kernel (rotation, quantization and
 * GEMM in one launch, no codes written to the workspace), else 0 (also for shapes w4_linear
 * rejects).  Host-only query: launches nothing, needs no stream. */
int w4_linear_fused(int64_t M, int64_t N, int64_t K, int g, int act_bits, int x_dtype);

/* Human-readable name of a status code (static string). */
const char *w4_status_string(int status);
/* Message describing the calling thread's last error ("" if none). */
const char *w4_last_error(void);
/* Library version string (static). */
const char *w4_version(void);


#ifdef __cplusplus
}
#endif

#endif /* W4_H */
