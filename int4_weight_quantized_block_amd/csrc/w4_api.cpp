// C ABI of the W4 linear layer: argument checks, workspace layout, regime dispatch.
// Declarations and the meaning of every argument: include/w4.h.
#include "w4.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return W4_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(W4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

#define W4_CHECK_PTR(p)                                                         \
    do {                                                                        \
        if (!(p)) return fail(W4_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);    \
        if (!aligned16(p)) return fail(W4_ERR_ALIGN, "%s: %s not 16-byte aligned", fn, #p); \
    } while (0)

#define W4_CHECK_OPT_PTR(p)                                                     \
    do {                                                                        \
        if ((p) && !aligned16(p)) return fail(W4_ERR_ALIGN, "%s: %s not 16-byte aligned", fn, #p); \
    } while (0)

int check_k(const char *fn, int64_t K, int g) {
    if (g != 64 && g != 256) return fail(W4_ERR_UNSUPPORTED, "%s: g=%d (supported: 64, 256)", fn, g);
    if (K < g || K % g) return fail(W4_ERR_SHAPE, "%s: K=%lld must be a positive multiple of g=%d", fn, (long long)K, g);
    if (K > W4_MAX_K) return fail(W4_ERR_SHAPE, "%s: K=%lld exceeds %d", fn, (long long)K, W4_MAX_K);
    return W4_OK;
}

int check_linear_shape(const char *fn, int64_t M, int64_t N, int64_t K, int act_bits) {
    if (M < 0) return fail(W4_ERR_SHAPE, "%s: M=%lld < 0", fn, (long long)M);
    if (N < 1) return fail(W4_ERR_SHAPE, "%s: N=%lld < 1", fn, (long long)N);
    if (K < 64 || K % 64) return fail(W4_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 64", fn, (long long)K);
    if (K > W4_MAX_K) return fail(W4_ERR_SHAPE, "%s: K=%lld exceeds %d", fn, (long long)K, W4_MAX_K);
    if (act_bits != 4 && act_bits != 8) return fail(W4_ERR_UNSUPPORTED, "%s: act_bits=%d (supported: 4, 8)", fn, act_bits);
    if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31) return fail(W4_ERR_SHAPE, "%s: M or N too large", fn);
    return W4_OK;
}

}  // namespace

extern "C" {

const char *w4_version(void) { return "w4 0.1 (gfx950)"; }

const char *w4_last_error(void) { return g_last_error.c_str(); }

const char *w4_status_string(int status) {
    switch (status) {
        case W4_OK: return "W4_OK";
        case W4_ERR_INVALID_ARG: return "W4_ERR_INVALID_ARG";
        case W4_ERR_SHAPE: return "W4_ERR_SHAPE";
        case W4_ERR_UNSUPPORTED: return "W4_ERR_UNSUPPORTED";
        case W4_ERR_ALIGN: return "W4_ERR_ALIGN";
        case W4_ERR_HIP: return "W4_ERR_HIP";
        case W4_ERR_WORKSPACE: return "W4_ERR_WORKSPACE";
        default: return "W4_ERR_UNKNOWN";
    }
}

size_t w4_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits, int r) {
    if (M <= 0) return 0;
    const size_t t = r > 0 ? align256((size_t)M * (size_t)r * sizeof(float)) : 0;
    const size_t part = N <= 0 || K <= 0 ? 0
                        : M <= 64      ? align256(w4::gemv_workspace_bytes(M, N, K, act_bits))
                                       : align256(w4::gemm_workspace_bytes(M, N, K));
    return t + part;
}

size_t w4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits, int r) {
    if (M <= 0) return 0;
    const size_t qb = act_bits == 4 ? (size_t)M * (size_t)(K / 2) : (size_t)M * (size_t)K;
    return align256(qb) + 2 * align256((size_t)M * 4) + w4_workspace_bytes(M, N, K, act_bits, r);
}

int w4_linear_fused(int64_t M, int64_t N, int64_t K, int g, int act_bits, int x_dtype) {
    if ((x_dtype != W4_F32 && x_dtype != W4_BF16) || N < 1 || K < 1 || (g != 64 && g != 256) || K % g)
        return 0;
    return w4::gemv_fusable(M, N, K, g, act_bits, x_dtype == W4_F32) ? 1 : 0;
}

int w4_pack_weights(const void *W, int w_dtype, int64_t N, int64_t K, int g, int wmode, uint8_t *packed,
                    float *row_scale, uint8_t *zp, void *stream) {
    const char *fn = "w4_pack_weights";
    if (w_dtype != W4_F32 && w_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: w_dtype=%d", fn, w_dtype);
    if (wmode != W4_SYM && wmode != W4_ASYM) return fail(W4_ERR_INVALID_ARG, "%s: wmode=%d", fn, wmode);
    if (N < 1) return fail(W4_ERR_SHAPE, "%s: N=%lld < 1", fn, (long long)N);
    if (N > (int64_t)1 << 31) return fail(W4_ERR_SHAPE, "%s: N too large", fn);
    if (int e = check_k(fn, K, g)) return e;
    W4_CHECK_PTR(W);
    W4_CHECK_PTR(packed);
    W4_CHECK_PTR(row_scale);
    if (wmode == W4_ASYM) {
        W4_CHECK_PTR(zp);
    } else if (zp) {
        return fail(W4_ERR_INVALID_ARG, "%s: zp must be NULL for W4_SYM", fn);
    }
    return hip_status(w4::launch_pack(W, w_dtype == W4_F32, N, K, g, wmode == W4_ASYM, packed, row_scale, zp,
                                      static_cast<hipStream_t>(stream)),
                      fn);
}

int w4_rotate_quant_act(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits, void *q,
                        float *tok_scale, int32_t *tok_rowsum, void *stream) {
    const char *fn = "w4_rotate_quant_act";
    if (x_dtype != W4_F32 && x_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: x_dtype=%d", fn, x_dtype);
    if (act_bits != 4 && act_bits != 8) return fail(W4_ERR_UNSUPPORTED, "%s: act_bits=%d", fn, act_bits);
    if (M < 0) return fail(W4_ERR_SHAPE, "%s: M=%lld < 0", fn, (long long)M);
    if (M > (int64_t)1 << 31) return fail(W4_ERR_SHAPE, "%s: M too large", fn);
    if (int e = check_k(fn, K, g)) return e;
    if (!w4::rotquant_supported(K, g))
        return fail(W4_ERR_UNSUPPORTED, "%s: K=%lld has no supported split for g=%d", fn, (long long)K, g);
    if (M == 0) return ok();
    W4_CHECK_PTR(X);
    W4_CHECK_PTR(q);
    W4_CHECK_PTR(tok_scale);
    W4_CHECK_PTR(tok_rowsum);
    return hip_status(w4::launch_rotquant(X, x_dtype == W4_F32, M, K, g, act_bits, q, tok_scale, tok_rowsum,
                                          static_cast<hipStream_t>(stream)),
                      fn);
}

int w4_lowrank_down(const void *x, const void *l1, int64_t M, int64_t K, int r, float *t, void *stream) {
    const char *fn = "w4_lowrank_down";
    if (M < 0 || K < 8 || K % 8 || K > W4_MAX_K)
        return fail(W4_ERR_SHAPE, "%s: M=%lld K=%lld (K must be a positive multiple of 8)", fn, (long long)M,
                    (long long)K);
    if (r < 1 || r > 64) return fail(W4_ERR_UNSUPPORTED, "%s: r=%d (supported 1..64)", fn, r);
    if (M == 0) return ok();
    W4_CHECK_PTR(x);
    W4_CHECK_PTR(l1);
    W4_CHECK_PTR(t);
    return hip_status(w4::launch_lowrank_down(x, l1, M, K, r, t, static_cast<hipStream_t>(stream)), fn);
}

int w4_probe_mfma_rate(int64_t blocks, int iters, int random_operands, int32_t *sink, void *stream) {
    const char *fn = "w4_probe_mfma_rate";
    if (blocks < 1 || blocks > (int64_t)1 << 24 || iters < 1)
        return fail(W4_ERR_INVALID_ARG, "%s: blocks=%lld iters=%d", fn, (long long)blocks, iters);
    W4_CHECK_PTR(sink);
    return hip_status(w4::launch_mfma_rate(blocks, iters, random_operands != 0, sink, static_cast<hipStream_t>(stream)),
                      fn);
}

// xf: NULL, or bf16 X for the fused small-M kernel (rotation and quantization inside the GEMM
// launch; q, tok_scale and tok_rowsum are then not read).
static int linear_impl(const char *fn, const void *q, const float *tok_scale, const int32_t *tok_rowsum,
                       int act_bits, const uint8_t *packed, const float *row_scale, const uint8_t *zp,
                       const void *bias, int bias_dtype, const w4_lowrank *lr, int64_t M, int64_t N, int64_t K,
                       void *Y, int y_kind, void *ws, size_t ws_bytes, hipStream_t st, const void *xf = nullptr,
                       int g = 0) {
    if (y_kind != W4_OUT_BF16 && y_kind != W4_OUT_I32) return fail(W4_ERR_INVALID_ARG, "%s: y_kind=%d", fn, y_kind);
    if (bias && bias_dtype != W4_F32 && bias_dtype != W4_BF16)
        return fail(W4_ERR_INVALID_ARG, "%s: bias_dtype=%d", fn, bias_dtype);
    W4_CHECK_PTR(q);
    W4_CHECK_PTR(tok_scale);
    W4_CHECK_PTR(tok_rowsum);
    W4_CHECK_PTR(packed);
    W4_CHECK_PTR(row_scale);
    W4_CHECK_OPT_PTR(zp);
    W4_CHECK_OPT_PTR(bias);
    W4_CHECK_PTR(Y);
    const float *t = nullptr;
    const uint16_t *l2 = nullptr;
    int r = 0;
    size_t tbytes = 0;  // workspace bytes taken by the low-rank t
    if (lr && y_kind == W4_OUT_BF16) {
        r = lr->r;
        if (r < 1 || r > 64) return fail(W4_ERR_UNSUPPORTED, "%s: lowrank r=%d (supported 1..64)", fn, r);
        if (!lr->l2) return fail(W4_ERR_INVALID_ARG, "%s: lowrank l2 is NULL", fn);
        if (!aligned16(lr->l2)) return fail(W4_ERR_ALIGN, "%s: lowrank l2 not 16-byte aligned", fn);
        l2 = static_cast<const uint16_t *>(lr->l2);
        if (lr->t) {
            if (!aligned16(lr->t)) return fail(W4_ERR_ALIGN, "%s: lowrank t not 16-byte aligned", fn);
            t = lr->t;
        } else {
            if (!lr->x || !lr->l1) return fail(W4_ERR_INVALID_ARG, "%s: lowrank needs t or (x, l1)", fn);
            if (!aligned16(lr->x) || !aligned16(lr->l1))
                return fail(W4_ERR_ALIGN, "%s: lowrank x / l1 not 16-byte aligned", fn);
            tbytes = align256((size_t)M * (size_t)r * sizeof(float));
            if (!ws || ws_bytes < tbytes)
                return fail(W4_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, tbytes);
        }
    }
    if (ws && !aligned16(ws)) return fail(W4_ERR_ALIGN, "%s: ws not 16-byte aligned", fn);
    if (M == 0) return ok();
    if (lr && y_kind == W4_OUT_BF16 && !t) {
        float *tw = static_cast<float *>(ws);
        hipError_t e = w4::launch_lowrank_down(lr->x, lr->l1, M, K, r, tw, st);
        if (e != hipSuccess) return hip_status(e, fn);
        t = tw;
    }
    w4::LinearArgs a;
    a.A = static_cast<const uint8_t *>(q);
    a.sx = tok_scale;
    a.rowsum = tok_rowsum;
    a.B = packed;
    a.sw = row_scale;
    a.zp = zp;
    a.bias = y_kind == W4_OUT_BF16 ? bias : nullptr;
    a.bias_bf16 = bias_dtype == W4_BF16;
    a.lr_t = t;
    a.lr_l2 = l2;
    a.lr_r = r;
    a.Y = Y;
    a.y_i32 = y_kind == W4_OUT_I32;
    a.M = M;
    a.N = N;
    a.K = K;
    // the rest of the workspace (if any) holds the K-split partial sums (small-M path, or the
    // last partial round of tiles of the large-M path)
    void *gws = ws ? static_cast<uint8_t *>(ws) + tbytes : nullptr;
    const size_t gbytes = ws ? ws_bytes - tbytes : 0;
    hipError_t e = xf        ? w4::launch_gemv_fused(a, xf, g, act_bits, st)
                   : M <= 64 ? w4::launch_gemv(a, act_bits, gws, gbytes, st)
                             : w4::launch_gemm(a, act_bits, gws, gbytes, st);
    return hip_status(e, fn);
}

int w4_linear_cached_rot(const void *q, const float *tok_scale, const int32_t *tok_rowsum, int act_bits,
                         const uint8_t *packed, const float *row_scale, const uint8_t *zp, const void *bias,
                         int bias_dtype, const w4_lowrank *lr, int64_t M, int64_t N, int64_t K, void *Y, int y_kind,
                         void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "w4_linear_cached_rot";
    if (int e = check_linear_shape(fn, M, N, K, act_bits)) return e;
    if (M == 0 && y_kind != W4_OUT_BF16 && y_kind != W4_OUT_I32)
        return fail(W4_ERR_INVALID_ARG, "%s: y_kind=%d", fn, y_kind);
    return linear_impl(fn, q, tok_scale, tok_rowsum, act_bits, packed, row_scale, zp, bias, bias_dtype, lr, M, N, K,
                       Y, y_kind, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int w4_linear(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits, const uint8_t *packed,
              const float *row_scale, const uint8_t *zp, const void *bias, int bias_dtype, const w4_lowrank *lr,
              int64_t N, void *Y, int y_kind, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "w4_linear";
    if (x_dtype != W4_F32 && x_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: x_dtype=%d", fn, x_dtype);
    if (int e = check_linear_shape(fn, M, N, K, act_bits)) return e;
    if (int e = check_k(fn, K, g)) return e;
    if (!w4::rotquant_supported(K, g))
        return fail(W4_ERR_UNSUPPORTED, "%s: K=%lld has no supported split for g=%d", fn, (long long)K, g);
    if (y_kind != W4_OUT_BF16 && y_kind != W4_OUT_I32) return fail(W4_ERR_INVALID_ARG, "%s: y_kind=%d", fn, y_kind);
    if (M == 0) return ok();
    W4_CHECK_PTR(X);
    const int r = (lr && !lr->t && y_kind == W4_OUT_BF16) ? lr->r : 0;
    const size_t need = w4_linear_workspace_bytes(M, N, K, act_bits, r > 0 ? r : 0);
    if (!ws || ws_bytes < need) return fail(W4_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    if (!aligned16(ws)) return fail(W4_ERR_ALIGN, "%s: ws not 16-byte aligned", fn);
    uint8_t *base = static_cast<uint8_t *>(ws);
    const size_t qb = align256(act_bits == 4 ? (size_t)M * (size_t)(K / 2) : (size_t)M * (size_t)K);
    void *qbuf = base;
    float *sx = reinterpret_cast<float *>(base + qb);
    int32_t *rs = reinterpret_cast<int32_t *>(base + qb + align256((size_t)M * 4));
    uint8_t *rest = base + qb + 2 * align256((size_t)M * 4);
    const size_t rest_bytes = ws_bytes - (size_t)(rest - base);
    // Check everything the GEMM half will check before launching the first kernel.
    {
        W4_CHECK_PTR(packed);
        W4_CHECK_PTR(row_scale);
        W4_CHECK_OPT_PTR(zp);
        W4_CHECK_OPT_PTR(bias);
        W4_CHECK_PTR(Y);
        if (bias && bias_dtype != W4_F32 && bias_dtype != W4_BF16)
            return fail(W4_ERR_INVALID_ARG, "%s: bias_dtype=%d", fn, bias_dtype);
        if (lr && y_kind == W4_OUT_BF16) {
            if (lr->r < 1 || lr->r > 64) return fail(W4_ERR_UNSUPPORTED, "%s: lowrank r=%d", fn, lr->r);
            if (!lr->l2) return fail(W4_ERR_INVALID_ARG, "%s: lowrank l2 is NULL", fn);
            if (!lr->t && (!lr->x || !lr->l1)) return fail(W4_ERR_INVALID_ARG, "%s: lowrank needs t or (x, l1)", fn);
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    // a few tokens: one launch rotates, quantizes and multiplies (same result, no codes written)
    if (w4::gemv_fusable(M, N, K, g, act_bits, x_dtype == W4_F32))
        return linear_impl(fn, qbuf, sx, rs, act_bits, packed, row_scale, zp, bias, bias_dtype, lr, M, N, K, Y, y_kind,
                           rest, rest_bytes, st, X, g);
    hipError_t e = w4::launch_rotquant(X, x_dtype == W4_F32, M, K, g, act_bits, qbuf, sx, rs, st);
    if (e != hipSuccess) return hip_status(e, fn);
    return linear_impl(fn, qbuf, sx, rs, act_bits, packed, row_scale, zp, bias, bias_dtype, lr, M, N, K, Y, y_kind,
                       rest, rest_bytes, st);
}

}  // extern "C"
