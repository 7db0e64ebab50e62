// C ABI of the W4 linear layer: argument checks, workspace layout, regime dispatch.
// Declarations and the meaning of every argument: include/w4.h.
#include "w4.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
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

bool rot_size_ok(int g) { return g == 16 || g == 64 || g == 256 || g == 1024 || g == 4096; }

int check_k(const char *fn, int64_t K, int g) {
    if (!rot_size_ok(g)) return fail(W4_ERR_UNSUPPORTED, "%s: g=%d (supported: 16, 64, 256, 1024, 4096)", fn, g);
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

// ---------------------------------------------------------------------------------------
// Scratch for w4_linear_noalloc: the workspace of w4_linear (activation codes, token scales,
// row sums, low-rank t, K-split partials) in a file-scope device array, so that callers who
// cannot allocate need not pass one.  Every GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` is only a host-side stand-in for the symbol;
// kernels get the device address from hipGetSymbolAddress, looked up once per device with
// that device current.  Nothing in it has to start at zero: every byte a call reads was
// written earlier in the same call.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The stream's device must be the current one (the symbol address is per device).
int scratch_for_stream(const char *fn, hipStream_t st, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (st) {
        hipDevice_t sdev = 0;
        e = hipStreamGetDevice(st, &sdev);
        if (e != hipSuccess) return hip_status(e, fn);
        if ((int)sdev != dev)
            return fail(W4_ERR_INVALID_ARG, "%s: stream is on device %d, current device is %d", fn, (int)sdev, dev);
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(W4_ERR_INVALID_ARG, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, fn);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4_OK;
}

}  // namespace

extern "C" {

const char *w4_version(void) { return "w4 0.2 (gfx950)"; }

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

int w4_rotate_quant_act_lowrank(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits, void *q,
                                float *tok_scale, int32_t *tok_rowsum, const void *l1, int r, float *t, int64_t ldt,
                                void *stream) {
    const char *fn = "w4_rotate_quant_act_lowrank";
    if (x_dtype != W4_BF16) return fail(W4_ERR_UNSUPPORTED, "%s: the low-rank branch takes bf16 X", fn);
    if (act_bits != 4 && act_bits != 8) return fail(W4_ERR_UNSUPPORTED, "%s: act_bits=%d", fn, act_bits);
    if (M < 0) return fail(W4_ERR_SHAPE, "%s: M=%lld < 0", fn, (long long)M);
    if (M > (int64_t)1 << 31) return fail(W4_ERR_SHAPE, "%s: M too large", fn);
    if (int e = check_k(fn, K, g)) return e;
    if (!w4::rotquant_supported(K, g))
        return fail(W4_ERR_UNSUPPORTED, "%s: K=%lld has no supported split for g=%d", fn, (long long)K, g);
    if (K % 8) return fail(W4_ERR_SHAPE, "%s: K=%lld must be a multiple of 8", fn, (long long)K);
    if (r < 1 || r > 64) return fail(W4_ERR_UNSUPPORTED, "%s: r=%d (supported 1..64)", fn, r);
    if (ldt != 0 && ldt < r) return fail(W4_ERR_INVALID_ARG, "%s: ldt=%lld < r=%d", fn, (long long)ldt, r);
    if (M == 0) return ok();
    W4_CHECK_PTR(X);
    W4_CHECK_PTR(q);
    W4_CHECK_PTR(tok_scale);
    W4_CHECK_PTR(tok_rowsum);
    W4_CHECK_PTR(l1);
    W4_CHECK_PTR(t);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t ld = ldt ? ldt : r;
    if (w4::rotquant_lr_fusable(K, g))
        return hip_status(w4::launch_rotquant_lr(X, M, K, g, act_bits, q, tok_scale, tok_rowsum, l1, r, t, ld, st), fn);
    hipError_t e = w4::launch_rotquant(X, false, M, K, g, act_bits, q, tok_scale, tok_rowsum, st);
    if (e != hipSuccess) return hip_status(e, fn);
    return hip_status(w4::launch_lowrank_down(X, l1, M, K, r, t, st, ld), fn);
}

int w4_rotate_quant_act_lowrank_fused(int64_t K, int g) { return w4::rotquant_lr_fusable(K, g) ? 1 : 0; }

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
    int ldt = 0;
    size_t tbytes = 0;  // workspace bytes taken by the low-rank t
    if (lr && y_kind == W4_OUT_BF16) {
        r = lr->r;
        if (r < 1 || r > 64) return fail(W4_ERR_UNSUPPORTED, "%s: lowrank r=%d (supported 1..64)", fn, r);
        if (!lr->l2) return fail(W4_ERR_INVALID_ARG, "%s: lowrank l2 is NULL", fn);
        if (!aligned16(lr->l2)) return fail(W4_ERR_ALIGN, "%s: lowrank l2 not 16-byte aligned", fn);
        l2 = static_cast<const uint16_t *>(lr->l2);
        if (lr->t) {
            if (!aligned16(lr->t)) return fail(W4_ERR_ALIGN, "%s: lowrank t not 16-byte aligned", fn);
            if (lr->ldt != 0 && lr->ldt < r) return fail(W4_ERR_INVALID_ARG, "%s: lowrank ldt=%d < r=%d", fn, lr->ldt, r);
            t = lr->t;
            ldt = lr->ldt ? lr->ldt : r;
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
        ldt = r;
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
    a.lr_ldt = ldt;
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

// The LinearArgs of one output of w4_linear_cached_rot_multi, after the checks linear_impl
// makes (a low-rank branch must supply t).
static int multi_args(const char *fn, int i, const void *q, const float *tok_scale, const int32_t *tok_rowsum,
                      int act_bits, int64_t M, int64_t K, const w4_linear_out &o, w4::LinearArgs &a) {
    if (int e = check_linear_shape(fn, M, o.N, K, act_bits)) return e;
    if (o.y_kind != W4_OUT_BF16 && o.y_kind != W4_OUT_I32)
        return fail(W4_ERR_INVALID_ARG, "%s: outs[%d].y_kind=%d", fn, i, o.y_kind);
    if (o.bias && o.bias_dtype != W4_F32 && o.bias_dtype != W4_BF16)
        return fail(W4_ERR_INVALID_ARG, "%s: outs[%d].bias_dtype=%d", fn, i, o.bias_dtype);
    const uint8_t *packed = o.packed, *zp = o.zp;
    const float *row_scale = o.row_scale;
    const void *bias = o.bias, *Y = o.Y;
    W4_CHECK_PTR(q);
    W4_CHECK_PTR(tok_scale);
    W4_CHECK_PTR(tok_rowsum);
    W4_CHECK_PTR(packed);
    W4_CHECK_PTR(row_scale);
    W4_CHECK_OPT_PTR(zp);
    W4_CHECK_OPT_PTR(bias);
    W4_CHECK_PTR(Y);
    a = w4::LinearArgs{};
    const w4_lowrank *lr = o.lr;
    if (lr && o.y_kind == W4_OUT_BF16) {
        if (lr->r < 1 || lr->r > 64) return fail(W4_ERR_UNSUPPORTED, "%s: outs[%d] lowrank r=%d", fn, i, lr->r);
        if (!lr->l2 || !lr->t) return fail(W4_ERR_INVALID_ARG, "%s: outs[%d] lowrank needs t and l2", fn, i);
        if (!aligned16(lr->l2) || !aligned16(lr->t))
            return fail(W4_ERR_ALIGN, "%s: outs[%d] lowrank t / l2 not 16-byte aligned", fn, i);
        if (lr->ldt != 0 && lr->ldt < lr->r)
            return fail(W4_ERR_INVALID_ARG, "%s: outs[%d] lowrank ldt=%d < r=%d", fn, i, lr->ldt, lr->r);
        a.lr_t = lr->t;
        a.lr_l2 = static_cast<const uint16_t *>(lr->l2);
        a.lr_r = lr->r;
        a.lr_ldt = lr->ldt ? lr->ldt : lr->r;
    }
    a.A = static_cast<const uint8_t *>(q);
    a.sx = tok_scale;
    a.rowsum = tok_rowsum;
    a.B = packed;
    a.sw = row_scale;
    a.zp = zp;
    a.bias = o.y_kind == W4_OUT_BF16 ? bias : nullptr;
    a.bias_bf16 = o.bias_dtype == W4_BF16;
    a.Y = o.Y;
    a.y_i32 = o.y_kind == W4_OUT_I32;
    a.M = M;
    a.N = o.N;
    a.K = K;
    return W4_OK;
}

int w4_linear_cached_rot_multi(const void *q, const float *tok_scale, const int32_t *tok_rowsum, int act_bits,
                               int64_t M, int64_t K, int count, const w4_linear_out *outs, void *ws,
                               size_t ws_bytes, void *stream) {
    const char *fn = "w4_linear_cached_rot_multi";
    if (count < 1 || count > W4_MULTI_MAX) return fail(W4_ERR_INVALID_ARG, "%s: count=%d (1..%d)", fn, count, W4_MULTI_MAX);
    if (!outs) return fail(W4_ERR_INVALID_ARG, "%s: outs is NULL", fn);
    if (ws && !aligned16(ws)) return fail(W4_ERR_ALIGN, "%s: ws not 16-byte aligned", fn);
    w4::LinearArgs args[W4_MULTI_MAX];
    for (int i = 0; i < count; ++i)
        if (int e = multi_args(fn, i, q, tok_scale, tok_rowsum, act_bits, M, K, outs[i], args[i])) return e;
    if (M == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < count;) {
        if (i + 1 < count && w4::gemm_pairable(args[i], args[i + 1])) {
            if (int e = hip_status(w4::launch_gemm_pair(args[i], args[i + 1], act_bits, st), fn)) return e;
            i += 2;
            continue;
        }
        const w4::LinearArgs &a = args[i];
        const hipError_t e = M <= 64 ? w4::launch_gemv(a, act_bits, ws, ws ? ws_bytes : 0, st)
                                     : w4::launch_gemm(a, act_bits, ws, ws ? ws_bytes : 0, st);
        if (int r = hip_status(e, fn)) return r;
        ++i;
    }
    return ok();
}

// The whole layer: rotate-quantize into the front of ws, then the GEMM half.  The codes,
// token scales, row sums and (when computed here) the low-rank t must fit ws; the K-split
// partial sums take whatever room is left (with less, the kernels do not split K).
// noalloc == false: ws must also hold the partials, as w4_linear documents.  noalloc == true:
// ws and ws_bytes are ignored; after every argument check the device's scratch array is used.
static int linear_whole(const char *fn, const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits,
                        const uint8_t *packed, const float *row_scale, const uint8_t *zp, const void *bias,
                        int bias_dtype, const w4_lowrank *lr, int64_t N, void *Y, int y_kind, void *ws,
                        size_t ws_bytes, hipStream_t st, bool noalloc) {
    if (x_dtype != W4_F32 && x_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: x_dtype=%d", fn, x_dtype);
    if (int e = check_linear_shape(fn, M, N, K, act_bits)) return e;
    if (int e = check_k(fn, K, g)) return e;
    if (!w4::rotquant_supported(K, g))
        return fail(W4_ERR_UNSUPPORTED, "%s: K=%lld has no supported split for g=%d", fn, (long long)K, g);
    if (y_kind != W4_OUT_BF16 && y_kind != W4_OUT_I32) return fail(W4_ERR_INVALID_ARG, "%s: y_kind=%d", fn, y_kind);
    if (M == 0) return ok();
    W4_CHECK_PTR(X);
    const int r = (lr && !lr->t && y_kind == W4_OUT_BF16) ? lr->r : 0;
    const size_t qb = align256(act_bits == 4 ? (size_t)M * (size_t)(K / 2) : (size_t)M * (size_t)K);
    const size_t front = qb + 2 * align256((size_t)M * 4);
    if (noalloc) {
        const size_t need = front + (r > 0 ? align256((size_t)M * (size_t)r * sizeof(float)) : 0);
        if (need > kScratchBytes)
            return fail(W4_ERR_WORKSPACE, "%s: needs %zu bytes of scratch (codes, token scales, row sums%s), the "
                        "limit is %zu", fn, need, r > 0 ? ", low-rank t" : "", kScratchBytes);
        ws = nullptr;  // looked up after every other check
        ws_bytes = kScratchBytes;
    } else {
        const size_t need = w4_linear_workspace_bytes(M, N, K, act_bits, r > 0 ? r : 0);
        if (!ws || ws_bytes < need) return fail(W4_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
        if (!aligned16(ws)) return fail(W4_ERR_ALIGN, "%s: ws not 16-byte aligned", fn);
    }
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
    if (noalloc)
        if (int e = scratch_for_stream(fn, st, &ws)) return e;
    uint8_t *base = static_cast<uint8_t *>(ws);
    void *qbuf = base;
    float *sx = reinterpret_cast<float *>(base + qb);
    int32_t *rs = reinterpret_cast<int32_t *>(base + qb + align256((size_t)M * 4));
    uint8_t *rest = base + front;
    const size_t rest_bytes = ws_bytes - front;
    // a few tokens: one launch rotates, quantizes and multiplies (same result, no codes written)
    if (w4::gemv_fusable(M, N, K, g, act_bits, x_dtype == W4_F32))
        return linear_impl(fn, qbuf, sx, rs, act_bits, packed, row_scale, zp, bias, bias_dtype, lr, M, N, K, Y, y_kind,
                           rest, rest_bytes, st, X, g);
    hipError_t e = w4::launch_rotquant(X, x_dtype == W4_F32, M, K, g, act_bits, qbuf, sx, rs, st);
    if (e != hipSuccess) return hip_status(e, fn);
    return linear_impl(fn, qbuf, sx, rs, act_bits, packed, row_scale, zp, bias, bias_dtype, lr, M, N, K, Y, y_kind,
                       rest, rest_bytes, st);
}

int w4_linear(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits, const uint8_t *packed,
              const float *row_scale, const uint8_t *zp, const void *bias, int bias_dtype, const w4_lowrank *lr,
              int64_t N, void *Y, int y_kind, void *ws, size_t ws_bytes, void *stream) {
    return linear_whole("w4_linear", X, x_dtype, M, K, g, act_bits, packed, row_scale, zp, bias, bias_dtype, lr, N, Y,
                        y_kind, ws, ws_bytes, static_cast<hipStream_t>(stream), false);
}

size_t w4_noalloc_scratch_bytes(void) { return kScratchBytes; }

int w4_linear_noalloc(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits, const uint8_t *packed,
                      const float *row_scale, const uint8_t *zp, const void *bias, int bias_dtype,
                      const w4_lowrank *lr, int64_t N, void *Y, int y_kind, void *stream) {
    return linear_whole("w4_linear_noalloc", X, x_dtype, M, K, g, act_bits, packed, row_scale, zp, bias, bias_dtype,
                        lr, N, Y, y_kind, nullptr, 0, static_cast<hipStream_t>(stream), true);
}

// ------------------------------------------------------------------------------------------
// Grouped-scale weight format

static int check_gw(const char *fn, int64_t K, int gw) {
    if (gw != 32 && gw != 64 && gw != 128 && gw != 256)
        return fail(W4_ERR_UNSUPPORTED, "%s: gw=%d (supported: 32, 64, 128, 256)", fn, gw);
    if (K < 64 || K % 64 || K % gw)
        return fail(W4_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 64 and of gw=%d", fn, (long long)K, gw);
    if (K > W4_MAX_K) return fail(W4_ERR_SHAPE, "%s: K=%lld exceeds %d", fn, (long long)K, W4_MAX_K);
    return W4_OK;
}

size_t w4_grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits, int gw, int r) {
    (void)act_bits;
    if (M <= 0) return 0;
    const size_t t = r > 0 ? align256((size_t)M * (size_t)r * sizeof(float)) : 0;
    const size_t part = N <= 0 || K <= 0 || gw <= 0 ? 0 : align256(w4::grouped_workspace_bytes(M, N, K, gw));
    return t + part;
}

size_t w4_linear_grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_bits, int gw, int r) {
    if (M <= 0) return 0;
    const size_t codes = act_bits == 16 ? 0
                         : align256(act_bits == 4 ? (size_t)M * (size_t)(K / 2) : (size_t)M * (size_t)K) +
                               2 * align256((size_t)M * 4);
    return codes + w4_grouped_workspace_bytes(M, N, K, act_bits, gw, r);
}

int w4_pack_weights_grouped(const void *W, int w_dtype, int64_t N, int64_t K, int g, int gw, uint8_t *packed,
                            uint16_t *group_scale, void *stream) {
    const char *fn = "w4_pack_weights_grouped";
    if (w_dtype != W4_F32 && w_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: w_dtype=%d", fn, w_dtype);
    if (N < 1) return fail(W4_ERR_SHAPE, "%s: N=%lld < 1", fn, (long long)N);
    if (N > (int64_t)1 << 31) return fail(W4_ERR_SHAPE, "%s: N too large", fn);
    if (int e = check_gw(fn, K, gw)) return e;
    if (g != 0) {
        if (int e = check_k(fn, K, g)) return e;
    }
    W4_CHECK_PTR(W);
    W4_CHECK_PTR(packed);
    W4_CHECK_PTR(group_scale);
    return hip_status(w4::launch_pack_grouped(W, w_dtype == W4_F32, N, K, g, gw, packed, group_scale,
                                              static_cast<hipStream_t>(stream)),
                      fn);
}

// act: int8 / packed int4 codes (act_bits 8 / 4, with tok_scale) or bf16 X (act_bits 16).
static int grouped_impl(const char *fn, const void *act, const float *tok_scale, int act_bits, const uint8_t *packed,
                        const uint16_t *group_scale, int gw, const void *bias, int bias_dtype, const w4_lowrank *lr,
                        int64_t M, int64_t N, int64_t K, void *Y, int y_kind, void *ws, size_t ws_bytes,
                        hipStream_t st) {
    if (y_kind != W4_OUT_BF16 && y_kind != W4_OUT_I32) return fail(W4_ERR_INVALID_ARG, "%s: y_kind=%d", fn, y_kind);
    if (act_bits == 16 && y_kind == W4_OUT_I32)
        return fail(W4_ERR_INVALID_ARG, "%s: W4_OUT_I32 needs integer activations", fn);
    if (bias && bias_dtype != W4_F32 && bias_dtype != W4_BF16)
        return fail(W4_ERR_INVALID_ARG, "%s: bias_dtype=%d", fn, bias_dtype);
    W4_CHECK_PTR(act);
    if (act_bits != 16) W4_CHECK_PTR(tok_scale);
    W4_CHECK_PTR(packed);
    W4_CHECK_PTR(group_scale);
    W4_CHECK_OPT_PTR(bias);
    W4_CHECK_PTR(Y);
    const float *t = nullptr;
    const uint16_t *l2 = nullptr;
    int r = 0;
    int ldt = 0;
    size_t tbytes = 0;
    if (lr && y_kind == W4_OUT_BF16) {
        r = lr->r;
        if (r < 1 || r > 64) return fail(W4_ERR_UNSUPPORTED, "%s: lowrank r=%d (supported 1..64)", fn, r);
        if (!lr->l2) return fail(W4_ERR_INVALID_ARG, "%s: lowrank l2 is NULL", fn);
        if (!aligned16(lr->l2)) return fail(W4_ERR_ALIGN, "%s: lowrank l2 not 16-byte aligned", fn);
        l2 = static_cast<const uint16_t *>(lr->l2);
        if (lr->t) {
            if (!aligned16(lr->t)) return fail(W4_ERR_ALIGN, "%s: lowrank t not 16-byte aligned", fn);
            if (lr->ldt != 0 && lr->ldt < r) return fail(W4_ERR_INVALID_ARG, "%s: lowrank ldt=%d < r=%d", fn, lr->ldt, r);
            t = lr->t;
            ldt = lr->ldt ? lr->ldt : r;
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
    if (r && !t) {
        float *tw = static_cast<float *>(ws);
        hipError_t e = w4::launch_lowrank_down(lr->x, lr->l1, M, K, r, tw, st);
        if (e != hipSuccess) return hip_status(e, fn);
        t = tw;
        ldt = r;
    }
    w4::GroupedArgs a{};
    a.A = act;
    a.sx = tok_scale;
    a.B = packed;
    a.gs = group_scale;
    a.gw = gw;
    a.bias = y_kind == W4_OUT_BF16 ? bias : nullptr;
    a.bias_bf16 = bias_dtype == W4_BF16;
    a.lr_t = t;
    a.lr_l2 = l2;
    a.lr_r = r;
    a.lr_ldt = ldt;
    a.Y = Y;
    a.y_i32 = y_kind == W4_OUT_I32;
    a.M = M;
    a.N = N;
    a.K = K;
    void *gws = ws ? static_cast<uint8_t *>(ws) + tbytes : nullptr;
    const size_t gbytes = ws ? ws_bytes - tbytes : 0;
    return hip_status(w4::launch_gemm_grouped(a, act_bits, gws, gbytes, st), fn);
}

int w4_linear_cached_rot_grouped(const void *q, const float *tok_scale, int act_bits, const uint8_t *packed,
                                 const uint16_t *group_scale, int gw, const void *bias, int bias_dtype,
                                 const w4_lowrank *lr, int64_t M, int64_t N, int64_t K, void *Y, int y_kind, void *ws,
                                 size_t ws_bytes, void *stream) {
    const char *fn = "w4_linear_cached_rot_grouped";
    if (act_bits != 4 && act_bits != 8)
        return fail(W4_ERR_UNSUPPORTED, "%s: act_bits=%d (supported: 4, 8)", fn, act_bits);
    if (int e = check_linear_shape(fn, M, N, K, act_bits)) return e;
    if (int e = check_gw(fn, K, gw)) return e;
    return grouped_impl(fn, q, tok_scale, act_bits, packed, group_scale, gw, bias, bias_dtype, lr, M, N, K, Y, y_kind,
                        ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int w4_linear_grouped(const void *X, int x_dtype, int64_t M, int64_t K, int g, int act_bits, const uint8_t *packed,
                      const uint16_t *group_scale, int gw, const void *bias, int bias_dtype, const w4_lowrank *lr,
                      int64_t N, void *Y, int y_kind, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "w4_linear_grouped";
    if (x_dtype != W4_F32 && x_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: x_dtype=%d", fn, x_dtype);
    if (act_bits != 4 && act_bits != 8 && act_bits != 16)
        return fail(W4_ERR_UNSUPPORTED, "%s: act_bits=%d (supported: 4, 8, 16)", fn, act_bits);
    if (int e = check_linear_shape(fn, M, N, K, act_bits == 16 ? 8 : act_bits)) return e;
    if (int e = check_gw(fn, K, gw)) return e;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (act_bits == 16) {
        // W4A16: the unrotated bf16 activations go straight into the bf16 GEMM
        if (g != 0) return fail(W4_ERR_UNSUPPORTED, "%s: W4A16 takes unrotated weights (g = 0), got g=%d", fn, g);
        if (x_dtype != W4_BF16) return fail(W4_ERR_UNSUPPORTED, "%s: W4A16 takes bf16 activations", fn);
        return grouped_impl(fn, X, nullptr, 16, packed, group_scale, gw, bias, bias_dtype, lr, M, N, K, Y, y_kind, ws,
                            ws_bytes, st);
    }
    if (int e = check_k(fn, K, g)) return e;
    if (!w4::rotquant_supported(K, g))
        return fail(W4_ERR_UNSUPPORTED, "%s: K=%lld has no supported split for g=%d", fn, (long long)K, g);
    if (y_kind != W4_OUT_BF16 && y_kind != W4_OUT_I32) return fail(W4_ERR_INVALID_ARG, "%s: y_kind=%d", fn, y_kind);
    if (M == 0) return ok();
    W4_CHECK_PTR(X);
    const int r = (lr && !lr->t && y_kind == W4_OUT_BF16) ? lr->r : 0;
    const size_t need = w4_linear_grouped_workspace_bytes(M, N, K, act_bits, gw, r > 0 ? r : 0);
    if (!ws || ws_bytes < need) return fail(W4_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    if (!aligned16(ws)) return fail(W4_ERR_ALIGN, "%s: ws not 16-byte aligned", fn);
    {
        W4_CHECK_PTR(packed);
        W4_CHECK_PTR(group_scale);
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
    uint8_t *base = static_cast<uint8_t *>(ws);
    const size_t qb = align256(act_bits == 4 ? (size_t)M * (size_t)(K / 2) : (size_t)M * (size_t)K);
    float *sx = reinterpret_cast<float *>(base + qb);
    int32_t *rs = reinterpret_cast<int32_t *>(base + qb + align256((size_t)M * 4));
    uint8_t *rest = base + qb + 2 * align256((size_t)M * 4);
    hipError_t e = w4::launch_rotquant(X, x_dtype == W4_F32, M, K, g, act_bits, base, sx, rs, st);
    if (e != hipSuccess) return hip_status(e, fn);
    return grouped_impl(fn, base, sx, act_bits, packed, group_scale, gw, bias, bias_dtype, lr, M, N, K, Y, y_kind, rest,
                        ws_bytes - (size_t)(rest - base), st);
}

}  // extern "C"
