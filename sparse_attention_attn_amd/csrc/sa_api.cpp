// sa_api.cpp -- the C ABI declared in include/sparse_attn.h.
//
// Every entry point validates all of its arguments on the host before anything is
// enqueued (akol1/TensorFold pull request 4, first commit message: encoding refuses
// a pipeline that cannot take the launch; TensorFold pull request 1206 shows the
// same stance with an explicit Unsupported refusal rather than a silent fallback).
// On error nothing is launched and the outputs are untouched.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sa_internal.h"
#include "sparse_attn.h"

namespace sa {
int device_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}
}  // namespace sa

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_last_error[0] = '\0';
    return SA_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxGrid = 0x7fffffff;

int check_attn(int dtype, const void *q, const void *k, const void *v, int64_t n_ctx, const int32_t *idx,
               const int32_t *nsel, int32_t kmax, const float *sinks, float scale, int32_t rows, int32_t H,
               int32_t D, float *out, void *ws, size_t ws_bytes, bool shared) {
    (void)nsel;
    (void)scale;
    if (rows > 0 && (!q || !k || !v || !idx || !sinks || !out))
        return fail(SA_ERR_NULL, "q, k_cache, v_cache, idx, sinks and out must be non-NULL");
    if (dtype != SA_BF16 && dtype != SA_F32) return fail(SA_ERR_UNSUPPORTED, "dtype %d is not SA_BF16 or SA_F32", dtype);
    if (D != SA_HEAD_DIM) return fail(SA_ERR_UNSUPPORTED, "head width %d: only %d is implemented", D, SA_HEAD_DIM);
    if (H < 1 || H > SA_MAX_HEADS) return fail(SA_ERR_SHAPE, "heads %d outside [1, %d]", H, SA_MAX_HEADS);
    if (rows < 0) return fail(SA_ERR_SHAPE, "row count %d is negative", rows);
    if (kmax < 1 || kmax > SA_MAX_KMAX) return fail(SA_ERR_SHAPE, "kmax %d outside [1, %d]", kmax, SA_MAX_KMAX);
    if (n_ctx < 1 || n_ctx > 0x7fffffff) return fail(SA_ERR_SHAPE, "n_ctx %lld outside [1, 2^31)", (long long)n_ctx);
    const int64_t elt = dtype == SA_BF16 ? 2 : 4;
    const int64_t caches = shared ? 1 : rows;
    if (caches > 0 && n_ctx > INT64_MAX / D / elt / caches) return fail(SA_ERR_SHAPE, "cache size overflows");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(SA_ERR_UNSUPPORTED, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (!aligned(idx, 4) || !aligned(sinks, 4) || (nsel && !aligned(nsel, 4)))
        return fail(SA_ERR_UNSUPPORTED, "idx, nsel and sinks must be 4-byte aligned");
    size_t need = 0;
    if (dtype == SA_BF16) {
        // The gathers address a cache through a 32-bit byte range (1 KiB per position).
        if (n_ctx > SA_BF16_MAX_CTX)
            return fail(SA_ERR_UNSUPPORTED, "n_ctx %lld: bf16 caches hold at most %d positions", (long long)n_ctx,
                        SA_BF16_MAX_CTX);
        const sa::AttnPlan p = sa::plan_attn_bf16(rows, H, kmax);
        if (p.units > kMaxGrid) return fail(SA_ERR_SHAPE, "too many rows for one launch");
        need = p.ws_bytes;
    } else {
        if (n_ctx > SA_F32_MAX_CTX)
            return fail(SA_ERR_UNSUPPORTED, "n_ctx %lld: float32 caches hold at most %d positions", (long long)n_ctx,
                        SA_F32_MAX_CTX);
        if ((int64_t)rows * ((H + 15) / 16) > kMaxGrid) return fail(SA_ERR_SHAPE, "too many rows for one launch");
        if (sa::f32_split_applies(rows, H, kmax)) need = sa::f32_split_workspace_bytes(rows, H, kmax);
    }
    (void)shared;
    if (ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (need > 0 && !ws) return fail(SA_ERR_NULL, "this launch needs a workspace of %zu bytes", need);
    if (need > 0 && !aligned(ws, 16)) return fail(SA_ERR_UNSUPPORTED, "the workspace must be 16-byte aligned");
    return SA_OK;
}

int run_attn(int dtype, const void *q, const void *k, const void *v, int64_t n_ctx, const int32_t *idx,
             const int32_t *nsel, int32_t kmax, const float *sinks, float scale, int32_t rows, int32_t H,
             int32_t D, float *out, void *ws, size_t ws_bytes, void *stream, bool shared) {
    int rc = check_attn(dtype, q, k, v, n_ctx, idx, nsel, kmax, sinks, scale, rows, H, D, out, ws, ws_bytes, shared);
    if (rc != SA_OK) return rc;
    sa::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cache_stride = shared ? 0 : n_ctx * D;
    a.n_ctx = n_ctx;
    a.idx = idx;
    a.nsel = nsel;
    a.kmax = kmax;
    a.sinks = sinks;
    a.scale = scale;
    a.rows = rows;
    a.H = H;
    a.out = out;
    a.ws = ws;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == SA_BF16 ? sa::launch_attn_bf16(a, s) : sa::launch_attn_f32(a, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

namespace sa {
int check_decode(int dtype, const void *q, const void *k_cache, const void *v_cache, int64_t n_ctx, const int32_t *idx,
                 const int32_t *nsel, int32_t kmax, const float *sinks, float scale, int32_t B, int32_t H, int32_t D,
                 float *out, void *ws, size_t ws_bytes) {
    const int rc = check_attn(dtype, q, k_cache, v_cache, n_ctx, idx, nsel, kmax, sinks, scale, B, H, D, out, ws,
                              ws_bytes, false);
    return rc == SA_OK ? ok() : rc;
}
int run_decode(int dtype, const void *q, const void *k_cache, const void *v_cache, int64_t n_ctx, const int32_t *idx,
               const int32_t *nsel, int32_t kmax, const float *sinks, float scale, int32_t B, int32_t H, int32_t D,
               float *out, void *ws, size_t ws_bytes, void *stream) {
    return run_attn(dtype, q, k_cache, v_cache, n_ctx, idx, nsel, kmax, sinks, scale, B, H, D, out, ws, ws_bytes,
                    stream, false);
}
int fail_with(int code, const char *msg) { return fail(code, "%s", msg); }
}  // namespace sa

extern "C" {

int sparse_attn_abi_version(void) { return SA_ABI_VERSION; }

const char *sparse_attn_status_string(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_NULL: return "null pointer";
        case SA_ERR_SHAPE: return "invalid size";
        case SA_ERR_UNSUPPORTED: return "unsupported configuration";
        case SA_ERR_WORKSPACE: return "workspace too small";
        case SA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *sparse_attn_last_error(void) { return g_last_error; }

size_t sparse_attn_workspace_bytes(int op, int64_t rows, int32_t heads, int32_t head_dim, int32_t kmax,
                                   int64_t n_ctx) {
    (void)head_dim;
    (void)n_ctx;
    if (op != SA_OP_DECODE && op != SA_OP_PREFILL) return 0;
    if (rows <= 0 || heads < 1 || heads > SA_MAX_HEADS || kmax < 1 || kmax > SA_MAX_KMAX) return 0;
    return sa::plan_attn_bf16(rows, heads, kmax).ws_bytes;
}

int sparse_attn_decode(int dtype, const void *q, const void *k_cache, const void *v_cache, int64_t n_ctx,
                       const int32_t *idx, const int32_t *nsel, int32_t kmax, const float *sinks, float scale,
                       int32_t B, int32_t H, int32_t D, float *out, void *ws, size_t ws_bytes, void *stream) {
    return run_attn(dtype, q, k_cache, v_cache, n_ctx, idx, nsel, kmax, sinks, scale, B, H, D, out, ws, ws_bytes,
                    stream, false);
}

int sparse_attn_prefill(int dtype, const void *q, const void *k_cache, const void *v_cache, int64_t n_ctx,
                        const int32_t *idx, const int32_t *nsel, int32_t kmax, const float *sinks, float scale,
                        int32_t T, int32_t H, int32_t D, float *out, void *ws, size_t ws_bytes, void *stream) {
    return run_attn(dtype, q, k_cache, v_cache, n_ctx, idx, nsel, kmax, sinks, scale, T, H, D, out, ws, ws_bytes,
                    stream, true);
}

int sparse_attn_topk(const float *scores, int64_t rows, int64_t n, int64_t ld, const int32_t *valid_len, int32_t k,
                     int32_t *idx_out, int32_t *count_out, void *ws, size_t ws_bytes, void *stream) {
    (void)ws;
    if (rows < 0 || rows > kMaxGrid) return fail(SA_ERR_SHAPE, "rows %lld outside [0, 2^31)", (long long)rows);
    if (rows > 0 && (!scores || !idx_out)) return fail(SA_ERR_NULL, "scores and idx_out must be non-NULL");
    if (n < 0 || n > 0x7fffffff) return fail(SA_ERR_SHAPE, "n %lld outside [0, 2^31)", (long long)n);
    if (ld < n) return fail(SA_ERR_SHAPE, "ld %lld < n %lld", (long long)ld, (long long)n);
    if (k < 1) return fail(SA_ERR_SHAPE, "k %d must be >= 1", k);
    if (!aligned(scores, 4) || !aligned(idx_out, 4) || (valid_len && !aligned(valid_len, 4)) ||
        (count_out && !aligned(count_out, 4)))
        return fail(SA_ERR_UNSUPPORTED, "top-k arrays must be 4-byte aligned");
    const size_t need = sparse_attn_workspace_bytes(SA_OP_TOPK, rows, 0, 0, k, n);
    if (ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    sa::TopkArgs a{scores, rows, n, ld, valid_len, k, idx_out, count_out};
    const hipError_t e = sa::launch_topk(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int sparse_attn_pad_heads(int dtype, const void *q, int64_t rows, int32_t h_real, int32_t h_pad, int32_t D,
                          const float *sinks, void *q_pad, float *sinks_pad, void *stream) {
    if (!sinks || !sinks_pad || (rows > 0 && (!q || !q_pad)))
        return fail(SA_ERR_NULL, "q, sinks, q_pad and sinks_pad must be non-NULL");
    if (dtype != SA_BF16 && dtype != SA_F32) return fail(SA_ERR_UNSUPPORTED, "dtype %d", dtype);
    if (D != SA_HEAD_DIM) return fail(SA_ERR_UNSUPPORTED, "head width %d: only %d is implemented", D, SA_HEAD_DIM);
    if (h_real < 1 || h_pad < h_real || h_pad > SA_MAX_HEADS)
        return fail(SA_ERR_SHAPE, "need 1 <= h_real (%d) <= h_pad (%d) <= %d", h_real, h_pad, SA_MAX_HEADS);
    if (rows < 0 || rows > ((int64_t)1 << 40)) return fail(SA_ERR_SHAPE, "rows %lld", (long long)rows);
    if (!aligned(q, 16) || !aligned(q_pad, 16) || !aligned(sinks, 4) || !aligned(sinks_pad, 4))
        return fail(SA_ERR_UNSUPPORTED, "q and q_pad must be 16-byte aligned, sinks 4-byte aligned");
    const hipError_t e = sa::launch_pad_heads(dtype, q, rows, h_real, h_pad, sinks, q_pad, sinks_pad,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int sparse_attn_unpad_heads(const float *out_pad, int64_t rows, int32_t h_pad, int32_t h_real, int32_t D,
                            float *out, void *stream) {
    if (rows > 0 && (!out_pad || !out)) return fail(SA_ERR_NULL, "out_pad and out must be non-NULL");
    if (D != SA_HEAD_DIM) return fail(SA_ERR_UNSUPPORTED, "head width %d: only %d is implemented", D, SA_HEAD_DIM);
    if (h_real < 1 || h_pad < h_real || h_pad > SA_MAX_HEADS)
        return fail(SA_ERR_SHAPE, "need 1 <= h_real (%d) <= h_pad (%d) <= %d", h_real, h_pad, SA_MAX_HEADS);
    if (rows < 0 || rows > ((int64_t)1 << 40)) return fail(SA_ERR_SHAPE, "rows %lld", (long long)rows);
    if (!aligned(out_pad, 16) || !aligned(out, 16)) return fail(SA_ERR_UNSUPPORTED, "out_pad and out must be 16-byte aligned");
    const hipError_t e = sa::launch_unpad_heads(out_pad, rows, h_pad, h_real, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
