// sa_noalloc.hip -- sparse_attn_decode_noalloc: decode whose workspace is a static device array
// of this library, for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array (scratch, SA_NOALLOC_SCRATCH_BYTES) exists once per GPU that the library runs on and
// stays until the process ends. Its device address is looked up once per device, with that
// device current, by hipGetSymbolAddress; only that address is ever passed to a kernel (the
// array's name is a host-side stand-in on the host). Every call on one GPU shares the array, so
// two calls in flight at once on one GPU (on different streams, or from different threads) race.
// The kernels that use it are the bf16 and float32 split paths. The float32 path writes every
// byte it reads in the same call. The bf16 path also keeps sequence words there between calls,
// and accepts any earlier contents for them, so nothing has to be cleared between calls.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "sa_internal.h"
#include "sparse_attn.h"

namespace {

constexpr size_t kScratchBytes = SA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// This device's copy of scratch (the calling thread's current device, dev).
hipError_t scratch_on(int dev, void **ptr) {
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = p;
    });
    *ptr = g_scratch[dev];
    return g_scratch_err[dev];
}

}  // namespace

extern "C" int sparse_attn_decode_noalloc(int dtype, const void *q, const void *k_cache, const void *v_cache,
                                          int64_t n_ctx, const int32_t *idx, const int32_t *nsel, int32_t kmax,
                                          const float *sinks, float scale, int32_t B, int32_t H, int32_t D,
                                          float *out, void *stream) {
    // The workspace this call needs (run_decode validates every argument; sizes it would refuse
    // need none here).
    size_t need = 0;
    if (dtype == SA_BF16)
        need = sparse_attn_workspace_bytes(SA_OP_DECODE, B, H, D, kmax, n_ctx);
    else if (dtype == SA_F32 && B > 0 && H >= 1 && H <= SA_MAX_HEADS && kmax >= 1 && kmax <= SA_MAX_KMAX &&
             sa::f32_split_applies(B, H, kmax))
        need = sa::f32_split_workspace_bytes(B, H, kmax);
    if (need > kScratchBytes) {
        char msg[160];
        snprintf(msg, sizeof msg, "this call needs %zu bytes of workspace, more than the %zu of the static scratch",
                 need, kScratchBytes);
        return sa::fail_with(SA_ERR_WORKSPACE, msg);
    }
    // Every argument is checked before the scratch's address is looked up (a HIP call), so that
    // an invalid call reports its own status; the placeholder only stands for that address.
    void *const placeholder = reinterpret_cast<void *>(uintptr_t{256});
    const int rc = sa::check_decode(dtype, q, k_cache, v_cache, n_ctx, idx, nsel, kmax, sinks, scale, B, H, D, out,
                                    need > 0 ? placeholder : nullptr, need > 0 ? kScratchBytes : 0);
    if (rc != SA_OK) return rc;
    void *ws = nullptr;
    if (need > 0) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return sa::fail_with(SA_ERR_HIP, "no current HIP device (or its ordinal is 64 or more)");
        const hipError_t e = scratch_on(dev, &ws);
        if (e != hipSuccess || !ws) return sa::fail_with(SA_ERR_HIP, "the static scratch has no device address");
    }
    return sa::run_decode(dtype, q, k_cache, v_cache, n_ctx, idx, nsel, kmax, sinks, scale, B, H, D, out, ws,
                          need > 0 ? kScratchBytes : 0, stream);
}
