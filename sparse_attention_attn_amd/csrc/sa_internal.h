// sa_internal.h -- declarations shared by the library's own translation units
// (host API layer and HIP kernel files). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Arguments of one attention launch (decode or prefill; the kernels are the same).
struct AttnArgs {
    const void *q;          // [rows, H, 512]
    const void *k;          // cache base; row r's cache starts at r * cache_stride elements
    const void *v;
    int64_t cache_stride;   // elements between consecutive rows' caches (0: one shared cache)
    int64_t n_ctx;          // rows in each cache
    const int32_t *idx;     // [rows, kmax]
    const int32_t *nsel;    // [rows] or nullptr
    int32_t kmax;
    const float *sinks;     // [H]
    float scale;
    int32_t rows;
    int32_t H;
    float *out;             // [rows, H, 512]
};

struct TopkArgs {
    const float *scores;    // [rows, ld]
    int64_t rows, n, ld;
    const int32_t *valid_len;
    int32_t k;
    int32_t *idx_out;       // [rows, k]
    int32_t *count_out;     // [rows] or nullptr
};

// Enqueue helpers; they assume validated arguments and return the HIP launch status.
// launch_attn_bf16 runs the aliased-cache kernel when a.k == a.v (one cache serving as keys
// and values: each selected row is gathered once).
hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t s);
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
hipError_t launch_pad_heads(int dtype, const void *q, int64_t rows, int h_real, int h_pad,
                            const float *sinks, void *q_pad, float *sinks_pad, hipStream_t s);
hipError_t launch_unpad_heads(const float *out_pad, int64_t rows, int h_pad, int h_real, float *out,
                              hipStream_t s);

// Launch geometry of the bf16 attention kernel for a given problem (exposed for the
// host-side tests through sparse_attn_plan in the API layer).
struct AttnPlan {
    int heads_per_wg;       // 16, 32 or 64
    int cols_per_wg;        // 64, 128, 256 or 512
    int64_t units;          // (row, head group, column slice) work units; the launch runs
                            // min(units, compute units) persistent workgroups over them
    int threads;            // per workgroup
    int lds_bytes;          // static LDS per workgroup, separate K and V caches
    int lds_bytes_aliased;  // the same for one cache serving as both
};
AttnPlan plan_attn_bf16(int64_t rows, int H);

// Compute units of the current device, cached per device (256 if the query fails).
int device_cu_count();

}  // namespace sa
