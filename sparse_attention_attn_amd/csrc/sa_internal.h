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
    void *ws;               // workspace of the split path (score tiles), or nullptr
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

// Launch geometry of the bf16 attention for a given problem. Small batches take the split
// path (sa_attn_split.hip, one launch): the score contraction of every 64-key tile in its own
// workgroup, the scores through the workspace, then the softmax and values per (row, 16-head
// group, 64-column slice). Larger ones take the persistent kernels (sa_attn.hip). Both give
// the same bits, so the choice is free to follow the batch size.
struct AttnPlan {
    int split;              // 1: the split path
    int heads_per_wg;       // persistent kernels: 16, 32 or 64
    int cols_per_wg;        // persistent kernels: 64, 128, 256 or 512
    int64_t units;          // persistent kernels: (row, head group, column slice) work units; the
                            // launch runs min(units, compute units) workgroups over them
    int threads;            // per workgroup
    int lds_bytes;          // static LDS per workgroup, separate K and V caches
    int lds_bytes_aliased;  // the same for one cache serving as both
    size_t ws_bytes;        // workspace the launch needs (0 for the persistent kernels)
};
// The split path takes rows whose index lists hold at most kSplitMaxK entries (a consumer
// workgroup keeps a row's list in LDS), when there are fewer than kSplitMaxUnits (row, 64-head
// block) pairs: measured on the decode shape (64 heads, k = 640, back-to-back launches), it
// takes 11 us at 1 row, 15 at 8, 23 at 16 and 35 at 23 against 31-38 us for the persistent
// kernels, and breaks even near 24 rows. This choice depends on the sizes only, never on the
// device, so that the workspace a call needs does too.
constexpr int kSplitMaxK = 1024;
constexpr int64_t kSplitMaxUnits = 24;
AttnPlan plan_attn_bf16(int64_t rows, int H, int32_t kmax);
size_t split_workspace_bytes(int64_t rows, int H, int32_t kmax);
hipError_t launch_attn_split(const AttnArgs &a, hipStream_t s);

// The float32 split path (sa_attn_f32_split.hip) for small batches: launches with fewer than
// kF32SplitMaxUnits (row, 64-head block) pairs and index lists of more than kF32SplitMinK (and
// at most kSplitMaxK) entries, a subset of the bf16 split's launches, so that
// sparse_attn_workspace_bytes, which has no dtype, stays an upper bound. Measured on 64 heads at
// k = 640 over 4,096 positions: 22 us at 1 row, 57 at 16 and 75-77 at 17-23 rows, against about
// 86 us for attn_f32_kernel at 17-23 rows (each workgroup a chain of twenty 32-key tiles), so the
// float32 split takes every launch the bf16 split takes. Index lists of at most four tiles are
// as fast in attn_f32_kernel. The score tiles take rows x ceil(kmax / 32) x ceil(H / 16) x
// 2 KiB of workspace, never more than the bf16 split's. Both float32 paths give the same bits.
constexpr int64_t kF32SplitMaxUnits = 24;
constexpr int32_t kF32SplitMinK = 128;
static_assert(kF32SplitMaxUnits <= kSplitMaxUnits, "the float32 split's launches are the bf16 split's");
bool f32_split_applies(int64_t rows, int H, int32_t kmax);
size_t f32_split_workspace_bytes(int64_t rows, int H, int32_t kmax);
hipError_t launch_attn_f32_split(const AttnArgs &a, hipStream_t s);

// Compute units of the current device, cached per device (256 if the query fails).
int device_cu_count();

// The validated decode call behind sparse_attn_decode (for the allocation-free variant in
// sa_noalloc.hip), its validation alone (nothing enqueued, no HIP call), and a way for that file
// to set the calling thread's last error.
int check_decode(int dtype, const void *q, const void *k_cache, const void *v_cache, int64_t n_ctx, const int32_t *idx,
                 const int32_t *nsel, int32_t kmax, const float *sinks, float scale, int32_t B, int32_t H, int32_t D,
                 float *out, void *ws, size_t ws_bytes);
int run_decode(int dtype, const void *q, const void *k_cache, const void *v_cache, int64_t n_ctx, const int32_t *idx,
               const int32_t *nsel, int32_t kmax, const float *sinks, float scale, int32_t B, int32_t H, int32_t D,
               float *out, void *ws, size_t ws_bytes, void *stream);
int fail_with(int code, const char *msg);

}  // namespace sa
