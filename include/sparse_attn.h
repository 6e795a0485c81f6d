/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) gathered sparse-attention library.
 *
 * The operation (akol1/TensorFold pull request 4, "DeepSeek V4.1: sparse attention
 * on eight SIMD groups, the same bytes", first commit message): for each query
 * row and head, attend over a selected list of cached key/value rows, scored in
 * 64-key tiles against a 512-wide head made of sixteen 32-wide output column
 * groups, keeping a running maximum, a tile sum and a value sum in a fixed
 * order. Each head carries a sink logit (TensorFold pull request 1206, "What
 * changes": padded heads get zero sinks). The selected rows come from an indexer's
 * top-k (pull request 4 names the indexer's merge and finish, "the same picks").
 *
 * What each attention entry point returns, for row r, head h, with
 * n = nsel[r] (or kmax) selected cache rows i_0..i_{n-1}:
 *     s_j = scale * dot(q[r,h,:], K[c(r), i_j, :])
 *     o[r,h,:] = sum_j exp(s_j - M) V[c(r), i_j, :] / (exp(sink_h - M) + sum_j exp(s_j - M))
 * with M the maximum of sink_h and the s_j. The sink is an extra logit with a
 * zero value vector and is not multiplied by `scale`. c(r) = r for decode (each
 * row has its own cache) and 0 for prefill (all rows share one cache).
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller. The library
 *     allocates nothing, keeps no pointer after it returns and has no state
 *     apart from a per-thread last-error message.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream). Calls
 *     only enqueue kernels on it and never synchronise; results are ready once
 *     the caller has synchronised that stream.
 *   - A call with zero rows enqueues nothing and succeeds; its per-row arrays
 *     (and, for decode, the caches) may then be NULL.
 *   - Every argument is validated on the host before anything is enqueued. On
 *     error nothing is enqueued and no output is touched; the return value is
 *     one of the SA_ERR_* codes and sparse_attn_last_error() describes it.
 *   - Arrays are dense, row-major, with the shapes given below. q, k_cache,
 *     v_cache and out must be 16-byte aligned; idx, nsel, sinks, scores and the
 *     top-k outputs 4-byte aligned.
 *   - Device-data contract (cannot be checked on the host): an index outside
 *     [0, n_ctx) among a row's first nsel[r] entries makes that row's whole
 *     output (every head) NaN; the kernel never reads out of bounds for it.
 *     nsel[r] values are clamped to [0, kmax]. Duplicate indices count twice.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 2

/* Status codes. */
#define SA_OK 0
#define SA_ERR_NULL 1        /* a required pointer is NULL */
#define SA_ERR_SHAPE 2       /* a size is negative, zero where it must not be, or too large */
#define SA_ERR_UNSUPPORTED 3 /* valid but not implemented: head width != 512, dtype, alignment */
#define SA_ERR_WORKSPACE 4   /* workspace smaller than sparse_attn_workspace_bytes() */
#define SA_ERR_HIP 5         /* the HIP runtime reported an error while enqueueing */

/* Storage types of q, k_cache and v_cache. Accumulation and output are float32. */
#define SA_F32 0
#define SA_BF16 1

/* Operation ids for sparse_attn_workspace_bytes(). */
#define SA_OP_DECODE 0
#define SA_OP_PREFILL 1
#define SA_OP_TOPK 2

/* The only head width implemented: sixteen 32-wide output column groups. */
#define SA_HEAD_DIM 512
/* Largest number of heads one call accepts. */
#define SA_MAX_HEADS 128
/* Largest kmax (index-list length) one attention call accepts: the kernels address a row's
   list and its 64-key tiles with 32-bit offsets. */
#define SA_MAX_KMAX (1 << 24)
/* Largest n_ctx (cache positions) of a bf16 call: 4 GiB of cache per 1 KiB position row.
   Larger bf16 caches are refused with SA_ERR_UNSUPPORTED. */
#define SA_BF16_MAX_CTX 4194303
/* Largest n_ctx of a float32 call (2 KiB per position row). */
#define SA_F32_MAX_CTX 2097151

/* Returns SA_ABI_VERSION of the loaded library. */
int sparse_attn_abi_version(void);

/* Static description of a status code (never NULL). */
const char *sparse_attn_status_string(int status);

/* Detailed message for the last error returned on the calling thread ("" if none). */
const char *sparse_attn_last_error(void);

/*
 * Bytes of device workspace an attention call (op SA_OP_DECODE or SA_OP_PREFILL)
 * with these sizes needs; 0 for SA_OP_TOPK and for invalid sizes. Pass a buffer
 * of at least this size, 16-byte aligned, as ws / ws_bytes (NULL / 0 when it is
 * 0). The workspace is scratch for the call's kernels only: whatever it held
 * before a call never changes the result, the caller needs neither to clear it
 * nor to keep it, and two calls in flight at once (on different streams) need
 * different workspaces.
 *
 * Small batches (fewer than 24 rows per block of 64 heads, index lists of at most
 * 1,024 entries) split the keys of every row across workgroups of one launch: each
 * 64-key tile is scored in its own workgroup and the raw scores and tile maxima go
 * through the workspace, before the softmax and value products fold them in key
 * order. The workspace holds 6 KiB of sequence and ready words (the launch's
 * workgroups wait on them; every call accepts any earlier contents), then
 * rows x ceil(kmax / 64) x ceil(heads / 16) x 4,224 bytes. Larger batches need no
 * workspace. A row's result is the same, bit for bit, on either path (the ds4
 * commit log for ds4_tp.c: a split that follows the launch must not change the
 * output bytes). On the bf16 split path a workgroup that waits more than 200 ms
 * for its row's scores (a device held by other work beyond any normal load) stops
 * waiting and writes its part of the row as NaN, so a call always completes.
 * Float32 launches with fewer than 17 rows per block of 64 heads and index lists
 * of 129 to 1,024 entries split the same way, with 32-key tiles of 2 KiB (rows x
 * ceil(kmax / 32) x ceil(heads / 16) x 2 KiB, never more than the bf16 figure).
 * The value depends only on (op, rows, heads, kmax) and covers both storage types.
 */
size_t sparse_attn_workspace_bytes(int op, int64_t rows, int32_t heads, int32_t head_dim,
                                   int32_t kmax, int64_t n_ctx);

/*
 * Decode: B independent sequences, each with its own cache (pull request 4,
 * first commit message: one attention per head and row).
 *   dtype     SA_BF16 or SA_F32: storage type of q, k_cache, v_cache
 *   q         [B, H, D]
 *   k_cache   [B, n_ctx, D]   row b's keys; may be the same pointer as v_cache
 *   v_cache   [B, n_ctx, D]
 *   idx       [B, kmax] int32 selected cache rows of each sequence
 *   nsel      [B] int32 number of valid entries of each idx row, or NULL (kmax for all)
 *   sinks     [H] float32 per-head sink logits
 *   scale     multiplies q.k (not the sinks)
 *   out       [B, H, D] float32
 *   ws        device workspace of ws_bytes >= sparse_attn_workspace_bytes(SA_OP_DECODE, B, H,
 *             D, kmax, n_ctx) bytes (SA_ERR_WORKSPACE if smaller); NULL when that is 0
 * Requires D == 512, 1 <= H <= 128, B >= 0, 1 <= kmax <= SA_MAX_KMAX, n_ctx >= 1
 * (n_ctx <= SA_BF16_MAX_CTX for SA_BF16, <= SA_F32_MAX_CTX for SA_F32).
 */
int sparse_attn_decode(int dtype, const void *q, const void *k_cache, const void *v_cache,
                       int64_t n_ctx, const int32_t *idx, const int32_t *nsel, int32_t kmax,
                       const float *sinks, float scale, int32_t B, int32_t H, int32_t D,
                       float *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Decode without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The same call as sparse_attn_decode, with the same results bit for bit, except that its
 * workspace is a static device array of the library, SA_NOALLOC_SCRATCH_BYTES per GPU, held
 * until the process ends. It allocates nothing. Every call on one GPU shares that GPU's
 * array: calls in flight at once on one GPU race and must not overlap. A call whose
 * workspace would exceed the array returns SA_ERR_WORKSPACE before anything is enqueued.
 */
#define SA_NOALLOC_SCRATCH_BYTES (8u << 20)
int sparse_attn_decode_noalloc(int dtype, const void *q, const void *k_cache, const void *v_cache,
                               int64_t n_ctx, const int32_t *idx, const int32_t *nsel, int32_t kmax,
                               const float *sinks, float scale, int32_t B, int32_t H, int32_t D,
                               float *out, void *stream);

/*
 * Prefill: T query rows over ONE shared cache (TensorFold pull request 1206,
 * "What changes": a prefill segment runs the 32-head attention for all its rows).
 * Identical to decode except that every row reads the same cache:
 *   q         [T, H, D]
 *   k_cache   [n_ctx, D], v_cache [n_ctx, D]
 *   idx       [T, kmax], nsel [T] or NULL; a causal caller keeps row t's indices <= its position
 *   out       [T, H, D] float32
 *   ws        as for decode, sized by sparse_attn_workspace_bytes(SA_OP_PREFILL, T, ...)
 * Each row's result equals what decode returns for that row with the shared
 * cache as its own (the same kernel runs both).
 */
int sparse_attn_prefill(int dtype, const void *q, const void *k_cache, const void *v_cache,
                        int64_t n_ctx, const int32_t *idx, const int32_t *nsel, int32_t kmax,
                        const float *sinks, float scale, int32_t T, int32_t H, int32_t D,
                        float *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Exact top-k of each row of indexer scores (pull request 4 names the indexer's
 * merge and finish per row with "the same picks"; selection is exact with ties
 * going to the lower position).
 *   scores     [rows, ld] float32; row r's candidates are positions [0, valid_len[r])
 *   valid_len  [rows] int32 or NULL (n for every row); values are clamped to [0, n]
 *   k          positions to select per row, k >= 1
 *   idx_out    [rows, k] int32: the selected positions in ascending order, then -1
 *   count_out  [rows] int32 or NULL: min(k, valid_len[r])
 * Order used: larger score first; NaN below -inf; -0 equal to +0; equal scores
 * by lower position. Requires rows >= 0, n >= 0, ld >= n, n < 2^31.
 */
int sparse_attn_topk(const float *scores, int64_t rows, int64_t n, int64_t ld,
                     const int32_t *valid_len, int32_t k, int32_t *idx_out, int32_t *count_out,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Head padding (TensorFold pull request 1206, "What changes": the real queries
 * go into a zero-padded 32-head buffer, the extra sinks are zero, and the real
 * output groups are copied out afterwards).
 * sparse_attn_pad_heads copies q [rows, h_real, D] into q_pad [rows, h_pad, D]
 * with heads h_real..h_pad-1 zero, and sinks [h_real] into sinks_pad [h_pad]
 * with the extra sinks zero. Requires 1 <= h_real <= h_pad <= 128, D == 512.
 */
int sparse_attn_pad_heads(int dtype, const void *q, int64_t rows, int32_t h_real, int32_t h_pad,
                          int32_t D, const float *sinks, void *q_pad, float *sinks_pad,
                          void *stream);

/* Copies heads 0..h_real-1 of out_pad [rows, h_pad, D] (float32) into out [rows, h_real, D]. */
int sparse_attn_unpad_heads(const float *out_pad, int64_t rows, int32_t h_pad, int32_t h_real,
                            int32_t D, float *out, void *stream);

/*
 * Measurement only (not part of the method): the decode kernels' gathers alone. For each of
 * `rows` sequences with caches k_cache / v_cache [rows, n_ctx, 512] bf16, reads the K and V
 * rows that idx [rows, kmax] selects (an index outside [0, n_ctx) reads nothing) with the same
 * direct-to-LDS DMAs as sparse_attn_decode, rows_in_flight (8 or 16) of each per wave, and
 * discards them. Its duration over a batch is the most the decode kernels could reach for that
 * access pattern; benchmarks report the decode rate against it next to the HBM peak.
 */
int sparse_attn_gather_probe(const void *k_cache, const void *v_cache, int64_t n_ctx,
                             const int32_t *idx, int32_t rows, int32_t kmax, int32_t rows_in_flight,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
