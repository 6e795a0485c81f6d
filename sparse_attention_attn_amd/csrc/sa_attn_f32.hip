// sa_attn_f32.hip -- gathered sparse attention with per-head sinks for float32 inputs, on the
// float32 matrix cores (v_mfma_f32_16x16x4_f32).
//
// What it computes: akol1/TensorFold pull request 4 ("DeepSeek V4.1: sparse attention on eight
// SIMD groups, the same bytes"), first commit message: the selected keys are scored in tiles
// against a 512-wide head, with a running maximum, a tile sum and a value sum in a fixed order;
// TensorFold pull request 1206, "What changes": a sink logit per head. Everything stays in float32
// (the weights are never rounded to a narrower type), which is what the 1e-5 bound on float32
// inputs needs.
//
// How it maps to CDNA4. One workgroup serves one query row and one group of 16 heads, so every
// selected cache row is gathered from HBM once for 16 heads (the key/value latent is shared by
// all heads), not once per head. A tile is 32 keys (a float32 row is 2 KiB: a 32-row K tile and
// a 32-row V tile fill 128 KiB of LDS). Eight waves, two per SIMD:
//   * Scores S^T = K Q^T, 16 keys x 16 heads per block, two blocks per tile: wave w computes block
//     b = w & 1 over the dimension quarter dq = w >> 1 (32 MFMA steps of 4 dimensions) and leaves
//     the partial tile in LDS; each wave then sums the four partials in quarter order (one fixed
//     reduction order). The contraction's k index runs over dimensions 128 g + kk for lane group g
//     and step kk, so that a lane reads four steps' K operands with one 16-byte LDS read.
//   * K slots are ordered so that lane group g's four scores of block b are keys g + 16b + 4j
//     (j < 4): the lane's eight scores are exactly the weights its value MFMA operand needs (the
//     operand's k index is key 4s + g at step s). No score or weight moves between lanes.
//   * Every wave computes the tile's online-softmax step for its 16 heads (the same values in all
//     waves): tile maximum over 32 keys (in-lane, then two lane swaps), m' = max(m, tile max),
//     reference r = m' (0 if m' = -inf), alpha = exp(m - r), p = exp(s - r), l = alpha l + sum p,
//     acc = alpha acc + P V. It starts from m = sink, l = exp(sink - r(sink)).
//   * Values O^T = V^T P^T: wave w owns 64 of the 512 columns (four 16-column blocks), 8 MFMA steps
//     of 4 keys per block and tile.
// Tile j+1's K rows are gathered during tile j's softmax and values, tile j's V rows during its
// scores. Keys past a row's count, and out-of-range indices, gather zeros through the buffer
// range (an out-of-range index inside the count makes the row NaN).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_attn_f32_common.h"
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kVStrF = kRowF + 64;         // V row stride: the four lane groups' rows on four bank windows
constexpr int kWavesF = 8;
static_assert(kT32 * kKStrF + kT32 * kVStrF + kWavesF * 4 * 64 * 4 <= 160 * 1024, "LDS budget");

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_f32_kernel(AttnArgs a, int n_hg) {
    __shared__ __attribute__((aligned(16))) char k_lds[kT32 * kKStrF];
    __shared__ __attribute__((aligned(16))) char v_lds[kT32 * kVStrF];
    __shared__ f32x4 part_lds[4][2][64];   // [dimension quarter][block][lane]
    __shared__ int bad_lds[kWavesF];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int b_own = w & 1;
    const int dq = w >> 1;
    // XCD-aware order (each XCD takes every eighth workgroup id; xcd_remap gives it a contiguous
    // range of units): the head groups of one row run on one XCD, so that their gathers of the
    // same cache rows share that XCD's L2 instead of each fetching them from beyond it.
    const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t row = u / n_hg;
    const int hg = (int)(u % n_hg);
    const int head = 16 * hg + l16;
    const bool head_ok = head < a.H;

    int n = a.nsel ? a.nsel[row] : a.kmax;
    n = n < 0 ? 0 : (n > a.kmax ? a.kmax : n);
    const int ntiles = (n + kT32 - 1) / kT32;
    const int32_t *irow = a.idx + row * a.kmax;

    // The query for this wave's dimension quarter: lane (g, l16) holds dims 128 g + 32 dq .. +31
    // of head 16 hg + l16 (zero for heads past H).
    float qv[32];
    {
        const float *qrow = (const float *)a.q + (row * a.H + (head_ok ? head : 0)) * kHeadDim + 128 * g + 32 * dq;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const f32x4 x = head_ok ? *(const f32x4 *)(qrow + 4 * i) : (f32x4){};
            qv[4 * i] = x[0];
            qv[4 * i + 1] = x[1];
            qv[4 * i + 2] = x[2];
            qv[4 * i + 3] = x[3];
        }
    }
    const float sink = head_ok ? a.sinks[head] : 0.0f;

    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)a.k + row * a.cache_stride * 4), 0, (int)(uint32_t)(a.n_ctx * kRowF), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)a.v + row * a.cache_stride * 4), 0, (int)(uint32_t)(a.n_ctx * kRowF), kBufferFlags);
    // Tile t's index list: lane l holds entry 32 t + (l & 31), loaded asynchronously (the
    // address clamped to the row) and resolved once an explicit wait covers it: -1 for a masked
    // or out-of-range entry, which gathers zeros; bad: a live entry is out of range.
    bool bad = false;
    auto load_idx = [&](int t, float &raw) {
        const int p = t * kT32 + (lane & 31);
        load4_async(raw, irow + (p < a.kmax ? p : a.kmax - 1));
    };
    auto resolve = [&](int t, float &raw) {
        register_ready(raw);
        const int p = t * kT32 + (lane & 31);
        const int iv = __float_as_int(raw);
        const bool live = p < n;
        const bool inr = iv >= 0 && (int64_t)iv < a.n_ctx;
        bad = bad || __builtin_amdgcn_ballot_w64(live && !inr) != 0;
        return (live && inr) ? iv : -1;
    };
    // Wave w gathers tile keys 4w .. 4w+3 of K (two 1 KiB DMAs per row) or of V.
    auto dma_k = [&](int iv) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int kap = 4 * w + i;
            const uint32_t off = ((uint32_t)__builtin_amdgcn_readlane(iv, kap) << 11) + ((uint32_t)lane << 4);
            const uint32_t dst = lds_addr((SA_LDS char *)k_lds + kslot32(kap) * kKStrF);
            dma16_buf(rk, off, dst);
            dma16_buf(rk, off + 1024u, dst + 1024u);
        }
    };
    auto dma_v = [&](int iv) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int kap = 4 * w + i;
            const uint32_t off = ((uint32_t)__builtin_amdgcn_readlane(iv, kap) << 11) + ((uint32_t)lane << 4);
            const uint32_t dst = lds_addr((SA_LDS char *)v_lds + kap * kVStrF);
            dma16_buf(rv, off, dst);
            dma16_buf(rv, off + 1024u, dst + 1024u);
        }
    };

    // Online-softmax state (per lane: head l16) and the wave's 64 output columns 64 w + 16 cb +
    // 4 g + 0..3 of head l16.
    float m = sink;
    float ref = f32_ref(sink);
    float l = expf(sink - ref);
    f32x4 acc[4] = {};

    float raw_next;
    int iv_cur = -1;
    if (ntiles > 0) {
        load_idx(0, raw_next);
        wait_vmcnt<0>();
        iv_cur = resolve(0, raw_next);
        dma_k(iv_cur);
    }
    const float scale = a.scale;
    // Per-lane LDS read bases. Scores: slot 16 b_own + l16, dims 128 g + 32 dq + 4i (16 bytes).
    const SA_LDS char *krow = (const SA_LDS char *)k_lds + (16 * b_own + l16) * kKStrF + (128 * g + 32 * dq) * 4;
    // Values: row (key) 4s + g, column 64 w + 16 cb + l16.
    const SA_LDS char *vrow = (const SA_LDS char *)v_lds + g * kVStrF + (64 * w + l16) * 4;

    for (int t = 0; t < ntiles; t++) {
        wait_vmcnt<0>();   // K(t) has landed (the only operations in flight)
        lds_barrier();     // every wave's K(t) rows have landed; every wave is done with V(t-1)
        const bool more = t + 1 < ntiles;
        if (more) load_idx(t + 1, raw_next);  // I(t+1), then V(t) during the scores
        dma_v(iv_cur);
        // ---- partial scores of block b_own over the dimension quarter dq
        f32x4 sp = {};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const f32x4 kx = *(const SA_LDS f32x4 *)(krow + 16 * i);
#pragma unroll
            for (int e = 0; e < 4; e++)
                sp = __builtin_amdgcn_mfma_f32_16x16x4f32(kx[e], qv[4 * i + e], sp, 0, 0, 0);
        }
        part_lds[dq][b_own][lane] = sp;
        lds_barrier();     // all partials are in LDS; every wave is done with K(t)
        int iv_next = -1;
        if (more) {
            wait_vmcnt<8>();  // I(t+1) has landed (after it: the eight V(t) gathers)
            iv_next = resolve(t + 1, raw_next);
            dma_k(iv_next);   // K(t+1), during the softmax and the values
        }
        // ---- scores: the four quarters in order; lane (g, l16): keys g + 4e of the tile
        float tot[8];
#pragma unroll
        for (int bb = 0; bb < 2; bb++) {
            const f32x4 p0 = part_lds[0][bb][lane], p1 = part_lds[1][bb][lane];
            const f32x4 p2 = part_lds[2][bb][lane], p3 = part_lds[3][bb][lane];
#pragma unroll
            for (int j = 0; j < 4; j++) tot[4 * bb + j] = f32_score_sum(p0[j], p1[j], p2[j], p3[j]);
        }
        float s[8];
        const float mt = f32_tile_scores(tot, t * kT32 + g, n, scale, s);
        const float m_new = fmaxf(m, mt);
        const float ref_new = f32_ref(m_new);
        const float alpha = expf(m - ref_new);
        float pe[8];
        const float psum = f32_tile_weights(s, ref_new, pe);
        l = f32_l_step(alpha, l, psum);
        m = m_new;
        ref = ref_new;
        // ---- values: V(t) has landed (after it only K(t+1) is in flight)
        if (more) wait_vmcnt<8>(); else wait_vmcnt<0>();
        lds_barrier();
        f32x4 tv[4] = {};
#pragma unroll
        for (int st = 0; st < 8; st++) {
#pragma unroll
            for (int cb = 0; cb < 4; cb++) {
                const float vx = *(const SA_LDS float *)(vrow + 4 * st * kVStrF + 64 * cb);
                tv[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vx, pe[st], tv[cb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int cb = 0; cb < 4; cb++) acc[cb] = f32_acc_step(acc[cb], alpha, tv[cb]);
        iv_cur = iv_next;
    }
    wait_vmcnt<0>();
    (void)ref;

    // Whole-row NaN for an out-of-range index (any wave saw one), else acc / l.
    if (lane == 0) bad_lds[w] = bad;
    lds_barrier();
    bool row_bad = false;
#pragma unroll
    for (int i = 0; i < kWavesF; i++) row_bad = row_bad || bad_lds[i] != 0;
    if (head_ok) {
        float *orow = a.out + (row * a.H + head) * kHeadDim + 64 * w + 4 * g;
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = row_bad ? __uint_as_float(0x7fc00000u) : acc[cb][e] / l;
            *(f32x4 *)(orow + 16 * cb) = o;
        }
    }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t s) {
    if (f32_split_applies(a.rows, a.H, a.kmax)) return launch_attn_f32_split(a, s);
    const int n_hg = (a.H + 15) / 16;
    const int64_t grid = (int64_t)a.rows * n_hg;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)grid), dim3(512), 0, s, a, n_hg);
    return hipGetLastError();
}

}  // namespace sa
