// sa_attn_split.hip -- the bf16 attention path for small batches: the keys of a row are split
// across workgroups for the score contraction, and the softmax and value products then fold the
// score tiles in key order. Same results, bit for bit, as the persistent kernels of sa_attn.hip.
//
// What it computes is the same as sa_attn.hip (akol1/TensorFold pull request 4, "DeepSeek V4.1:
// sparse attention on eight SIMD groups, the same bytes", first commit message: 64-key tiles,
// running maximum, tile sum, value sum; TensorFold pull request 1206, "What changes": a sink per
// head). The ds4 commit log for ds4_tp.c (the attention split of 8 against 32 groups) shows
// why a split may not follow the launch: its outputs changed with the group count. Here the
// split is the 64-key tile, a constant of the method, and no arithmetic changes with it.
//
// Why: a row of the decode shape (64 heads, k = 640) is ten 64-key tiles. In the persistent
// kernels one workgroup walks them in a chain, each tile waiting twice for rows gathered from
// HBM, so a launch of one or a few rows takes about 30 us whatever the chip's size. Here:
//   1. attn_split_scores_kernel: one workgroup per (row, tile, block of 64 heads). Its eight
//      waves gather the tile's 64 K rows once and compute the score MFMA chain exactly as the
//      persistent kernel does (same wave roles: key half kh = w >> 2, 16-head group w & 3; same
//      K slot order and operand layout), then store each wave's raw scores, in its lane layout,
//      to the workspace: [row][tile][16-head group][key half][lane][8] fp32, 4 KiB per tile and
//      head group. All tiles of all rows run at once.
//   2. attn_split_values_kernel: one workgroup per (row, 16-head group, 64-column slice). It
//      loads the row's index list, gathers the V column slices of a round of up to ten tiles
//      and their score tiles into LDS in one go, then runs, per wave (key half kh = w >> 2,
//      16-column part w & 3), the same online-softmax steps and value MFMAs on each tile in
//      order (the four waves of a key half share the weights), and the same fixed-order fold of
//      the two key halves (sa_attn_common.h).
// Every (row, head, column) thus sees the same operations, on the same operands, in the same
// order as in the persistent kernels: which path a launch takes never changes its bits.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_attn_common.h"
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kSplitCols = 64;                 // output columns per values workgroup
constexpr int kSplitSlices = kHeadDim / kSplitCols;
constexpr int kVRowB = kSplitCols * 2;         // bytes of a V row slice
constexpr int kVTileB = kTile * kVRowB;        // one tile's V slices: 8 KiB
constexpr int kSTileB = 2 * 64 * 8 * 4;        // one tile's scores for a 16-head group: 4 KiB
constexpr int kRing = 10;                      // tiles per round of the values kernel
static_assert(kSplitCols == 64 && kVRowB == 128, "the values kernel's waves own 16 columns each");

// Chunk swizzle of a V row slice in LDS (8 chunks of 16 bytes): the chunk c of the slice in
// slot s is stored at chunk c ^ (s & 7). The four keys one 16-lane group reads in a
// transposing read sit in four consecutive slots, which then use four different chunks.
__device__ __forceinline__ int vswz(int s) { return s & 7; }

// Score tiles: [row][tile][head group][key half][lane][8] fp32.
__device__ __forceinline__ size_t score_block(int64_t row, int tile, int hg, int ntiles_max, int n_hg) {
    return (((size_t)row * ntiles_max + tile) * n_hg + hg) * (kSTileB / 4);
}

// The row's count, by a scalar (constant address space) load: it waits on the scalar counter,
// not on the vector-memory counter that the gathers in flight hold.
__device__ __forceinline__ int row_count(const AttnArgs &a, int64_t row) {
    int n = a.nsel ? *(const __attribute__((address_space(4))) int32_t *)(a.nsel + row) : a.kmax;
    return n < 0 ? 0 : (n > a.kmax ? a.kmax : n);
}

// One workgroup per (row, tile, block of 64 heads), blocks fastest. A tile past the row's
// count has no selected key: its workgroup leaves at once (the values kernel never reads it).
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_split_scores_kernel(AttnArgs a, int ntiles_max, int n_hb, int n_hg) {
    __shared__ __attribute__((aligned(16))) char k_lds[kTile * kKStride];
    __shared__ int idx_lds[kWaves][64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int wi = w & 3;
    const int kh = w >> 2;
    const int64_t b = blockIdx.x;
    const int hb = (int)(b % n_hb);
    const int tile = (int)((b / n_hb) % ntiles_max);
    const int64_t row = b / ((int64_t)n_hb * ntiles_max);
    const int hg = 4 * hb + wi;

    // The query, the tile's index list and the row's count go out together (one memory round
    // trip); a tile past the count then leaves, once its loads have landed.
    bf16x8 qreg[16];
    float sink_unused;
    load_q_async(a, row, 16 * hg, g, l16, qreg, sink_unused);
    {
        const int p = tile * kTile + lane;
        const int pc = p < a.kmax ? p : a.kmax - 1;
        dma4(a.idx + row * a.kmax, (uint32_t)pc * 4u, lds_addr(&idx_lds[w][0]));
    }
    const int n = row_count(a, row);
    wait_vmcnt<0>();
    if (tile * kTile >= n) return;
    q_ready(qreg, sink_unused);
    __builtin_amdgcn_s_waitcnt(0);
    // Row to gather for entry tile*64 + lane, or -1 (masked or out of range: gathers zeros,
    // as in the persistent kernels; the values kernel marks a row with a live out-of-range
    // entry as NaN).
    const int iv_raw = idx_lds[w][lane];
    const bool live = tile * kTile + lane < n;
    const int iv = (live && iv_raw >= 0 && (int64_t)iv_raw < a.n_ctx) ? iv_raw : -1;

    // Wave w gathers tile keys 8w .. 8w+7 (its key half) into the K slots of the persistent
    // kernels: key 32kh + kap goes to slot 32kh + kslot_of_key(kap).
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)a.k + row * a.cache_stride * 2), 0, (int)(uint32_t)(a.n_ctx * kRowBytes), kBufferFlags);
#pragma unroll
    for (int i = 0; i < kRows; i++) {
        const int ij = __builtin_amdgcn_readlane(iv, kRows * w + i);
        const int slot = 32 * kh + kslot_of_key(8 * wi + i);
        dma16_buf(rk, ((uint32_t)ij << 10) + ((uint32_t)lane << 4), lds_addr((SA_LDS char *)k_lds + slot * kKStride));
    }
    wait_vmcnt<0>();
    lds_barrier();  // every wave's K rows have landed
    if (hg >= n_hg) return;

    const SA_LDS char *krow = (const SA_LDS char *)k_lds + (32 * kh + l16) * kKStride + 16 * g;
    f32x4 sacc0, sacc1;
    score_chain(krow, qreg, sacc0, sacc1, [](int) {});
    f32x4 *dst = (f32x4 *)((float *)a.ws + score_block(row, tile, hg, ntiles_max, n_hg) + (kh * 64 + lane) * 8);
    dst[0] = sacc0;
    dst[1] = sacc1;
}

// One workgroup per (row, 16-head group, 64-column slice), in an order that keeps the
// workgroups of one row and head group on one XCD (they read the same score tiles). Eight
// waves, two per SIMD: wave w takes key half kh = w >> 2 and the 16 columns cs*64 + 16(w & 3)
// .. +15 (one MFMA block). The four waves of a key half split a round's tiles for the
// expensive part of the online softmax (scaled scores, tile maxima, weights), share them
// through LDS, and each runs the cheap sequential parts (reference scan, tile sums) itself.
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_split_values_kernel(AttnArgs a, int ntiles_max, int n_hg) {
    __shared__ __attribute__((aligned(16))) char v_lds[kRing * kVTileB];
    // A tile's scores, then (same slot, same lane layout: 32 bytes per lane and key half) its
    // weights as the two bf16 parts of the value MFMA's P^T operand.
    __shared__ __attribute__((aligned(16))) char s_lds[kRing * kSTileB];
    __shared__ float mloc_lds[2][kRing][64];   // per key half and tile: the tile's maximum
    __shared__ float psum_lds[2][kRing][64];   // per key half and tile: the tile sum
    __shared__ int idx_lds[kSplitMaxK];
    __shared__ float meta_lds[4][3][16];
    __shared__ f32x4 xch_lds[4][64];
    __shared__ int bad_lds[kWaves];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int cq = w & 3;
    const int kh = w >> 2;
    // Residue (mod 4) of the round's tiles this wave weighs: the two waves of a SIMD (w and
    // w ^ 4) take different residues, so every SIMD weighs five of ten tiles.
    const int qv = (cq + 2 * kh) & 3;
    const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
    const int cs = (int)(u % kSplitSlices);
    const int hg = (int)((u / kSplitSlices) % n_hg);
    const int64_t row = u / ((int64_t)kSplitSlices * n_hg);
    const int head = 16 * hg + l16;

    // First memory round trip: the first round's score tiles, the row's index list (the first
    // ntiles_max * 64 entries, the offsets clamped to the row), the sink and the row's count,
    // all in flight together. Score tiles past the row's count are never written by the
    // scores kernel; reading them stays inside the workspace, and they are not used.
    const int nt_first = ntiles_max < kRing ? ntiles_max : kRing;
    const float *sws = (const float *)a.ws + score_block(row, 0, hg, ntiles_max, n_hg);
    const uint32_t v_base = lds_addr((SA_LDS char *)v_lds);
    const uint32_t s_base = lds_addr((SA_LDS char *)s_lds);
    // Each wave moves 512 bytes of every 4 KiB score tile, in two 256-byte pieces.
    auto issue_scores = [&](int t, int slot) {
        const uint32_t off = (uint32_t)t * (uint32_t)(n_hg * kSTileB) + 512u * w + 4u * lane;
        dma4(sws, off, s_base + slot * kSTileB + 512 * w);
        dma4(sws, off + 256u, s_base + slot * kSTileB + 512 * w + 256);
    };
    for (int i = 0; i < nt_first; i++) issue_scores(i, i);
    // Index list: wave w moves tiles w and w + 8 (64 entries each) into LDS.
#pragma unroll
    for (int r = 0; r < 2; r++) {
        const int p = (w + 8 * r) * kTile + lane;
        const int pc = p < a.kmax ? p : a.kmax - 1;
        dma4(a.idx + row * a.kmax, (uint32_t)pc * 4u, lds_addr(&idx_lds[p - lane]));
    }
    float sink;
    load4_async(sink, head < a.H ? a.sinks + head : (const float *)g_zero_row);
    const int n = row_count(a, row);
    const int ntiles = (n + kTile - 1) / kTile;
    wait_vmcnt<0>();
    register_ready(sink);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // every wave's index pieces have landed

    HalfState st;
    f32x4 acc[1];
    half_start(st, acc, kh == 0, sink);
    const float scale2 = a.scale * kLog2e;

    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)a.v + row * a.cache_stride * 2 + (int64_t)cs * kVRowB), 0,
        (int)(uint32_t)(a.n_ctx * kRowBytes - (int64_t)cs * kVRowB), kBufferFlags);
    // DMA lane roles: lane (r8, c) = (lane >> 3, lane & 7) moves chunk c ^ vswz(slot) of the
    // slice of tile key (and V slot) 8w + r8 to chunk c of that slot.
    const int dslot = 8 * w + (lane >> 3);
    const uint32_t dchunk = (uint32_t)((lane & 7) ^ vswz(dslot)) << 4;
    // Value operand: lane (g, l16) reads key 32kh + 8g + 4t2 + (l16 >> 2) of the tile at columns
    // 16cq + 4(l16 & 3) .. +3 of the slice (chunk 2cq + (l16 & 3)/2, 8 bytes in for odd l16);
    // the transposing read returns column 16cq + l16 of keys 8g + 4t2 + 0..3 of the half.
    uint32_t vaddr[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; t2++) {
        const int slot = 32 * kh + 8 * g + 4 * t2 + (l16 >> 2);
        const int chunk = 2 * cq + ((l16 & 3) >> 1);
        vaddr[t2] = (uint32_t)(slot * kVRowB + 16 * (chunk ^ vswz(slot)) + 8 * (l16 & 1));
    }
    // An entry inside the count that is out of range makes the whole row NaN, as in the
    // persistent kernels (bad_w: one of this wave's entries is); masked entries (past the
    // count) gather zeros.
    bool bad_w = false;

    for (int t0 = 0; t0 < ntiles; t0 += kRing) {
        const int nt = ntiles - t0 < kRing ? ntiles - t0 : kRing;
        // Second memory round trip: the round's V slices (and, after the first round, its
        // score tiles). The round's index entries are read from LDS first, so that the gathers
        // then go out back to back.
        if (t0 > 0)
            for (int i = 0; i < nt; i++) issue_scores(t0 + i, i);
        int raw[kRing];
#pragma unroll
        for (int i = 0; i < kRing; i++) {
            const int p = (t0 + i) * kTile + dslot;
            raw[i] = (i < nt && p < n) ? idx_lds[p] : -1;
        }
#pragma unroll
        for (int i = 0; i < kRing; i++) {
            if (i < nt) {
                const int p = (t0 + i) * kTile + dslot;
                const bool inr = raw[i] >= 0 && (int64_t)raw[i] < a.n_ctx;
                bad_w = bad_w || __builtin_amdgcn_ballot_w64(p < n && !inr) != 0;
                const int iv = inr ? raw[i] : -1;  // -1: an offset past the range, zeros
                dma16_buf(rv, ((uint32_t)iv << 10) + dchunk, v_base + i * kVTileB + w * 1024);
            }
        }
        wait_vmcnt<0>();
        lds_barrier();  // every wave's slices and score pieces have landed

        // Phase 1: scaled scores and the tile maximum of this wave's tiles of the round (qv,
        // qv + 4, qv + 8); the maxima go to LDS for the reference scan. Every LDS read of a phase
        // goes out before the first use (a slot past the round's tiles is read and not used), so
        // the reads' latencies overlap instead of adding up tile by tile.
        constexpr int kMine = (kRing + 3) / 4;
        float sk[kMine][8];
        f32x4 sraw[kMine][2];
#pragma unroll
        for (int j = 0; j < kMine; j++) {
            const int i = qv + 4 * j < kRing ? qv + 4 * j : kRing - 1;
            const SA_LDS f32x4 *sp = lds_at<f32x4>(s_base + i * kSTileB + (kh * 64 + lane) * 32);
            sraw[j][0] = sp[0];
            sraw[j][1] = sp[1];
        }
#pragma unroll
        for (int j = 0; j < kMine; j++) {
            const int i = qv + 4 * j;
            if (i < nt) {
                const int t = t0 + i;
                mloc_lds[kh][i][lane] = tile_scores(sraw[j][0], sraw[j][1], t * kTile + 32 * kh + 8 * g, n,
                                                    (t + 1) * kTile <= n, scale2, sk[j]);
            }
        }
        lds_barrier();
        // Phase 2: the reference scan over the round's tiles in key order (every wave of a key
        // half computes the same values), then the weights of this wave's tiles against their
        // references, written over their scores.
        float ref_t[kRing], refp_t[kRing], mloc_t[kRing];
        uint32_t resc = 0;
#pragma unroll
        for (int i = 0; i < kRing; i++) mloc_t[i] = mloc_lds[kh][i][lane];
#pragma unroll
        for (int i = 0; i < kRing; i++) {
            if (i < nt) {
                float rp;
                const bool r = tile_reference(st, mloc_t[i], rp);
                ref_t[i] = st.ref;
                refp_t[i] = rp;
                resc |= (uint32_t)r << i;
            }
        }
#pragma unroll
        for (int j = 0; j < kMine; j++) {
            const int i = qv + 4 * j;
            if (i < nt) {
                // ref_t[qv + 4j], picked with static indices
                float ref = ref_t[4 * j];
#pragma unroll
                for (int q = 1; q < 4; q++)
                    if (4 * j + q < kRing && qv == q) ref = ref_t[4 * j + q < kRing ? 4 * j + q : 0];
                bf16x8 ph, pl;
                const float psum = tile_weights(sk[j], ref, ph, pl);
                SA_LDS bf16x8 *pp = (SA_LDS bf16x8 *)lds_at<bf16x8>(s_base + i * kSTileB + (kh * 64 + lane) * 32);
                pp[0] = ph;
                pp[1] = pl;
                psum_lds[kh][i][lane] = psum;
            }
        }
        lds_barrier();
        // Phase 3: tile sums, rescales and value MFMAs in key order. The tile sums are read up
        // front, and each tile's weights and value operand one tile ahead of its MFMAs.
        float psum_t[kRing];
#pragma unroll
        for (int i = 0; i < kRing; i++) psum_t[i] = psum_lds[kh][i][lane];
        auto operands = [&](int i, bf16x8 &ph, bf16x8 &pl, bf16x8 &vop) {
            const SA_LDS bf16x8 *pp = lds_at<bf16x8>(s_base + i * kSTileB + (kh * 64 + lane) * 32);
            ph = pp[0];
            pl = pp[1];
            const uint32_t vt = v_base + i * kVTileB;
            const bf16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4 *)lds_at<bf16x4>(vt + vaddr[0]));
            const bf16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4 *)lds_at<bf16x4>(vt + vaddr[1]));
            vop = (bf16x8){r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        };
        bf16x8 ph_c, pl_c, v_c;
        operands(0, ph_c, pl_c, v_c);
#pragma unroll
        for (int i = 0; i < kRing; i++) {
            if (i < nt) {
                bf16x8 ph_n = ph_c, pl_n = pl_c, v_n = v_c;
                if (i + 1 < kRing) operands(i + 1, ph_n, pl_n, v_n);
                const bool r = (resc >> i) & 1u;
                const float alpha = tile_alpha(r, st.l, refp_t[i], ref_t[i]);
                tile_accumulate(st, r, alpha, psum_t[i], acc);
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_c, ph_c, acc[0], 0, 0, 0);
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_c, pl_c, acc[0], 0, 0, 0);
                ph_c = ph_n;
                pl_c = pl_n;
                v_c = v_n;
            }
        }
        lds_barrier();  // every wave is done with this round's buffers
    }

    // Fold of the two key halves (half 0, half 1) and store: half 1 hands its state to half 0.
    if (kh == 1) {
        if (g == 0) {
            meta_lds[cq][0][l16] = st.m;
            meta_lds[cq][1][l16] = st.ref;
            meta_lds[cq][2][l16] = st.l;
        }
        xch_lds[cq][lane] = acc[0];
    }
    if (lane == 0) bad_lds[w] = bad_w;
    lds_barrier();
    if (kh == 0 && head < a.H) {
        bool bad = false;
#pragma unroll
        for (int i = 0; i < kWaves; i++) bad = bad || bad_lds[i] != 0;
        const uint64_t bad_mask = __builtin_amdgcn_readfirstlane(bad ? 1 : 0) ? ~0ull : 0ull;
        const HalfFold f = fold_scales(st.m, st.ref, st.l, meta_lds[cq][0][l16], meta_lds[cq][1][l16],
                                       meta_lds[cq][2][l16]);
        const f32x4 x1 = xch_lds[cq][lane];
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = fold_elem(f, acc[0][e], x1[e], bad_mask);
        // Lane (g, l16): head 16hg + l16, columns cs*64 + 16cq + 4g + 0..3.
        float *dst = a.out + (row * a.H + head) * kHeadDim + cs * kSplitCols + 16 * cq + 4 * g;
        __builtin_nontemporal_store(o, (f32x4 *)dst);
    }
}

}  // namespace

hipError_t launch_attn_split(const AttnArgs &a, hipStream_t s) {
    const int ntiles_max = (a.kmax + kTile - 1) / kTile;
    const int n_hg = (a.H + 15) / 16;
    const int n_hb = (n_hg + 3) / 4;
    const int64_t g1 = (int64_t)a.rows * ntiles_max * n_hb;
    const int64_t g2 = (int64_t)a.rows * n_hg * kSplitSlices;
    if (g1 == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_split_scores_kernel, dim3((unsigned)g1), dim3(512), 0, s, a, ntiles_max, n_hb, n_hg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_split_values_kernel, dim3((unsigned)g2), dim3(512), 0, s, a, ntiles_max, n_hg);
    return hipGetLastError();
}

size_t split_workspace_bytes(int64_t rows, int H, int32_t kmax) {
    const int64_t ntiles_max = (kmax + kTile - 1) / kTile;
    const int64_t n_hg = (H + 15) / 16;
    return (size_t)(rows * ntiles_max * n_hg) * kSTileB;
}

}  // namespace sa
