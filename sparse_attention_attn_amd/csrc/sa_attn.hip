// sa_attn.hip -- gathered sparse attention with per-head sinks, bf16 storage, for gfx950:
// every tile's keys split between two halves of an eight-wave workgroup. One kernel reads
// separate K and V caches, the other one cache serving as both (each selected row is then
// gathered once).
//
// What it computes: akol1/TensorFold pull request 4 ("DeepSeek V4.1: sparse attention on
// eight SIMD groups, the same bytes"), first commit message: for a query row and its heads,
// the selected keys are scored in 64-key tiles against a 512-wide head (sixteen 32-wide
// output column groups), with a running maximum, a tile sum and a value sum. TensorFold
// pull request 1206, "What changes": every head has a sink logit (zero for padded heads).
//
// How it maps to CDNA4 (this is not the pages' one-SIMD-group-per-head design):
//   * One workgroup serves one query row, a block of 16*HQ heads (HQ = 4, 2 or 1) and
//     512/NS output columns, on eight waves, two per SIMD, because the key/value latent is
//     shared by all heads of a row: each selected cache row is gathered from HBM once per
//     row, not once per head. Wave w takes key half kh = w>>2 of every 64-key tile (keys
//     32kh .. 32kh+31), and with wi = w&3, heads 16(wi % HQ) .. +15 of the block and column
//     quarter / half wi / HQ of the slice (one of 4/HQ). Each wave keeps its own online
//     softmax over its key half; at the end of a unit the two waves that hold the same
//     heads and columns combine their states through LDS, in a fixed order (half 0, half 1).
//   * S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16 with the 16 heads on
//     the N side. The query (16 heads x 512) stays in 64 registers, so every score is
//     contracted over the full head width inside one wave.
//   * K rows sit in the order that makes each lane's four scores of a 16-slot block, for
//     blocks 0 and 1, exactly the eight weights of its P^T operand (keys 8g .. 8g+7 of
//     lane group g). So no score, maximum, sum or weight crosses a wave inside a tile: the
//     row maximum and the tile sum are in-lane reductions plus two lane swaps
//     (v_permlane16_swap, v_permlane32_swap). The barriers left are those that hand a
//     gathered buffer from the waves that filled it to the waves that read it, and back.
//   * Gathers are index-driven direct-to-LDS DMAs through buffer resources (a masked key
//     reads zeros), issued one row at a time inside the MFMA loops.
//   * With fewer than four 16-head groups per block (HQ < 4), several waves of a key half
//     hold the same heads; each 16-key block of their score tile is then contracted by one
//     wave and handed to the others through LDS, so no score is computed twice.
//   * In these kernels, splitting work across workgroups or waves only ever splits heads and
//     output columns (every score is contracted over the whole head width in one wave); the
//     keys of a tile always go to the same two halves. The small-batch path
//     (sa_attn_split.hip) scores each 64-key tile in its own workgroup with the same score
//     chain and then runs the same per-tile steps in key order. So results are bit-identical
//     across launch shapes, head counts, paths and repeats, and the two kernels here give the
//     same bits on equal contents.
//
// Numerics, in log2 units (x2 = x * log2 e), per wave and 32-key half tile: m' = max(m,
// max_j s_j); the exponent reference r moves to m' (0 if m' = -inf) with alpha = 2^(r - r')
// (0 while nothing has been accumulated) when m' > r + 8 or r > m' > -inf for one of the
// wave's 16 heads, else alpha = 1; p_j = 2^(s_j - r) split into hi + lo, both bf16; l =
// alpha*l + sum_j (hi + lo); acc = alpha*acc + (hi + lo) V. Half 0 starts from the sink
// (m = sink, r = sink or 0 if -inf, l = 2^(sink - r)), half 1 from nothing (m = -inf, r = 0,
// l = 0). End: with R the reference of the half holding the larger maximum and a_h =
// 2^(r_h - R) (0 for a half with l = 0), out = (a_0 acc_0 + a_1 acc_1) / (a_0 l_0 + a_1 l_1).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "sa_attn_common.h"
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

// Row rotation by 8 inside each 16-lane row (DPP row_ror:8): lane l16 receives lane l16 ^ 8.
__device__ __forceinline__ float ror8(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
}

// End of a unit: combine the two key halves and store. The pair (w, w ^ 4) holds the same
// heads; wave kh finalises column blocks OWN*kh .. OWN*kh + OWN-1 in two rounds of OWN/2.
// Per round each wave writes the partner's blocks (16-byte pieces, lane-major) into its
// slot of xch (a free gathered buffer) and reads its own from the partner's slot. Lane
// (g, l16) then holds head l16, columns 16cb + 4g + 0..3 of every block. For a pair of
// blocks (2p, 2p+1) a DPP row rotation trades the halves of the 16-lane rows, so that one
// store writes whole 128-byte lines (columns 32p .. 32p+31) of heads 0..7 and the next of
// heads 8..15: lane (g, l16) stores head (l16 & 7) [+ 8], columns 32p + 4(g + 4(l16 >> 3)).
// The stores go through a buffer resource spanning the output row; a head past H stores
// past its end, which the hardware drops, so every wave issues exactly OWN stores.
template <int KH, int CB>
__device__ __forceinline__ void combine_store(const HalfState &st, const f32x4 (&acc)[CB], float (*meta)[3][16],
                                              f32x4 *xch, int w, int lane, int g, int l16, float *orow, int H,
                                              int head0, int col0, bool bad) {
    constexpr int OWN = CB / 2;
    constexpr int HALF = OWN / 2;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(orow, 0, H * kHeadDim * 4, kBufferFlags);
    if (g == 0) {
        meta[w][0][l16] = st.m;
        meta[w][1][l16] = st.ref;
        meta[w][2][l16] = st.l;
    }
    const uint64_t bad_mask = __builtin_amdgcn_readfirstlane(bad ? 1 : 0) ? ~0ull : 0ull;
    const bool lo_row = l16 < 8;
    // Output addresses. One block: head head0 + l16, columns col0 + 16cb + 4g. A pair:
    // heads head0 + (l16 & 7) and + 8, columns col0 + 32p + 4(g + 4(l16 >> 3)).
    const int h1 = head0 + l16;
    const int hA = head0 + (l16 & 7), hB = hA + 8;
    const int base1 = h1 < H ? (h1 * kHeadDim + col0 + 4 * g) * 4 : -1;
    const int baseA = hA < H ? (hA * kHeadDim + col0 + 4 * (g + 4 * (l16 >> 3))) * 4 : -1;
    const int baseB = hB < H ? (hB * kHeadDim + col0 + 4 * (g + 4 * (l16 >> 3))) * 4 : -1;
    auto at = [](int base, int bytes) { return base < 0 ? kDropOffset : base + bytes; };
    HalfFold fold{0.0f, 0.0f, 1.0f};
#pragma unroll
    for (int r = 0; r < 2; r++) {
        // Round 0: every wave is past its value products (the buffer is free).
        // Round 1: every partner has read round 0.
        lds_barrier();
#pragma unroll
        for (int i = 0; i < HALF; i++) xch[(w * HALF + i) * 64 + lane] = acc[OWN * (1 - KH) + r * HALF + i];
        lds_barrier();
        if (r == 0) {
            const int p = w ^ 4;
            const float mp = meta[p][0][l16], rp = meta[p][1][l16], lp = meta[p][2][l16];
            const float m0 = KH ? mp : st.m, r0 = KH ? rp : st.ref, l0 = KH ? lp : st.l;
            const float m1 = KH ? st.m : mp, r1 = KH ? st.ref : rp, l1 = KH ? st.l : lp;
            fold = fold_scales(m0, r0, l0, m1, r1, l1);
        }
        auto finish = [&](int cb, const f32x4 &par) {
            const f32x4 own = acc[cb];
            const f32x4 x0 = KH ? par : own;
            const f32x4 x1 = KH ? own : par;
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = fold_elem(fold, x0[e], x1[e], bad_mask);
            return o;
        };
        // The partner reads go out four at a time ahead of their first use, so their LDS
        // latency overlaps instead of adding up block by block.
        constexpr int GRP = HALF < 4 ? HALF : 4;
#pragma unroll
        for (int i0 = 0; i0 < HALF; i0 += GRP) {
            f32x4 parts[GRP];
#pragma unroll
            for (int i = 0; i < GRP; i++) parts[i] = xch[((w ^ 4) * HALF + i0 + i) * 64 + lane];
            if constexpr (GRP >= 2) {
#pragma unroll
                for (int i = 0; i < GRP; i += 2) {
                    const int cb = OWN * KH + r * HALF + i0 + i;  // even
                    const f32x4 x = finish(cb, parts[i]);
                    const f32x4 y = finish(cb + 1, parts[i + 1]);
                    f32x4 sa, sb;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float xr = ror8(x[e]), yr = ror8(y[e]);
                        sa[e] = lo_row ? x[e] : yr;
                        sb[e] = lo_row ? xr : y[e];
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sa), rsrc, at(baseA, 64 * cb), 0,
                                                           kStoreNT);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sb), rsrc, at(baseB, 64 * cb), 0,
                                                           kStoreNT);
                }
            } else {
                const int cb = OWN * KH + r * HALF + i0;
                const f32x4 o = finish(cb, parts[0]);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rsrc, at(base1, 64 * cb), 0,
                                                       kStoreNT);
            }
        }
    }
}

// Work items shared by both kernels. A unit is one (query row, head group of 64, column
// slice); a workgroup serves units base, base + G, ... as one stream of 64-key tiles (at
// least one per unit; a row with no selected key runs one all-masked tile, which changes
// nothing). useq counts the units this workgroup has started, to tell whose bad-index
// flag a resolved list belongs to.
struct Item {              // all fields wave-uniform
    int64_t unit;          // < 0: none
    int64_t row;
    int tile, ntiles, n, hg, cs, useq;
};

template <int NS>
struct Stream {
    const AttnArgs &a;
    int n_hg;
    int64_t units, G;
    __device__ Item make(int64_t u, int useq) const {
        Item it{};
        it.unit = u;
        it.useq = useq;
        if (u < 0 || u >= units) { it.unit = -1; return it; }
        it.cs = (int)(u % NS);
        it.hg = (int)((u / NS) % n_hg);
        it.row = u / ((int64_t)NS * n_hg);
        // A scalar (constant address space) load: it waits on the LDS/scalar counter, not
        // on the vector-memory counter that the in-flight gathers hold.
        int n = a.nsel ? *(const __attribute__((address_space(4))) int32_t *)(a.nsel + it.row) : a.kmax;
        n = n < 0 ? 0 : (n > a.kmax ? a.kmax : n);
        it.n = n;
        it.tile = 0;
        it.ntiles = n > 0 ? (n + kTile - 1) / kTile : 1;
        return it;
    }
    __device__ Item next(const Item &it) const {
        if (it.unit < 0) return it;
        if (it.tile + 1 < it.ntiles) { Item nx = it; nx.tile++; return nx; }
        return make(it.unit + G, it.useq + 1);
    }
};

// Index list of an item's tile into one of this wave's LDS slots: lane l fetches entry
// tile*64 + l (address clamped to the row). Always issued, also when there is no item (then
// the fallback's list is re-read), so that every wave issues the same number of
// vector-memory operations per tile.
__device__ __forceinline__ void dma_idx(const AttnArgs &a, const Item &it, const Item &fallback, int *slot, int lane) {
    const Item &src = it.unit >= 0 ? it : fallback;
    const int p = (it.unit >= 0 ? it.tile : 0) * kTile + lane;
    const int pc = p < a.kmax ? p : a.kmax - 1;
    dma4(a.idx + src.row * a.kmax, (uint32_t)pc * 4u, lds_addr(slot));
}
// Row to gather for entry tile*64 + l, or -1 (masked or out of range: gather zeros); bad is
// set when a live entry (inside the row's count) is out of range.
__device__ __forceinline__ int resolve(const AttnArgs &a, const Item &it, const int *slot, int lane, bool &bad) {
    const int iv = slot[lane];
    const int p = it.tile * kTile + lane;
    const bool live = p < it.n;
    const bool inr = iv >= 0 && (int64_t)iv < a.n_ctx;
    bad = __builtin_amdgcn_ballot_w64(live && !inr) != 0;
    return (live && inr) ? iv : -1;
}

// ---------------------------------------------------------------------------------------
// Separate K and V caches. One K buffer and one V buffer of 64 rows each: V(j) is gathered
// while the scores of tile j run, K(j+1) while its values are applied. Two barriers per
// tile: "K(j) landed, V buffer free" and "V(j) landed, K buffer free".
// When every row reads one shared cache (prefill), tile j+1's rows are also prefetched into
// L2 as soon as its index list is resolved (mid tile j), so that their gathers mostly hit
// L2: 11-18% shorter at 2,048 rows. With a cache per row (decode) the gathers already run at
// the HBM rate, and the extra L2 traffic measured 7-22% slower, so there is no prefetch.
template <int HQ, int NS>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_kernel(AttnArgs a, int n_hg, int64_t units) {
    constexpr int CQ = 4 / HQ;                 // column parts per key half
    constexpr int COLS = kHeadDim / NS;        // output columns per workgroup
    constexpr int WCOLS = COLS / CQ;           // output columns per wave
    constexpr int CB = WCOLS / 16;             // 16-column blocks of the value MFMA per wave
    constexpr int VROW = COLS * 2;             // bytes of one V row slice
    constexpr int VSTRIDE = vstride_of(VROW);
    constexpr int VCHUNKS = VROW / 16;         // 16-byte pieces of a V row slice
    constexpr int kStores = CB / 2;            // output stores per wave per unit
    static_assert(kRows == 8 && CB >= 4 && HQ * CQ == 4, "tile split");
    static_assert(kWaves * (CB / 4) * 1024 <= kTile * VSTRIDE, "the exchange fits the V buffer");
    static_assert(kStores + kRows < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) char k_lds[kTile * kKStride];
    __shared__ __attribute__((aligned(16))) char v_lds[kTile * VSTRIDE];
    __shared__ int idx_lds[kWaves][2][64];   // each wave's own copy of a tile's index list
    __shared__ float meta_lds[kWaves][3][16];
    __shared__ uint32_t pf_lds[kWaves][64];  // where the L2 prefetches land (never read)
    // With fewer than four 16-head groups the waves of a key half share heads: each of the two
    // 16-slot blocks of a group's score tile is computed by one wave and handed to the others
    // here, [key half][head group][block], instead of every wave computing the whole tile.
    constexpr bool kShareScores = HQ < 4;
    __shared__ f32x4 xs_lds[kShareScores ? 2 * HQ * 2 : 1][64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int wi = w & 3;
    const int hq = wi % HQ;
    const int cq = wi / HQ;
    const int kh = w >> 2;
    const Stream<NS> str{a, n_hg, units, (int64_t)gridDim.x};
    // The score block this wave computes, or -1. 32 heads: each of the two waves of a head
    // group (column parts 0, 1) takes one block. 16 heads: in key half 0 the waves of column
    // parts 0 and 1 take blocks 0 and 1, in half 1 those of parts 2 and 3, so that every SIMD
    // (which holds one wave of each half with the same wi) runs one block.
    const int sblock = HQ == 2 ? cq : (HQ == 1 ? (kh == 0 ? (cq < 2 ? cq : -1) : (cq >= 2 ? cq - 2 : -1)) : 0);

    // Wave w gathers tile keys 8w .. 8w+7 (all in its own key half) into both buffers: key
    // 32kh + kap goes to K slot 32kh + kslot_of_key(kap) and to V slot 32kh + swap23(kap).
    // One DMA instruction moves one cache row (64 lanes x 16 bytes) or its column slice. The
    // buffer resource spans the row's cache; a masked key (-1) has a wrapped-around offset
    // past its end and arrives as zeros.
    auto rsrc_k = [&](const Item &it) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)a.k + it.row * a.cache_stride * 2), 0,
                                                 (int)(uint32_t)(a.n_ctx * kRowBytes), kBufferFlags);
    };
    auto rsrc_v = [&](const Item &it) {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const char *)a.v + it.row * a.cache_stride * 2 + (int64_t)it.cs * VROW), 0,
            (int)(uint32_t)(a.n_ctx * kRowBytes - (int64_t)it.cs * VROW), kBufferFlags);
    };
    auto dma_k_row = [&](__amdgpu_buffer_rsrc_t rsrc, int iv, int i) {
        const int ij = __builtin_amdgcn_readlane(iv, kRows * w + i);
        const int slot = 32 * kh + kslot_of_key(8 * wi + i);
        dma16_buf(rsrc, ((uint32_t)ij << 10) + ((uint32_t)lane << 4), lds_addr((SA_LDS char *)k_lds + slot * kKStride));
    };
    auto dma_v_row = [&](__amdgpu_buffer_rsrc_t rsrc, int iv, int i) {
        const int ij = __builtin_amdgcn_readlane(iv, kRows * w + i);
        const int slot = 32 * kh + swap23(8 * wi + i);
        if (VCHUNKS == 64 || lane < VCHUNKS)
            dma16_buf(rsrc, ((uint32_t)ij << 10) + ((uint32_t)lane << 4), lds_addr((SA_LDS char *)v_lds + slot * VSTRIDE));
    };

    const bool shared_cache = a.cache_stride == 0;
    // Prefetch lanes: lane l takes tile key 8w + l/8 (the rows this wave gathers) and its
    // 128-byte line l%8; V lines past the slice get an offset past the range (nothing).
    const uint32_t pf_line = (uint32_t)(lane & 7) << 7;
    const bool pf_v_line = (int)pf_line < VROW;
    const float scale2 = a.scale * kLog2e;
    bf16x8 qreg[16];
    f32x4 acc[CB];       // head l16, columns 16cb + 4g + 0..3 of the slice
    HalfState st;
    float sink_n;

    // Issue order per wave: Q/sink(0), I(0) | drain | K(0), I(1); then in tile j: V(j)
    // spread through the scores; with a shared cache, once I(j+1) is resolved, the two L2
    // prefetches of tile j+1; on a unit's last tile the next unit's query and sink
    // (kQLoads) once V(j) has landed; K(j+1) spread through the values; then I(j+2),
    // followed on a unit's last tile by its kStores output stores. Each wait below counts
    // exactly the operations issued after the one it needs.
    Item cur = str.make(xcd_remap(blockIdx.x, str.G), 0);
    Item nx = str.next(cur);
    Item nx2 = str.next(nx);
    bool bad = false, bad_next = false;
    load_q_async(a, cur.row, cur.hg * 16 * HQ + 16 * hq, g, l16, qreg, sink_n);
    dma_idx(a, cur, cur, &idx_lds[w][0][0], lane);
    wait_vmcnt<0>();
    q_ready(qreg, sink_n);
    half_start(st, acc, kh == 0, sink_n);
    __builtin_amdgcn_s_waitcnt(0);  // nothing the compiler tracks is pending in the loop
    bool starting = false;          // the next unit's query is in flight; its stores follow I(j+1)
    int iv_cur = resolve(a, cur, &idx_lds[w][0][0], lane, bad);
    {
        const __amdgpu_buffer_rsrc_t rk = rsrc_k(cur);
#pragma unroll
        for (int i = 0; i < kRows; i++) dma_k_row(rk, iv_cur, i);
        dma_idx(a, nx, cur, &idx_lds[w][1][0], lane);
    }

    // Per-lane LDS read bases. Scores: slot 32kh + 16b + l16, dims 32kk + 8g + 0..7.
    const SA_LDS char *krow = (const SA_LDS char *)k_lds + (32 * kh + l16) * kKStride + 16 * g;
    // Values: lane (g, l16) addresses the V slot of key 8g + 4t2 + l16/4 of its half and
    // columns 16cb + 4(l16%4) .. +3 of the wave's part; the transposing read returns column
    // 16cb + l16 of keys 8g + 4t2 + 0..3, which are elements 4t2 + 0..3 of the V^T operand.
    const SA_LDS char *vrow = (const SA_LDS char *)v_lds + (32 * kh + swap23(8 * g + (l16 >> 2))) * VSTRIDE +
                              2 * cq * WCOLS + 8 * (l16 & 3);

    for (int j = 0; cur.unit >= 0; j++) {
        const bool more = nx.unit >= 0;
        const bool last_of_unit = !more || nx.unit != cur.unit;
        // K(j) has landed for this wave, and with it a unit's query and sink when tile j
        // starts one. After K(j) come I(j+1) and, when tile j starts a unit, the previous
        // unit's stores.
        if (starting) wait_vmcnt<vm_clamp(1 + kStores)>(); else wait_vmcnt<1>();
        if (starting) {
            q_ready(qreg, sink_n);
            half_start(st, acc, kh == 0, sink_n);
        }
        lds_barrier();  // every wave's K(j) has landed; every wave is done with V(j-1)

        // ---- scores of the wave's 32 keys for its 16 heads over the full head width.
        f32x4 sacc0, sacc1;
        {
            // The tile's V rows go out in the score steps, in the matrix pipe's shadow (every
            // wave finished the previous tile's values before the barrier): one every two of a
            // 16-step block chain, one every four of the 32-step two-block chain.
            const __amdgpu_buffer_rsrc_t rv = rsrc_v(cur);
            if constexpr (kShareScores) {
                auto hook = [&](int kk) {
                    if (kk % 2 == 0) dma_v_row(rv, iv_cur, kk / 2);
                };
                f32x4 *xs = xs_lds[(kh * HQ + hq) * 2];
                if (sblock >= 0) {
                    f32x4 sb;
                    score_block_chain(krow + sblock * 16 * kKStride, qreg, sb, hook);
                    xs[sblock * 64 + lane] = sb;
                } else {
#pragma unroll
                    for (int kk = 0; kk < 16; kk++) hook(kk);
                }
                lds_barrier();  // both blocks of every head group's score tile are in LDS
                sacc0 = xs[lane];
                sacc1 = xs[64 + lane];
            } else {
                score_chain(krow, qreg, sacc0, sacc1, [&](int i) {
                    if (i % 4 == 0) dma_v_row(rv, iv_cur, i / 4);
                });
            }
        }

        // Indices of item j+1 have landed (after them: [stores], V(j)).
        if (starting) wait_vmcnt<vm_clamp(kStores + kRows)>(); else wait_vmcnt<kRows>();
        starting = false;
        int iv_n = 0;
        const bool q_now = last_of_unit && more;
        if (more) {
            bool b;
            iv_n = resolve(a, nx, &idx_lds[w][(j + 1) & 1][0], lane, b);
            if (nx.unit == cur.unit) bad = bad || b; else bad_next = bad_next || b;
            if (shared_cache) {
                const int ij = __builtin_amdgcn_ds_bpermute((kRows * w + (lane >> 3)) << 2, iv_n);
                const uint32_t off = ((uint32_t)ij << 10) + pf_line;
                prefetch4_buf(rsrc_k(nx), off, lds_addr(&pf_lds[w][0]));
                prefetch4_buf(rsrc_v(nx), pf_v_line ? off : 0xffffff80u, lds_addr(&pf_lds[w][0]));
            }
        }

        bf16x8 ph, pl;
        half_tile(sacc0, sacc1, cur.tile * kTile + 32 * kh + 8 * g, cur.n, (cur.tile + 1) * kTile <= cur.n, scale2,
                  st, acc, ph, pl);

        // V(j) has landed: after it come only the two prefetches, when issued.
        if (shared_cache && more) wait_vmcnt<2>(); else wait_vmcnt<0>();
        // On a unit's last tile: the next unit's query (the scores were qreg's last use),
        // ahead of the K rows, so the wait for K(j+1) covers it too.
        if (q_now) load_q_async(a, nx.row, nx.hg * 16 * HQ + 16 * hq, g, l16, qreg, sink_n);
        lds_barrier();  // every wave's V(j) has landed; every wave is done with K(j)

        // ---- values O^T += V^T P^T over the wave's 32 keys, one MFMA per part of P.
        {
            const __amdgpu_buffer_rsrc_t rk = rsrc_k(nx);
            auto read_v = [&](int cb) -> bf16x8 {
                const bf16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4 *)(vrow + 32 * cb));
                const bf16x4 t1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4 *)(vrow + 8 * VSTRIDE + 32 * cb));
                return (bf16x8){t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
            };
            bf16x8 vcur = read_v(0);
#pragma unroll
            for (int cb = 0; cb < CB; cb++) {
                bf16x8 vnxt = vcur;
                if (cb + 1 < CB) vnxt = read_v(cb + 1);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur, ph, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur, pl, acc[cb], 0, 0, 0);
                // The next tile's K rows go out here, in the matrix pipe's shadow (every
                // wave is past this tile's scores: the K buffer is free).
                if (more) {
#pragma unroll
                    for (int r = cb * kRows / CB; r < (cb + 1) * kRows / CB; r++) dma_k_row(rk, iv_n, r);
                }
                __builtin_amdgcn_sched_barrier(0);
                vcur = vnxt;
            }
        }

        dma_idx(a, nx2, cur, &idx_lds[w][j & 1][0], lane);  // slot j&1 held item j's list
        iv_cur = iv_n;
        starting = q_now;
        if (last_of_unit) {
            float *orow = a.out + cur.row * a.H * kHeadDim;
            const int head0 = cur.hg * 16 * HQ + 16 * hq;
            const int col0 = cur.cs * COLS + cq * WCOLS;
            f32x4 *xch = (f32x4 *)v_lds;
            if (kh) combine_store<1>(st, acc, meta_lds, xch, w, lane, g, l16, orow, a.H, head0, col0, bad);
            else combine_store<0>(st, acc, meta_lds, xch, w, lane, g, l16, orow, a.H, head0, col0, bad);
            bad = bad_next;
            bad_next = false;
        }
        cur = nx;
        nx = nx2;
        nx2 = str.next(nx2);
    }
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------------------
// One cache as K and V. Two tile buffers of 64 full rows alternate: tile j+1 is gathered
// during all of tile j (half of its rows in the scores, half in the values), and one
// barrier per tile hands buffers over ("T(j) landed; every wave is done with tile j-1, so
// its buffer may be refilled"). Index lists run two tiles ahead of the compute. Rows are
// stored with stride 1024 and the chunk swizzle tswz (applied on the gather side: lane i
// of a row's DMA fetches chunk i ^ tswz(slot)), and the LDS reads undo it by XOR.
template <int HQ, int NS>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_alias_kernel(AttnArgs a, int n_hg, int64_t units) {
    constexpr int CQ = 4 / HQ;
    constexpr int COLS = kHeadDim / NS;
    constexpr int WCOLS = COLS / CQ;
    constexpr int CB = WCOLS / 16;
    constexpr int kStores = CB / 2;
    constexpr int kTileBytes = kTile * kRowBytes;
    static_assert(kRows == 8 && CB >= 4 && HQ * CQ == 4, "tile split");
    static_assert(kWaves * (CB / 4) * 1024 <= kTileBytes, "the exchange fits a tile buffer");

    __shared__ __attribute__((aligned(1024))) char t_lds[2 * kTileBytes];
    __shared__ int idx_lds[kWaves][2][64];
    __shared__ float meta_lds[kWaves][3][16];
    // Score blocks shared between the waves of a key half that hold the same heads (fewer than
    // four 16-head groups), as in the separate-cache kernel: [key half][head group][block].
    constexpr bool kShareScores = HQ < 4;
    __shared__ f32x4 xs_lds[kShareScores ? 2 * HQ * 2 : 1][64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int wi = w & 3;
    const int hq = wi % HQ;
    const int cq = wi / HQ;
    const int kh = w >> 2;
    const Stream<NS> str{a, n_hg, units, (int64_t)gridDim.x};
    const uint32_t t_base = lds_addr((SA_LDS char *)t_lds);
    const int sblock = HQ == 2 ? cq : (HQ == 1 ? (kh == 0 ? (cq < 2 ? cq : -1) : (cq >= 2 ? cq - 2 : -1)) : 0);

    auto rsrc_t = [&](const Item &it) {
        if (it.unit < 0) return __builtin_amdgcn_make_buffer_rsrc((void *)a.k, 0, 0, kBufferFlags);
        return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)a.k + it.row * a.cache_stride * 2), 0,
                                                 (int)(uint32_t)(a.n_ctx * kRowBytes), kBufferFlags);
    };
    // Wave w gathers tile keys 8w .. 8w+7 of its key half into K slots (as the separate
    // kernel's K buffer), whole rows, swizzled.
    auto dma_t_row = [&](__amdgpu_buffer_rsrc_t rsrc, int iv, int buf, int i) {
        const int ij = __builtin_amdgcn_readlane(iv, kRows * w + i);
        const int slot = 32 * kh + kslot_of_key(8 * wi + i);
        const uint32_t src_chunk = (uint32_t)(lane ^ tswz(slot));
        dma16_buf(rsrc, ((uint32_t)ij << 10) + (src_chunk << 4), t_base + buf * kTileBytes + slot * kRowBytes);
    };

    const float scale2 = a.scale * kLog2e;
    bf16x8 qreg[16];
    f32x4 acc[CB];
    HalfState st;
    float sink_n;

    // Read bases within a buffer (XOR with the per-step column offset; bits 4-9 only).
    // Scores: slot 32kh + 16b + l16, chunk 4kk + g, stored at (4kk + g) ^ tswz(l16).
    const uint32_t kbase = (uint32_t)((32 * kh + l16) * kRowBytes + 16 * (g ^ tswz(l16)));
    // Values: lane (g, l16) reads the slot of key 8g + 4t2 + l16/4 of its half, which is
    // K slot 16t2 + 4g + l16/4, columns 16cb + 4(l16%4) .. +3: chunk 2cb + h (h = (l16%4)/2),
    // stored at (2cb + h) ^ tswz(slot), plus 8 bytes for odd l16.
    const int vslot = 32 * kh + 4 * g + (l16 >> 2);
    const uint32_t vbase =
        (uint32_t)(vslot * kRowBytes + 8 * (l16 & 1) + 16 * (((l16 & 3) >> 1) ^ tswz(vslot)));

    // Issue order per wave: Q/sink(0), I(0), I(1) | drain | T(0), I(2); then in tile j:
    // half of T(j+1) through the scores, on a unit's last tile the next unit's query and
    // sink (kQLoads), the rest of T(j+1) through the values, then I(j+3) and on a unit's
    // last tile its kStores output stores.
    Item cur = str.make(xcd_remap(blockIdx.x, str.G), 0);
    Item nx = str.next(cur);
    Item nx2 = str.next(nx);
    bool bad0 = false, bad1 = false, bad2 = false;  // units cur.useq, +1, +2
    int cur_useq = 0;
    auto note_bad = [&](const Item &it, bool b) {
        const int d = it.useq - cur_useq;
        bad0 = bad0 || (b && d == 0);
        bad1 = bad1 || (b && d == 1);
        bad2 = bad2 || (b && d == 2);
    };
    load_q_async(a, cur.row, cur.hg * 16 * HQ + 16 * hq, g, l16, qreg, sink_n);
    dma_idx(a, cur, cur, &idx_lds[w][0][0], lane);
    dma_idx(a, nx, cur, &idx_lds[w][1][0], lane);
    wait_vmcnt<0>();
    q_ready(qreg, sink_n);
    half_start(st, acc, kh == 0, sink_n);
    __builtin_amdgcn_s_waitcnt(0);
    int iv_next = 0;  // rows of the tile after the current one
    {
        bool b;
        const int iv0 = resolve(a, cur, &idx_lds[w][0][0], lane, b);
        note_bad(cur, b);
        if (nx.unit >= 0) {
            iv_next = resolve(a, nx, &idx_lds[w][1][0], lane, b);
            note_bad(nx, b);
        }
        const __amdgpu_buffer_rsrc_t rt = rsrc_t(cur);
#pragma unroll
        for (int i = 0; i < kRows; i++) dma_t_row(rt, iv0, 0, i);
        dma_idx(a, nx2, cur, &idx_lds[w][0][0], lane);
    }
    bool starting = false;      // tile j starts a unit whose query was loaded in tile j-1
    bool stores_prev = false;   // tile j-1 ended a unit: its stores follow I(j+2)

    for (int j = 0; cur.unit >= 0; j++) {
        const int buf = j & 1;
        const bool more = nx.unit >= 0;
        const bool last_of_unit = !more || nx.unit != cur.unit;
        const bool q_now = last_of_unit && more;
        // T(j) has landed for this wave (and the query, issued before its last rows).
        // After T(j) come I(j+2) and, when tile j-1 ended a unit, its stores.
        if (stores_prev) wait_vmcnt<vm_clamp(1 + kStores)>(); else wait_vmcnt<1>();
        if (starting) {
            q_ready(qreg, sink_n);
            half_start(st, acc, kh == 0, sink_n);
        }
        lds_barrier();  // every wave's T(j) has landed; every wave is done with tile j-1

        const uint32_t tb = t_base + buf * kTileBytes;
        const __amdgpu_buffer_rsrc_t rt = rsrc_t(nx);
        // ---- scores of the wave's 32 keys for its 16 heads over the full head width.
        f32x4 sacc0 = (f32x4){}, sacc1 = (f32x4){};
        if (!kShareScores) {
            // Block 0's chain, then block 1's (each the same MFMAs on the same operands in the same
            // order as interleaved), with the K operand read kAhead reads ahead of its MFMA.
            const uint32_t kb = tb + kbase;
            constexpr int kAhead = 2;
            // Block 1's base: adding 16 rows changes no bit that the step's XOR touches.
            const uint32_t kb1 = kb + 16 * kRowBytes;
            auto kread = [&](int i) {
                const int kk = i & 15;
                return *lds_at<bf16x8>((i >> 4 ? kb1 : kb) ^ (64u * kk));
            };
            bf16x8 ring[kAhead + 1];
#pragma unroll
            for (int i = 0; i < kAhead; i++) ring[i] = kread(i);
#pragma unroll
            for (int i = 0; i < 32; i++) {
                if (i + kAhead < 32) ring[(i + kAhead) % (kAhead + 1)] = kread(i + kAhead);
                const int kk = i & 15;
                if (i < 16) sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[i % (kAhead + 1)], qreg[kk], sacc0, 0, 0, 0);
                else sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[i % (kAhead + 1)], qreg[kk], sacc1, 0, 0, 0);
                // Rows 0..3 of T(j+1), one every eight steps.
                if (more && i % 8 == 0) dma_t_row(rt, iv_next, buf ^ 1, i / 8);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // One block of the head group's score tile per computing wave (block b's chain: the
            // same operands in the same order), handed to the other waves through LDS.
            f32x4 *xs = xs_lds[(kh * HQ + hq) * 2];
            if (sblock >= 0) {
                const uint32_t kb = tb + kbase + (uint32_t)(sblock * 16 * kRowBytes);
                f32x4 sb = (f32x4){};
                bf16x8 k0 = *lds_at<bf16x8>(kb);
#pragma unroll
                for (int kk = 0; kk < 16; kk++) {
                    bf16x8 n0 = k0;
                    if (kk + 1 < 16) n0 = *lds_at<bf16x8>(kb ^ (64u * (kk + 1)));
                    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qreg[kk], sb, 0, 0, 0);
                    if (more && kk % 4 == 0) dma_t_row(rt, iv_next, buf ^ 1, kk / 4);
                    __builtin_amdgcn_sched_barrier(0);
                    k0 = n0;
                }
                xs[sblock * 64 + lane] = sb;
            } else {
#pragma unroll
                for (int kk = 0; kk < 16; kk += 4)
                    if (more) dma_t_row(rt, iv_next, buf ^ 1, kk / 4);
            }
            lds_barrier();  // both blocks of every head group's score tile are in LDS
            sacc0 = xs[lane];
            sacc1 = xs[64 + lane];
        }
        // The scores were the last use of qreg in this unit.
        if (q_now) load_q_async(a, nx.row, nx.hg * 16 * HQ + 16 * hq, g, l16, qreg, sink_n);

        bf16x8 ph, pl;
        half_tile(sacc0, sacc1, cur.tile * kTile + 32 * kh + 8 * g, cur.n, (cur.tile + 1) * kTile <= cur.n, scale2,
                  st, acc, ph, pl);

        // ---- values O^T += V^T P^T over the wave's 32 keys, one MFMA per part of P.
        {
            const uint32_t vb = tb + vbase;
            const uint32_t cbase = (uint32_t)(cur.cs * COLS * 2 + cq * WCOLS * 2);
            auto read_v = [&](int cb) -> bf16x8 {
                const uint32_t ad = vb ^ (cbase + 32u * cb);
                const bf16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4 *)lds_at<bf16x4>(ad));
                const bf16x4 t1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4 *)lds_at<bf16x4>(ad + 16 * kRowBytes));
                return (bf16x8){t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
            };
            bf16x8 vcur = read_v(0);
#pragma unroll
            for (int cb = 0; cb < CB; cb++) {
                bf16x8 vnxt = vcur;
                if (cb + 1 < CB) vnxt = read_v(cb + 1);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur, ph, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur, pl, acc[cb], 0, 0, 0);
                // Rows 4..7 of T(j+1).
                if (more) {
#pragma unroll
                    for (int r = cb * 4 / CB; r < (cb + 1) * 4 / CB; r++) dma_t_row(rt, iv_next, buf ^ 1, 4 + r);
                }
                __builtin_amdgcn_sched_barrier(0);
                vcur = vnxt;
            }
        }

        // Indices of item j+2 have landed: after I(j+2) came [stores of tile j-1's unit],
        // T(j+1) (when there is a tile j+1) and [the next unit's query].
        if (nx2.unit >= 0) {
            wait_vmcnt_dyn((stores_prev ? kStores : 0) + (more ? kRows : 0) + (q_now ? kQLoads : 0));
            bool b;
            iv_next = resolve(a, nx2, &idx_lds[w][buf][0], lane, b);
            note_bad(nx2, b);
        }
        const Item nx3 = str.next(nx2);
        dma_idx(a, nx3, cur, &idx_lds[w][buf ^ 1][0], lane);  // slot buf^1 held I(j+1)
        stores_prev = last_of_unit;
        starting = q_now;
        if (last_of_unit) {
            float *orow = a.out + cur.row * a.H * kHeadDim;
            const int head0 = cur.hg * 16 * HQ + 16 * hq;
            const int col0 = cur.cs * COLS + cq * WCOLS;
            f32x4 *xch = (f32x4 *)(t_lds + buf * kTileBytes);
            if (kh) combine_store<1>(st, acc, meta_lds, xch, w, lane, g, l16, orow, a.H, head0, col0, bad0);
            else combine_store<0>(st, acc, meta_lds, xch, w, lane, g, l16, orow, a.H, head0, col0, bad0);
            bad0 = bad1;
            bad1 = bad2;
            bad2 = false;
            cur_useq++;
        }
        cur = nx;
        nx = nx2;
        nx2 = nx3;
    }
    wait_vmcnt<0>();
}

template <int HQ, int NS, bool ALIAS>
hipError_t launch_variant(const AttnArgs &a, int64_t units, hipStream_t s) {
    const int n_hg = (a.H + 16 * HQ - 1) / (16 * HQ);
    const int64_t cus = device_cu_count();
    const dim3 grid((unsigned)(units < cus ? units : cus));
    if (ALIAS)
        hipLaunchKernelGGL((attn_bf16_alias_kernel<HQ, NS>), grid, dim3(512), 0, s, a, n_hg, units);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<HQ, NS>), grid, dim3(512), 0, s, a, n_hg, units);
    return hipGetLastError();
}

template <bool ALIAS>
hipError_t launch_plan(const AttnArgs &a, const AttnPlan &p, hipStream_t s) {
    const int ns = kHeadDim / p.cols_per_wg;
    switch (p.heads_per_wg) {
        case 64:
            switch (ns) {
                case 1: return launch_variant<4, 1, ALIAS>(a, p.units, s);
                case 2: return launch_variant<4, 2, ALIAS>(a, p.units, s);
                case 4: return launch_variant<4, 4, ALIAS>(a, p.units, s);
                case 8: return launch_variant<4, 8, ALIAS>(a, p.units, s);
            }
            break;
        case 32:
            switch (ns) {
                case 1: return launch_variant<2, 1, ALIAS>(a, p.units, s);
                case 2: return launch_variant<2, 2, ALIAS>(a, p.units, s);
                case 4: return launch_variant<2, 4, ALIAS>(a, p.units, s);
            }
            break;
        case 16:
            switch (ns) {
                case 1: return launch_variant<1, 1, ALIAS>(a, p.units, s);
                case 2: return launch_variant<1, 2, ALIAS>(a, p.units, s);
            }
            break;
    }
    return hipErrorInvalidValue;
}

constexpr int kSmallLds = kWaves * 2 * 64 * 4 + kWaves * 3 * 16 * 4;

}  // namespace

AttnPlan plan_attn_bf16(int64_t rows, int H, int32_t kmax) {
    AttnPlan p{};
    const int64_t n_hb = (H + 63) / 64;
    if (kmax <= kSplitMaxK && rows * n_hb < kSplitMaxUnits) {
        p.split = 1;
        p.threads = 512;
        p.ws_bytes = split_workspace_bytes(rows, H, kmax);
        return p;
    }
    const int hq = H > 32 ? 4 : (H > 16 ? 2 : 1);
    p.heads_per_wg = 16 * hq;
    const int64_t n_hg = (H + p.heads_per_wg - 1) / p.heads_per_wg;
    const int64_t rows_hg = rows * n_hg;
    // One workgroup per CU fits (the K tile alone is 65 KiB of LDS). With fewer
    // (row, head block) pairs than CUs, column slices add units; every slice gathers the
    // full K tile but only its own V columns. The slice count is the largest that keeps all
    // units in one round of workgroups (a unit is a latency-bound chain of tiles, so a second
    // round costs a whole chain: 72 us at 48 rows with 8 slices, against 39 us at 32 rows).
    // A wave keeps at least 64 columns, so blocks of fewer heads (more column parts per wave
    // pair) allow fewer slices. The slice count never changes a result's bits.
    const int64_t cus = device_cu_count();
    const int ns_max = 2 * hq;
    int ns = 1;
    while (ns < ns_max && rows_hg * (2 * ns) <= cus) ns *= 2;
    p.cols_per_wg = kHeadDim / ns;
    p.units = rows_hg * ns;
    p.threads = 512;
    p.lds_bytes = kTile * kKStride + kTile * vstride_of(2 * p.cols_per_wg) + kSmallLds + kWaves * 64 * 4;
    p.lds_bytes_aliased = 2 * kTile * kRowBytes + kSmallLds;
    return p;
}

hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t s) {
    const AttnPlan p = plan_attn_bf16(a.rows, a.H, a.kmax);
    if (p.split) return launch_attn_split(a, s);
    if (p.units == 0) return hipSuccess;
    return a.k == a.v ? launch_plan<true>(a, p, s) : launch_plan<false>(a, p, s);
}

}  // namespace sa
