// sa_attn_split.hip -- the bf16 attention path for small batches: the keys of a row are split
// across workgroups for the score contraction, and the softmax and value products then fold the
// score tiles in key order, all in one launch. Same results, bit for bit, as the persistent
// kernels of sa_attn.hip.
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
// HBM, so a launch of one or a few rows takes about 30 us whatever the chip's size. Here every
// workgroup of attn_split_kernel takes one or two roles:
//   * producer of (row, tile, block of 16 HPB heads, HPB = 1, 2 or 4): its eight waves gather
//     the tile's 64 K rows once, and 2 HPB of them run the score MFMA chain exactly as the
//     persistent kernel does (one key half and one 16-head group each; same K slot order and
//     operand layout). The block's query goes through LDS once (one 1 KiB DMA per head). It
//     stores each scoring wave's scaled scores (log2 units, masked past the row's count: the
//     persistent kernels' tile_scores), in its lane layout, and each key half's tile maximum
//     per head, then publishes the tile's ready word. A narrower block puts each score
//     chain on a SIMD of its own, and the launch takes the narrowest that still fits the chip in
//     one round of workgroups (one row: 16 heads, 10.6 against 12.5 us for 64).
//   * consumer of (row, 16-head group, 64-column slice): it loads the row's index list and
//     gathers the V column slices of a round of up to ten tiles while the producers run, waits
//     for the ready words of the row's tiles, loads the scaled scores of the tiles it weighs and
//     every tile's maxima straight into registers, then runs, per wave
//     (key half kh = w >> 2, 16-column part w & 3), the same online-softmax steps and value MFMAs
//     on each tile in order (the four waves of a key half share the weights), and the same
//     fixed-order fold of the two key halves (sa_attn_common.h).
// Every (row, head, column) thus sees the same operations, on the same operands, in the same
// order as in the persistent kernels: which path a launch takes never changes its bits.
//
// Workgroup order. All producers come first (padded to a multiple of eight), then the consumers,
// remapped so that the consumers of one row and head group run on one XCD (the hardware places
// workgroup i on XCD i % 8). A consumer therefore only ever waits for workgroups with lower ids,
// which the hardware dispatches first (workgroups of a grid go out in id order) and which wait
// for nothing. Every wait is also bounded in time: past 200 ms the row is reported as NaN.
// (A layout that lets the first consumers of each row run the next row's producer tasks first,
// so that eight decode rows need 266 workgroups instead of 336, measured slower: 15.9 against
// 14.5 us; without the XCD remap, eight rows took 16.1 us.)
//
// Synchronisation through the workspace. Its first kSyncBytes hold, per (row, producer block),
// a sequence number E, a consumer count U and one ready word per tile. Every workgroup reads E
// at its start; a producer stores its scores and maxima with device-scope (sc1) stores, waits
// until they have completed, and then stores the ready word ready_word(E, tile); a consumer
// polls the ready words of its row's tiles with device-scope loads until all match, then reads
// the scores with device-scope loads. The producer of tile 0 first resets U; every consumer adds
// one to U once its reads of sync words are done (the add's round trip runs beside the value
// products), and the one that brings U to the group's consumer count stores E + 1 at its end,
// so the next launch on this workspace waits for different words. The words are mixed
// with the tile index, so that no earlier contents of the workspace (zeros, a repeated byte,
// data of another launch shape) can pass for a ready word except by a 64-bit coincidence.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_attn_common.h"
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kSplitCols = 64;                 // output columns per consumer
constexpr int kSplitSlices = kHeadDim / kSplitCols;
constexpr int kVRowB = kSplitCols * 2;         // bytes of a V row slice
constexpr int kVTileB = kTile * kVRowB;        // one tile's V slices: 8 KiB
constexpr int kSTileB = 2 * 64 * 8 * 4;        // one tile's scores for a 16-head group: 4 KiB
constexpr int kMTileB = 2 * 16 * 4;            // one tile's maxima for a 16-head group: [key half][head]
constexpr int kRing = 10;                      // tiles per round of a consumer
constexpr int kMaxTiles = kSplitMaxK / kTile;
static_assert(kSplitCols == 64 && kVRowB == 128, "a consumer's waves own 16 columns each");

// Sync words: 32 per (row, producer block): [0] E, [1] U, [2 + t] the ready word of tile t.
constexpr int kSyncGroupWords = 32;
constexpr size_t kSyncBytes = (size_t)kSplitMaxUnits * kSyncGroupWords * 8;
static_assert(2 + kMaxTiles <= kSyncGroupWords, "the ready words fit a group");
// Bound of every wait: 200 ms of the 100 MHz constant clock (s_memrealtime).
constexpr long long kWaitTicks = 20000000;

__device__ __forceinline__ uint64_t ready_word(uint64_t e, int t) {
    return (e + 1) ^ (0x9E3779B97F4A7C15ull * (uint64_t)(t + 1));
}

// Chunk swizzle of a V row slice in LDS (8 chunks of 16 bytes): the chunk c of the slice in
// slot s is stored at chunk c ^ (s & 7). The four keys one 16-lane group reads in a
// transposing read sit in four consecutive slots, which then use four different chunks.
__device__ __forceinline__ int vswz(int s) { return s & 7; }

// Workspace after the sync words: scaled score tiles [row][tile][head group][key half][lane][8] fp32,
// then tile maxima [row][tile][head group][key half][head] fp32.
__device__ __forceinline__ size_t score_block(int64_t row, int tile, int hg, int ntiles_max, int n_hg) {
    return (((size_t)row * ntiles_max + tile) * n_hg + hg) * (kSTileB / 4);
}
__device__ __forceinline__ size_t maxima_offset(int64_t rows, int ntiles_max, int n_hg) {
    return kSyncBytes + (size_t)rows * ntiles_max * n_hg * kSTileB;
}

// The row's count, by a scalar (constant address space) load: it waits on the scalar counter,
// not on the vector-memory counter that the gathers in flight hold.
__device__ __forceinline__ int row_count(const AttnArgs &a, int64_t row) {
    int n = a.nsel ? *(const __attribute__((address_space(4))) int32_t *)(a.nsel + row) : a.kmax;
    return n < 0 ? 0 : (n > a.kmax ? a.kmax : n);
}

constexpr int kStoreDevice = 16;   // cache policy sc1 of a buffer load or store: device scope
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Device-scope atomic add returning the old value asynchronously: old may be used only after
// an explicit vector-memory wait that covers it, followed by register_ready.
__device__ __forceinline__ void atomic_add_async(uint64_t &old, uint64_t *p, uint64_t v) {
    asm volatile("global_atomic_add_x2 %0, %1, %2, off sc0" : "=v"(old) : "v"(p), "v"(v) : "memory");
}
#pragma clang diagnostic pop

// LDS of the two roles, one array (a workgroup takes one role).
// Consumer: V ring, weight ring, tile sums, index list, fold metadata, the fold exchange,
// bad-index flags. Producer: K tile, index lists, the block's query.
constexpr int kOffV = 0;
constexpr int kOffS = kOffV + kRing * kVTileB;
constexpr int kOffPsum = kOffS + kRing * kSTileB;
constexpr int kOffIdx = kOffPsum + 2 * kRing * 64 * 4;
constexpr int kOffMeta = kOffIdx + kSplitMaxK * 4;
constexpr int kOffXch = kOffMeta + 4 * 3 * 16 * 4;
constexpr int kOffBad = kOffXch + 4 * 64 * 16;
constexpr int kLdsConsumer = kOffBad + kWaves * 4;
constexpr int kOffPIdx = kTile * kKStride;
constexpr int kOffQ = kOffPIdx + kWaves * 64 * 4;
constexpr int kLdsProducer = kOffQ + 64 * kRowBytes;
constexpr int kLdsBytes = kLdsConsumer > kLdsProducer ? kLdsConsumer : kLdsProducer;
static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");

// Producer task b of the launch: (row, tile, head block of 16 HPB heads), head blocks fastest.
template <int HPB>
__device__ __forceinline__ void producer(const AttnArgs &a, char *lds, int64_t b, int ntiles_max, int n_hb, int n_hg,
                                         uint64_t *sync) {
    char *k_lds = lds;
    int (*idx_lds)[64] = (int (*)[64])(lds + kOffPIdx);
    char *q_lds = lds + kOffQ;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    // Score roles: wave w < 2 HPB takes key half kh = w / HPB and head group wi = w % HPB of
    // the block; gather roles: wave w gathers tile keys 8w .. 8w+7.
    const int wi = w % HPB;
    const int kh = w / HPB;
    const int hb = (int)(b % n_hb);
    const int tile = (int)((b / n_hb) % ntiles_max);
    const int64_t row = b / ((int64_t)n_hb * ntiles_max);
    const int hg = HPB * hb + wi;
    uint64_t *sg = sync + (row * n_hb + hb) * kSyncGroupWords;

    // First memory round trip: E, the tile's index list and the row's count; the block's query
    // follows (16 HPB heads x 1 KiB into LDS, 2 HPB per wave) and may still be in
    // flight while the K rows are gathered. Head h's row is stored rotated by h chunks of 16
    // bytes, so that 16 heads read at one column hit 16 different bank groups.
    const uint64_t e = __hip_atomic_load(sg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    {
        const int p = tile * kTile + lane;
        const int pc = p < a.kmax ? p : a.kmax - 1;
        dma4(a.idx + row * a.kmax, (uint32_t)pc * 4u, lds_addr(&idx_lds[w][0]));
    }
#pragma unroll
    for (int i = 0; i < 2 * HPB; i++) {
        const int hl = 2 * HPB * w + i;
        const int h = 16 * HPB * hb + hl;
        const void *src = h < a.H ? (const void *)((const uint16_t *)a.q + (row * a.H + h) * kHeadDim)
                                  : (const void *)g_zero_row;
        dma16(src, (uint32_t)((lane - hl) & 63) << 4, lds_addr(q_lds + hl * kRowBytes));
    }
    const int n = row_count(a, row);
    wait_vmcnt<2 * HPB>();  // E and the index list; the query's rows may still be in flight
    // Tiles past the row's count have no selected key and no consumer waits for them; tile 0
    // always publishes (its producer resets the group's consumer count).
    const int nwait = n > 0 ? (n + kTile - 1) / kTile : 1;
    if (tile >= nwait) {
        wait_vmcnt<0>();  // no DMA may land in LDS after this task
        return;
    }
    if (tile * kTile < n) {
        // Row to gather for entry tile*64 + lane, or -1 (masked or out of range: gathers zeros,
        // as in the persistent kernels; the consumers mark a row with a live out-of-range entry
        // as NaN).
        const int iv_raw = idx_lds[w][lane];
        const bool live = tile * kTile + lane < n;
        const int iv = (live && iv_raw >= 0 && (int64_t)iv_raw < a.n_ctx) ? iv_raw : -1;
        // Wave w gathers tile keys 8w .. 8w+7 (key half w >> 2) into the K slots of the
        // persistent kernels: key 32kh + kap goes to slot 32kh + kslot_of_key(kap).
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const char *)a.k + row * a.cache_stride * 2), 0, (int)(uint32_t)(a.n_ctx * kRowBytes),
            kBufferFlags);
#pragma unroll
        for (int i = 0; i < kRows; i++) {
            const int ij = __builtin_amdgcn_readlane(iv, kRows * w + i);
            const int slot = 32 * (w >> 2) + kslot_of_key(8 * (w & 3) + i);
            dma16_buf(rk, ((uint32_t)ij << 10) + ((uint32_t)lane << 4),
                      lds_addr((SA_LDS char *)k_lds + slot * kKStride));
        }
        wait_vmcnt<kRows>();  // this wave's query rows (its K rows may still be in flight)
        lds_barrier();        // every wave's query rows have landed
        bf16x8 qreg[16];      // lane (g, l16): head 16 wi + l16, dims 32 kk + 8 g + 0..7
        {
            const int hl = 16 * wi + l16;
#pragma unroll
            for (int kk = 0; kk < 16; kk++)
                qreg[kk] = *lds_at<bf16x8>(lds_addr(q_lds + hl * kRowBytes) + (((4 * kk + g + hl) & 63) << 4));
        }
        wait_vmcnt<0>();
        lds_barrier();  // every wave's K rows have landed
        if (kh < 2 && hg < n_hg) {
            const SA_LDS char *krow = (const SA_LDS char *)k_lds + (32 * kh + l16) * kKStride + 16 * g;
            f32x4 sacc0, sacc1;
            score_chain(krow, qreg, sacc0, sacc1, [](int) {});
            // The half tile's scaled scores and their maximum per head: tile_scores on the same
            // operands as in the persistent kernels (the consumers take both instead of computing
            // them).
            float sk[8];
            const float mt = tile_scores(sacc0, sacc1, tile * kTile + 32 * kh + 8 * g, n, (tile + 1) * kTile <= n,
                                         a.scale * kLog2e, sk);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((float *)((char *)a.ws + kSyncBytes) + score_block(row, tile, hg, ntiles_max, n_hg)), 0,
                kSTileB, kBufferFlags);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, (f32x4){sk[0], sk[1], sk[2], sk[3]}), rs,
                                                   (kh * 64 + lane) * 32, 0, kStoreDevice);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, (f32x4){sk[4], sk[5], sk[6], sk[7]}), rs,
                                                   (kh * 64 + lane) * 32 + 16, 0, kStoreDevice);
            const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((char *)a.ws + maxima_offset(a.rows, ntiles_max, n_hg) +
                         (((size_t)row * ntiles_max + tile) * n_hg + hg) * kMTileB),
                0, kMTileB, kBufferFlags);
            if (g == 0)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mt), rm, (kh * 16 + l16) * 4, 0, kStoreDevice);
        }
    }
    // Publish: every wave's device-scope stores have completed, then the tile's ready word (after
    // the reset of the consumer count, for tile 0).
    wait_vmcnt<0>();
    lds_barrier();
    if (w == 0 && lane == 0) {
        if (tile == 0) __hip_atomic_store(sg + 1, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_vmcnt<0>();
        __hip_atomic_store(sg + 2 + tile, ready_word(e, tile), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Consumer task u of the launch: (row, 16-head group, 64-column slice), slices fastest. Eight
// waves, two per SIMD: wave w takes key half kh = w >> 2 and the 16 columns cs*64 + 16(w & 3)
// .. +15 (one MFMA block). The four waves of a key half split a round's tiles for the
// expensive part of the online softmax (the weights), share the weights through
// LDS, and each runs the cheap sequential parts (reference scan, tile sums) itself.
template <int HPB>
__device__ __forceinline__ void consumer(const AttnArgs &a, char *lds, int64_t u, int ntiles_max, int n_hb, int n_hg,
                                         uint64_t *sync) {
    char *v_lds = lds + kOffV;
    char *s_lds = lds + kOffS;
    float (*psum_lds)[kRing][64] = (float (*)[kRing][64])(lds + kOffPsum);
    int *idx_lds = (int *)(lds + kOffIdx);
    float (*meta_lds)[3][16] = (float (*)[3][16])(lds + kOffMeta);
    f32x4 (*xch_lds)[64] = (f32x4 (*)[64])(lds + kOffXch);
    int *bad_lds = (int *)(lds + kOffBad);

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int cq = w & 3;
    const int kh = w >> 2;
    // Residue (mod 4) of the round's tiles this wave weighs: the two waves of a SIMD (w and
    // w ^ 4) take different residues, so every SIMD weighs five of ten tiles.
    const int qv = (cq + 2 * kh) & 3;
    const int cs = (int)(u % kSplitSlices);
    const int hg = (int)((u / kSplitSlices) % n_hg);
    const int64_t row = u / ((int64_t)kSplitSlices * n_hg);
    const int head = 16 * hg + l16;
    const int hb = hg / HPB;
    uint64_t *sg = sync + (row * n_hb + hb) * kSyncGroupWords;

    // First memory round trip: E, the row's index list (the first ntiles_max * 64 entries, the
    // offsets clamped to the row), the sink and the row's count.
    const uint64_t e = __hip_atomic_load(sg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    const int nwait = ntiles > 0 ? ntiles : 1;
    wait_vmcnt<0>();
    register_ready(sink);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // every wave's index pieces have landed

    HalfState st;
    f32x4 acc[1];
    half_start(st, acc, kh == 0, sink);

    const float *sws = (const float *)((const char *)a.ws + kSyncBytes) + score_block(row, 0, hg, ntiles_max, n_hg);
    const float *mws = (const float *)((const char *)a.ws + maxima_offset(a.rows, ntiles_max, n_hg)) +
                       ((size_t)row * ntiles_max * n_hg + hg) * (kMTileB / 4);
    const uint32_t v_base = lds_addr((SA_LDS char *)v_lds);
    const uint32_t s_base = lds_addr((SA_LDS char *)s_lds);
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
    // persistent kernels (bad_w: one of this wave's entries is, or its wait ran out); masked
    // entries (past the count) gather zeros.
    bool bad_w = false;
    // The V slices of a round: the round's index entries are read from LDS first, so that the
    // gathers then go out back to back.
    auto issue_v = [&](int t0, int nt) {
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
    };
    if (ntiles > 0) issue_v(0, ntiles < kRing ? ntiles : kRing);

    // Wait until every tile of the row has been scored: wave 0 polls the ready words (lane t
    // tile t), the others wait at the barrier. Bounded: past kWaitTicks the row is NaN.
    if (w == 0) {
        const long long t_start = wall_clock64();
        bool late = false;
        for (;;) {
            bool pend = false;
            if (lane < nwait) {
                const uint64_t f = __hip_atomic_load(sg + 2 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                pend = f != ready_word(e, lane);
            }
            if (__builtin_amdgcn_ballot_w64(pend) == 0) break;
            if (wall_clock64() - t_start > kWaitTicks) {
                late = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        bad_w = bad_w || late;
    }
    lds_barrier();

    // This consumer's count for the group (U): the one that brings it to the group's consumer
    // count advances E at its end. It goes out once every read of sync words is done, at a
    // point where no later wait covers it until the end.
    const int hgs = n_hg - HPB * hb < HPB ? n_hg - HPB * hb : HPB;
    const uint64_t nv = (uint64_t)hgs * kSplitSlices;
    uint64_t u_old = 0;
    if (ntiles == 0 && w == 0 && lane == 0) atomic_add_async(u_old, sg + 1, 1);
    for (int t0 = 0; t0 < ntiles; t0 += kRing) {
        const int nt = ntiles - t0 < kRing ? ntiles - t0 : kRing;
        if (t0 > 0) issue_v(t0, nt);
        // This wave's tiles' scores (qv, qv + 4, qv + 8) and every tile's maxima of its key half,
        // by device-scope loads straight into registers (a slot past the round's tiles reloads
        // its last tile and is not used).
        constexpr int kMine = (kRing + 3) / 4;
        const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)sws, 0, ((ntiles_max - 1) * n_hg + 1) * kSTileB, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rmx = __builtin_amdgcn_make_buffer_rsrc(
            (void *)mws, 0, ((ntiles_max - 1) * n_hg + 1) * kMTileB, kBufferFlags);
        f32x4 sraw[kMine][2];
#pragma unroll
        for (int j = 0; j < kMine; j++) {
            const int i = qv + 4 * j < nt ? qv + 4 * j : nt - 1;
            const int off = (t0 + i) * n_hg * kSTileB + (kh * 64 + lane) * 32;
            sraw[j][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, off, 0, kStoreDevice));
            sraw[j][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, off + 16, 0, kStoreDevice));
        }
        float ref_t[kRing], refp_t[kRing], mloc_t[kRing];
        uint32_t resc = 0;
#pragma unroll
        for (int i = 0; i < kRing; i++) {
            const int ic = i < nt ? i : nt - 1;
            mloc_t[i] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rmx, (t0 + ic) * n_hg * kMTileB + (kh * 16 + l16) * 4, 0, kStoreDevice));
        }
        // The reference scan over the round's tiles in key order (every wave of a key half
        // computes the same values), then the weights of this wave's tiles against their
        // references, into the weight ring.
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
                float sk[8];
#pragma unroll
                for (int e = 0; e < 8; e++) sk[e] = e < 4 ? sraw[j][0][e] : sraw[j][1][e - 4];
                bf16x8 ph, pl;
                const float psum = tile_weights(sk, ref, ph, pl);
                SA_LDS bf16x8 *pp = (SA_LDS bf16x8 *)lds_at<bf16x8>(s_base + i * kSTileB + (kh * 64 + lane) * 32);
                pp[0] = ph;
                pp[1] = pl;
                psum_lds[kh][i][lane] = psum;
            }
        }
        // Every register load of the round counts as used here, so that the compiler has no load
        // of its own in flight past this point (its next wait would cover the count below).
#pragma unroll
        for (int i = 0; i < kRing; i++) asm volatile("" ::"v"(mloc_t[i]));
#pragma unroll
        for (int j = 0; j < kMine; j++) asm volatile("" ::"v"(sraw[j][0]), "v"(sraw[j][1]));
        wait_vmcnt<0>();  // this wave's V slices
        if (t0 + kRing >= ntiles && w == 0 && lane == 0) atomic_add_async(u_old, sg + 1, 1);
        lds_barrier();
        // Tile sums, rescales and value MFMAs in key order. The tile sums are read up front, and
        // each tile's weights and value operand one tile ahead of its MFMAs.
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
        for (int i = 0; i < 4; i++) o[i] = fold_elem(f, acc[0][i], x1[i], bad_mask);
        // Lane (g, l16): head 16hg + l16, columns cs*64 + 16cq + 4g + 0..3.
        float *dst = a.out + (row * a.H + head) * kHeadDim + cs * kSplitCols + 16 * cq + 4 * g;
        __builtin_nontemporal_store(o, (f32x4 *)dst);
    }
    // The last consumer of the group advances E for the next launch on this workspace (every
    // read of this launch's ready words is done by then).
    if (w == 0) {
        wait_vmcnt<0>();
        register_ready(u_old);
        if (lane == 0 && u_old == nv - 1) __hip_atomic_store(sg, e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Workgroups 0 .. n_prod-1 are producer tasks, n_prod .. n_prod_pad-1 idle, the others consumer
// tasks.
template <int HPB>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_split_kernel(AttnArgs a, int ntiles_max, int n_hb, int n_hg, int64_t n_prod, int64_t n_prod_pad) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
    uint64_t *sync = (uint64_t *)a.ws;
    const int64_t b = blockIdx.x;
    if (b < n_prod_pad) {
        if (b < n_prod) producer<HPB>(a, lds, b, ntiles_max, n_hb, n_hg, sync);
    } else
        consumer<HPB>(a, lds, xcd_remap(b - n_prod_pad, gridDim.x - n_prod_pad), ntiles_max, n_hb, n_hg, sync);
}

}  // namespace

hipError_t launch_attn_split(const AttnArgs &a, hipStream_t s) {
    const int ntiles_max = (a.kmax + kTile - 1) / kTile;
    const int n_hg = (a.H + 15) / 16;
    const int64_t n_cons = (int64_t)a.rows * n_hg * kSplitSlices;
    if (a.rows <= 0 || ntiles_max == 0) return hipSuccess;
    // Producer blocks of 16, 32 or 64 heads: the narrowest whose launch fits the chip in one
    // round of workgroups (a narrower block runs its score chains on fewer SIMDs at once).
    const int64_t cus = device_cu_count();
    int hpb = 4;
    for (int c = 1; c < 4; c *= 2) {
        const int64_t nhb = (n_hg + c - 1) / c;
        if (a.rows * nhb < kSplitMaxUnits && a.rows * ntiles_max * nhb + n_cons <= cus) {
            hpb = c;
            break;
        }
    }
    const int n_hb = (n_hg + hpb - 1) / hpb;
    const int64_t n_prod = (int64_t)a.rows * ntiles_max * n_hb;
    const int64_t n_prod_pad = (n_prod + 7) & ~(int64_t)7;
    const dim3 grid((unsigned)(n_prod_pad + n_cons));
    if (hpb == 1)
        hipLaunchKernelGGL(attn_split_kernel<1>, grid, dim3(512), 0, s, a, ntiles_max, n_hb, n_hg, n_prod, n_prod_pad);
    else if (hpb == 2)
        hipLaunchKernelGGL(attn_split_kernel<2>, grid, dim3(512), 0, s, a, ntiles_max, n_hb, n_hg, n_prod, n_prod_pad);
    else
        hipLaunchKernelGGL(attn_split_kernel<4>, grid, dim3(512), 0, s, a, ntiles_max, n_hb, n_hg, n_prod, n_prod_pad);
    return hipGetLastError();
}

size_t split_workspace_bytes(int64_t rows, int H, int32_t kmax) {
    const int64_t ntiles_max = (kmax + kTile - 1) / kTile;
    const int64_t n_hg = (H + 15) / 16;
    if (rows <= 0) return 0;
    return kSyncBytes + (size_t)(rows * ntiles_max * n_hg) * (kSTileB + kMTileB);
}

}  // namespace sa
