// sa_attn_f32_split.hip -- the float32 attention path for small batches: the keys of a row are
// split across workgroups for the score contraction, then the softmax and the value products
// run over the score tiles in key order. Same results, bit for bit, as attn_f32_kernel
// (sa_attn_f32.hip).
//
// What it computes is sa_attn_f32_common.h's: akol1/TensorFold pull request 4 ("DeepSeek V4.1:
// sparse attention on eight SIMD groups, the same bytes"), first commit message: keys scored in
// tiles with a running maximum, a tile sum and a value sum; TensorFold pull request 1206,
// "What changes": a sink per head; float32 throughout. The ds4 commit log for ds4_tp.c (the
// attention split of 8 against 32 groups) shows why a split may not follow the launch: its
// outputs changed with the group count. Here the split unit is the 32-key tile, a constant of
// the method, and no operation changes with the launch.
//
// Why: attn_f32_kernel runs one workgroup per (row, 16-head group), a chain of k/32 tiles that
// waits twice per tile for gathered rows; eight rows of 64 heads are 32 workgroups on a 256-CU
// part. Here:
//   1. attn_f32_split_scores_kernel: one workgroup per (row, tile, block of one, two or four
//      16-head groups). Its eight waves gather the tile's 32 K rows once for the block and run
//      attn_f32_kernel's score contraction for each head group and 16-key block over each
//      dimension quarter (the same MFMA steps on the same operands): wave w takes quarter
//      w >> 1 and, with one head group, key block w & 1; with two or four, half of the head
//      groups (w & 1) and both key blocks, so that no two waves load the same query columns.
//      Wave i then sums head group i's quarters in order and stores the raw sums, in
//      attn_f32_kernel's lane layout (lane (g, l16): tile keys g + 4e of head l16), to the
//      workspace: [row][tile][16-head group][lane][8] fp32, 2 KiB per tile and head group.
//   2. attn_f32_split_values_kernel: one workgroup per (row, 16-head group, 64-column slice),
//      four waves, one 16-column block each, in rounds of up to twelve tiles. Each wave gathers
//      its own columns of the round's V rows and loads the score sums of its share of the tiles;
//      then (a) each wave scales and masks the scores of every fourth tile and takes their
//      maxima, (b) every wave walks the running maximum over the round's tiles (each tile's
//      reference and alpha), and each wave weighs its own tiles, and (c) every wave runs the
//      tile sums, rescales and value MFMAs in key order, as attn_f32_kernel does for its
//      columns, refilling its V slots with the next round's tiles as it goes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_attn_f32_common.h"
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kSplitColsF = 64;                  // output columns per values workgroup
constexpr int kSlicesF = kHeadDim / kSplitColsF;
constexpr int kSTileF = 64 * 8 * 4;              // one tile's scores for a 16-head group: 2 KiB
constexpr int kRingF = 12;                       // tiles per round of the values kernel
constexpr int kMineF = kRingF / 4;               // tiles each of the four waves scales and weighs
static_assert(kRingF % 4 == 0, "every wave weighs the same number of a round's tiles");
static_assert(kRingF * (kT32 * kSplitColsF * 4 + kSTileF + 2 * 64 * 4) + kSplitMaxK * 4 <= 150 * 1024, "LDS budget");

// LDS pointer from a 32-bit LDS byte address.
template <typename T>
__device__ __forceinline__ SA_LDS T *lds_ptr(uint32_t addr) {
    return (SA_LDS T *)(uintptr_t)addr;
}

// Score tiles: [row][tile][head group][lane][8] fp32 (offset in floats).
__device__ __forceinline__ size_t score_block_f32(int64_t row, int tile, int hg, int ntiles_max, int n_hg) {
    return (((size_t)row * ntiles_max + tile) * n_hg + hg) * (kSTileF / 4);
}

// The row's count, by a scalar (constant address space) load.
__device__ __forceinline__ int row_count_f32(const AttnArgs &a, int64_t row) {
    int n = a.nsel ? *(const __attribute__((address_space(4))) int32_t *)(a.nsel + row) : a.kmax;
    return n < 0 ? 0 : (n > a.kmax ? a.kmax : n);
}

// One workgroup per (row, tile, block of HPB 16-head groups), blocks fastest. A tile past the
// row's count has no selected key: its workgroup leaves at once (the values kernel never reads
// it). HPB trades the K tile's gathers (once per block) against the spread of the score MFMAs
// over the chip: a tile's 64 heads are 2.1 MFLOP of float32 matrix work, 3.4 us on one CU.
template <int HPB>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_f32_split_scores_kernel(AttnArgs a, int ntiles_max, int n_hb, int n_hg) {
    __shared__ __attribute__((aligned(16))) char k_lds[kT32 * kKStrF];
    __shared__ f32x4 part_lds[HPB][4][2][64];  // [head group][dimension quarter][block][lane]

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    // One head group: wave w takes key block w & 1. Two or four: head groups HW (w & 1) .. +HW-1
    // of the block (HW = HPB / 2) and both key blocks.
    constexpr int HW = HPB == 1 ? 1 : HPB / 2;
    constexpr int NB = HPB == 1 ? 1 : 2;
    const int half = w & 1;
    const int dq = w >> 1;
    // XCD-aware order: the head blocks of one tile run on one XCD, where their gathers of the
    // same K rows share its L2.
    const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int hb = (int)(bid % n_hb);
    const int tile = (int)((bid / n_hb) % ntiles_max);
    const int64_t row = bid / ((int64_t)n_hb * ntiles_max);
    const int hg0 = HPB * hb;
    const int ng = n_hg - hg0 < HPB ? n_hg - hg0 : HPB;  // head groups in the block

    // The tile's index entry (lane l: entry 32 tile + (l & 31)), the queries of the block's head
    // groups and the row's count go out together.
    const int p = tile * kT32 + (lane & 31);
    float raw;
    load4_async(raw, a.idx + row * a.kmax + (p < a.kmax ? p : a.kmax - 1));
    // Query of this wave's head group j (block head group jg) for its dimension quarter: lane
    // (g, l16) holds dims 128 g + 32 dq .. +31 of head 16 (hg0 + jg) + l16 (zero for heads past H).
    auto group_of = [&](int j) { return HPB == 1 ? 0 : HW * half + j; };
    float qv[HW][32];
#pragma unroll
    for (int j = 0; j < HW; j++) {
        const int i = group_of(j);
        const int head = 16 * (hg0 + i) + l16;
        const bool ok = i < ng && head < a.H;
        const float *qrow = (const float *)a.q + (row * a.H + (ok ? head : 0)) * kHeadDim + 128 * g + 32 * dq;
#pragma unroll
        for (int c = 0; c < 8; c++) {
            const f32x4 x = ok ? *(const f32x4 *)(qrow + 4 * c) : (f32x4){};
            qv[j][4 * c] = x[0];
            qv[j][4 * c + 1] = x[1];
            qv[j][4 * c + 2] = x[2];
            qv[j][4 * c + 3] = x[3];
        }
    }
    const int n = row_count_f32(a, row);
    wait_vmcnt<0>();
    register_ready(raw);
    if (tile * kT32 >= n) return;
    // Row to gather for the entry, or -1 (masked or out of range: gathers zeros, as in
    // attn_f32_kernel; the values kernel marks a row with a live out-of-range entry as NaN).
    const int iv_raw = __float_as_int(raw);
    const bool live = p < n;
    const int iv = (live && iv_raw >= 0 && (int64_t)iv_raw < a.n_ctx) ? iv_raw : -1;

    // Wave w gathers tile keys 4w .. 4w+3 (two 1 KiB DMAs per 2 KiB row) into attn_f32_kernel's
    // K slots.
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)a.k + row * a.cache_stride * 4), 0, (int)(uint32_t)(a.n_ctx * kRowF), kBufferFlags);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int kap = 4 * w + i;
        const uint32_t off = ((uint32_t)__builtin_amdgcn_readlane(iv, kap) << 11) + ((uint32_t)lane << 4);
        const uint32_t dst = lds_addr((SA_LDS char *)k_lds + kslot32(kap) * kKStrF);
        dma16_buf(rk, off, dst);
        dma16_buf(rk, off + 1024u, dst + 1024u);
    }
    wait_vmcnt<0>();
    lds_barrier();  // every wave's K rows have landed

    // Partial scores over the dimension quarter dq of this wave's (head group, key block) pairs:
    // HW x NB independent accumulation chains (a group past the heads contracts a zero query and
    // is not stored), each in attn_f32_kernel's step order.
    const int b0 = HPB == 1 ? (w & 1) : 0;
    const SA_LDS char *krow = (const SA_LDS char *)k_lds + (16 * b0 + l16) * kKStrF + (128 * g + 32 * dq) * 4;
    f32x4 sp[HW][NB] = {};
#pragma unroll
    for (int c = 0; c < 8; c++) {
        f32x4 kx[NB];
#pragma unroll
        for (int bb = 0; bb < NB; bb++) kx[bb] = *(const SA_LDS f32x4 *)(krow + 16 * bb * kKStrF + 16 * c);
#pragma unroll
        for (int e = 0; e < 4; e++) {
#pragma unroll
            for (int j = 0; j < HW; j++)
#pragma unroll
                for (int bb = 0; bb < NB; bb++)
                    sp[j][bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kx[bb][e], qv[j][4 * c + e], sp[j][bb], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < HW; j++)
#pragma unroll
        for (int bb = 0; bb < NB; bb++)
            if (group_of(j) < ng) part_lds[group_of(j)][dq][b0 + bb][lane] = sp[j][bb];
    lds_barrier();  // every head group's partials are in LDS

    // Wave i sums head group i's four quarters in order and stores the raw sums.
    if (w < ng) {
        float tot[8];
#pragma unroll
        for (int bb = 0; bb < 2; bb++) {
            const f32x4 p0 = part_lds[w][0][bb][lane], p1 = part_lds[w][1][bb][lane];
            const f32x4 p2 = part_lds[w][2][bb][lane], p3 = part_lds[w][3][bb][lane];
#pragma unroll
            for (int j = 0; j < 4; j++) tot[4 * bb + j] = f32_score_sum(p0[j], p1[j], p2[j], p3[j]);
        }
        f32x4 *dst =
            (f32x4 *)((float *)a.ws + score_block_f32(row, tile, hg0 + w, ntiles_max, n_hg) + lane * 8);
        dst[0] = (f32x4){tot[0], tot[1], tot[2], tot[3]};
        dst[1] = (f32x4){tot[4], tot[5], tot[6], tot[7]};
    }
}

// One workgroup per (row, 16-head group, 64-column slice), in an order that keeps the
// workgroups of one row and head group on one XCD (they read the same score tiles). Four waves:
// wave w owns the 16 columns cs*64 + 16w .. +15 (one MFMA block) and gathers only those columns
// of every selected V row, into LDS slots of its own (32 keys x 64 bytes per tile: the four keys
// one value read takes sit in one 256-byte window, on distinct banks). A wave's slot of a tile
// is then free as soon as its own value MFMAs of that tile have read it: the next round's V
// slices go out in the value phase, tile by tile, with no barrier, and the wave's share of the
// next round's score tiles is loaded into registers in the same phase.
__global__ void __launch_bounds__(256)
attn_f32_split_values_kernel(AttnArgs a, int ntiles_max, int n_hg) {
    constexpr int kVPriv = kT32 * 16 * 4;   // a wave's 16 columns of a tile: 2 KiB
    __shared__ __attribute__((aligned(16))) char v_lds[kRingF][4][kVPriv];
    __shared__ f32x4 pe_lds[kRingF][64][2];  // per tile: its weights, lane layout (keys g + 4e)
    __shared__ float mt_lds[kRingF][64];     // per tile: its maximum
    __shared__ float psum_lds[kRingF][64];   // per tile: its sum
    __shared__ int idx_lds[kSplitMaxK];
    __shared__ int bad_lds[4];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int64_t u = xcd_remap(blockIdx.x, gridDim.x);
    const int cs = (int)(u % kSlicesF);
    const int hg = (int)((u / kSlicesF) % n_hg);
    const int64_t row = u / ((int64_t)kSlicesF * n_hg);
    const int head = 16 * hg + l16;
    const bool head_ok = head < a.H;

    // This wave's raw score sums of the tiles w, w + 4, w + 8 of the round starting at tile t0
    // (lane layout: 32 bytes per lane); tiles past ntiles_max are not read. Tiles past the row's
    // count are never written by the scores kernel; reading them stays inside the workspace, and
    // they are not used.
    const float *sws = (const float *)a.ws + score_block_f32(row, 0, hg, ntiles_max, n_hg);
    f32x4 sraw[kMineF][2];
    auto load_scores = [&](int t0) {
#pragma unroll
        for (int j = 0; j < kMineF; j++) {
            const int t = t0 + w + 4 * j;
            if (t < ntiles_max) {
                const f32x4 *src = (const f32x4 *)(sws + (size_t)t * n_hg * (kSTileF / 4) + lane * 8);
                sraw[j][0] = src[0];
                sraw[j][1] = src[1];
            }
        }
    };

    // First memory round trip: this wave's score sums of the first round, the row's index list
    // (the first ntiles_max * 32 entries, the offsets clamped to the row), the sink and the
    // row's count, all in flight together.
    load_scores(0);
    const int npieces = (ntiles_max * kT32 + 63) / 64;  // index pieces of 64 entries; piece j: wave j & 3
    for (int j = w; j < npieces; j += 4) {
        const int pp = j * 64 + lane;
        const int pc = pp < a.kmax ? pp : a.kmax - 1;
        dma4(a.idx + row * a.kmax, (uint32_t)pc * 4u, lds_addr(&idx_lds[j * 64]));
    }
    float sink;
    load4_async(sink, head_ok ? a.sinks + head : (const float *)g_zero_row);
    const int n = row_count_f32(a, row);
    const int ntiles = (n + kT32 - 1) / kT32;
    wait_vmcnt<0>();
    register_ready(sink);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // every wave's index pieces have landed

    float m = sink;
    float l = expf(sink - f32_ref(sink));
    f32x4 acc = {};
    const float scale = a.scale;

    const int64_t col_b = ((int64_t)cs * kSplitColsF + 16 * w) * 4;  // byte offset of the wave's columns
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)a.v + row * a.cache_stride * 4 + col_b), 0, (int)(uint32_t)(a.n_ctx * kRowF - col_b),
        kBufferFlags);
    const uint32_t v_base = lds_addr((SA_LDS char *)&v_lds[0][w][0]);
    // An entry inside the count that is out of range makes the whole row NaN, as in
    // attn_f32_kernel (bad_w: one of the row's entries is; every wave sees every entry).
    bool bad_w = false;
    // Tile t's V columns of this wave into slot i: two DMAs of sixteen keys; lane l moves the
    // 16-byte chunk l & 3 of key 16h + (l >> 2) (masked or out-of-range entries gather zeros).
    auto issue_v = [&](int t, int i) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int pos = t * kT32 + 16 * h + (lane >> 2);
            const int raw = pos < n ? idx_lds[pos] : -1;
            const bool inr = raw >= 0 && (int64_t)raw < a.n_ctx;
            bad_w = bad_w || __builtin_amdgcn_ballot_w64(pos < n && !inr) != 0;
            const int iv = inr ? raw : -1;  // -1: an offset past the range, zeros
            dma16_buf(rv, ((uint32_t)iv << 11) + ((uint32_t)(lane & 3) << 4),
                      v_base + (uint32_t)(i * 4 * kVPriv + h * 1024));
        }
    };
    {
        const int nt0 = ntiles < kRingF ? ntiles : kRingF;
        for (int i = 0; i < nt0; i++) issue_v(i, i);
    }

    for (int t0 = 0; t0 < ntiles; t0 += kRingF) {
        const int nt = ntiles - t0 < kRingF ? ntiles - t0 : kRingF;
        wait_vmcnt<0>();  // this wave's V slices of the round (and its score loads) have landed

        // (a) Scaled scores and the maxima of this wave's tiles of the round (w, w + 4, w + 8).
        float sk[kMineF][8];
#pragma unroll
        for (int j = 0; j < kMineF; j++) {
            const int i = w + 4 * j;
            if (i < nt) {
                const float tot[8] = {sraw[j][0][0], sraw[j][0][1], sraw[j][0][2], sraw[j][0][3],
                                      sraw[j][1][0], sraw[j][1][1], sraw[j][1][2], sraw[j][1][3]};
                mt_lds[i][lane] = f32_tile_scores(tot, (t0 + i) * kT32 + g, n, scale, sk[j]);
            }
        }
        lds_barrier();
        // (b) The running maximum over the round's tiles in key order (every wave computes the
        // same values), then the weights of this wave's tiles.
        float ref_t[kRingF], alpha_t[kRingF], mt_t[kRingF];
#pragma unroll
        for (int i = 0; i < kRingF; i++) mt_t[i] = mt_lds[i][lane];
#pragma unroll
        for (int i = 0; i < kRingF; i++) {
            if (i < nt) {
                const float m_new = fmaxf(m, mt_t[i]);
                ref_t[i] = f32_ref(m_new);
                alpha_t[i] = expf(m - ref_t[i]);
                m = m_new;
            }
        }
#pragma unroll
        for (int j = 0; j < kMineF; j++) {
            const int i = w + 4 * j;
            if (i < nt) {
                // ref_t[w + 4j], picked with static indices
                float ref = ref_t[4 * j];
#pragma unroll
                for (int q = 1; q < 4; q++)
                    if (w == q) ref = ref_t[4 * j + q];
                float pe[8];
                const float psum = f32_tile_weights(sk[j], ref, pe);
                pe_lds[i][lane][0] = (f32x4){pe[0], pe[1], pe[2], pe[3]};
                pe_lds[i][lane][1] = (f32x4){pe[4], pe[5], pe[6], pe[7]};
                psum_lds[i][lane] = psum;
            }
        }
        lds_barrier();
        // The next round's score sums go out now (sraw is free).
        const int t1 = t0 + kRingF;
        if (t1 < ntiles) load_scores(t1);
        // (c) Tile sums, rescales and value MFMAs in key order. The tile sums are read up front,
        // and each tile's weights and value operands one tile ahead of its MFMAs. Once tile i's
        // MFMAs have read the wave's slot i, the next round's tile i goes into it.
        float psum_t[kRingF];
#pragma unroll
        for (int i = 0; i < kRingF; i++) psum_t[i] = psum_lds[i][lane];
        auto operands = [&](int i, f32x4 &pa, f32x4 &pb, float (&vx)[8]) {
            pa = pe_lds[i][lane][0];
            pb = pe_lds[i][lane][1];
#pragma unroll
            for (int st = 0; st < 8; st++)
                vx[st] = *lds_ptr<float>(v_base + (uint32_t)(i * 4 * kVPriv + (4 * st + g) * 64 + l16 * 4));
        };
        f32x4 pa_c, pb_c;
        float vx_c[8];
        operands(0, pa_c, pb_c, vx_c);
#pragma unroll
        for (int i = 0; i < kRingF; i++) {
            if (i < nt) {
                f32x4 pa_n = pa_c, pb_n = pb_c;
                float vx_n[8];
#pragma unroll
                for (int st = 0; st < 8; st++) vx_n[st] = vx_c[st];
                if (i + 1 < kRingF) operands(i + 1, pa_n, pb_n, vx_n);
                l = f32_l_step(alpha_t[i], l, psum_t[i]);
                const float pe[8] = {pa_c[0], pa_c[1], pa_c[2], pa_c[3], pb_c[0], pb_c[1], pb_c[2], pb_c[3]};
                f32x4 tv = {};
#pragma unroll
                for (int st = 0; st < 8; st++) tv = __builtin_amdgcn_mfma_f32_16x16x4f32(vx_c[st], pe[st], tv, 0, 0, 0);
                acc = f32_acc_step(acc, alpha_t[i], tv);
                // Slot i has been read (its values are in vx_c, used above): refill it.
                if (t1 + i < ntiles) issue_v(t1 + i, i);
                pa_c = pa_n;
                pb_c = pb_n;
#pragma unroll
                for (int st = 0; st < 8; st++) vx_c[st] = vx_n[st];
            }
        }
        lds_barrier();  // every wave is done with this round's weights
    }
    wait_vmcnt<0>();

    // Whole-row NaN for an out-of-range index (any wave saw one), else acc / l.
    if (lane == 0) bad_lds[w] = bad_w;
    lds_barrier();
    bool row_bad = false;
#pragma unroll
    for (int i = 0; i < 4; i++) row_bad = row_bad || bad_lds[i] != 0;
    if (head_ok) {
        float *dst = a.out + (row * a.H + head) * kHeadDim + cs * kSplitColsF + 16 * w + 4 * g;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = row_bad ? __uint_as_float(0x7fc00000u) : acc[e] / l;
        *(f32x4 *)dst = o;
    }
}

}  // namespace

bool f32_split_applies(int64_t rows, int H, int32_t kmax) {
    const int64_t n_hb = (H + 63) / 64;
    return kmax > kF32SplitMinK && kmax <= kSplitMaxK && rows * n_hb < kF32SplitMaxUnits;
}

size_t f32_split_workspace_bytes(int64_t rows, int H, int32_t kmax) {
    const int64_t ntiles_max = (kmax + kT32 - 1) / kT32;
    const int64_t n_hg = (H + 15) / 16;
    return (size_t)(rows * ntiles_max * n_hg) * kSTileF;
}

hipError_t launch_attn_f32_split(const AttnArgs &a, hipStream_t s) {
    const int ntiles_max = (a.kmax + kT32 - 1) / kT32;
    const int n_hg = (a.H + 15) / 16;
    const int64_t g2 = (int64_t)a.rows * n_hg * kSlicesF;
    if (g2 == 0) return hipSuccess;
    // Head groups per scores workgroup: the fewest (most workgroups) that keep the launch at one
    // workgroup per CU (two on one CU would share its matrix cores, whose rate sets a
    // workgroup's time). The choice never changes a bit.
    const int64_t slots = device_cu_count();
    int hpb = 1;
    while (hpb < 4 && (int64_t)a.rows * ntiles_max * ((n_hg + hpb - 1) / hpb) > slots) hpb *= 2;
    const int n_hb = (n_hg + hpb - 1) / hpb;
    const dim3 g1((unsigned)((int64_t)a.rows * ntiles_max * n_hb));
    if (hpb == 1)
        hipLaunchKernelGGL(attn_f32_split_scores_kernel<1>, g1, dim3(512), 0, s, a, ntiles_max, n_hb, n_hg);
    else if (hpb == 2)
        hipLaunchKernelGGL(attn_f32_split_scores_kernel<2>, g1, dim3(512), 0, s, a, ntiles_max, n_hb, n_hg);
    else
        hipLaunchKernelGGL(attn_f32_split_scores_kernel<4>, g1, dim3(512), 0, s, a, ntiles_max, n_hb, n_hg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_f32_split_values_kernel, dim3((unsigned)g2), dim3(256), 0, s, a, ntiles_max, n_hg);
    return hipGetLastError();
}

}  // namespace sa
