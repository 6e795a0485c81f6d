// sa_attn.hip -- gathered sparse attention with per-head sinks, bf16 storage, for gfx950.
//
// What it computes: akol1/TensorFold pull request 4 ("DeepSeek V4.1: sparse
// attention on eight SIMD groups, the same bytes"), first commit message: for a
// query row and its heads, the selected keys are scored in 64-key tiles against a
// 512-wide head (sixteen 32-wide output column groups), with a running maximum, a
// tile sum and a value sum kept in a fixed order. TensorFold pull request 1206,
// "What changes": every head has a sink logit (zero for padded heads).
//
// How it maps to CDNA4 (this is not the pages' one-SIMD-group-per-head design):
//   * One workgroup serves one query row and a block of 32 or 64 heads, because
//     the key/value latent is shared by all heads of a row: each selected cache
//     row is gathered from HBM once per row, not once per head.
//   * The gather is an index-driven direct-to-LDS DMA (global_load_lds_dwordx4):
//     one wave instruction moves one whole 1 KiB cache row (or the workgroup's
//     column slice of it), so every gather is a fully coalesced burst. K and V tiles sit in two LDS buffers; the next
//     tile's K is in flight while the current tile's values are applied, and the
//     next tile's V while the next scores are formed.
//   * S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_32x32x16_bf16 with the heads
//     on the N side, so every lane owns one head. The two waves of a head block each
//     hold the query for one half of the head width (64 VGPRs) and form partial
//     scores for all 64 keys; each hands the other the partials of its key half
//     through LDS, and both add (half 0 + half 1). The row maximum and the tile sum
//     are then an in-lane reduction over 16 scores, one exchange with lane^32, and a
//     fixed-order combine of the two key halves in LDS. V^T operands come from
//     ds_read_b64_tr_b16 transposing reads.
//   * Splitting work across workgroups only ever splits heads and output columns,
//     never keys, so each (row, head, column) is produced by the same sequence of
//     operations whatever the batch size or head count: results are bit-identical
//     across launch shapes and repeats, and no workspace or combine pass exists.
//
// Numerics (the fixed order), in log2 units (x2 = x * log2 e): per 64-key tile,
// m' = max(m, max_j s_j); the exponent reference r moves to m' (0 if m' = -inf), with
// alpha = 2^(r - r'), only when m' > r + 8 or r > m' > -inf for one of the wave's 32
// heads, else alpha = 1; p_j = 2^(s_j - r) rounded to bf16; l = alpha*l + sum_j p_j
// (the same rounded p); acc = alpha*acc + P V; m = m'. Start: m = sink, r = sink
// (0 if -inf), l = 2^(sink - r), acc = 0. End: acc / l. The moves of r change only
// rounding: every p stays below 2^8 and the ratio acc / l is what the definition gives.
// Keys past a row's count score -inf by select and gather a zero row, so a tail
// tile never multiplies a stale LDS value.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

// Kernel template.
//   HB: head blocks of 32 per workgroup (1 or 2); the workgroup has 2*HB waves.
//   NT: 32-column output groups per wave; the workgroup covers 64*NT columns.
// Wave w: head block hb = w/2; kb = w%2 picks the half of the head width the wave
// contracts for the scores, the 32-key block of each tile it finishes and
// normalises, and the half of the workgroup's columns it accumulates.
template <int HB, int NT>
__global__ void __launch_bounds__(128 * HB) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bf16_kernel(AttnArgs a, int n_hg, int64_t units) {
    constexpr int WAVES = 2 * HB;
    constexpr int COLS = 64 * NT;              // output columns per workgroup
    constexpr int VROW = COLS * 2;             // bytes of one V row slice
    constexpr int VSTRIDE = VROW + 64;         // padded V row stride in LDS
    constexpr int VCHUNKS = VROW / 16;         // 16-byte pieces of a V row slice
    constexpr int NK = kTile / WAVES;          // K rows gathered per wave per tile
    constexpr int NV = kTile / WAVES;          // V rows gathered per wave per tile
    constexpr int N_CS = kHeadDim / COLS;
    constexpr int kStores = 4 * NT;             // output stores per wave per unit
    static_assert(NK * WAVES == kTile, "tile split");
    static_assert(NV + 1 < 64 && NK < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) char k_lds[kTile * kKStride];
    __shared__ __attribute__((aligned(16))) char v_lds[kTile * VSTRIDE];
    // Per-wave 4 KiB exchange slot: first the partial scores a wave hands its partner,
    // later in the tile its P operand (the partner has read the partials by then).
    __shared__ __attribute__((aligned(16))) float xch_lds[WAVES][16][64];
    __shared__ float max_lds[WAVES][32];
    __shared__ float sum_lds[WAVES][32];
    __shared__ int idx_lds[WAVES][2][64];   // each wave's own copy of a tile's index list

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5;
    const int ln = lane & 31;
    const int hb = w >> 1;
    const int kb = w & 1;

    // A unit is one (query row, head group, column slice). This workgroup serves units
    // base, base + G, base + 2G, ... as one stream of 64-key tiles, so the next unit's
    // first gathers overlap the current unit's last tile. Every unit has at least one
    // tile (a row with no selected key runs one all-masked tile, which changes nothing).
    const int64_t G = (int64_t)gridDim.x;
    const int64_t base = xcd_remap(blockIdx.x, G);

    struct Item {          // one tile of one unit (all fields wave-uniform)
        int64_t unit;      // < 0: none
        int64_t row;
        int tile, ntiles, n, hg, cs;
    };
    auto make_item = [&](int64_t u) -> Item {
        Item it{};
        it.unit = u;
        if (u < 0 || u >= units) { it.unit = -1; return it; }
        it.cs = (int)(u % N_CS);
        it.hg = (int)((u / N_CS) % n_hg);
        it.row = u / ((int64_t)N_CS * n_hg);
        // A scalar (constant address space) load: it waits on the LDS/scalar counter,
        // not on the vector-memory counter that the in-flight gathers hold.
        int n = a.nsel ? *(const __attribute__((address_space(4))) int32_t *)(a.nsel + it.row) : a.kmax;
        n = n < 0 ? 0 : (n > a.kmax ? a.kmax : n);
        it.n = n;
        it.tile = 0;
        it.ntiles = n > 0 ? (n + kTile - 1) / kTile : 1;
        return it;
    };
    auto next_item = [&](const Item &it) -> Item {
        if (it.unit < 0) return it;
        if (it.tile + 1 < it.ntiles) { Item nx = it; nx.tile++; return nx; }
        return make_item(it.unit + G);
    };
    auto idx_row = [&](const Item &it) { return a.idx + it.row * a.kmax; };
    auto kbase_of = [&](const Item &it) { return (const char *)a.k + it.row * a.cache_stride * 2; };
    auto vbase_of = [&](const Item &it) {
        return (const char *)a.v + it.row * a.cache_stride * 2 + (int64_t)it.cs * VROW;
    };

    // Index list of an item's tile into this wave's slot buf: lane l fetches entry
    // tile*64 + l (address clamped to the row). Always issued, also when there is no
    // item (then the current row's list is re-read), so that every wave issues the same
    // number of vector-memory operations per tile.
    auto dma_idx = [&](const Item &it, const Item &fallback, int buf) {
        const Item &src = it.unit >= 0 ? it : fallback;
        const int p = (it.unit >= 0 ? it.tile : 0) * kTile + lane;
        const int pc = p < a.kmax ? p : a.kmax - 1;
        dma4(idx_row(src), (uint32_t)pc * 4u, lds_addr(&idx_lds[w][buf][0]));
    };
    // Row to gather for entry tile*64 + l, or -1 (masked or out of range: gather zeros).
    auto resolve = [&](const Item &it, int buf, bool &bad) -> int {
        const int iv = idx_lds[w][buf][lane];
        const int p = it.tile * kTile + lane;
        const bool live = p < it.n;
        const bool inr = iv >= 0 && (int64_t)iv < a.n_ctx;
        if (__builtin_amdgcn_ballot_w64(live && !inr)) bad = true;
        return (live && inr) ? iv : -1;
    };
    // One DMA instruction gathers one cache row (64 lanes x 16 bytes = 1 KiB) into an
    // LDS slot; lane i moves bytes [16i, 16i + 16) of the row. Wave w gathers keys
    // NK*w + i. The buffer resource spans the row's cache; a masked key (-1) has a
    // wrapped-around offset past its end and arrives as zeros.
    // Row DMAs are issued one at a time, spread through the tile's compute, so that the
    // CU's address unit (16 cycles per 1 KiB row) never queues a burst of them.
    auto rsrc_k = [&](const Item &it) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)kbase_of(it), 0, (int)(uint32_t)(a.n_ctx * kRowBytes),
                                                 kBufferFlags);
    };
    auto rsrc_v = [&](const Item &it) {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)vbase_of(it), 0, (int)(uint32_t)(a.n_ctx * kRowBytes - (int64_t)it.cs * VROW), kBufferFlags);
    };
    auto dma_k_row = [&](__amdgpu_buffer_rsrc_t rsrc, int iv, int i) {
        const int ij = __builtin_amdgcn_readlane(iv, NK * w + i);
        dma16_buf(rsrc, ((uint32_t)ij << 10) + ((uint32_t)lane << 4),
                  lds_addr((SA_LDS char *)k_lds + (NK * w + swap23(i)) * kKStride));
    };
    // V rows keep the tile's key order; only the unit's column slice is moved.
    auto dma_v_row = [&](__amdgpu_buffer_rsrc_t rsrc, int iv, int i) {
        const int j = w * NV + i;
        const int ij = __builtin_amdgcn_readlane(iv, j);
        if (VCHUNKS == 64 || lane < VCHUNKS)
            dma16_buf(rsrc, ((uint32_t)ij << 10) + ((uint32_t)lane << 4), lds_addr(v_lds + j * VSTRIDE));
    };

    // Per-unit state. Query operand of S^T = K Q^T over this wave's half kb of the head
    // width: lane (head ln, half g) holds d = 256 kb + 128 g + 8 kk + 0..7, kk < 16.
    // Softmax state in log2 units: scores and the sink are multiplied by log2(e) so that
    // exp(x - y) = exp2(x2 - y2) runs on v_exp_f32. m_run is the running maximum, ref the
    // exponent reference that l_run and acc are relative to (see the tile update).
    const float scale2 = a.scale * kLog2e;
    bf16x8 qreg[16];
    f32x16 acc[NT];
    float m_run, ref, l_run;
    // The next unit's query and sink are loaded asynchronously (load_q_async, then
    // start_unit once a wait has covered them), so a unit boundary needs no drain. The
    // query lands in qreg itself: the previous unit's last scores have been formed.
    float sink_n;
    int head_n;
    bool head_ok_n;
    auto load_q_async = [&](const Item &it) {
        head_n = (it.hg * HB + hb) * 32 + ln;
        head_ok_n = head_n < a.H;
        // Heads past H read zeros (query and sink) from the static zero row.
        const uint16_t *qrow = head_ok_n ? (const uint16_t *)a.q + (it.row * a.H + head_n) * kHeadDim
                                         : (const uint16_t *)g_zero_row;
        qrow += 256 * kb + 128 * g;
#pragma unroll
        for (int kk = 0; kk < 16; kk++) load16_async(qreg[kk], qrow + 8 * kk);
        load4_async(sink_n, head_ok_n ? a.sinks + head_n : (const float *)g_zero_row);
    };
    // After a vector-memory wait that covers load_q_async: the loaded registers become
    // ordinary values (register_ready), and the unit's state starts from its sink.
    auto start_unit = [&]() {
#pragma unroll
        for (int kk = 0; kk < 16; kk++) register_ready(qreg[kk]);
        register_ready(sink_n);
        const float sink2 = sink_n * kLog2e;
        m_run = sink2;
        ref = (sink2 == -INFINITY) ? 0.0f : sink2;
        l_run = exp2_hw(sink2 - ref);
#pragma unroll
        for (int nt = 0; nt < NT; nt++) acc[nt] = (f32x16){};
    };
    // Normalise and store. Lane (g, ln) holds head ln, columns 32nt + 8eq + 4g + 0..3 of
    // the wave's slice, for eq < 4. Per 32-column group nt the wave's 32 x 32 block goes
    // through its own 4 KiB exchange slot: written by MFMA lane, read back so that eight
    // lanes hold one head's 128 contiguous bytes, then stored as whole 128-byte lines.
    // In the slot, 16-byte chunk c of head row r sits at chunk c ^ ((r >> 1) & 7): both the
    // writes (sixteen rows, one chunk) and the reads (two rows, eight chunks) of every
    // sixteen lanes then touch sixteen different bank groups.
    // The stores go through a buffer resource spanning the unit's output row; a lane
    // whose head is past H stores past its end, which the hardware drops. So every wave
    // issues exactly kStores stores, which the vector-memory waits below count on.
    auto leave_unit = [&](const Item &it, bool bad) {
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            a.out + it.row * a.H * kHeadDim, 0, a.H * kHeadDim * 4, kBufferFlags);
        SA_LDS char *slot = (SA_LDS char *)&xch_lds[w][0][0];
        // x * 1 is x exactly and x * NaN is NaN: a select of constants, so the divide is
        // not put behind a branch and the store count stays the same on every path.
        const float poison = bad ? NAN : 1.0f;
        const int rd_row = lane >> 3, rd_chunk = lane & 7;
        const int head0 = (it.hg * HB + hb) * 32;
        const int col0 = it.cs * COLS + kb * NT * 32;
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
#pragma unroll
            for (int eq = 0; eq < 4; eq++) {
                f32x4 o;
#pragma unroll
                for (int i = 0; i < 4; i++) o[i] = (acc[nt][4 * eq + i] / l_run) * poison;
                const int c = 2 * eq + g;
                *(SA_LDS f32x4 *)(slot + ln * 128 + 16 * (c ^ ((ln >> 1) & 7))) = o;
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = 8 * i + rd_row;
                const f32x4 o = *(const SA_LDS f32x4 *)(slot + r * 128 + 16 * (rd_chunk ^ ((r >> 1) & 7)));
                const int h = head0 + r;
                const int off = h < a.H ? (h * kHeadDim + col0 + 32 * nt + 4 * rd_chunk) * 4 : kDropOffset;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rsrc, off, 0, kStoreNT);
            }
        }
    };

    // Issue order per wave: Q/sink(0), I(0) | drain | K(0), I(1); then in tile j: V(j)
    // spread through the scores; on a unit's last tile the next unit's query and sink
    // (kQLoads) once V(j) has landed; K(j+1) spread through the values; then I(j+2),
    // followed on a unit's last tile by its kStores output stores. Each wait below counts
    // exactly the operations issued after the one it needs.
    Item cur = make_item(base);
    Item nx = next_item(cur);
    Item nx2 = next_item(nx);
    bool bad = false, bad_next = false;
    load_q_async(cur);
    dma_idx(cur, cur, 0);
    wait_vmcnt<0>();
    start_unit();
    __builtin_amdgcn_s_waitcnt(0);  // nothing the compiler tracks is pending in the loop
    bool starting = false;          // the next unit's query is in flight
    bool stores_out = false;        // the previous tile ended a unit: its stores follow I(j+1)
    int iv_cur = resolve(cur, 0, bad);  // rows of the current tile (its V goes out with the scores)
    {
        const __amdgpu_buffer_rsrc_t rk = rsrc_k(cur);
#pragma unroll
        for (int i = 0; i < NK; i++) dma_k_row(rk, iv_cur, i);
        dma_idx(nx, cur, 1);
    }

    for (int j = 0; cur.unit >= 0; j++) {
        const bool more = nx.unit >= 0;
        const bool last_of_unit = !more || nx.unit != cur.unit;
        // K(j) has landed for this wave, and with it a unit's query and sink when tile j
        // starts one (issued just before K(j)). After K(j) come I(j+1) and, when tile j
        // starts a unit, the previous unit's stores.
        if (starting) wait_vmcnt<vm_clamp(1 + kStores)>(); else wait_vmcnt<1>();
        if (starting) {
            start_unit();
            starting = false;
        }
        lds_barrier();

        // ---- partial scores over this wave's half kb of the head width, for both
        // 32-key blocks of the tile: S^T (keys) x (32 heads); K from LDS, Q in registers.
        f32x16 sacc0 = (f32x16){}, sacc1 = (f32x16){};
        {
            // Software-pipelined: the operands of step kk+1 are read before the two
            // MFMAs of step kk issue, so LDS latency hides behind the matrix pipe.
            // The tile's V rows go out here, NV / 16 per step, in the matrix pipe's shadow
            // (every wave finished the previous tile's values before the barrier above).
            const __amdgpu_buffer_rsrc_t rv = rsrc_v(cur);
            const SA_LDS char *krow = (const SA_LDS char *)k_lds + ln * kKStride + 512 * kb + 256 * g;
            bf16x8 k0 = *(const SA_LDS bf16x8 *)(krow);
            bf16x8 k1 = *(const SA_LDS bf16x8 *)(krow + 32 * kKStride);
#pragma unroll
            for (int kk = 0; kk < 16; kk++) {
                bf16x8 n0 = k0, n1 = k1;
                if (kk + 1 < 16) {
                    n0 = *(const SA_LDS bf16x8 *)(krow + 16 * (kk + 1));
                    n1 = *(const SA_LDS bf16x8 *)(krow + 32 * kKStride + 16 * (kk + 1));
                }
                sacc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qreg[kk], sacc0, 0, 0, 0);
                sacc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qreg[kk], sacc1, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < NV / 16; r++) dma_v_row(rv, iv_cur, kk * (NV / 16) + r);
                __builtin_amdgcn_sched_barrier(0);
                k0 = n0;
                k1 = n1;
            }
        }
        // Hand the partner (the other half of the head width) its key block's partials.
        {
            const f32x16 give = kb ? sacc0 : sacc1;
#pragma unroll
            for (int c = 0; c < 4; c++)  // chunk c of every lane is contiguous: 16-byte writes
                ((f32x4 *)&xch_lds[w][0][0])[64 * c + lane] =
                    (f32x4){give[4 * c], give[4 * c + 1], give[4 * c + 2], give[4 * c + 3]};
        }
        lds_barrier();  // partials exchanged; every wave is also done reading k_lds

        // Indices of item j+1 have landed (after them: [stores], V(j)).
        if (stores_out) wait_vmcnt<vm_clamp(kStores + NV)>(); else wait_vmcnt<NV>();
        int iv_n = 0;
        const bool q_now = last_of_unit && more;
        if (more) iv_n = resolve(nx, (j + 1) & 1, nx.unit == cur.unit ? bad : bad_next);
        const __amdgpu_buffer_rsrc_t rk = rsrc_k(nx);

        // Full scores of key block kb: (half 0 + half 1) of the head width, the same
        // sum in both waves of the pair. Element e of this lane is key
        // kb*32 + 16*(e/8) + 8g + e%8 of the tile.
        const f32x16 own = kb ? sacc1 : sacc0;
        f32x4 part[4];
#pragma unroll
        for (int c = 0; c < 4; c++) part[c] = ((const f32x4 *)&xch_lds[w ^ 1][0][0])[64 * c + lane];
        float s[16];
        float mloc = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const float full = own[e] + part[e >> 2][e & 3];
            const int p = cur.tile * kTile + kb * 32 + 16 * (e >> 3) + 8 * g + (e & 7);
            s[e] = p < cur.n ? full * scale2 : -INFINITY;
            mloc = fmaxf(mloc, s[e]);
        }
        mloc = max_xor32(mloc);
        if (g == 0) max_lds[w][ln] = mloc;
        lds_barrier();  // maxima exchanged; every wave is done reading the partials

        // ---- online softmax with the sink, fixed order. The reference follows the
        // running maximum lazily: it moves (and l_run, acc are rescaled by alpha) only
        // when the maximum has risen more than kLazy above it, or when it sits above a
        // finite maximum (only possible from the start value 0 of a -inf sink); the
        // decision is taken for the wave's 32 heads together. Otherwise alpha = 1 and
        // the accumulators are left alone; every p stays <= 2^kLazy.
        const float mt = fmaxf(max_lds[2 * hb][ln], max_lds[2 * hb + 1][ln]);
        const float m_new = fmaxf(m_run, mt);
        const bool move = m_new > ref + kLazy || (m_new < ref && m_new != -INFINITY);
        const bool rescale = __builtin_amdgcn_ballot_w64(move) != 0;
        float alpha = 1.0f;
        if (rescale) {
            const float ref_new = (m_new == -INFINITY) ? 0.0f : m_new;
            // Nothing accumulated yet (l = 0, from a -inf sink): the old reference may be
            // arbitrarily far above the new one, and 0 (not 2^(r - r'), which can overflow
            // to inf and make inf * 0) keeps l and acc at 0.
            alpha = l_run == 0.0f ? 0.0f : exp2_hw(ref - ref_new);
            ref = ref_new;
        }
        // p = hi + lo with both parts bf16, so the value product (one MFMA per part) sees
        // p to about 16 significant bits and l sums the same hi + lo. For p > 0 both parts
        // are positive, so an infinite value times a positive weight stays infinite (never
        // inf - inf or 0 * inf): hi is p truncated toward zero and lo = bf16(p - hi); when
        // p is itself a bf16 value, hi is the next bf16 below it and lo its last unit, so
        // hi + lo = p exactly (exact sums stay exact).
        bf16x8 ph0, ph1, pl0, pl1;
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const float pf = exp2_hw(s[e] - ref);
            const uint32_t pbits = __float_as_uint(pf);
            const uint32_t trunc = pbits >> 16;  // a NaN stays a NaN after either step below
            const bool exact = (pbits & 0xffffu) == 0u && pf > 0.0f;
            const uint32_t hb = exact ? trunc - 1u : trunc;
            const float hif = __uint_as_float(hb << 16);
            const __bf16 hi = __builtin_bit_cast(__bf16, (uint16_t)hb);
            const __bf16 lo = (__bf16)(pf - hif);
            psum += hif + (float)lo;
            if (e < 8) { ph0[e] = hi; pl0[e] = lo; } else { ph1[e - 8] = hi; pl1[e - 8] = lo; }
        }
        psum = sum_xor32(psum);
        bf16x8 *p_out = (bf16x8 *)&xch_lds[w][0][0];
        p_out[lane] = ph0;
        p_out[64 + lane] = ph1;
        p_out[128 + lane] = pl0;
        p_out[192 + lane] = pl1;
        if (g == 0) sum_lds[w][ln] = psum;

        // V(j) has landed: nothing was issued after it.
        wait_vmcnt<0>();
        // On a unit's last tile: the next unit's query (the scores were qreg's last use),
        // ahead of the K rows, so the wait for K(j+1) covers it too.
        if (q_now) load_q_async(nx);
        lds_barrier();

        l_run = alpha * l_run + (sum_lds[2 * hb][ln] + sum_lds[2 * hb + 1][ln]);
        m_run = m_new;

        if (rescale) [[unlikely]] {
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                acc[nt] *= alpha;
                __builtin_amdgcn_sched_barrier(0);  // one 16-register group at a time
            }
        }

        // ---- values O^T += V^T P^T over the tile's four 16-key steps.
        bf16x8 pop[4], pol[4];  // hi and lo parts of P
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const bf16x8 *src = (const bf16x8 *)&xch_lds[2 * hb + (ks >> 1)][0][0];
            pop[ks] = src[64 * (ks & 1) + lane];
            pol[ks] = src[128 + 64 * (ks & 1) + lane];
        }
        // Lane (g, ch, l16) addresses row 16ks + 8g + 4t2 + l16/4 and columns
        // 32nt + 16ch + 4(l16%4) .. +3 of the wave's half of the slice; the
        // transposing read returns column 32nt + 16ch + l16 of rows +0..3.
        const int l16 = lane & 15;
        const int ch = (lane >> 4) & 1;
        const SA_LDS char *vrow = (const SA_LDS char *)v_lds + (8 * g + (l16 >> 2)) * VSTRIDE +
                                  2 * (kb * NT * 32 + 16 * ch + 4 * (l16 & 3));
        // Software-pipelined over the column groups: the four V^T operands of group
        // nt+1 (eight transposing reads) are issued before the four MFMAs of group nt.
        auto read_v = [&](int nt, bf16x8 (&vop)[4]) {
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
#pragma unroll
                for (int t2 = 0; t2 < 2; t2++) {
                    const bf16x4 part = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (SA_LDS bf16x4 *)(vrow + (16 * ks + 4 * t2) * VSTRIDE + 64 * nt));
                    vop[ks][4 * t2 + 0] = part[0];
                    vop[ks][4 * t2 + 1] = part[1];
                    vop[ks][4 * t2 + 2] = part[2];
                    vop[ks][4 * t2 + 3] = part[3];
                }
            }
        };
        bf16x8 vcur[4], vnxt[4];
        read_v(0, vcur);
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            if (nt + 1 < NT) read_v(nt + 1, vnxt);
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur[ks], pop[ks], acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur[ks], pol[ks], acc[nt], 0, 0, 0);
            }
            // The next tile's K rows go out here, NK / NT per column group, in the matrix
            // pipe's shadow (every wave is past this tile's scores: the K buffer is free).
            if (more) {
#pragma unroll
                for (int r = 0; r < NK / NT; r++) dma_k_row(rk, iv_n, nt * (NK / NT) + r);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 4; ks++) vcur[ks] = vnxt[ks];
        }
        lds_barrier();  // every wave is done with v_lds and the P operands

        dma_idx(nx2, cur, j & 1);  // slot j&1 held item j's list, consumed above
        iv_cur = iv_n;
        stores_out = last_of_unit;
        starting = q_now;
        if (last_of_unit) {
            leave_unit(cur, bad);
            bad = bad_next;
            bad_next = false;
        }
        cur = nx;
        nx = nx2;
        nx2 = next_item(nx2);
    }
    wait_vmcnt<0>();
}

template <int HB, int NT>
hipError_t launch_variant(const AttnArgs &a, int64_t units, int64_t grid, hipStream_t s) {
    const int n_hg = (a.H + 32 * HB - 1) / (32 * HB);
    hipLaunchKernelGGL((attn_bf16_kernel<HB, NT>), dim3((unsigned)grid), dim3(128 * HB), 0, s, a, n_hg, units);
    return hipGetLastError();
}

constexpr int lds_bytes_of(int HB, int NT) {
    return kTile * kKStride + kTile * (128 * NT + 64) + 2 * HB * 4096 + 2 * 2 * HB * 32 * 4 + 2 * HB * 512;
}

}  // namespace

AttnPlan plan_attn_bf16(int64_t rows, int H) {
    AttnPlan p{};
    const int hb = H > 32 ? 2 : 1;
    p.heads_per_wg = 32 * hb;
    const int64_t n_hg = (H + p.heads_per_wg - 1) / p.heads_per_wg;
    const int64_t rows_hg = rows * n_hg;
    // One workgroup per CU fits (the K tile alone is 64 KiB of LDS). With fewer
    // (row, head block) pairs than CUs, column slices add units; every slice gathers
    // the full K tile but only its own V columns.
    int nt = 8;
    if (rows_hg < 64) nt = 1;
    else if (rows_hg < 128) nt = 2;
    else if (rows_hg < 256) nt = 4;
    p.cols_per_wg = 64 * nt;
    p.units = rows_hg * (kHeadDim / p.cols_per_wg);
    if (hb == 2) {  // the eight-wave kernel
        p.threads = 512;
        p.lds_bytes = attn_bf16_ks_lds_bytes(p.cols_per_wg, false);
        return p;
    }
    p.threads = 128 * hb;
    p.lds_bytes = lds_bytes_of(hb, nt);
    return p;
}

namespace {
// Compute units of the current device (cached per device): the persistent grid size,
// since one workgroup of this kernel occupies a CU's LDS.
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}
}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t s) {
    const AttnPlan p = plan_attn_bf16(a.rows, a.H);
    if (p.units == 0) return hipSuccess;
    const int64_t grid = p.units < cu_count() ? p.units : cu_count();
    const int nt = p.cols_per_wg / 64;
    if (p.heads_per_wg == 64) return launch_attn_bf16_ks(a, p.cols_per_wg, p.units, s);
    switch (nt) {
        case 1: return launch_variant<1, 1>(a, p.units, grid, s);
        case 2: return launch_variant<1, 2>(a, p.units, grid, s);
        case 4: return launch_variant<1, 4>(a, p.units, grid, s);
        default: return launch_variant<1, 8>(a, p.units, grid, s);
    }
}

}  // namespace sa
