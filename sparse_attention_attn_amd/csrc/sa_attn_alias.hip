// sa_attn_alias.hip -- gathered sparse attention with per-head sinks when the key and
// value caches are one tensor (a shared latent that serves as both), bf16, gfx950.
//
// What it computes is exactly what sa_attn.hip computes (akol1/TensorFold pull
// request 4, first commit message: 64-key tiles, a running maximum, a tile sum and a
// value sum in a fixed order; TensorFold pull request 1206, "What changes": a sink logit
// per head), with K = V. The pages do not say whether the latent is both; when the
// caller passes the same cache for both, each selected row is gathered once per query
// row instead of twice, which halves the gathered bytes.
//
// Differences from sa_attn.hip, all in the data movement; the per-tile arithmetic
// (scores, softmax with the lazy reference, values, normalisation) is the same code
// in the same order, so an aliased call gives the same bits as a separate-cache call
// with equal contents:
//   * one LDS tile holds the 64 gathered rows and serves both products: the score
//     reads use it as K (slot s holds key (s & 32) | swap23(s & 31)), the transposing
//     value reads use it as V (the four consecutive keys of a ds_read_b64_tr_b16 are
//     four consecutive slots, since swap23 moves whole groups of four);
//   * the row stride is 1104 bytes (80 mod 256): the K reads (sixteen slots at one
//     column) stay conflict-free, the V^T reads (four rows x 64 bytes) see at most a
//     two-way bank conflict;
//   * two tile buffers alternate: tile j+1 is in flight during all of tile j, and tile
//     j+2 is issued as soon as tile j's values are done with its buffer. Index lists
//     run two tiles ahead of the gathers (three ahead of the compute);
//   * every wait names its operation by counting what was issued after it, including
//     the next unit's query (issued after a unit's last scores) and a unit's output
//     stores (issued after the next gathers); the count is formed at run time and
//     dispatched to an s_waitcnt immediate.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kTStride = kRowBytes + 80;  // 1104: 80 (mod 256)

// Kernel template: HB head blocks of 32 (2*HB waves), NT 32-column output groups per
// wave. Wave w: head block hb = w/2, kb = w%2 (half of the head width for the scores,
// key block it finishes, half of the columns it accumulates), as in sa_attn.hip.
template <int HB, int NT>
__global__ void __launch_bounds__(128 * HB) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bf16_alias_kernel(AttnArgs a, int n_hg, int64_t units) {
    constexpr int WAVES = 2 * HB;
    constexpr int COLS = 64 * NT;              // output columns per workgroup
    constexpr int NR = kTile / WAVES;          // rows gathered per wave per tile
    constexpr int N_CS = kHeadDim / COLS;
    constexpr int kStores = 4 * NT;            // output stores per wave per unit
    static_assert(NR * WAVES == kTile, "tile split");

    __shared__ __attribute__((aligned(16))) char t_lds[2][kTile * kTStride];
    __shared__ __attribute__((aligned(16))) float xch_lds[WAVES][16][64];
    __shared__ float max_lds[WAVES][32];
    __shared__ float sum_lds[WAVES][32];
    __shared__ int idx_lds[WAVES][2][64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5;
    const int ln = lane & 31;
    const int hb = w >> 1;
    const int kb = w & 1;

    const int64_t G = (int64_t)gridDim.x;
    const int64_t base = xcd_remap(blockIdx.x, G);

    struct Item {          // one tile of one unit (all fields wave-uniform)
        int64_t unit;      // < 0: none
        int64_t row;
        int tile, ntiles, n, hg, cs;
        int useq;          // how many units this workgroup started before this one
    };
    auto make_item = [&](int64_t u, int useq) -> Item {
        Item it{};
        it.unit = u;
        it.useq = useq;
        if (u < 0 || u >= units) { it.unit = -1; return it; }
        it.cs = (int)(u % N_CS);
        it.hg = (int)((u / N_CS) % n_hg);
        it.row = u / ((int64_t)N_CS * n_hg);
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
        return make_item(it.unit + G, it.useq + 1);
    };

    // Index list of an item's tile into this wave's slot buf (always issued: with no
    // item the fallback's list is re-read).
    auto dma_idx = [&](const Item &it, const Item &fallback, int buf) {
        const bool has = it.unit >= 0;
        const int64_t row = has ? it.row : fallback.row;  // values, not a reference: stays in SGPRs
        const int p = (has ? it.tile : 0) * kTile + lane;
        const int pc = p < a.kmax ? p : a.kmax - 1;
        dma4(a.idx + row * a.kmax, (uint32_t)pc * 4u, lds_addr(&idx_lds[w][buf][0]));
    };
    // bad[d]: the unit d units after the current one has an index out of range.
    bool bad0 = false, bad1 = false, bad2 = false;
    int cur_useq = 0;
    auto resolve = [&](const Item &it, int buf) -> int {
        if (it.unit < 0) return -1;
        const int iv = idx_lds[w][buf][lane];
        const int p = it.tile * kTile + lane;
        const bool live = p < it.n;
        const bool inr = iv >= 0 && (int64_t)iv < a.n_ctx;
        if (__builtin_amdgcn_ballot_w64(live && !inr)) {
            const int d = it.useq - cur_useq;  // flags set by value (no pointer select)
            bad0 = bad0 || d == 0;
            bad1 = bad1 || d == 1;
            bad2 = bad2 || d >= 2;
        }
        return (live && inr) ? iv : -1;
    };
    // One DMA instruction per cache row (1 KiB): wave w gathers keys NR*w + i into slots
    // NR*w + swap23(i) of buffer buf. The buffer resource spans the row's cache; a masked
    // key (-1) has a wrapped-around offset past its end and arrives as zeros, and so does
    // every row when there is no item (the resource is then empty). The rows of one tile
    // are issued one or two at a time through the next tile's scores, so the CU's address
    // unit (16 cycles per 1 KiB row) never queues a burst of them.
    auto rsrc_tile = [&](const Item &it) {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const char *)a.k + (it.unit >= 0 ? it.row * a.cache_stride * 2 : 0)), 0,
            it.unit >= 0 ? (int)(uint32_t)(a.n_ctx * kRowBytes) : 0, kBufferFlags);
    };
    auto dma_tile_row = [&](__amdgpu_buffer_rsrc_t rsrc, int iv, int buf, int i) {
        const int ij = __builtin_amdgcn_readlane(iv, NR * w + i);
        dma16_buf(rsrc, ((uint32_t)ij << 10) + ((uint32_t)lane << 4),
                  lds_addr((SA_LDS char *)&t_lds[buf][0] + (NR * w + swap23(i)) * kTStride));
    };

    const float scale2 = a.scale * kLog2e;
    bf16x8 qreg[16];
    f32x16 acc[NT];
    float m_run, ref, l_run;
    float sink_n;
    auto load_q_async = [&](const Item &it) {
        const int head = (it.hg * HB + hb) * 32 + ln;
        const bool ok = head < a.H;
        const uint16_t *qrow = ok ? (const uint16_t *)a.q + (it.row * a.H + head) * kHeadDim
                                  : (const uint16_t *)g_zero_row;
        qrow += 256 * kb + 128 * g;
#pragma unroll
        for (int kk = 0; kk < 16; kk++) load16_async(qreg[kk], qrow + 8 * kk);
        load4_async(sink_n, ok ? a.sinks + head : (const float *)g_zero_row);
    };
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
    // Normalise, transpose through the wave's exchange slot into whole 128-byte lines,
    // store non-temporally through a buffer resource (lanes past H are dropped by the
    // range check): exactly kStores stores per wave, as in sa_attn.hip.
    auto leave_unit = [&](const Item &it, bool bad) {
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            a.out + it.row * a.H * kHeadDim, 0, a.H * kHeadDim * 4, kBufferFlags);
        SA_LDS char *slot = (SA_LDS char *)&xch_lds[w][0][0];
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

    // Issue order per wave (S(j) = tile j's scores; mid(j) = after them; end(j) = after its
    // values):
    //   prologue: Q(0), I(0), I(1) | drain | T(0), I(2)
    //   S(j):     T(j+1), spread through the score steps
    //   mid(j):   Q(next unit) when j is a unit's last tile
    //   end(j):   wait I(j+2); I(j+3), then the unit's stores when j is its last
    // The top of tile j waits for T(j) (and for Q when j starts a unit).
    Item cur = make_item(base, 0);
    Item nx = next_item(cur);
    Item nx2 = next_item(nx);
    Item nx3 = next_item(nx2);
    load_q_async(cur);
    dma_idx(cur, cur, 0);
    dma_idx(nx, cur, 1);
    wait_vmcnt<0>();
    start_unit();
    __builtin_amdgcn_s_waitcnt(0);  // nothing the compiler tracks is pending in the loop
    int iv_next;                    // rows of tile j+1, gathered during tile j's scores
    {
        const int iv0 = resolve(cur, 0);
        iv_next = resolve(nx, 1);
        const __amdgpu_buffer_rsrc_t r0 = rsrc_tile(cur);
#pragma unroll
        for (int i = 0; i < NR; i++) dma_tile_row(r0, iv0, 0, i);
        dma_idx(nx2, cur, 0);
    }
    bool last1 = false;  // tile j-1 ended a unit (its stores follow I(j+2); Q(j-1) precedes I(j+2))

    for (int j = 0; cur.unit >= 0; j++) {
        const bool more = nx.unit >= 0;
        const bool last_of_unit = !more || nx.unit != cur.unit;
        const int buf = j & 1;
        // T(j) has landed, and the query of a unit that starts here. Issued after T(j):
        // [Q(j-1)] I(j+2) [stores(j-1)]; when tile j starts a unit, the wait is for Q(j-1),
        // after which come I(j+2) and the stores.
        if (last1) wait_vmcnt<vm_clamp(1 + kStores)>(); else wait_vmcnt<1>();
        if (last1) start_unit();
        lds_barrier();

        const __amdgpu_buffer_rsrc_t rt = rsrc_tile(nx);  // T(j+1)
        // ---- partial scores over this wave's half of the head width (tile as K).
        f32x16 sacc0 = (f32x16){}, sacc1 = (f32x16){};
        {
            // The first half of T(j+1) goes out here into the other buffer (every wave
            // finished tile j-1's values, which used it, before the barrier above); the
            // second half goes out during this tile's values.
            const SA_LDS char *krow = (const SA_LDS char *)&t_lds[buf][0] + ln * kTStride + 512 * kb + 256 * g;
            bf16x8 k0 = *(const SA_LDS bf16x8 *)(krow);
            bf16x8 k1 = *(const SA_LDS bf16x8 *)(krow + 32 * kTStride);
#pragma unroll
            for (int kk = 0; kk < 16; kk++) {
                bf16x8 n0 = k0, n1 = k1;
                if (kk + 1 < 16) {
                    n0 = *(const SA_LDS bf16x8 *)(krow + 16 * (kk + 1));
                    n1 = *(const SA_LDS bf16x8 *)(krow + 32 * kTStride + 16 * (kk + 1));
                }
                sacc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qreg[kk], sacc0, 0, 0, 0);
                sacc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qreg[kk], sacc1, 0, 0, 0);
#pragma unroll
                for (int r = kk * (NR / 2) / 16; r < (kk + 1) * (NR / 2) / 16; r++)
                    dma_tile_row(rt, iv_next, buf ^ 1, r);
                __builtin_amdgcn_sched_barrier(0);
                k0 = n0;
                k1 = n1;
            }
        }
        {
            const f32x16 give = kb ? sacc0 : sacc1;
#pragma unroll
            for (int c = 0; c < 4; c++)  // chunk c of every lane is contiguous: 16-byte writes
                ((f32x4 *)&xch_lds[w][0][0])[64 * c + lane] =
                    (f32x4){give[4 * c], give[4 * c + 1], give[4 * c + 2], give[4 * c + 3]};
        }
        lds_barrier();

        // The scores were the last use of qreg in this unit.
        const bool q_now = last_of_unit && more;
        if (q_now) load_q_async(nx);

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
        lds_barrier();

        // ---- online softmax with the sink (the same code and order as sa_attn.hip).
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
            const uint32_t trunc = pbits >> 16;
            const bool exact = (pbits & 0xffffu) == 0u && pf > 0.0f;
            const uint32_t hb = pf != pf ? 0x7fc0u : (exact ? trunc - 1u : trunc);
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
        lds_barrier();

        l_run = alpha * l_run + (sum_lds[2 * hb][ln] + sum_lds[2 * hb + 1][ln]);
        m_run = m_new;

        if (rescale) [[unlikely]] {
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                acc[nt] *= alpha;
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- values O^T += V^T P^T with the same tile read as V. Step ks covers keys
        // 16ks..16ks+15; lane (g, ch, l16) addresses slot 16ks + 8t2 + 4g + l16/4 (key
        // 16ks + 8g + 4t2 + l16/4) at column 32nt + 16ch + 4(l16%4) of the wave's columns.
        // Key steps outside, column groups inside: only one step's P parts and two V
        // operands are live. Each accumulator still takes its eight MFMAs in the same
        // order (step 0 hi, lo, step 1 hi, lo, ...), so the bits are those of sa_attn.hip.
        const int l16 = lane & 15;
        const int ch = (lane >> 4) & 1;
        const SA_LDS char *vrow = (const SA_LDS char *)&t_lds[buf][0] + (4 * g + (l16 >> 2)) * kTStride +
                                  2 * (cur.cs * COLS + kb * NT * 32 + 16 * ch + 4 * (l16 & 3));
        auto read_v = [&](int ks, int nt) -> bf16x8 {
            bf16x8 v;
#pragma unroll
            for (int t2 = 0; t2 < 2; t2++) {
                const bf16x4 part = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (SA_LDS bf16x4 *)(vrow + (16 * ks + 8 * t2) * kTStride + 64 * nt));
                v[4 * t2 + 0] = part[0];
                v[4 * t2 + 1] = part[1];
                v[4 * t2 + 2] = part[2];
                v[4 * t2 + 3] = part[3];
            }
            return v;
        };
        bf16x8 vc = read_v(0, 0);
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const bf16x8 *src = (const bf16x8 *)&xch_lds[2 * hb + (ks >> 1)][0][0];
            const bf16x8 ph = src[64 * (ks & 1) + lane];
            const bf16x8 pl = src[128 + 64 * (ks & 1) + lane];
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                bf16x8 vn = vc;
                if (nt + 1 < NT) vn = read_v(ks, nt + 1);
                else if (ks + 1 < 4) vn = read_v(ks + 1, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc, ph, acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc, pl, acc[nt], 0, 0, 0);
                // Second half of T(j+1), spread over the 4 NT key-step x column-group pairs.
                {
                    constexpr int kSteps = 4 * NT;
                    const int st = ks * NT + nt;
#pragma unroll
                    for (int r = st * (NR / 2) / kSteps; r < (st + 1) * (NR / 2) / kSteps; r++)
                        dma_tile_row(rt, iv_next, buf ^ 1, NR / 2 + r);
                }
                __builtin_amdgcn_sched_barrier(0);
                vc = vn;
            }
        }
        lds_barrier();  // every wave is done with this tile buffer and the P operands

        // I(j+2) has landed: after it come [stores(j-1)], T(j+1), [Q(j)].
        wait_vmcnt_dyn((last1 ? kStores : 0) + NR + (q_now ? kQLoads : 0));
        iv_next = resolve(nx2, buf);
        dma_idx(nx3, cur, buf ^ 1);  // slot buf^1 held I(j+1), resolved at end(j-1)
        if (last_of_unit) {
            leave_unit(cur, bad0);
            bad0 = bad1;
            bad1 = bad2;
            bad2 = false;
            cur_useq++;
        }
        last1 = last_of_unit;
        cur = nx;
        nx = nx2;
        nx2 = nx3;
        nx3 = next_item(nx3);
    }
    wait_vmcnt<0>();
}

template <int HB, int NT>
hipError_t launch_variant(const AttnArgs &a, int64_t units, int64_t grid, hipStream_t s) {
    const int n_hg = (a.H + 32 * HB - 1) / (32 * HB);
    hipLaunchKernelGGL((attn_bf16_alias_kernel<HB, NT>), dim3((unsigned)grid), dim3(128 * HB), 0, s, a, n_hg, units);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16_alias(const AttnArgs &a, hipStream_t s) {
    // Same work split as the separate-cache kernel (plan_attn_bf16).
    const AttnPlan p = plan_attn_bf16(a.rows, a.H);
    if (p.units == 0) return hipSuccess;
    const int64_t cus = device_cu_count();
    const int64_t grid = p.units < cus ? p.units : cus;
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
