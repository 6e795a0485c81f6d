// sa_topk.hip -- exact per-row top-k selection of indexer scores for gfx950.
//
// akol1/TensorFold pull request 4 (PR body) names the indexer's merge and finish
// done by one threadgroup per row with "the same picks". Selection here is exact:
// every score maps to an order-preserving 32-bit key (NaN lowest, -0 == +0); the
// k-th largest key T and the number `need` of keys equal to T to take are found
// exactly; then one pass in position order selects keys > T and the first `need`
// keys == T and compacts their positions with ballot/popcount prefix sums, so the
// output is ascending by construction and ties go to the lower position. Every
// count is an integer, so the result is the unique exact answer.
//
// Two kernels find T:
//   * topk_regs_kernel (rows of up to 32,768 scores): each lane keeps 16 to 64 keys
//     in registers; T is built bit by bit, from the top, as the largest value with
//     at least k keys >= it: a bisection over all keys until few enough share T's
//     leading bits, then over those few alone. A row takes 1 to 8 waves; several
//     waves add their counts through LDS.
//   * topk_radix_kernel (longer rows): four 8-bit radix passes with LDS
//     histograms, the keys cached in LDS when the row fits (32,768 scores) and
//     re-read from memory otherwise.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 32768;

// Order-preserving key: NaN -> 0 (below -inf), -0 -> the key of +0, negative values
// bit-inverted, non-negative values with the sign bit set. Straight-line selects.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    u = u == 0x80000000u ? 0u : u;
    const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return x != x ? 0u : key;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Per 16-bit half h of h2: 1 if h > c, else 0, for both halves of cx2 equal to c:
// min(sat(h - c), 1) on packed unsigned 16-bit lanes (v_pk_sub_u16 with clamp, then
// v_pk_min_u16). Written out because the compiler otherwise turns it into a compare and
// select per half.
__device__ __forceinline__ u16x2 ge_pair(uint32_t h2, uint32_t cx2, uint32_t one2) {
    uint32_t t;
    asm("v_pk_sub_u16 %0, %1, %2 clamp\n\tv_pk_min_u16 %0, %0, %3" : "=&v"(t) : "v"(h2), "s"(cx2), "s"(one2));
    return __builtin_bit_cast(u16x2, t);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ void __launch_bounds__(kThreads) topk_radix_kernel(TopkArgs a) {
    __shared__ uint32_t keys[kLdsKeys];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wtot[2][kWaves];
    __shared__ uint32_t pick[2];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int64_t row = blockIdx.x;
    const float *srow = a.scores + row * a.ld;
    int32_t *orow = a.idx_out + row * a.k;

    int64_t vl64 = a.valid_len ? (int64_t)a.valid_len[row] : a.n;
    vl64 = vl64 < 0 ? 0 : (vl64 > a.n ? a.n : vl64);
    const int vl = (int)vl64;
    const int k = a.k;

    if (vl <= k) {  // every candidate is selected
        for (int i = t; i < k; i += kThreads) orow[i] = i < vl ? i : -1;
        if (t == 0 && a.count_out) a.count_out[row] = vl;
        return;
    }

    const bool in_lds = vl <= kLdsKeys;
    if (in_lds) {
        for (int i = t; i < vl; i += kThreads) keys[i] = order_key(srow[i]);
    }
    auto key_at = [&](int i) -> uint32_t { return in_lds ? keys[i] : order_key(srow[i]); };

    // ---- radix select of the k-th largest key.
    uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (t < 256) hist[t] = 0u;
        __syncthreads();
        for (int i = t; i < vl; i += kThreads) {
            const uint32_t u = key_at(i);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        // Inclusive scan of the bins from the top (x_t = hist[255 - t]) by threads 0..255:
        // a shuffle scan inside each wave, then the four wave totals through LDS.
        uint32_t x = 0u;
        if (t < 256) {
            x = hist[255 - t];
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(x, off);
                if (lane >= off) x += y;
            }
            if (lane == 63) wtot[0][w] = x;
        }
        __syncthreads();
        if (t < 256) {
            uint32_t before = 0u;
            for (int ww = 0; ww < w; ww++) before += wtot[0][ww];
            const uint32_t incl = before + x;
            const uint32_t excl = incl - hist[255 - t];
            if (incl >= krem && excl < krem) {
                pick[0] = 255u - (uint32_t)t;
                pick[1] = excl;
            }
        }
        __syncthreads();
        prefix |= pick[0] << shift;
        mask |= 255u << shift;
        krem -= pick[1];
        __syncthreads();
    }
    const uint32_t T = prefix;
    const uint32_t need = krem;  // keys equal to T to take, lowest positions first

    // ---- ordered compaction.
    uint32_t base_eq = 0u, base_sel = 0u;
    for (int b0 = 0; b0 < vl; b0 += kThreads) {
        const int i = b0 + t;
        const uint32_t u = i < vl ? key_at(i) : 0u;
        const bool gt = i < vl && u > T;
        const bool eq = i < vl && u == T;

        const uint64_t meq = __builtin_amdgcn_ballot_w64(eq);
        if (lane == 0) wtot[0][w] = (uint32_t)__builtin_popcountll(meq);
        __syncthreads();
        uint32_t eq_before = 0u, eq_total = 0u;
        for (int ww = 0; ww < kWaves; ww++) {
            const uint32_t c = wtot[0][ww];
            eq_before += ww < w ? c : 0u;
            eq_total += c;
        }
        const uint32_t eq_rank = base_eq + eq_before + lanes_below(meq);
        const bool sel = gt || (eq && eq_rank < need);

        const uint64_t msel = __builtin_amdgcn_ballot_w64(sel);
        if (lane == 0) wtot[1][w] = (uint32_t)__builtin_popcountll(msel);
        __syncthreads();
        uint32_t sel_before = 0u, sel_total = 0u;
        for (int ww = 0; ww < kWaves; ww++) {
            const uint32_t c = wtot[1][ww];
            sel_before += ww < w ? c : 0u;
            sel_total += c;
        }
        const uint32_t pos = base_sel + sel_before + lanes_below(msel);
        if (sel && pos < (uint32_t)k) orow[pos] = i;  // exactly k are selected; the bound is a guard
        base_eq += eq_total;
        base_sel += sel_total;
        __syncthreads();
    }
    if (t == 0 && a.count_out) a.count_out[row] = k;
}


// Sum over the wave of a per-lane count: DPP row shifts build each 16-lane row's
// inclusive sum, the two row broadcasts carry rows 0 and 0..1 upward, and lane 63
// ends with the total.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// WAVES waves per row, KPL keys per lane: a wave covers 64 * KPL positions.
//
// The threshold T (the k-th largest key) is the largest value with at least k keys
// at or above it. It is found in two phases that keep the bracket lo <= T < hi,
// hi = lo + 2^b, with c_lo / c_hi the numbers of keys at or above lo / hi:
//   coarse: bisection over every key, one bit per step from the top, each step a
//     per-lane count (compare + add) summed over the row; it stops as soon as at
//     most kCand keys fall inside the bracket;
//   fine: those keys (sharing T's upper bits) are compacted through LDS, every wave
//     loads all of them (at most four per lane), and the remaining bits are decided
//     over them alone, plus the fixed count of keys above the bracket it started from.
// At the end hi = T + 1, so c_hi keys are > T and c_lo - c_hi equal T; when all ties
// are taken (the usual case), the selection is simply key >= T.
template <int WAVES, int KPL>
__global__ void __launch_bounds__(64 * WAVES) topk_regs_kernel(TopkArgs a) {
    static_assert(KPL % 4 == 0, "keys per lane pair up twice in the packed count");
    constexpr int kWaveSpan = 64 * KPL;
    constexpr int kCandPerLane = 4;
    constexpr uint32_t kCand = 64 * kCandPerLane;
    __shared__ uint32_t cnt_lds[2][WAVES];
    __shared__ uint32_t tot_lds[WAVES];
    constexpr int kStage = 4096;
    __shared__ uint32_t cand_lds[kCand + 64];
    __shared__ int32_t out_lds[kStage + 64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;
    const float *srow = a.scores + row * a.ld;
    int32_t *orow = a.idx_out + row * a.k;

    int64_t vl64 = a.valid_len ? (int64_t)a.valid_len[row] : a.n;
    vl64 = vl64 < 0 ? 0 : (vl64 > a.n ? a.n : vl64);
    const int vl = (int)vl64;
    const uint32_t k = (uint32_t)a.k;

    if ((uint32_t)vl <= k) {  // every candidate is selected
        for (int i = threadIdx.x; i < a.k; i += 64 * WAVES) orow[i] = i < vl ? i : -1;
        if (threadIdx.x == 0 && a.count_out) a.count_out[row] = vl;
        return;
    }

    // Register r of lane l holds position w * 64 * KPL + 64 r + l (key 0 past the row).
    const int base = w * kWaveSpan + lane;
    // Every load is issued (positions past the row read position 0, which exists since
    // vl > k >= 1) so that all of them are in flight together; the key is masked after.
    // live(p) = all ones when p < vl, else 0 (arithmetic, so no per-key branch).
    auto live = [&](int p) -> uint32_t { return (uint32_t)((p - vl) >> 31); };
    float x[KPL];
#pragma unroll
    for (int r = 0; r < KPL; r++) {
        const int p = base + 64 * r;
        x[r] = srow[p & (int)live(p)];
    }
    uint32_t key[KPL];
#pragma unroll
    for (int r = 0; r < KPL; r++) key[r] = order_key(x[r]) & live(base + 64 * r);

    // Row-wide sum of one per-wave value, in wave order; the slot alternates so that one
    // barrier per call suffices.
    auto row_total = [&](uint32_t c, int slot) -> uint32_t {
        if constexpr (WAVES == 1) {
            return c;
        } else {
            if (lane == 0) cnt_lds[slot][w] = c;
            __syncthreads();
            uint32_t t = 0u;
#pragma unroll
            for (int ww = 0; ww < WAVES; ww++) t += cnt_lds[slot][ww];
            return t;
        }
    };

    // ---- coarse phase. Every tested value is >= 1, so the zero keys past the row never
    // count; NaN keys (also 0) count only towards c_lo = vl at the start.
    uint32_t lo = 0u, c_lo = (uint32_t)vl, c_hi = 0u;
    int bit = 32;  // the bracket is [lo, lo + 2^bit)
    {
        // While the tested bit is 16 or higher, the candidate's low half is zero, so
        // key >= cand compares the upper halves only: two keys per register, counted by
        // min(sat(h - (c - 1)), 1) on packed 16-bit lanes (1 iff h >= c), no lane masks.
        uint32_t hk[KPL / 2];
#pragma unroll
        for (int i = 0; i < KPL / 2; i++) hk[i] = (key[2 * i] >> 16) | (key[2 * i + 1] & 0xffff0000u);
        const uint32_t one2 = 0x00010001u;
        while (bit > 16 && c_lo - c_hi > kCand) {
            bit--;
            const uint32_t cand = lo | (1u << bit);
            const uint32_t cm1 = (cand >> 16) - 1u;
            const uint32_t cm1x2 = cm1 | (cm1 << 16);
            u16x2 acc0 = (u16x2){0, 0}, acc1 = (u16x2){0, 0};  // two chains in flight
#pragma unroll
            for (int i = 0; i < KPL / 2; i += 2) {
                acc0 += ge_pair(hk[i], cm1x2, one2);
                acc1 += ge_pair(hk[i + 1], cm1x2, one2);
            }
            const u16x2 acc = acc0 + acc1;
            uint32_t c = (uint32_t)acc[0] + (uint32_t)acc[1];
            c = row_total(wave_sum(c), bit & 1);
            if (c >= k) { lo = cand; c_lo = c; } else { c_hi = c; }
        }
    }
    while (bit > 0 && c_lo - c_hi > kCand) {
        bit--;
        const uint32_t cand = lo | (1u << bit);
        uint32_t c = 0u;
#pragma unroll
        for (int r = 0; r < KPL; r++) c += key[r] >= cand ? 1u : 0u;
        c = row_total(wave_sum(c), bit & 1);
        if (c >= k) { lo = cand; c_lo = c; } else { c_hi = c; }
    }

    // ---- fine phase over the keys inside the bracket (at most kCand of them).
    // Per-key predicates are combined with & (not &&) and every LDS write is issued, to a
    // spare slot per lane when the key is not taken, so these loops have no branches.
    if (bit > 0) {
        const uint32_t span_m1 = bit >= 32 ? 0xffffffffu : (1u << bit) - 1u;
        auto inside = [&](int r) { return (key[r] - lo <= span_m1) & (base + 64 * r < vl); };
        uint32_t before = 0u;
        if constexpr (WAVES > 1) {
            uint32_t mine = 0u;
#pragma unroll
            for (int r = 0; r < KPL; r++) mine += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(inside(r)));
            if (lane == 0) tot_lds[w] = mine;
            __syncthreads();
#pragma unroll
            for (int ww = 0; ww < WAVES; ww++) before += ww < w ? tot_lds[ww] : 0u;
        }
#pragma unroll
        for (int r = 0; r < KPL; r++) {
            const bool in = inside(r);
            const uint64_t m = __builtin_amdgcn_ballot_w64(in);
            const uint32_t j = before + lanes_below(m);
            // exactly c_lo - c_hi keys are inside; the bound is a guard
            cand_lds[(in & (j < kCand)) ? j : kCand + lane] = key[r];
            before += (uint32_t)__builtin_popcountll(m);
        }
        __syncthreads();
        const uint32_t ncand = c_lo - c_hi;
        uint32_t ck[kCandPerLane];
#pragma unroll
        for (int i = 0; i < kCandPerLane; i++) {
            const uint32_t j = 64u * i + lane;
            ck[i] = j < ncand ? cand_lds[j] : 0u;
        }
        const uint32_t c_above = c_hi;  // keys >= the bracket's upper end at entry
        while (bit > 0) {
            bit--;
            const uint32_t cand = lo | (1u << bit);
            uint32_t c = c_above;
#pragma unroll
            for (int i = 0; i < kCandPerLane; i++)
                c += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(ck[i] >= cand));
            if (c >= k) { lo = cand; c_lo = c; } else { c_hi = c; }
        }
    }
    const uint32_t T = lo;
    const uint32_t need = k - c_hi;           // keys equal to T to take, lowest positions first
    const bool all_ties = need == c_lo - c_hi;

    // ---- ordered selection. Selected before this wave: every key > T there, and its
    // share of the first `need` ties.
    uint32_t sel_base = 0u, eq_base = 0u;
    if constexpr (WAVES > 1) {
        __syncthreads();  // every wave has read the last coarse totals from cnt_lds
        uint32_t gt_w = 0u, eq_w = 0u;
#pragma unroll
        for (int r = 0; r < KPL; r++) {
            gt_w += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key[r] > T));
            eq_w += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64((key[r] == T) & (base + 64 * r < vl)));
        }
        if (lane == 0) { cnt_lds[0][w] = gt_w; cnt_lds[1][w] = eq_w; }
        __syncthreads();
        uint32_t gt_before = 0u;
#pragma unroll
        for (int ww = 0; ww < WAVES; ww++) {
            gt_before += ww < w ? cnt_lds[0][ww] : 0u;
            eq_base += ww < w ? cnt_lds[1][ww] : 0u;
        }
        sel_base = gt_before + (eq_base < need ? eq_base : need);
    }
    // Selected positions go to out_lds[pos] (a spare slot per lane otherwise) when the
    // output row fits there, and leave in coalesced stores; else straight to memory.
    const bool staged = k <= (uint32_t)kStage;
    auto emit = [&](bool sel, uint32_t pos, int p) {
        if (staged) {
            out_lds[(sel & (pos < k)) ? pos : kStage + lane] = p;
        } else if (sel && pos < k) {  // exactly k are selected; the bound is a guard
            orow[pos] = p;
        }
    };
    if (all_ties) {
#pragma unroll
        for (int r = 0; r < KPL; r++) {
            const int p = base + 64 * r;
            const bool sel = (key[r] >= T) & (p < vl);
            const uint64_t msel = __builtin_amdgcn_ballot_w64(sel);
            emit(sel, sel_base + lanes_below(msel), p);
            sel_base += (uint32_t)__builtin_popcountll(msel);
        }
    } else {
#pragma unroll
        for (int r = 0; r < KPL; r++) {
            const int p = base + 64 * r;
            const bool eq = (key[r] == T) & (p < vl);
            const uint64_t meq = __builtin_amdgcn_ballot_w64(eq);
            const bool sel = (key[r] > T) | (eq & (eq_base + lanes_below(meq) < need));
            const uint64_t msel = __builtin_amdgcn_ballot_w64(sel);
            emit(sel, sel_base + lanes_below(msel), p);
            eq_base += (uint32_t)__builtin_popcountll(meq);
            sel_base += (uint32_t)__builtin_popcountll(msel);
        }
    }
    if (staged) {
        __syncthreads();
        for (int i = threadIdx.x; i < (int)k; i += 64 * WAVES) orow[i] = out_lds[i];
    }
    if (threadIdx.x == 0 && a.count_out) a.count_out[row] = (int32_t)k;
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    const dim3 grid((unsigned)a.rows);
    if (a.n <= 64 * 64) {
        // One wave per row has the most rows in flight; with at most four rows per CU,
        // four waves per row shorten each row's chain of dependent steps instead.
        if (a.rows <= 4 * (int64_t)device_cu_count())
            hipLaunchKernelGGL((topk_regs_kernel<4, 16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((topk_regs_kernel<1, 64>), grid, dim3(64), 0, s, a);
    } else if (a.n <= 4 * 64 * 64) {
        hipLaunchKernelGGL((topk_regs_kernel<4, 64>), grid, dim3(256), 0, s, a);
    } else if (a.n <= 8 * 64 * 64) {
        hipLaunchKernelGGL((topk_regs_kernel<8, 64>), grid, dim3(512), 0, s, a);
    } else {
        hipLaunchKernelGGL(topk_radix_kernel, grid, dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace sa
