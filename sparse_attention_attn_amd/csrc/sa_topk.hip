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
//   * topk_regs_kernel (rows of up to 32,768 scores): each lane keeps 32 or 64 keys
//     in registers; T is built bit by bit, from the top, as the largest value with
//     at least k keys >= it (32 counting steps of v_cmp + ballot + popcount). Rows
//     of up to 4,096 scores take one wave and no barrier at all; longer rows take 4
//     or 16 waves that add their counts through LDS at each step.
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


// WAVES waves per row, KPL keys per lane: a wave covers 64 * KPL positions.
template <int WAVES, int KPL>
__global__ void __launch_bounds__(64 * WAVES) topk_regs_kernel(TopkArgs a) {
    constexpr int kKeysPerLane = KPL;
    constexpr int kWaveSpan = 64 * KPL;
    __shared__ uint32_t cnt_lds[2][WAVES];
    __shared__ uint32_t tot_lds[2][WAVES];

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
    float x[kKeysPerLane];
#pragma unroll
    for (int r = 0; r < kKeysPerLane; r++) {
        const int p = base + 64 * r;
        x[r] = srow[p & (int)live(p)];
    }
    uint32_t key[kKeysPerLane];
#pragma unroll
    for (int r = 0; r < kKeysPerLane; r++) key[r] = order_key(x[r]) & live(base + 64 * r);

    auto wave_count = [&](auto pred) -> uint32_t {
        uint32_t c = 0u;
#pragma unroll
        for (int r = 0; r < kKeysPerLane; r++) c += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(pred(r)));
        return c;
    };
    // Sum of one count per wave, in wave order; slot alternates so one barrier suffices.
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

    // T = the k-th largest key: the largest value with at least k keys >= it.
    uint32_t T = 0u;
    for (int bit = 31; bit >= 0; bit--) {
        const uint32_t cand = T | (1u << bit);
        const uint32_t c = row_total(wave_count([&](int r) { return key[r] >= cand; }), bit & 1);
        if (c >= k) T = cand;
    }

    // Counts above T and equal to T (within the row) per wave, then each wave's offsets.
    const uint32_t gt_w = wave_count([&](int r) { return key[r] > T; });
    const uint32_t eq_w = wave_count([&](int r) { return key[r] == T && base + 64 * r < vl; });
    uint32_t gt_before = 0u, gt_all = gt_w, eq_before = 0u;
    if constexpr (WAVES > 1) {
        if (lane == 0) { cnt_lds[0][w] = gt_w; tot_lds[0][w] = eq_w; }
        __syncthreads();
        gt_all = 0u;
#pragma unroll
        for (int ww = 0; ww < WAVES; ww++) {
            const uint32_t g = cnt_lds[0][ww], e = tot_lds[0][ww];
            gt_all += g;
            gt_before += ww < w ? g : 0u;
            eq_before += ww < w ? e : 0u;
        }
    }
    const uint32_t need = k - gt_all;  // keys equal to T to take, lowest positions first
    // Selected before this wave: every key > T there, and its share of the first `need` ties.
    uint32_t sel_base = gt_before + (eq_before < need ? eq_before : need);
    uint32_t eq_base = eq_before;
#pragma unroll
    for (int r = 0; r < kKeysPerLane; r++) {
        const int p = base + 64 * r;
        const bool eq = key[r] == T && p < vl;
        const uint64_t meq = __builtin_amdgcn_ballot_w64(eq);
        const bool sel = key[r] > T || (eq && eq_base + lanes_below(meq) < need);
        const uint64_t msel = __builtin_amdgcn_ballot_w64(sel);
        const uint32_t pos = sel_base + lanes_below(msel);
        if (sel && pos < k) orow[pos] = p;  // exactly k are selected; the bound is a guard
        eq_base += (uint32_t)__builtin_popcountll(meq);
        sel_base += (uint32_t)__builtin_popcountll(msel);
    }
    if (threadIdx.x == 0 && a.count_out) a.count_out[row] = (int32_t)k;
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    const dim3 grid((unsigned)a.rows);
    if (a.n <= 64 * 64) {
        hipLaunchKernelGGL((topk_regs_kernel<1, 64>), grid, dim3(64), 0, s, a);
    } else if (a.n <= 4 * 64 * 64) {
        hipLaunchKernelGGL((topk_regs_kernel<4, 64>), grid, dim3(256), 0, s, a);
    } else if (a.n <= 16 * 64 * 32) {
        hipLaunchKernelGGL((topk_regs_kernel<16, 32>), grid, dim3(1024), 0, s, a);
    } else {
        hipLaunchKernelGGL(topk_radix_kernel, grid, dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace sa
