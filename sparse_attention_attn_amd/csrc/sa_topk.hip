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
//   * topk_regs_kernel (rows of up to 32,768 scores): each lane keeps 8 to 64 keys
//     in registers; T is found by three radix passes from the top (11, 11 and 10
//     bits), each an LDS histogram of the keys that share the digits found so far
//     and one scan that locates the digit where the count from the top reaches k.
//     A row takes 4, 8 or 16 waves (topk_rows8_kernel: 8 waves and 8 keys per lane, held to
//     eight waves per SIMD so that four rows share a CU; 16 waves for rows of more than 4,096
//     scores when there is at most one row per CU).
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
        for (int64_t i = t; i < k; i += kThreads) orow[i] = i < vl ? (int32_t)i : -1;
        if (t == 0 && a.count_out) a.count_out[row] = vl;
        return;
    }

    const bool in_lds = vl <= kLdsKeys;
    if (in_lds) {
        for (int i = t; i < vl; i += kThreads) keys[i] = order_key(srow[i]);  // vl <= kLdsKeys here
    }
    // Loop counters over a row are 64-bit: a row may hold up to 2^31 - 1 scores, and a 32-bit
    // counter stepping past its end would overflow.
    auto key_at = [&](int64_t i) -> uint32_t { return in_lds ? keys[i] : order_key(srow[i]); };

    // ---- radix select of the k-th largest key.
    uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (t < 256) hist[t] = 0u;
        __syncthreads();
        for (int64_t i = t; i < vl; i += kThreads) {
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
    for (int64_t b0 = 0; b0 < vl; b0 += kThreads) {
        const int64_t i = b0 + t;
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
        if (sel && pos < (uint32_t)k) orow[pos] = (int32_t)i;  // exactly k are selected; the bound is a guard
        base_eq += eq_total;
        base_sel += sel_total;
        __syncthreads();
    }
    if (t == 0 && a.count_out) a.count_out[row] = k;
}


// Inclusive prefix sum over the wave's lanes: DPP row shifts build each 16-lane row's
// inclusive sum, the two row broadcasts carry rows 0 and 0..1 upward, and lane 63
// ends with the total.
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// WAVES waves per row, KPL keys per lane: a wave covers 64 * KPL positions.
//
// The threshold T (the k-th largest key) is fixed 11, 11 and 10 bits at a time from the
// top. Pass p counts, in an LDS histogram over its digit, the row's keys whose higher
// digits equal those already fixed; every thread then owns 2048 / (64 WAVES) consecutive
// bins, a prefix sum over the threads gives each thread the count of keys in the bins
// above its own, and the one thread whose bins hold the crossing (fewer than krem keys
// above a bin, at least krem with it) publishes the digit and the count above it.
// krem, the number of keys still to take, starts at k and loses that count every pass;
// at the end krem keys equal to T are taken (the lowest positions first) and k - krem
// keys are greater than T.
template <int WAVES, int KPL>
__device__ __forceinline__ void topk_regs_row(TopkArgs a) {
    constexpr int kWaveSpan = 64 * KPL;
    constexpr int kBins = 2048;
    constexpr int kBinsPerThread = kBins / (64 * WAVES);
    constexpr int kVW = kBinsPerThread >= 4 ? 4 : kBinsPerThread;  // bins per LDS access
    static_assert(kVW >= 2 && kBinsPerThread % kVW == 0, "bins are read and cleared 8 or 16 bytes at a time");
    __shared__ uint32_t cnt_lds[2][WAVES];
    __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
    __shared__ uint32_t pick_lds[4];  // digit, count above it, count in it; T (early exit)
    constexpr int kStage = 4096;
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
        for (int64_t i = threadIdx.x; i < a.k; i += 64 * WAVES) orow[i] = i < vl ? (int32_t)i : -1;
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

    // ---- radix passes. hist starts at zero and every thread clears the bins it read.
    typedef uint32_t binv __attribute__((ext_vector_type(kVW)));
    binv *hv = (binv *)&hist[threadIdx.x * kBinsPerThread];
#pragma unroll
    for (int i = 0; i < kBinsPerThread / kVW; i++) hv[i] = (binv){};
    uint32_t prefix = 0u, krem = k, t_count = 0u;
#pragma unroll
    for (int pass = 0; pass < 3; pass++) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
        const int hi_shift = pass == 0 ? 32 : (pass == 1 ? 21 : 10);
        __syncthreads();  // the bins are clear; pick_lds of the last pass has been read
#pragma unroll
        for (int r = 0; r < KPL; r++) {
            const bool in = (base + 64 * r < vl) & (pass == 0 || (key[r] >> hi_shift) == prefix);
            if (in) atomicAdd(&hist[(key[r] >> shift) & dmask], 1u);
        }
        __syncthreads();
        uint32_t h[kBinsPerThread];
        uint32_t mine = 0u;
#pragma unroll
        for (int i = 0; i < kBinsPerThread / kVW; i++) {
            const binv v = hv[i];
            hv[i] = (binv){};
#pragma unroll
            for (int e = 0; e < kVW; e++) {
                h[kVW * i + e] = v[e];
                mine += v[e];
            }
        }
        const uint32_t incl = wave_scan(mine);
        if constexpr (WAVES > 1) {
            if (lane == 63) cnt_lds[pass & 1][w] = incl;
        }
        __syncthreads();
        uint32_t before = 0u, total = incl;
        if constexpr (WAVES > 1) {
            total = 0u;
#pragma unroll
            for (int ww = 0; ww < WAVES; ww++) {
                const uint32_t c = cnt_lds[pass & 1][ww];
                before += ww < w ? c : 0u;
                total += c;
            }
        } else {
            total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        }
        uint32_t run = total - (before + incl);  // keys in the bins above this thread's
#pragma unroll
        for (int i = kBinsPerThread - 1; i >= 0; i--) {
            if (run < krem && run + h[i] >= krem) {
                pick_lds[0] = (uint32_t)(threadIdx.x * kBinsPerThread + i);
                pick_lds[1] = run;
                pick_lds[2] = h[i];
            }
            run += h[i];
        }
        __syncthreads();
        prefix = (prefix << (pass == 2 ? 10 : 11)) | pick_lds[0];
        krem -= pick_lds[1];
        t_count = pick_lds[2];
        // One key has the digits found so far: it is T (and krem = 1). Its owner publishes
        // it, which replaces the remaining passes. (Not with 64 keys per lane, where the
        // extra loop costs more registers than the pass it saves.) It goes to its own slot:
        // other waves may still be reading slot 0 of this pass.
        if (KPL <= 16 && pass < 2 && t_count == 1u) {
#pragma unroll
            for (int r = 0; r < KPL; r++)
                if ((base + 64 * r < vl) & ((key[r] >> shift) == prefix)) pick_lds[3] = key[r];
            __syncthreads();
            prefix = pick_lds[3];
            break;
        }
    }
    const uint32_t T = prefix;
    const uint32_t need = krem;               // keys equal to T to take, lowest positions first
    const bool all_ties = need == t_count;

    // ---- ordered selection. Every wave has read the last pass's totals from cnt_lds
    // before the barrier that ended that pass, so cnt_lds is free again.
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
        // The usual case: every key >= T is taken; selected before this wave = the
        // selected keys of the waves before it. With up to 16 keys per lane the ballots are
        // kept (in scalar registers) for the emit loop, else formed again there.
        constexpr bool kKeep = KPL <= 16;
        auto ballot_sel = [&](int r) { return __builtin_amdgcn_ballot_w64((key[r] >= T) & (base + 64 * r < vl)); };
        uint64_t msel[kKeep ? KPL : 1];
        uint32_t cnt = 0u;
#pragma unroll
        for (int r = 0; r < KPL; r++) {
            const uint64_t m = ballot_sel(r);
            if constexpr (kKeep) msel[r] = m;
            cnt += (uint32_t)__builtin_popcountll(m);
        }
        uint32_t sel_base = 0u;
        if constexpr (WAVES > 1) {
            if (lane == 0) cnt_lds[0][w] = cnt;
            __syncthreads();
#pragma unroll
            for (int ww = 0; ww < WAVES; ww++) sel_base += ww < w ? cnt_lds[0][ww] : 0u;
        }
#pragma unroll
        for (int r = 0; r < KPL; r++) {
            uint64_t m;
            if constexpr (kKeep) m = msel[r]; else m = ballot_sel(r);
            emit(((m >> lane) & 1u) != 0u, sel_base + lanes_below(m), base + 64 * r);
            sel_base += (uint32_t)__builtin_popcountll(m);
        }
    } else {
        // Selected before this wave: every key > T there, and its share of the first
        // `need` ties.
        uint32_t sel_base = 0u, eq_base = 0u;
        if constexpr (WAVES > 1) {
            uint32_t gt_w = 0u, eq_w = 0u;
#pragma unroll
            for (int r = 0; r < KPL; r++) {
                gt_w += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key[r] > T));
                eq_w += (uint32_t)__builtin_popcountll(
                    __builtin_amdgcn_ballot_w64((key[r] == T) & (base + 64 * r < vl)));
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

template <int WAVES, int KPL>
__global__ void __launch_bounds__(64 * WAVES) topk_regs_kernel(TopkArgs a) {
    topk_regs_row<WAVES, KPL>(a);
}
// Eight waves per row, eight keys per lane, held to eight waves per SIMD (the compiler
// otherwise takes 105 scalar registers, which allows seven): four rows then share a CU, so
// up to four rows per CU run in one round (1,024 rows of 4,096: 11.4 -> 10.7 us, measured).
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(8, 8))) topk_rows8_kernel(TopkArgs a) {
    topk_regs_row<8, 8>(a);
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    const dim3 grid((unsigned)a.rows);
    const int64_t cus = device_cu_count();
    if (a.n <= 64 * 64) {
        // With at most four rows per CU, eight waves per row shorten each row's chain;
        // beyond that, four waves per row keep more rows in flight.
        if (a.rows <= 4 * cus)
            hipLaunchKernelGGL(topk_rows8_kernel, grid, dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((topk_regs_kernel<4, 16>), grid, dim3(256), 0, s, a);
    } else if (a.n <= 16 * 64 * 16 && a.rows <= cus) {
        // At most one row per CU: sixteen waves per row, 16 or 32 keys per lane, shorten each
        // row's chain (8 x 16,384: 18.4 -> 9.9 us; 8 x 32,768: 20.3 -> 17.5 us, measured).
        hipLaunchKernelGGL((topk_regs_kernel<16, 16>), grid, dim3(1024), 0, s, a);
    } else if (a.n <= 4 * 64 * 64) {
        hipLaunchKernelGGL((topk_regs_kernel<4, 64>), grid, dim3(256), 0, s, a);
    } else if (a.n <= 16 * 64 * 32 && a.rows <= cus) {
        hipLaunchKernelGGL((topk_regs_kernel<16, 32>), grid, dim3(1024), 0, s, a);
    } else if (a.n <= 8 * 64 * 64) {
        hipLaunchKernelGGL((topk_regs_kernel<8, 64>), grid, dim3(512), 0, s, a);
    } else {
        hipLaunchKernelGGL(topk_radix_kernel, grid, dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace sa
