// sa_topk.hip -- exact per-row top-k selection of indexer scores for gfx950.
//
// akol1/TensorFold pull request 4 (PR body) names the indexer's merge and finish
// done by one threadgroup per row with "the same picks". Here one workgroup of
// 1024 threads selects the k largest of a row exactly:
//   1. map every score to an order-preserving 32-bit key (NaN lowest, -0 == +0)
//      and keep the row's keys in LDS (rows of up to 32,768 scores, 128 KiB);
//   2. four 8-bit radix passes, most significant first, find the k-th largest key
//      T and how many keys equal to T must be taken (need);
//   3. one pass in position order selects keys > T and the first `need` keys == T,
//      and compacts their positions with ballot/popcount prefix sums, so the output
//      is ascending by construction and ties go to the lower position.
// Every count is an integer, so the result is the unique exact answer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 32768;

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (x != x) return 0u;               // NaN ranks below -inf
    if (u == 0x80000000u) u = 0u;        // -0 ties +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a) {
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

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.rows), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
