// sa_attn_f32_common.h -- the float32 attention steps shared by the float32 kernels: the
// one-workgroup-per-row kernel (sa_attn_f32.hip) and the split path for small batches
// (sa_attn_f32_split.hip). Both evaluate these functions on the same operands in the same
// order, so a row's result has the same bits whichever runs it.
//
// What they compute: akol1/TensorFold pull request 4 ("DeepSeek V4.1: sparse attention on
// eight SIMD groups, the same bytes"), first commit message: keys scored in tiles, a running
// maximum, a tile sum and a value sum; TensorFold pull request 1206, "What changes": a sink
// logit per head. Float32 throughout (the weights are never rounded to a narrower type). Per
// 32-key tile: m' = max(m, tile maximum), reference r = m' (0 while m' = -inf), alpha =
// exp(m - r), p = exp(s - r) (0 for a masked key), l = alpha l + sum p, acc = alpha acc + P V
// (the tile's P V summed on its own first).
// Contraction is off here: a product followed by a sum is never fused, in any caller.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_device.h"

namespace sa {

constexpr int kT32 = 32;                   // keys per float32 tile
constexpr int kRowF = kHeadDim * 4;        // bytes of a float32 cache row
constexpr int kKStrF = kRowF + 16;         // K slot stride: 16 slots of one read on 16 bank groups

// K slot of tile key kap (0..31): key g + 16b + 4j sits in slot 16b + 4g + j, so that lane
// group g's four scores of 16-key block b are the keys g + 4e its value operand needs.
__device__ __forceinline__ int kslot32(int kap) {
    const int b = kap >> 4, r = kap & 15;
    return 16 * b + 4 * (r & 3) + (r >> 2);
}

// A score from the four dimension-quarter partial sums of its MFMA chains, in quarter order.
__device__ __forceinline__ float f32_score_sum(float p0, float p1, float p2, float p3) {
#pragma clang fp contract(off)
    return ((p0 + p1) + p2) + p3;
}

// Scaled scores of a lane's eight keys (tile keys g + 4e at positions p0 + 4e; -inf past the
// row's count n) and the tile maximum over the tile's 32 keys (the four lane groups).
__device__ __forceinline__ float f32_tile_scores(const float (&tot)[8], int p0, int n, float scale,
                                                 float (&s)[8]) {
#pragma clang fp contract(off)
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        s[e] = p0 + 4 * e < n ? tot[e] * scale : -INFINITY;
        mt = fmaxf(mt, s[e]);
    }
    return max_xor32(max_xor16(mt));
}

// Exponent reference of a running maximum.
__device__ __forceinline__ float f32_ref(float m) { return m == -INFINITY ? 0.0f : m; }

// Weights of a lane's eight keys against the reference, and the tile sum over 32 keys.
__device__ __forceinline__ float f32_tile_weights(const float (&s)[8], float ref, float (&pe)[8]) {
#pragma clang fp contract(off)
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        pe[e] = s[e] == -INFINITY ? 0.0f : expf(s[e] - ref);
        psum += pe[e];
    }
    return sum_xor32(sum_xor16(psum));
}

// Tile sum step: alpha l + psum, a product then a sum.
__device__ __forceinline__ float f32_l_step(float alpha, float l, float psum) {
#pragma clang fp contract(off)
    return alpha * l + psum;
}

// Value sum step: the tile's P V (its own MFMA chain, started from zero) added once to the
// rescaled running sum, a product then a sum. The running sum thus takes one rounding per
// tile, not one per MFMA step of four keys: with many equal weights (a short cache, duplicate
// indices), per-step roundings at the running sum's magnitude add up past 1e-5.
__device__ __forceinline__ f32x4 f32_acc_step(const f32x4 &acc, float alpha, const f32x4 &tile) {
#pragma clang fp contract(off)
    return acc * alpha + tile;
}

}  // namespace sa
