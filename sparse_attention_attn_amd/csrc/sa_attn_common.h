// sa_attn_common.h -- the per-element arithmetic of the bf16 attention kernels, shared by the
// persistent kernels (sa_attn.hip) and the split path for small batches (sa_attn_split.hip).
// Not part of the public ABI.
//
// What it computes: akol1/TensorFold pull request 4 ("DeepSeek V4.1: sparse attention on eight
// SIMD groups, the same bytes"), first commit message: the selected keys are scored in 64-key
// tiles against a 512-wide head, with a running maximum, a tile sum and a value sum; TensorFold
// pull request 1206, "What changes": a sink logit per head.
//
// Every kernel that includes this header runs, for each (row, head, column), the same sequence
// of operations: the score MFMA chain, half_tile on each 32-key half tile, the value MFMAs
// and the fixed-order combine of the two key halves. Floating-point contraction is switched
// off inside these helpers, so that the compiler cannot fuse a multiply into a later add in
// one kernel and not in another: the bits of a result never depend on which kernel (or which
// template instance) produced it.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kWaves = 8;
constexpr int kRows = kTile / kWaves;   // rows each wave gathers per tile (per buffer)

// K slot, within a 32-key half, of key kap = 8g + 4b + r: slot 16b + 4g + r. Row 4g + r of
// the score MFMA over slots 16b .. 16b+15 lands in lane group g, element r, which is the
// P^T operand's element 4b + r (key 8g + 4b + r).
__device__ __forceinline__ int kslot_of_key(int kap) { return ((kap & 4) << 2) | ((kap >> 3) << 2) | (kap & 3); }

// LDS row stride of the separate kernel's V buffer: the row bytes plus 32, an odd multiple
// of 32 for every slice width. A transposing read of the value MFMA's operand touches
// eight consecutive V slots (V slot of key kap: swap23(kap)) at one 32-byte column
// window; with an odd multiple of 32 as stride they land on eight different bank windows.
constexpr int vstride_of(int vrow) { return vrow + 32; }

// Chunk swizzle of the aliased kernel's tile rows (stride 1024): the 16-byte chunk c of
// the row in slot s is stored at chunk c ^ tswz(s). The score reads (sixteen slots
// 16b .. 16b+15, one chunk) see sixteen different values of tswz and so sixteen bank
// groups; the value reads (slots 16t2 + 0..7, or + 8..15, one aligned 32-byte window) see
// eight different even (or odd) values, which keep each window whole and move the eight
// windows to eight different places.
__device__ __forceinline__ int tswz(int s) { return ((s & 7) << 1) | ((s >> 3) & 1); }

template <typename T>
__device__ __forceinline__ const SA_LDS T *lds_at(uint32_t addr) {
    return (const SA_LDS T *)(uintptr_t)addr;
}

// Online-softmax state of one wave over its key half, relative to the reference ref.
struct HalfState {
    float m, ref, l;
};

template <int CB>
__device__ __forceinline__ void half_start(HalfState &st, f32x4 (&acc)[CB], bool with_sink, float sink) {
#pragma clang fp contract(off)
    if (with_sink) {
        const float sink2 = sink * kLog2e;
        st.m = sink2;
        st.ref = (sink2 == -INFINITY) ? 0.0f : sink2;
        st.l = exp2_hw(sink2 - st.ref);
    } else {
        st.m = -INFINITY;
        st.ref = 0.0f;
        st.l = 0.0f;
    }
#pragma unroll
    for (int cb = 0; cb < CB; cb++) acc[cb] = (f32x4){};
}

// The pieces of one half tile's online-softmax step, in the order half_tile runs them. The
// split paths run the same pieces for a tile spread over workgroups, waves and phases; every piece
// computes the same values from the same inputs, so the results are the same bits.
//
// Scaled scores (log2 units) of one half tile and their maximum over the wave's 32 keys. s0,
// s1: the score MFMA blocks; element 4b + r of this lane is key p0 + 4b + r of the row's list
// (p0 = 64 tile + 32 kh + 8 g); keys at or past n are masked (whole: the tile lies inside the
// row's count, so nothing is).
__device__ __forceinline__ float tile_scores(const f32x4 &s0, const f32x4 &s1, int p0, int n, bool whole,
                                             float scale2, float (&s)[8]) {
#pragma clang fp contract(off)
    float mloc = -INFINITY;
    if (whole) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            s[e] = (e < 4 ? s0[e] : s1[e - 4]) * scale2;
            mloc = fmaxf(mloc, s[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float full = e < 4 ? s0[e] : s1[e - 4];
            s[e] = p0 + e < n ? full * scale2 : -INFINITY;
            mloc = fmaxf(mloc, s[e]);
        }
    }
    return max_xor32(max_xor16(mloc));
}

// Reference step: the running maximum takes the tile's maximum, and the exponent reference
// follows it lazily: it moves only when the maximum has risen more than kLazy above it, or
// when it sits above a finite maximum (from the start value 0); the decision is taken for the
// wave's 16 heads together (wave-uniform result). Otherwise every p stays <= 2^kLazy. On a
// move, ref_prev keeps the old reference for the rescale factor.
__device__ __forceinline__ bool tile_reference(HalfState &st, float mloc, float &ref_prev) {
#pragma clang fp contract(off)
    const float m_new = fmaxf(st.m, mloc);
    // Bitwise forms and a select: no exec-mask branches in a chain that a wave may walk tile
    // after tile (the same values as the short-circuit form).
    const bool move = (m_new > st.ref + kLazy) | ((m_new < st.ref) & (m_new != -INFINITY));
    const bool rescale = __builtin_amdgcn_ballot_w64(move) != 0;
    ref_prev = st.ref;
    const float ref_new = (m_new == -INFINITY) ? 0.0f : m_new;
    st.ref = rescale ? ref_new : st.ref;
    st.m = m_new;
    return rescale;
}

// Weights of one half tile against the reference ref: p = hi + lo with both parts bf16, so the
// value product (one MFMA per part) sees p to about 16 significant bits, and psum (the tile
// sum, reduced over the wave's four lane groups) sums the same hi + lo. hi is p truncated
// toward zero and lo = bf16(p - hi); when p is itself a positive bf16 value, hi is the next
// bf16 below it and lo its last unit, so hi + lo = p exactly, and an infinite value times a
// positive weight stays infinite. For p >= 0 both cases are the top half of bits(p) - 1,
// saturated at 0 (p = 0 gives hi = lo = 0; a NaN stays a NaN).
__device__ __forceinline__ float tile_weights(const float (&s)[8], float ref, bf16x8 &ph, bf16x8 &pl) {
#pragma clang fp contract(off)
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const float pf = exp2_hw(s[e] - ref);
        const uint32_t pbits = __float_as_uint(pf);
        const uint32_t hb = __builtin_elementwise_sub_sat(pbits, 1u);
        const float hif = __uint_as_float(hb & 0xffff0000u);
        const __bf16 hi = __builtin_bit_cast(__bf16, (uint16_t)(hb >> 16));
        const __bf16 lo = (__bf16)(pf - hif);
        psum += hif + (float)lo;
        ph[e] = hi;
        pl[e] = lo;
    }
    return sum_xor32(sum_xor16(psum));
}

// Rescale factor of a tile: 1 without a reference move, else 2^(ref_prev - ref); 0 while
// nothing has been accumulated (l = 0): the old reference may then be arbitrarily far from
// the new one, and 0 (not 2^(r - r'), which can overflow) keeps acc at 0.
__device__ __forceinline__ float tile_alpha(bool rescale, float l, float ref_prev, float ref) {
#pragma clang fp contract(off)
    return rescale ? (l == 0.0f ? 0.0f : exp2_hw(ref_prev - ref)) : 1.0f;
}

// Tile sum step and accumulator rescale (before the tile's value MFMAs).
template <int CB>
__device__ __forceinline__ void tile_accumulate(HalfState &st, bool rescale, float alpha, float psum,
                                                f32x4 (&acc)[CB]) {
#pragma clang fp contract(off)
    st.l = __builtin_fmaf(alpha, st.l, psum);
    if (rescale) [[unlikely]] {
#pragma unroll
        for (int cb = 0; cb < CB; cb++) acc[cb] *= alpha;
    }
}

// One half tile: scores, reference, weights, tile sum and rescale. Returns the two bf16 parts
// of the weights as the P^T operand of the value MFMAs that follow.
template <int CB>
__device__ __forceinline__ void half_tile(const f32x4 &s0, const f32x4 &s1, int p0, int n, bool whole, float scale2,
                                          HalfState &st, f32x4 (&acc)[CB], bf16x8 &ph, bf16x8 &pl) {
    float s[8];
    const float mloc = tile_scores(s0, s1, p0, n, whole, scale2, s);
    float ref_prev;
    const float l_prev = st.l;
    const bool rescale = tile_reference(st, mloc, ref_prev);
    const float alpha = tile_alpha(rescale, l_prev, ref_prev, st.ref);
    const float psum = tile_weights(s, st.ref, ph, pl);
    tile_accumulate(st, rescale, alpha, psum, acc);
}

// The fold of the two key halves' states (half 0, half 1 in that order): R is the reference
// of the half with the larger maximum (half 0 on ties), a_h = 2^(r_h - R), 0 for a half that
// has accumulated nothing (l_h = 0), and the denominator a_0 l_0 + a_1 l_1 in an explicit
// fused form, so that the order of the two products is fixed.
struct HalfFold {
    float a0, a1, lsum;
};
__device__ __forceinline__ HalfFold fold_scales(float m0, float r0, float l0, float m1, float r1, float l1) {
#pragma clang fp contract(off)
    const float R = m0 >= m1 ? r0 : r1;
    HalfFold f;
    f.a0 = l0 == 0.0f ? 0.0f : exp2_hw(r0 - R);
    f.a1 = l1 == 0.0f ? 0.0f : exp2_hw(r1 - R);
    f.lsum = __builtin_fmaf(f.a0, l0, f.a1 * l1);
    return f;
}
// One output element: (a_0 x_0 + a_1 x_1) / (a_0 l_0 + a_1 l_1), or the quiet NaN 0x7fc00000
// where bad_mask (all ones or all zeros, in scalar registers) marks a row with an out-of-range index.
// The select is one v_cndmask_b32 written out, so that the compiler neither branches around
// the divides (it turns a select of a divide into a branch) nor lets a NaN payload depend on
// how it lowered the select: every kernel stores the same bits.
__device__ __forceinline__ float fold_elem(const HalfFold &f, float x0, float x1, uint64_t bad_mask) {
#pragma clang fp contract(off)
    const float v = __builtin_fmaf(f.a0, x0, f.a1 * x1) / f.lsum;
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(0x7fc00000u), "s"(bad_mask));
    return r;
}

// A row's query for one 16-head group and its sink, loaded asynchronously into qreg;
// usable after a wait that covers them and register_ready. Lane (g, l16) holds head
// head0 + l16, dims 32kk + 8g + 0..7 for kk < 16. Heads past H read zeros (query and sink)
// from the static zero row.
__device__ __forceinline__ void load_q_async(const AttnArgs &a, int64_t row, int head0, int g, int l16,
                                             bf16x8 (&qreg)[16], float &sink) {
    const int head = head0 + l16;
    const bool ok = head < a.H;
    const uint16_t *qrow =
        ok ? (const uint16_t *)a.q + (row * a.H + head) * kHeadDim : (const uint16_t *)g_zero_row;
    qrow += 8 * g;
#pragma unroll
    for (int kk = 0; kk < 16; kk++) load16_async(qreg[kk], qrow + 32 * kk);
    load4_async(sink, ok ? a.sinks + head : (const float *)g_zero_row);
}
__device__ __forceinline__ void q_ready(bf16x8 (&qreg)[16], float &sink) {
#pragma unroll
    for (int kk = 0; kk < 16; kk++) register_ready(qreg[kk]);
    register_ready(sink);
}

// Score MFMA chain of one wave: S^T = K Q^T for the 32 keys of its half (two 16-slot blocks)
// and its 16 heads, over the full head width (16 steps of 32 dimensions). krow: the lane's
// LDS base in the K buffer (slot 32kh + l16, dims 8g + 0..7; stride kKStride). Block 0's chain
// of 16 MFMAs runs first, then block 1's (the same MFMAs on the same operands, in the same order
// per block, as any interleaving of the two), each K operand read two reads ahead of its MFMA.
// After each of the 32 steps the caller's hook (step index 0..31) issues gathers in the matrix
// pipe's shadow.
template <typename Hook>
__device__ __forceinline__ void score_chain(const SA_LDS char *krow, const bf16x8 (&qreg)[16], f32x4 &sacc0,
                                            f32x4 &sacc1, Hook &&hook) {
    constexpr int kAhead = 2;
    sacc0 = (f32x4){};
    sacc1 = (f32x4){};
    auto kread = [&](int i) { return *(const SA_LDS bf16x8 *)(krow + (i >> 4) * 16 * kKStride + 64 * (i & 15)); };
    bf16x8 ring[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; i++) ring[i] = kread(i);
#pragma unroll
    for (int i = 0; i < 32; i++) {
        if (i + kAhead < 32) ring[(i + kAhead) % (kAhead + 1)] = kread(i + kAhead);
        if (i < 16) sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[i % (kAhead + 1)], qreg[i], sacc0, 0, 0, 0);
        else sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[i % (kAhead + 1)], qreg[i - 16], sacc1, 0, 0, 0);
        hook(i);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One 16-slot block of score_chain on its own: block b's MFMA chain, the same operands in the
// same order (kblk = krow + 16 b kKStride), for kernels that give the two blocks of a score tile
// to two waves.
template <typename Hook>
__device__ __forceinline__ void score_block_chain(const SA_LDS char *kblk, const bf16x8 (&qreg)[16], f32x4 &sacc,
                                                  Hook &&hook) {
    sacc = (f32x4){};
    bf16x8 k0 = *(const SA_LDS bf16x8 *)(kblk);
#pragma unroll
    for (int kk = 0; kk < 16; kk++) {
        bf16x8 n0 = k0;
        if (kk + 1 < 16) n0 = *(const SA_LDS bf16x8 *)(kblk + 64 * (kk + 1));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qreg[kk], sacc, 0, 0, 0);
        hook(kk);
        __builtin_amdgcn_sched_barrier(0);
        k0 = n0;
    }
}

}  // namespace
}  // namespace sa
