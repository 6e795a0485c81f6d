// sa_device.h -- device-side helpers of the bf16 attention kernels (sa_attn.hip: separate
// K and V caches, and one cache serving as both).
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define SA_LDS __attribute__((address_space(3)))

constexpr int kHeadDim = 512;   // sixteen 32-wide output column groups
constexpr int kTile = 64;       // keys per online-softmax tile
constexpr int kRowBytes = kHeadDim * 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;  // log2 units: p <= 256 between reference moves
constexpr int kQLoads = 17;      // per wave: sixteen 16-byte query pieces and one sink
// Word 3 of a raw buffer resource (32-bit data format, no swizzle) and an offset past any
// output row (stores there are dropped by the buffer range check).
constexpr int kBufferFlags = 0x00020000;
constexpr int kDropOffset = 0x7ffffff0;
// Cache policy of the output stores: non-temporal. The outputs are never read back by
// the kernel, and streaming them keeps them from contending with the gathers in the
// caches (a 12% shorter decode step at 1,024 rows, measured).
constexpr int kStoreNT = 2;
// s_waitcnt vmcnt holds at most 63: a larger count is clamped, which waits longer.
constexpr int vm_clamp(int n) { return n > 63 ? 63 : n; }

// 2^x on the hardware exponential (v_exp_f32); exp2(-inf) = 0, exp2(+inf) = inf, NaN stays NaN.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Source of the DMA for keys that are masked or invalid: 1 KiB of zeros.
__device__ __attribute__((aligned(16))) const uint32_t g_zero_row[kRowBytes / 4] = {0};

// All vector-memory traffic inside the tile loop is issued through the asm helpers
// below, so the compiler neither sees nor waits on it: the loop's only waits on the
// vector-memory counter are the explicit ones, each placed where one tile's
// gathers must have landed while the next tile's stay in flight.

// s_waitcnt vmcnt(N): this wave has at most N vector-memory operations outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n formed at run time (clamped to 0..63; a
// smaller count only waits longer).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    n = n < 0 ? 0 : (n > 63 ? 63 : n);
    switch (__builtin_amdgcn_readfirstlane(n)) {
#define SA_W(N) case N: wait_vmcnt<N>(); break;
        SA_W(0) SA_W(1) SA_W(2) SA_W(3) SA_W(4) SA_W(5) SA_W(6) SA_W(7) SA_W(8) SA_W(9)
        SA_W(10) SA_W(11) SA_W(12) SA_W(13) SA_W(14) SA_W(15) SA_W(16) SA_W(17) SA_W(18) SA_W(19)
        SA_W(20) SA_W(21) SA_W(22) SA_W(23) SA_W(24) SA_W(25) SA_W(26) SA_W(27) SA_W(28) SA_W(29)
        SA_W(30) SA_W(31) SA_W(32) SA_W(33) SA_W(34) SA_W(35) SA_W(36) SA_W(37) SA_W(38) SA_W(39)
        SA_W(40) SA_W(41) SA_W(42) SA_W(43) SA_W(44) SA_W(45) SA_W(46) SA_W(47) SA_W(48) SA_W(49)
        SA_W(50) SA_W(51) SA_W(52) SA_W(53) SA_W(54) SA_W(55) SA_W(56) SA_W(57) SA_W(58) SA_W(59)
        SA_W(60) SA_W(61) SA_W(62)
#undef SA_W
        default: wait_vmcnt<63>(); break;
    }
}

// Workgroup barrier for LDS traffic only: outstanding LDS operations complete,
// in-flight DMA gathers stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const SA_LDS void *)p;
}
__device__ __forceinline__ uint32_t lds_addr(const SA_LDS void *p) { return (uint32_t)(uintptr_t)p; }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The gathers below set M0 (the LDS base of a direct-to-LDS load) themselves and name it as
// clobbered. The compiler reserves M0 and may still warn about the clobber; it emits no M0
// use of its own in these kernels (every M0 write in the generated code is one of these).
//
// Direct-to-LDS gather through a buffer resource: lane i moves the 16 bytes at byte offset
// voff_i of the resource to LDS address lds + 16 i; lds is wave-uniform. An offset past the
// resource's range (a masked row's wrapped-around offset) reads as zeros, so masked rows need
// no separate source and every lane's access stays inside the resource. The load is
// non-temporal: a gathered cache row is used once per query row, and keeping the stream out
// of the caches' retained set measured 8% faster at 1,024 rows.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 ::"s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// L2 prefetch: lane i loads the 4 bytes at byte offset voff_i of the resource with the default
// cache policy (so the line stays in L2 for a later gather) into LDS address lds + 4 i, a
// per-wave slot that nothing reads. An offset past the resource's range fetches nothing.
__device__ __forceinline__ void prefetch4_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 ::"s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// Direct-to-LDS load of 4 bytes per lane, from sbase + voff_i to LDS address lds + 4 i (a
// tile's index list).
__device__ __forceinline__ void dma4(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
// Direct-to-LDS load of 16 bytes per lane, from sbase + voff_i to LDS address lds + 16 i.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
// Asynchronous loads into registers: the destination is written when the data
// returns, which the compiler does not model, so the value may be used only after an
// explicit vector-memory wait that covers the load, followed by register_ready on it.
// The compiler must also not copy or spill the destination before that wait (under
// register pressure it can); tests/test_isa_async_loads.py checks the built code for it.
__device__ __forceinline__ void load16_async(bf16x8 &dst, const void *p) {
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(dst) : "v"(p) : "memory");
}
__device__ __forceinline__ void load4_async(float &dst, const void *p) {
    asm volatile("global_load_dword %0, %1, off" : "=v"(dst) : "v"(p) : "memory");
}
#pragma clang diagnostic pop
// Orders every later use of v after the preceding (volatile) wait.
template <typename T>
__device__ __forceinline__ void register_ready(T &v) {
    asm volatile("" : "+v"(v));
}

// max(x[l], x[l ^ 32]) and x[l & 31] + x[l | 32] in every lane l: one v_permlane32_swap
// hands each half of the wave the other half's values (no LDS round trip), and both
// halves add in the same order, so the pair of lanes holds identical results.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same over lanes l and l ^ 16 with v_permlane16_swap: it hands rows 1 and 3 of the
// wave (16 lanes each) their even neighbour's values and the reverse, so the two results
// are the pair's values in some order, and a sum of the two is the same in both lanes.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Bits 2 and 3 of m exchanged (its own inverse). Key kap = 8g + 4t + q of a 32-key half
// sits in V slot swap23(kap) = 16(g >> 1) + 8t + 4(g & 1) + q, so the eight keys that one
// transposing read of the value operand takes (g in {0, 1} or {2, 3}, q < 4, fixed t) are
// eight consecutive slots.
__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// LDS row stride of the K buffer: padded by 16 bytes, so the 16 lanes of one ds_read_b128,
// which read 16 consecutive slots at the same column, land on 16 different 16-byte bank
// groups; each read is one base register plus an immediate offset.
constexpr int kKStride = kRowBytes + 16;

// Map the linear workgroup id so that the workgroups of one query row (its head
// groups and column slices, which gather the same cache rows) run on one XCD and
// share its L2. Dispatch places workgroup i on XCD i % 8.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t G) {
    const int64_t xcd = i & 7, slot = i >> 3;
    const int64_t per = G >> 3, rem = G & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace
}  // namespace sa
