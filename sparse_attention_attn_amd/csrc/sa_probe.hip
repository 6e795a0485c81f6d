// sa_probe.hip -- sparse_attn_gather_probe: the attention kernels' gathers alone, as a measured
// bandwidth reference for benchmarks. For each row it reads the selected K and V cache rows (1 KiB
// each in bf16) with the same direct-to-LDS, non-temporal buffer-resource DMAs, and discards them:
// no score, softmax or value product, and no output. Its rate is the most the attention kernels
// could reach for the same index-driven access pattern on this part.
//
// Four waves per workgroup; wave w of workgroup (row, piece) gathers entries piece*4*RIF + w*RIF
// .. + RIF - 1 of the row's list: RIF K rows and RIF V rows in flight per wave, into its own LDS
// slots, then waits for them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_internal.h"
#include "sparse_attn.h"

namespace sa {
namespace {

template <int RIF>
__global__ void __launch_bounds__(256) gather_probe_kernel(const void *k, const void *v, int64_t cache_stride,
                                                           int64_t n_ctx, const int32_t *idx, int32_t kmax,
                                                           int pieces) {
    __shared__ __attribute__((aligned(16))) char slots[4][2 * RIF][kRowBytes];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x / pieces;
    const int first = (int)(blockIdx.x % pieces) * 4 * RIF + w * RIF;
    const int p = first + (lane % RIF);
    int iv = p < kmax ? idx[row * kmax + p] : -1;
    iv = (iv >= 0 && (int64_t)iv < n_ctx) ? iv : -1;  // -1: an offset past the range, zeros
    const int64_t base = row * cache_stride * 2;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)k + base), 0, (int)(uint32_t)(n_ctx * kRowBytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)v + base), 0, (int)(uint32_t)(n_ctx * kRowBytes), kBufferFlags);
#pragma unroll
    for (int i = 0; i < RIF; i++) {
        const int ij = __builtin_amdgcn_readlane(iv, i);
        const uint32_t off = ((uint32_t)ij << 10) + ((uint32_t)lane << 4);
        dma16_buf(rk, off, lds_addr(&slots[w][2 * i][0]));
        dma16_buf(rv, off, lds_addr(&slots[w][2 * i + 1][0]));
    }
    wait_vmcnt<0>();
}

}  // namespace
}  // namespace sa

extern "C" int sparse_attn_gather_probe(const void *k_cache, const void *v_cache, int64_t n_ctx, const int32_t *idx,
                                        int32_t rows, int32_t kmax, int32_t rows_in_flight, void *stream) {
    if (rows < 0 || kmax < 1 || kmax > SA_MAX_KMAX || n_ctx < 1 || n_ctx > SA_BF16_MAX_CTX)
        return sa::fail_with(SA_ERR_SHAPE, "gather probe: rows >= 0, 1 <= kmax <= SA_MAX_KMAX, 1 <= n_ctx <= "
                                           "SA_BF16_MAX_CTX");
    if (rows > 0 && (!k_cache || !v_cache || !idx)) return sa::fail_with(SA_ERR_NULL, "gather probe: NULL array");
    if (rows_in_flight != 8 && rows_in_flight != 16)
        return sa::fail_with(SA_ERR_UNSUPPORTED, "gather probe: rows_in_flight is 8 or 16");
    if (rows == 0) return SA_OK;
    const int per = 4 * rows_in_flight;
    const int pieces = (kmax + per - 1) / per;
    if ((int64_t)rows * pieces > 0x7fffffff) return sa::fail_with(SA_ERR_SHAPE, "gather probe: too many rows");
    const dim3 grid((unsigned)((int64_t)rows * pieces));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t stride = n_ctx * SA_HEAD_DIM;
    if (rows_in_flight == 8)
        hipLaunchKernelGGL((sa::gather_probe_kernel<8>), grid, dim3(256), 0, s, k_cache, v_cache, stride, n_ctx, idx,
                           kmax, pieces);
    else
        hipLaunchKernelGGL((sa::gather_probe_kernel<16>), grid, dim3(256), 0, s, k_cache, v_cache, stride, n_ctx,
                           idx, kmax, pieces);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return sa::fail_with(SA_ERR_HIP, hipGetErrorString(e));
    return SA_OK;
}
