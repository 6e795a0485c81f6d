// sa_pad.hip -- head padding copies (TensorFold pull request 1206, "What changes":
// the real queries go into a zero-padded 32-head buffer, the extra sinks are zero,
// and the real output groups are copied out before the output projections).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kHeadDim = 512;

// q [rows, h_real, 512] -> q_pad [rows, h_pad, 512]; 16-byte units, zero for padded heads.
__global__ void __launch_bounds__(256)
pad_q_kernel(const uint4 *q, uint4 *q_pad, int64_t rows, int h_real, int h_pad, int units_per_head) {
    const int64_t total = rows * h_pad * units_per_head;
    for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total;
         u += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = u / ((int64_t)h_pad * units_per_head);
        const int rem = (int)(u % ((int64_t)h_pad * units_per_head));
        const int h = rem / units_per_head, c = rem % units_per_head;
        q_pad[u] = h < h_real ? q[(r * h_real + h) * units_per_head + c] : make_uint4(0, 0, 0, 0);
    }
}

__global__ void __launch_bounds__(128) pad_sinks_kernel(const float *sinks, float *sinks_pad, int h_real, int h_pad) {
    const int h = threadIdx.x;
    if (h < h_pad) sinks_pad[h] = h < h_real ? sinks[h] : 0.0f;
}

// out_pad [rows, h_pad, 512] -> out [rows, h_real, 512], float32 in 16-byte units.
__global__ void __launch_bounds__(256)
unpad_kernel(const float4 *out_pad, float4 *out, int64_t rows, int h_pad, int h_real) {
    constexpr int upr = kHeadDim / 4;
    const int64_t total = rows * h_real * upr;
    for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total;
         u += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = u / ((int64_t)h_real * upr);
        const int rem = (int)(u % ((int64_t)h_real * upr));
        out[u] = out_pad[(r * h_pad) * upr + rem];
    }
}

int64_t grid_for(int64_t units) {
    int64_t g = (units + 255) / 256;
    return g < 1 ? 1 : (g > 65536 ? 65536 : g);
}

}  // namespace

hipError_t launch_pad_heads(int dtype, const void *q, int64_t rows, int h_real, int h_pad,
                            const float *sinks, void *q_pad, float *sinks_pad, hipStream_t s) {
    const int elt = dtype == 1 ? 2 : 4;
    const int units_per_head = kHeadDim * elt / 16;
    const int64_t units = rows * h_pad * units_per_head;
    if (units > 0) {
        hipLaunchKernelGGL(pad_q_kernel, dim3((unsigned)grid_for(units)), dim3(256), 0, s,
                           (const uint4 *)q, (uint4 *)q_pad, rows, h_real, h_pad, units_per_head);
    }
    hipLaunchKernelGGL(pad_sinks_kernel, dim3(1), dim3(128), 0, s, sinks, sinks_pad, h_real, h_pad);
    return hipGetLastError();
}

hipError_t launch_unpad_heads(const float *out_pad, int64_t rows, int h_pad, int h_real, float *out,
                              hipStream_t s) {
    const int64_t units = rows * h_real * (kHeadDim / 4);
    if (units > 0) {
        hipLaunchKernelGGL(unpad_kernel, dim3((unsigned)grid_for(units)), dim3(256), 0, s,
                           (const float4 *)out_pad, (float4 *)out, rows, h_pad, h_real);
    }
    return hipGetLastError();
}

}  // namespace sa
