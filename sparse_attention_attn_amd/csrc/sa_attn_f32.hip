// sa_attn_f32.hip -- gathered sparse attention with per-head sinks for float32 inputs.
//
// Same definition and the same 64-key online-softmax order as the bf16 kernel
// (akol1/TensorFold pull request 4, first commit message: 64-key tiles, running
// maximum, tile sum, value sum; TensorFold pull request 1206, "What changes": a
// sink per head), computed entirely in float32 with no rounding of the
// probabilities. This is the precision path for float32 caches; the dense
// bf16 contractions of the throughput path are in sa_attn.hip.
//
// One workgroup (four waves) serves one (row, head). Per tile: the 64 scores are
// split four ways over the head width (fixed pairwise combine), the tile maximum
// and tile sum are taken over the 64 scores in key order, and each thread
// accumulates two output columns over the tile's keys in key order.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kHeadDim = 512;
constexpr int kTile = 64;

__global__ void __launch_bounds__(256) attn_f32_kernel(AttnArgs a) {
    __shared__ float q_lds[kHeadDim];
    __shared__ float s_lds[kTile];
    __shared__ int i_lds[kTile];

    const int t = threadIdx.x;
    const int64_t row = blockIdx.x / a.H;
    const int head = (int)(blockIdx.x % a.H);
    const float *qrow = (const float *)a.q + ((int64_t)row * a.H + head) * kHeadDim;
    const float *kc = (const float *)a.k + (int64_t)row * a.cache_stride;
    const float *vc = (const float *)a.v + (int64_t)row * a.cache_stride;
    const int32_t *irow = a.idx + (int64_t)row * a.kmax;
    int n = a.nsel ? a.nsel[row] : a.kmax;
    n = n < 0 ? 0 : (n > a.kmax ? a.kmax : n);

    q_lds[2 * t] = qrow[2 * t];
    q_lds[2 * t + 1] = qrow[2 * t + 1];

    const float sink = a.sinks[head];
    float m_run = sink;
    float l_run = expf(sink - ((sink == -INFINITY) ? 0.0f : sink));
    float acc0 = 0.0f, acc1 = 0.0f;
    int bad = 0;

    for (int t0 = 0; t0 < n; t0 += kTile) {
        int my_bad = 0;
        if (t < kTile) {
            const int p = t0 + t;
            int iv = -1;
            if (p < n) {
                iv = irow[p];
                if (iv < 0 || (int64_t)iv >= a.n_ctx) { my_bad = 1; iv = -1; }
            }
            i_lds[t] = iv;
        }
        bad |= __syncthreads_or(my_bad);

        // Score of key j = t/4 over the quarter c = t%4 of the head width.
        const int j = t >> 2, c = t & 3;
        const int iv = i_lds[j];
        float part = 0.0f;
        if (iv >= 0) {
            const float *krow = kc + (int64_t)iv * kHeadDim + 128 * c;
            for (int d = 0; d < 128; d++) part = fmaf(q_lds[128 * c + d], krow[d], part);
        }
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        if (c == 0) s_lds[j] = (t0 + j < n) ? part * a.scale : -INFINITY;
        __syncthreads();

        float mt = -INFINITY;
        for (int jj = 0; jj < kTile; jj++) mt = fmaxf(mt, s_lds[jj]);
        const float m_new = fmaxf(m_run, mt);
        const float ref = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = expf(m_run - ref);
        float ltile = 0.0f, v0 = 0.0f, v1 = 0.0f;
        for (int jj = 0; jj < kTile; jj++) {
            const int ij = i_lds[jj];
            if (ij < 0) continue;  // masked key: absent from the sum
            const float p = expf(s_lds[jj] - ref);
            ltile += p;
            const float *vrow = vc + (int64_t)ij * kHeadDim;
            v0 = fmaf(p, vrow[2 * t], v0);
            v1 = fmaf(p, vrow[2 * t + 1], v1);
        }
        l_run = alpha * l_run + ltile;
        acc0 = alpha * acc0 + v0;
        acc1 = alpha * acc1 + v1;
        m_run = m_new;
        __syncthreads();
    }

    float *orow = a.out + ((int64_t)row * a.H + head) * kHeadDim;
    orow[2 * t] = bad ? NAN : acc0 / l_run;
    orow[2 * t + 1] = bad ? NAN : acc1 / l_run;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t s) {
    const int64_t grid = (int64_t)a.rows * a.H;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
