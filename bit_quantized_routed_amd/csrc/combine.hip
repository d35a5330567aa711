// Weighted combine of the expert outputs (fixed order, deterministic):
//   y[slot] = sum_{s=0}^{nsplit-1} yp[s][slot]      (split partial sums, in order)
//   v[t] = sum_s shared[s][t] + sum_{k=0}^{K-1} g[t,k] * y[inv[t*K+k]]   (shared in partials)
//   out[t] = v[t]            (or out[t] + v[t] under residual accumulation)
#include "common.h"
#include "kernels.h"

// The K slot indices and gates are loaded first, then the K rows (independent
// loads in flight together), then the sums in fixed order.
#define CB_KMAX 16
__global__ void __launch_bounds__(256) k_combine(const float *__restrict__ y, int nsplit,
                                                 int64_t split_stride, const int32_t *__restrict__ inv,
                                                 const float *__restrict__ gate,
                                                 const float *__restrict__ shared, int sh_nsplit,
                                                 int64_t sh_stride, int H, int K, int accumulate,
                                                 float *out) {
    const int t = blockIdx.y;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= H / 4) return;
    int sl[CB_KMAX];
    float gk[CB_KMAX];
#pragma unroll
    for (int k = 0; k < CB_KMAX; ++k) {
        const int kk = min(k, K - 1);
        sl[k] = inv[t * K + kk];
        gk[k] = gate[t * K + kk];
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (shared) {
        v = ((const float4 *)(shared + (int64_t)t * H))[c];
        for (int sp = 1; sp < sh_nsplit; ++sp) {
            const float4 q = ((const float4 *)(shared + sp * sh_stride + (int64_t)t * H))[c];
            v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
        }
    }
    float4 yy[CB_KMAX];
#pragma unroll
    for (int k = 0; k < CB_KMAX; ++k) yy[k] = ((const float4 *)(y + (int64_t)sl[k] * H))[c];
    for (int sp = 1; sp < nsplit; ++sp) {
#pragma unroll
        for (int k = 0; k < CB_KMAX; ++k) {
            const float4 q = ((const float4 *)(y + sp * split_stride + (int64_t)sl[k] * H))[c];
            yy[k].x += q.x; yy[k].y += q.y; yy[k].z += q.z; yy[k].w += q.w;
        }
    }
#pragma unroll
    for (int k = 0; k < CB_KMAX; ++k) {
        if (k < K) {
            v.x = fmaf(gk[k], yy[k].x, v.x); v.y = fmaf(gk[k], yy[k].y, v.y);
            v.z = fmaf(gk[k], yy[k].z, v.z); v.w = fmaf(gk[k], yy[k].w, v.w);
        }
    }
    float4 *o = (float4 *)(out + (int64_t)t * H);
    if (accumulate) {
        const float4 a = o[c];
        v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
    }
    o[c] = v;
}

int mq_launch_combine(const float *y, int nsplit, int64_t split_stride, const int32_t *inv,
                      const float *gate, const float *shared, int sh_nsplit, int64_t sh_stride, int T, int H,
                      int K, int accumulate, float *out, hipStream_t st) {
    hipLaunchKernelGGL(k_combine, dim3((H / 4 + 255) / 256, T), dim3(256), 0, st, y, nsplit, split_stride,
                       inv, gate, shared, sh_nsplit, sh_stride, H, K, accumulate, out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
