// Weighted combine of the expert outputs (fixed order, deterministic):
//   v[t] = shared[t] + sum_{k=0}^{K-1} g[t,k] * y[inv[t*K+k]]
//   out[t] = v[t]            (or out[t] + v[t] under residual accumulation)
#include "common.h"
#include "kernels.h"

__global__ void __launch_bounds__(256) k_combine(const float *__restrict__ y,
                                                 const int32_t *__restrict__ inv,
                                                 const float *__restrict__ gate,
                                                 const float *__restrict__ shared, int H, int K,
                                                 int accumulate, float *out) {
    const int t = blockIdx.y;
    const float4 *sh = shared ? (const float4 *)(shared + (int64_t)t * H) : nullptr;
    float4 *o = (float4 *)(out + (int64_t)t * H);
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c < H / 4) {
        float4 v = sh ? sh[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k = 0; k < K; ++k) {
            const float g = gate[t * K + k];
            const float4 yy = ((const float4 *)(y + (int64_t)inv[t * K + k] * H))[c];
            v.x = fmaf(g, yy.x, v.x); v.y = fmaf(g, yy.y, v.y);
            v.z = fmaf(g, yy.z, v.z); v.w = fmaf(g, yy.w, v.w);
        }
        if (accumulate) {
            const float4 a = o[c];
            v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
        }
        o[c] = v;
    }
}

int mq_launch_combine(const float *y, const int32_t *inv, const float *gate, const float *shared,
                      int T, int H, int K, int accumulate, float *out, hipStream_t st) {
    hipLaunchKernelGGL(k_combine, dim3((H / 4 + 255) / 256, T), dim3(256), 0, st, y, inv, gate, shared, H,
                       K, accumulate, out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
