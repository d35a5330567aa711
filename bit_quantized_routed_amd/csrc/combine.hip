// Weighted combine of the expert outputs (fixed order, deterministic):
//   y[slot] = sum_{s=0}^{nsplit-1} yp[s][slot]      (split partial sums, in order)
//   v[t] = sum_s shared[s][t] + sum_{k=0}^{K-1} g[t,k] * y[inv[t*K+k]]   (shared in partials)
// (y in slot order when inv is null: y[t*K+k]).
//   out[t] = v[t]            (or out[t] + v[t] under residual accumulation)
#include "common.h"
#include "kernels.h"

// All loads are issued before the sums (split partials in batches of CB_SB, clamped
// indices); the sums then run in fixed order.  KMAX: 8 (top-K up to 8) or 16 (the
// indices past K are clamped to K - 1 and their terms skipped).
#define CB_SB 8
template <int CB_KMAX>
__global__ void __launch_bounds__(256) k_combine(const float *__restrict__ y, int nsplit,
                                                 int64_t split_stride, const int32_t *__restrict__ inv,
                                                 const float *__restrict__ gate,
                                                 const float *__restrict__ shared, int sh_nsplit,
                                                 int64_t sh_stride, int H, int K, int accumulate,
                                                 float *out) {
    const int t = blockIdx.y;
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= H / 4) return;
    int sl[CB_KMAX];
    float gk[CB_KMAX];
#pragma unroll
    for (int k = 0; k < CB_KMAX; ++k) {
        const int kk = min(k, K - 1);
        sl[k] = inv ? inv[t * K + kk] : t * K + kk;
        gk[k] = gate[t * K + kk];
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (shared) {
        const float4 *sp4 = (const float4 *)(shared + (int64_t)t * H) + c;
        for (int s0 = 0; s0 < sh_nsplit; s0 += CB_SB) {
            float4 q[CB_SB];
#pragma unroll
            for (int i = 0; i < CB_SB; ++i) q[i] = sp4[(int64_t)min(s0 + i, sh_nsplit - 1) * (sh_stride / 4)];
#pragma unroll
            for (int i = 0; i < CB_SB; ++i)
                if (s0 + i < sh_nsplit) { v.x += q[i].x; v.y += q[i].y; v.z += q[i].z; v.w += q[i].w; }
        }
    }
    // splits 0 and 1 loaded together; further splits (not used by the launches that
    // split the down projection at most twice) one after another
    float4 yy[CB_KMAX], y1[CB_KMAX];
#pragma unroll
    for (int k = 0; k < CB_KMAX; ++k) yy[k] = ((const float4 *)(y + (int64_t)sl[k] * H))[c];
    if (nsplit > 1) {
#pragma unroll
        for (int k = 0; k < CB_KMAX; ++k) y1[k] = ((const float4 *)(y + split_stride + (int64_t)sl[k] * H))[c];
#pragma unroll
        for (int k = 0; k < CB_KMAX; ++k) {
            yy[k].x += y1[k].x; yy[k].y += y1[k].y; yy[k].z += y1[k].z; yy[k].w += y1[k].w;
        }
    }
    for (int sp = 2; sp < nsplit; ++sp) {
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
    // few tokens: 64-thread work-groups, so that the loads of a row spread over more
    // compute units (the launch is latency- and load-issue-bound there)
    const int nb = T <= 8 ? 64 : 256;
    if (K <= 8)
        hipLaunchKernelGGL(k_combine<8>, dim3((H / 4 + nb - 1) / nb, T), dim3(nb), 0, st, y, nsplit,
                           split_stride, inv, gate, shared, sh_nsplit, sh_stride, H, K, accumulate, out);
    else
        hipLaunchKernelGGL(k_combine<16>, dim3((H / 4 + nb - 1) / nb, T), dim3(nb), 0, st, y, nsplit,
                           split_stride, inv, gate, shared, sh_nsplit, sh_stride, H, K, accumulate, out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
