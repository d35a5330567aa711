// Activation preparation for the decode kernels, and the RMSNorm of the
// residual stream.
//
// The decode dot product runs on v_dot2_f32_f16.  Weight codes enter as the fp16
// numbers 1024 + f*q (q in 0..3 sits in the mantissa with a position factor
// f in {1, 4, 16, 64, 256}, see ffn_dec.hip), so each activation is stored
// pre-divided by the same factor and by a per-row power-of-two scale s:
//   xq  = fp16(x_i / (s * f_i)), packed in the pair order the weights use;
//   gsum[j] = ( -1024 * sum_i xq_i ,  sum_i x_i / s )  per 16-element group j;
//   scale   = s = 2^(e - 10) with max|x| in (2^(e-1), 2^e]  (1 for an all-zero row).
// Then for a group with codes q, scale sc and min m:
//   sum_i (d*sc*q_i - dmin*m) x_i = s * ( d*sc*(S - 1024*sum xq) - dmin*m*sum x_i/s )
// where S = sum over the 8 code pairs of dot2(1024 + f*q, xq).
#include "common.h"
#include "kernels.h"

// pair p (0..7) holds group elements (p, p + 8); factor f_p:
__constant__ float mq_pair_inv_factor[8] = {1.0f, 0.25f, 0.0625f, 0.015625f, 0.00390625f,
                                            1.0f, 0.25f, 0.0625f};

template <int SRC>  // 0: fp32 rows, 1: bf16 rows
__global__ void __launch_bounds__(256) k_prep_act(const void *__restrict__ src, int nrows, int len,
                                                  int64_t src_ld, uint32_t *__restrict__ xq,
                                                  float2 *__restrict__ gsum,
                                                  float *__restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= nrows) return;
    const int G = len / 16;
    auto load16 = [&](int g, float *v) {
        if (SRC == 0) {
            const float4 *p = (const float4 *)((const float *)src + row * src_ld + g * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 a = p[i];
                v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
            }
        } else {
            const uint4 *p = (const uint4 *)((const uint16_t *)src + row * src_ld + g * 16);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 a = p[i];
                const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
                    v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
                }
            }
        }
    };
    float amax = 0.0f;
    for (int g = lane; g < G; g += 64) {
        float v[16];
        load16(g, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = mq_wave_max(amax);
    int ex = 0;
    if (amax > 0.0f) frexpf(amax, &ex);
    const float inv_s = amax > 0.0f ? ldexpf(1.0f, 10 - ex) : 1.0f;
    if (lane == 0) scale[row] = amax > 0.0f ? ldexpf(1.0f, ex - 10) : 1.0f;
    uint32_t *xr = xq + (int64_t)row * G * 8;
    float2 *gr = gsum + (int64_t)row * G;
    for (int g = lane; g < G; g += 64) {
        float v[16];
        load16(g, v);
        float X = 0.0f, Y = 0.0f;
        uint32_t w[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const float f = inv_s * mq_pair_inv_factor[p];
            const __half a = __float2half_rn(v[p] * f), b = __float2half_rn(v[p + 8] * f);
            w[p] = (uint32_t)__half_as_ushort(a) | ((uint32_t)__half_as_ushort(b) << 16);
            Y += __half2float(a) + __half2float(b);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) X += v[i] * inv_s;
        uint4 *o = (uint4 *)(xr + g * 8);
        o[0] = make_uint4(w[0], w[1], w[2], w[3]);
        o[1] = make_uint4(w[4], w[5], w[6], w[7]);
        gr[g] = make_float2(-1024.0f * Y, X);
    }
}

// x_bf16[t] = bf16(h[t] / sqrt(mean(h[t]^2) + eps)), one work-group per row.
// The bf16 rounding of each element is a decision on the exact quotient, so the
// sum of squares, the mean, the square root and the quotient are taken in fp64
// (rounding errors ~1e-16, far inside a bf16 half-ulp of 2^-9) and the quotient
// is rounded once, to nearest even, straight to bf16: an fp32 intermediate would
// round twice, and fp32 arithmetic moves ~1e-7 of the elements across a bf16
// rounding boundary.
__device__ __forceinline__ uint16_t mq_f64_to_bf16(double y) {
    // bf16 keeps 8 significant bits: spacing 2^(e-8) for |y| in [2^(e-1), 2^e),
    // 2^-133 below the smallest normal; y / spacing is exact, rint rounds it to
    // nearest even, and the rounded value is exact in fp32, whose top half is bf16
    int e = 0;
    (void)frexp(y, &e);
    e = e < -125 ? -125 : e;
    const double ulp = ldexp(1.0, e - 8);
    const float f = (float)(rint(y / ulp) * ulp);
    return (uint16_t)(__float_as_uint(f) >> 16);
}

__global__ void __launch_bounds__(256) k_rmsnorm_bf16(const float *__restrict__ h, int H, float eps,
                                                      uint16_t *__restrict__ x) {
    const int t = blockIdx.x;
    const float4 *hr = (const float4 *)(h + (int64_t)t * H);
    double ss = 0.0;
    for (int c = threadIdx.x; c < H / 4; c += 256) {
        const float4 v = hr[c];
        ss = fma((double)v.x, (double)v.x, ss); ss = fma((double)v.y, (double)v.y, ss);
        ss = fma((double)v.z, (double)v.z, ss); ss = fma((double)v.w, (double)v.w, ss);
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, MQ_WAVE);
    __shared__ double part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = (part[0] + part[1]) + (part[2] + part[3]);
    const double rs = sqrt(tot / (double)H + (double)eps);
    uint2 *xr = (uint2 *)(x + (int64_t)t * H);
    for (int c = threadIdx.x; c < H / 4; c += 256) {
        const float4 v = hr[c];
        xr[c] = make_uint2((uint32_t)mq_f64_to_bf16(v.x / rs) | ((uint32_t)mq_f64_to_bf16(v.y / rs) << 16),
                           (uint32_t)mq_f64_to_bf16(v.z / rs) | ((uint32_t)mq_f64_to_bf16(v.w / rs) << 16));
    }
}

int mq_launch_prep(const void *src, int src_bf16, int nrows, int len, int64_t src_ld, uint32_t *xq,
                   float2 *gsum, float *scale, hipStream_t st) {
    if (nrows <= 0) return MOE_Q2_OK;
    dim3 grid((nrows + 3) / 4);
    if (src_bf16)
        hipLaunchKernelGGL(k_prep_act<1>, grid, dim3(256), 0, st, src, nrows, len, src_ld, xq, gsum, scale);
    else
        hipLaunchKernelGGL(k_prep_act<0>, grid, dim3(256), 0, st, src, nrows, len, src_ld, xq, gsum, scale);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_rmsnorm(const float *h, int T, int H, float eps, uint16_t *x, hipStream_t st) {
    hipLaunchKernelGGL(k_rmsnorm_bf16, dim3(T), dim3(256), 0, st, h, H, eps, x);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

// fp32 -> two bf16 planes: hi = bf16(x), lo = bf16(x - hi) (x = hi + lo to ~16 bits).
__global__ void k_split_bf16(const float *__restrict__ x, int64_t n, uint16_t *__restrict__ hi,
                             uint16_t *__restrict__ lo) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float v = x[i];
        const uint16_t h = mq_f32_to_bf16(v);
        hi[i] = h;
        lo[i] = mq_f32_to_bf16(v - mq_bf16_to_f32(h));
    }
}

int mq_launch_split_bf16(const float *x, int64_t n, uint16_t *hi, uint16_t *lo, hipStream_t st) {
    const int grid = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_split_bf16, dim3(grid), dim3(256), 0, st, x, n, hi, lo);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
