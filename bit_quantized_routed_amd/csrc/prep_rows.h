// Activation digit preparation (one work-group per row), shared by the standalone
// preparation kernels and the router launch that also prepares the layer input.
#pragma once
#include "common.h"


// Two activation formats (ND = digits per element):
//  ND = 2 (15-bit, the default): s = 2^(e - 14) with max|x| in [2^(e-1), 2^e) (1 for
//   an all-zero row); a = rint(x / s) (|a| <= 2^14), hi = floor((a + 128) / 256),
//   lo = a - 256 hi: two int8 digits, a = 256 hi + lo exactly.
//  ND = 1 (Q8): s = 2^(e - 7); a = clamp(rint(x / s), -127, 127), one int8 digit.
// Both scales are powers of two, so x / s is exact and the rounding is a function of
// x alone (the oracle's Q8 mode takes the same decision).
// xdig[row][group][digit] = 16 bytes, byte b of dword s = digit of element 4b + s;
// xsum[row][block][quad][plane][4] = bf16 planes of A_j = sum of the group's a for
// the groups j = 4 quad .. 4 quad + 3 (hi plane bf16(A_j), lo plane bf16(A_j - hi)):
// one 16-byte vector per MFMA lane quad.
// One work-group per row (row == nrows: the all-zero row read by padding tokens).
// Thread i holds groups i, i + 256, ... (at most PD_NG) in registers: one pass of
// loads, a work-group max, then the digits from the registers.
// SRC 0: fp32 rows; 1: bf16 rows; 2: SwiGLU of split partial sums, row values
// silu(sum_s gate[s][row]) * sum_s up[s][row] (splits added in order; src = gate
// partials, src2 = up partials, split_stride apart).
#define PD_NG 4
// Work-groups after the zero row (SRC 2 only): the shared expert's SwiGLU, 256
// columns of one token each, h = silu(sum_s g[s][t]) * sum_s u[s][t] (splits in
// order, all partial loads in flight together), written as two bf16 planes
// (hi = bf16(h), lo = bf16(h - hi)).
struct MqSharedRows {
    const float *g, *u;
    int nsplit;
    int64_t split_stride;
    int Is;
    uint16_t *hi, *lo;
};

// Exponent offset of the row scale: 2^(e - MQ_ACT_BITS(ND)).
#define MQ_ACT_BITS(ND) ((ND) == 2 ? 14 : 7)

// The digits of 16 quantised elements a[0..15] of one group: ND 16-byte vectors.
template <int ND>
__device__ __forceinline__ void mq_group_digits(const int (&a)[16], mq_u32x4 *out) {
    mq_u32x4 hi, lo;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        uint32_t h = 0, l = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int x = a[4 * b + s4];
            const int dh = ND == 2 ? (x + 128) >> 8 : 0;
            const int dl = x - (dh << 8);
            h |= ((uint32_t)(dh & 0xFF)) << (8 * b);
            l |= ((uint32_t)(dl & 0xFF)) << (8 * b);
        }
        hi[s4] = h;
        lo[s4] = l;
    }
    if (ND == 2) {
        out[0] = hi;
        out[1] = lo;
    } else {
        out[0] = lo;
    }
}

// a = rint(v * inv_s), clamped to the int8 range for the one-digit format.
template <int ND>
__device__ __forceinline__ int mq_quant_act(float v, float inv_s) {
    const int x = (int)rintf(v * inv_s);
    return ND == 2 ? x : min(127, max(-127, x));
}

template <int SRC, int ND = 2>
__device__ __forceinline__ void mq_prep_digits_wg(const void *__restrict__ src, const void *__restrict__ src2,
                                                  int nsplit, int64_t split_stride, int nrows, int len,
                                                  int64_t src_ld, mq_u32x4 *__restrict__ xdig,
                                                  uint32_t *__restrict__ xsum, float *__restrict__ scale,
                                                  const MqSharedRows &sh, int row) {
    __shared__ float wmax[4];
    const int tid = threadIdx.x;
    if (SRC == 2 && row > nrows) {
        const int cb = (sh.Is + 255) / 256;
        const int t = (row - nrows - 1) / cb;
        const int c = ((row - nrows - 1) % cb) * 256 + tid;
        if (c >= sh.Is) return;
        const int64_t o = (int64_t)t * sh.Is + c;
        float g = 0.0f, u = 0.0f;
        for (int sp0 = 0; sp0 < sh.nsplit; sp0 += 16) {
            float gv[16], uv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t so = min(sp0 + j, sh.nsplit - 1) * sh.split_stride + o;
                gv[j] = sh.g[so];
                uv[j] = sh.u[so];
            }
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (sp0 + j < sh.nsplit) {
                    g += gv[j];
                    u += uv[j];
                }
        }
        const float h = g / (1.0f + expf(-g)) * u;
        const uint16_t hb = mq_f32_to_bf16(h);
        sh.hi[o] = hb;
        sh.lo[o] = mq_f32_to_bf16(h - mq_bf16_to_f32(hb));
        return;
    }
    const bool zero_row = row == nrows;
    const int G = len / 16;
    float v[PD_NG][16];
#pragma unroll
    for (int n = 0; n < PD_NG; ++n) {
        const int g = tid + 256 * n;
        if (zero_row || g >= G) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[n][i] = 0.0f;
        } else if (SRC == 2) {
            float gs[16], us[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) { gs[i] = 0.0f; us[i] = 0.0f; }
            // splits in order, four at a time with all their loads in flight
            for (int sp = 0; sp < nsplit; sp += 4) {
                float4 a[4][4], b[4][4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t off = min(sp + j, nsplit - 1) * split_stride + row * src_ld + g * 16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a[j][i] = ((const float4 *)((const float *)src + off))[i];
                        b[j][i] = ((const float4 *)((const float *)src2 + off))[i];
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (sp + j < nsplit) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            gs[4 * i] += a[j][i].x; gs[4 * i + 1] += a[j][i].y;
                            gs[4 * i + 2] += a[j][i].z; gs[4 * i + 3] += a[j][i].w;
                            us[4 * i] += b[j][i].x; us[4 * i + 1] += b[j][i].y;
                            us[4 * i + 2] += b[j][i].z; us[4 * i + 3] += b[j][i].w;
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) v[n][i] = gs[i] / (1.0f + expf(-gs[i])) * us[i];
        } else if (SRC == 0) {
            const float4 *p = (const float4 *)((const float *)src + row * src_ld + g * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 a = p[i];
                v[n][4 * i] = a.x; v[n][4 * i + 1] = a.y; v[n][4 * i + 2] = a.z; v[n][4 * i + 3] = a.w;
            }
        } else {
            const uint4 *p = (const uint4 *)((const uint16_t *)src + row * src_ld + g * 16);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 a = p[i];
                const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[n][8 * i + 2 * k] = __uint_as_float(w[k] << 16);
                    v[n][8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
                }
            }
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int n = 0; n < PD_NG; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[n][i]));
    amax = mq_wave_max(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    int ex = 0;
    if (amax > 0.0f) frexpf(amax, &ex);
    const float inv_s = amax > 0.0f ? ldexpf(1.0f, MQ_ACT_BITS(ND) - ex) : 1.0f;
    if (tid == 0) scale[row] = amax > 0.0f ? ldexpf(1.0f, ex - MQ_ACT_BITS(ND)) : 1.0f;
    mq_u32x4 *xr = xdig + (int64_t)row * G * ND;
    uint16_t *sr = (uint16_t *)(xsum + (int64_t)row * G);       // G/16 blocks x 32 bf16
#pragma unroll
    for (int n = 0; n < PD_NG; ++n) {
        const int g = tid + 256 * n;
        if (g >= G) break;
        int a[16];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            a[i] = mq_quant_act<ND>(v[n][i], inv_s);
            sum += a[i];
        }
        mq_group_digits<ND>(a, xr + ND * g);
        const float fs = (float)sum;                           // exact: |sum| <= 2^18
        const uint16_t bh = mq_f32_to_bf16(fs);
        const uint16_t bl = mq_f32_to_bf16(fs - mq_bf16_to_f32(bh));
        const int blk = g >> 4, j = g & 15;
        sr[blk * 32 + (j >> 2) * 8 + (j & 3)] = bh;
        sr[blk * 32 + (j >> 2) * 8 + 4 + (j & 3)] = bl;
    }
}

