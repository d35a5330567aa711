// Routed experts on the matrix cores, exact integer products of the 2-bit codes.
//
//   SWIGLU: h[p, r] = silu(x_t . Wg[r]) * (x_t . Wu[r])   for the slots p of an expert
//   PLAIN : y[p, r] = h_p . Wd[r]
//
// Each Q2 weight is w = d * sc_j * q - dmin * m_j, so for one 256-weight block
//   sum_i w_i a_i = d * sum_i (q_i sc_j) a_i  -  dmin * sum_j m_j A_j,   A_j = sum_{i in j} a_i.
// The activation row is quantised once per row to 15-bit integers a = rint(x / s)
// (s a power of two, |a| <= 2^14) and split into two int8 digits a = 256*hi + lo
// (lo in [-128, 127]).  The first sum is then exact on v_mfma_i32_16x16x64_i8:
// B = q*sc (0..45, an int8 built from the code dword with four mask/multiply
// pairs), A = hi and A = lo digits.  The min term is a 16-long product per block,
// done on v_mfma_f32_16x16x16_bf16 with B = m_j (exact) and A = A_j split into
// two bf16 planes.  Each block then folds d and dmin into an fp32 accumulator.
//
// MFMA roles: M = the unit's tokens (16), N = 16 weight rows, K = the reduction
// dimension.  Operand byte order inside a lane's 16-byte K slice follows the
// code dword: byte b of dword s is weight 4b + s of the group (the activation
// digits are stored in the same order).
//
// Work unit = (touched expert, 64-row tile of the tiled layout, up to 16 slots).
// Per work-group (4 waves): chunks of 4 block columns (21 KB, contiguous) stream
// HBM -> registers one chunk ahead of the compute and are copied to LDS; wave w
// computes block column w of the chunk for all 64 rows (4 N fragments), and the
// four waves' partial sums are added in a fixed order at the end.
#include "common.h"
#include "kernels.h"

typedef int32_t mq_i32x4 __attribute__((ext_vector_type(4)));
typedef short mq_s16x4 __attribute__((ext_vector_type(4)));

struct mq_pf6v { mq_u32x4 a, b, c, d, e, f; };

__device__ __forceinline__ void mq_ld6(const mq_u32x4 *__restrict__ src, int n16, int tid, mq_pf6v &pf) {
    pf.a = src[min(tid, n16 - 1)];
    pf.b = src[min(tid + 256, n16 - 1)];
    pf.c = src[min(tid + 512, n16 - 1)];
    pf.d = src[min(tid + 768, n16 - 1)];
    pf.e = src[min(tid + 1024, n16 - 1)];
    pf.f = src[min(tid + 1280, n16 - 1)];
}

__device__ __forceinline__ void mq_st6(mq_u32x4 *__restrict__ dst, int n16, int tid, const mq_pf6v &pf) {
    if (n16 == 4 * 336) {
        dst[tid] = pf.a;
        dst[tid + 256] = pf.b;
        dst[tid + 512] = pf.c;
        dst[tid + 768] = pf.d;
        dst[tid + 1024] = pf.e;
        if (__builtin_amdgcn_readfirstlane(tid >> 6) == 0) dst[tid + 1280] = pf.f;
        return;
    }
    if (tid < n16) dst[tid] = pf.a;
    if (tid + 256 < n16) dst[tid + 256] = pf.b;
    if (tid + 512 < n16) dst[tid + 512] = pf.c;
    if (tid + 768 < n16) dst[tid + 768] = pf.d;
    if (tid + 1024 < n16) dst[tid + 1024] = pf.e;
    if (tid + 1280 < n16) dst[tid + 1280] = pf.f;
}

// q*sc for the 16 weights of one group: dword s holds weights s, s+4, s+8, s+12.
__device__ __forceinline__ mq_i32x4 mq_codes_x_scale(uint32_t cw, uint32_t sc) {
    mq_i32x4 b;
    b[0] = (int32_t)((cw & 0x03030303u) * sc);
    b[1] = (int32_t)(((cw >> 2) & 0x03030303u) * sc);
    b[2] = (int32_t)(((cw >> 4) & 0x03030303u) * sc);
    b[3] = (int32_t)(((cw >> 6) & 0x03030303u) * sc);
    return b;
}

// m_j of 4 consecutive groups (one scale dword) as 4 bf16 (exact small integers).
__device__ __forceinline__ mq_s16x4 mq_mins_bf16(uint32_t swd) {
    const uint32_t m = (swd >> 4) & 0x0F0F0F0Fu;
    mq_s16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (short)(__float_as_uint((float)((m >> (8 * i)) & 0xFFu)) >> 16);
    return r;
}

template <bool SWIGLU>
__global__ void __launch_bounds__(256) k_q2_mma(const uint8_t *__restrict__ experts, int64_t expert_bytes,
                                                int64_t mat_off, int rows, int kblocks,
                                                const int32_t *__restrict__ units_hdr,
                                                const int4 *__restrict__ units,
                                                const int32_t *__restrict__ perm, int topk,
                                                const mq_u32x4 *__restrict__ xdig,
                                                const uint32_t *__restrict__ xsum,
                                                const float *__restrict__ xscale,
                                                float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint32_t stage[4 * 64 * MQ_BLOCK_DWORDS];
    __shared__ float red[4][16][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, q4 = lane >> 4;
    constexpr int ROW_TILE = SWIGLU ? 32 : 64;
    const int tiles = rows / ROW_TILE;
    const int U = units_hdr[0];
    const int G = kblocks * 16;                  // groups per activation row
    const int nchunks = (kblocks + 3) >> 2;
    const int64_t tile_bytes = (int64_t)kblocks * 64 * MQ_BLOCK_BYTES;

    for (int wu = blockIdx.x; wu < U * tiles; wu += gridDim.x) {
        const int u = wu / tiles, tile = wu - u * tiles;
        const int4 un = units[u];
        const int e = un.x, p0 = un.y, nt = un.z;
        const int r0 = tile * ROW_TILE;
        // A operand token of this lane: row l%16 of the M fragment
        const bool tok_ok = r16 < nt;
        const int arow = tok_ok ? (SWIGLU ? perm[p0 + r16] / topk : p0 + r16) : 0;
        const mq_u32x4 *xd = xdig + (int64_t)arow * G * 2;     // [G][2 digits] x 16 bytes
        const uint32_t *xs = xsum + (int64_t)arow * kblocks * 16; // [block][2 planes][16 bf16]
        const mq_u32x4 *tbase = (const mq_u32x4 *)(experts + (int64_t)e * expert_bytes + mat_off +
                                                   (int64_t)tile * tile_bytes);
        mq_f32x4 tot[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) tot[nf] = (mq_f32x4){0.f, 0.f, 0.f, 0.f};

        mq_pf6v pf;
        mq_ld6(tbase, min(4, kblocks) * 336, tid, pf);
        for (int c = 0; c < nchunks; ++c) {
            const int nb = min(4, kblocks - 4 * c);
            __syncthreads();
            mq_st6((mq_u32x4 *)stage, nb * 336, tid, pf);
            __syncthreads();
            if (c + 1 < nchunks)
                mq_ld6(tbase + (int64_t)(c + 1) * 4 * 336, min(4, kblocks - 4 * (c + 1)) * 336, tid, pf);
            if (wv < nb) {
                const int cb = 4 * c + wv;
                const uint32_t *bw = stage + wv * 64 * MQ_BLOCK_DWORDS;   // this wave's block column
                mq_i32x4 ahi[4], alo[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int g = cb * 16 + 4 * kk + q4;
                    if (tok_ok) {
                        const mq_u32x4 h = xd[2 * g], l = xd[2 * g + 1];
                        ahi[kk] = __builtin_bit_cast(mq_i32x4, h);
                        alo[kk] = __builtin_bit_cast(mq_i32x4, l);
                    } else {
                        ahi[kk] = (mq_i32x4){0, 0, 0, 0};
                        alo[kk] = (mq_i32x4){0, 0, 0, 0};
                    }
                }
                // bf16 planes of the group sums A_j, groups 4*q4 .. 4*q4+3 of block cb
                mq_s16x4 xh = {0, 0, 0, 0}, xl = {0, 0, 0, 0};
                if (tok_ok) {
                    const uint32_t *p = xs + cb * 16;                   // [2 planes][16 bf16] = 16 dwords
                    const uint2 vh = *(const uint2 *)(p + 2 * q4);
                    const uint2 vl = *(const uint2 *)(p + 8 + 2 * q4);
                    xh = __builtin_bit_cast(mq_s16x4, vh);
                    xl = __builtin_bit_cast(mq_s16x4, vl);
                }
#pragma unroll
                for (int nf = 0; nf < 4; ++nf) {
                    const uint32_t *blk = bw + (16 * nf + r16) * MQ_BLOCK_DWORDS;
                    mq_i32x4 ih = {0, 0, 0, 0}, il = {0, 0, 0, 0};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const uint32_t cw = blk[4 + 4 * kk + q4];
                        const uint32_t sc = (blk[kk] >> (8 * q4)) & 0xFu;
                        const mq_i32x4 b = mq_codes_x_scale(cw, sc);
                        ih = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi[kk], b, ih, 0, 0, 0);
                        il = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo[kk], b, il, 0, 0, 0);
                    }
                    const mq_s16x4 bm = mq_mins_bf16(blk[q4]);
                    mq_f32x4 am = {0.f, 0.f, 0.f, 0.f};
                    am = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, bm, am, 0, 0, 0);
                    am = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xl, bm, am, 0, 0, 0);
                    const uint32_t dd = blk[20];
                    const float d = mq_h2f((uint16_t)(dd & 0xFFFFu));
                    const float dmin = mq_h2f((uint16_t)(dd >> 16));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float qv = (float)((ih[i] << 8) + il[i]);
                        tot[nf][i] = fmaf(d, qv, fmaf(-dmin, am[i], tot[nf][i]));
                    }
                }
            }
        }
        // D layout: lane l, element i -> token 4*(l/16) + i, row slot 16*nf + l%16
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wv][4 * nf + i][lane] = tot[nf][i];
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * q4 + i;
                if (t < nt) {
                    const float s = xscale[SWIGLU ? perm[p0 + t] / topk : p0 + t];
                    float v[4];
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf)
                        v[nf] = ((red[0][4 * nf + i][lane] + red[1][4 * nf + i][lane]) +
                                 (red[2][4 * nf + i][lane] + red[3][4 * nf + i][lane])) * s;
                    float *o = out + (int64_t)(p0 + t) * rows + r0;
                    if (SWIGLU) {
                        // slots 0..31 gate rows, 32..63 up rows of the same 32 rows
#pragma unroll
                        for (int nf = 0; nf < 2; ++nf) {
                            const float g = v[nf], up = v[nf + 2];
                            o[16 * nf + r16] = g / (1.0f + expf(-g)) * up;
                        }
                    } else {
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf) o[16 * nf + r16] = v[nf];
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ activation digits
// Per row: s = 2^(e - 14) with max|x| in (2^(e-1), 2^e] (1 for an all-zero row);
// a = rint(x / s) (|a| <= 2^14), hi = floor((a + 128) / 256), lo = a - 256 hi.
// xdig[row][group][digit] = 16 bytes, byte b of dword s = digit of element 4b + s;
// xsum[row][block][plane][16] = bf16 planes of A_j = sum of the group's a (hi plane
// bf16(A_j), lo plane bf16(A_j - hi)).
template <int SRC>  // 0: fp32 rows, 1: bf16 rows
__global__ void __launch_bounds__(256) k_prep_digits(const void *__restrict__ src, int nrows, int len,
                                                     int64_t src_ld, mq_u32x4 *__restrict__ xdig,
                                                     uint32_t *__restrict__ xsum,
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
    const float inv_s = amax > 0.0f ? ldexpf(1.0f, 14 - ex) : 1.0f;
    if (lane == 0) scale[row] = amax > 0.0f ? ldexpf(1.0f, ex - 14) : 1.0f;
    mq_u32x4 *xr = xdig + (int64_t)row * G * 2;
    uint16_t *sr = (uint16_t *)(xsum + (int64_t)row * G);       // G/16 blocks x 32 bf16
    for (int g = lane; g < G; g += 64) {
        float v[16];
        load16(g, v);
        int a[16];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            a[i] = (int)rintf(v[i] * inv_s);
            sum += a[i];
        }
        mq_u32x4 hi, lo;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t h = 0, l = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int x = a[4 * b + s];
                const int dh = (x + 128) >> 8;
                const int dl = x - (dh << 8);
                h |= ((uint32_t)(dh & 0xFF)) << (8 * b);
                l |= ((uint32_t)(dl & 0xFF)) << (8 * b);
            }
            hi[s] = h;
            lo[s] = l;
        }
        xr[2 * g] = hi;
        xr[2 * g + 1] = lo;
        const float fs = (float)sum;                           // exact: |sum| <= 2^18
        const uint16_t bh = mq_f32_to_bf16(fs);
        const uint16_t bl = mq_f32_to_bf16(fs - mq_bf16_to_f32(bh));
        const int blk = g >> 4, j = g & 15;
        sr[blk * 32 + j] = bh;
        sr[blk * 32 + 16 + j] = bl;
    }
}

int mq_launch_prep_digits(const void *src, int src_bf16, int nrows, int len, int64_t src_ld,
                          void *xdig, uint32_t *xsum, float *scale, hipStream_t st) {
    if (nrows <= 0) return MOE_Q2_OK;
    dim3 grid((nrows + 3) / 4);
    if (src_bf16)
        hipLaunchKernelGGL(k_prep_digits<1>, grid, dim3(256), 0, st, src, nrows, len, src_ld,
                           (mq_u32x4 *)xdig, xsum, scale);
    else
        hipLaunchKernelGGL(k_prep_digits<0>, grid, dim3(256), 0, st, src, nrows, len, src_ld,
                           (mq_u32x4 *)xdig, xsum, scale);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_q2_mma(int swiglu, const void *experts, int64_t expert_bytes, int64_t mat_off,
                     int rows, int kblocks, const int32_t *units_hdr, const int4 *units,
                     int max_units, const int32_t *perm, int topk, const void *xdig,
                     const uint32_t *xsum, const float *xscale, float *out, int n_cu,
                     hipStream_t st) {
    const int tiles = rows / (swiglu ? 32 : 64);
    int64_t want = (int64_t)max_units * tiles;
    int64_t cap = (int64_t)n_cu * 8;
    const int grid = (int)(want < cap ? want : cap);
    if (grid <= 0) return MOE_Q2_OK;
    if (swiglu)
        hipLaunchKernelGGL(k_q2_mma<true>, dim3(grid), dim3(256), 0, st, (const uint8_t *)experts,
                           expert_bytes, mat_off, rows, kblocks, units_hdr, units, perm, topk,
                           (const mq_u32x4 *)xdig, xsum, xscale, out);
    else
        hipLaunchKernelGGL(k_q2_mma<false>, dim3(grid), dim3(256), 0, st, (const uint8_t *)experts,
                           expert_bytes, mat_off, rows, kblocks, units_hdr, units, perm, topk,
                           (const mq_u32x4 *)xdig, xsum, xscale, out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

// ------------------------------------------------------------------ prefill variant
// Same arithmetic as k_q2_mma, shaped for many tokens per expert.  Work unit =
// (expert, up to 16*MF slots); work item = (unit, super-tile of 4 consecutive
// 64-row tiles = 256 matrix rows).  Work-group = 8 waves: wave w owns tile w/2 and
// two 16-row fragments (SWIGLU: the gate fragment 16*(w%2).. and the up fragment
// 32 + 16*(w%2)..  of the same rows; PLAIN: fragments 2*(w%2), 2*(w%2)+1), times
// all MF token fragments.  Per block column, the 4 tiles' weights (21 KB) and the
// unit's activation digits + group sums (576 B per token) are staged in LDS, so a
// token's activations are read once per 256 rows; the next block column is
// prefetched into registers during the compute.
#define PF_TS 148   // LDS token stride in dwords: 576 B of data + 16 B pad (conflict-free reads)

template <bool SWIGLU, int MF>
__global__ void __launch_bounds__(512) k_q2_mma_pf(const uint8_t *__restrict__ experts,
                                                   int64_t expert_bytes, int64_t mat_off, int rows,
                                                   int kblocks, const int32_t *__restrict__ units_hdr,
                                                   const int4 *__restrict__ units,
                                                   const int32_t *__restrict__ perm, int topk,
                                                   const mq_u32x4 *__restrict__ xdig,
                                                   const uint32_t *__restrict__ xsum,
                                                   const float *__restrict__ xscale,
                                                   float *__restrict__ out) {
    constexpr int NTOK = 16 * MF;
    constexpr int NPB = (4 * 336 + 511) / 512;          // weight pieces per thread
    constexpr int NPA = (NTOK * 36 + 511) / 512;        // activation pieces per thread
    __shared__ __attribute__((aligned(16))) uint32_t sB[4 * 64 * MQ_BLOCK_DWORDS];
    __shared__ __attribute__((aligned(16))) uint32_t sA[NTOK * PF_TS];
    __shared__ int arow_s[NTOK];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, q4 = lane >> 4;
    const int tw = wv >> 1, hw = wv & 1;
    const int nslot0 = SWIGLU ? 16 * hw : 32 * hw;       // first fragment's slot
    const int nslot1 = SWIGLU ? 32 + 16 * hw : 32 * hw + 16;
    const int stiles = rows / (SWIGLU ? 32 : 64) / 4;
    const int U = units_hdr[0];
    const int G = kblocks * 16;
    const int64_t tile_bytes = (int64_t)kblocks * 64 * MQ_BLOCK_BYTES;

    for (int wu = blockIdx.x; wu < U * stiles; wu += gridDim.x) {
        const int u = wu / stiles, st = wu - u * stiles;
        const int4 un = units[u];
        const int e = un.x, p0 = un.y, nt = un.z;
        __syncthreads();
        for (int i = tid; i < NTOK; i += 512)
            arow_s[i] = i < nt ? (SWIGLU ? perm[p0 + i] / topk : p0 + i) : -1;
        __syncthreads();
        const uint8_t *tb = experts + (int64_t)e * expert_bytes + mat_off + (int64_t)(4 * st) * tile_bytes;
        const int nA = nt * 36;
        mq_u32x4 pb[NPB], pa[NPA];
        auto load = [&](int b) {
#pragma unroll
            for (int n = 0; n < NPB; ++n) {
                const int j = min(tid + 512 * n, 4 * 336 - 1);
                const int tl = j / 336, w = j - tl * 336;
                pb[n] = *(const mq_u32x4 *)(tb + (int64_t)tl * tile_bytes + (int64_t)b * 5376 + w * 16);
            }
#pragma unroll
            for (int n = 0; n < NPA; ++n) {
                const int j = min(tid + 512 * n, max(nA, 1) - 1);
                const int i = j / 36, w = j - i * 36;
                const int ar = max(arow_s[i], 0);
                if (w < 32)
                    pa[n] = xdig[((int64_t)ar * G + 16 * b) * 2 + w];
                else
                    pa[n] = *(const mq_u32x4 *)(xsum + ((int64_t)ar * kblocks + b) * 16 + (w - 32) * 4);
            }
        };
        mq_f32x4 tot[MF][2];
#pragma unroll
        for (int m = 0; m < MF; ++m) { tot[m][0] = (mq_f32x4){0.f, 0.f, 0.f, 0.f}; tot[m][1] = tot[m][0]; }
        load(0);
        for (int b = 0; b < kblocks; ++b) {
            __syncthreads();
#pragma unroll
            for (int n = 0; n < NPB; ++n) {
                const int j = tid + 512 * n;
                if (j < 4 * 336) *(mq_u32x4 *)(sB + 4 * j) = pb[n];
            }
#pragma unroll
            for (int n = 0; n < NPA; ++n) {
                const int j = tid + 512 * n;
                if (j < nA) {
                    const int i = j / 36, w = j - i * 36;
                    *(mq_u32x4 *)(sA + i * PF_TS + 4 * w) = pa[n];
                }
            }
            __syncthreads();
            if (b + 1 < kblocks) load(b + 1);
            const uint32_t *blk0 = sB + (tw * 64 + nslot0 + r16) * MQ_BLOCK_DWORDS;
            const uint32_t *blk1 = sB + (tw * 64 + nslot1 + r16) * MQ_BLOCK_DWORDS;
            mq_i32x4 hi[MF][2], lo[MF][2];
#pragma unroll
            for (int m = 0; m < MF; ++m)
#pragma unroll
                for (int f = 0; f < 2; ++f) { hi[m][f] = (mq_i32x4){0, 0, 0, 0}; lo[m][f] = hi[m][f]; }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int g = 4 * kk + q4;
                const mq_i32x4 b0 = mq_codes_x_scale(blk0[4 + g], (blk0[kk] >> (8 * q4)) & 0xFu);
                const mq_i32x4 b1 = mq_codes_x_scale(blk1[4 + g], (blk1[kk] >> (8 * q4)) & 0xFu);
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    if (16 * m < nt) {
                        const uint32_t *ap = sA + (16 * m + r16) * PF_TS + 8 * g;
                        const mq_i32x4 ah = __builtin_bit_cast(mq_i32x4, *(const mq_u32x4 *)ap);
                        const mq_i32x4 al = __builtin_bit_cast(mq_i32x4, *(const mq_u32x4 *)(ap + 4));
                        hi[m][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah, b0, hi[m][0], 0, 0, 0);
                        lo[m][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, b0, lo[m][0], 0, 0, 0);
                        hi[m][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah, b1, hi[m][1], 0, 0, 0);
                        lo[m][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, b1, lo[m][1], 0, 0, 0);
                    }
                }
            }
            const mq_s16x4 bm0 = mq_mins_bf16(blk0[q4]), bm1 = mq_mins_bf16(blk1[q4]);
            const uint32_t dd0 = blk0[20], dd1 = blk1[20];
            const float d0 = mq_h2f((uint16_t)(dd0 & 0xFFFFu)), m0 = mq_h2f((uint16_t)(dd0 >> 16));
            const float d1 = mq_h2f((uint16_t)(dd1 & 0xFFFFu)), m1 = mq_h2f((uint16_t)(dd1 >> 16));
#pragma unroll
            for (int m = 0; m < MF; ++m) {
                if (16 * m < nt) {
                    const uint32_t *xp = sA + (16 * m + r16) * PF_TS + 128;
                    const mq_s16x4 xh = __builtin_bit_cast(mq_s16x4, *(const uint2 *)(xp + 2 * q4));
                    const mq_s16x4 xl = __builtin_bit_cast(mq_s16x4, *(const uint2 *)(xp + 8 + 2 * q4));
                    mq_f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
                    a0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, bm0, a0, 0, 0, 0);
                    a0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xl, bm0, a0, 0, 0, 0);
                    a1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, bm1, a1, 0, 0, 0);
                    a1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xl, bm1, a1, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        tot[m][0][i] = fmaf(d0, (float)((hi[m][0][i] << 8) + lo[m][0][i]),
                                            fmaf(-m0, a0[i], tot[m][0][i]));
                        tot[m][1][i] = fmaf(d1, (float)((hi[m][1][i] << 8) + lo[m][1][i]),
                                            fmaf(-m1, a1[i], tot[m][1][i]));
                    }
                }
            }
        }
        // outputs: lane holds tokens 16m + 4*q4 + i of row slots (nslot0|nslot1) + r16
        const int trow = (4 * st + tw) * (SWIGLU ? 32 : 64);
#pragma unroll
        for (int m = 0; m < MF; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * m + 4 * q4 + i;
                if (t < nt) {
                    const float s = xscale[arow_s[t]];
                    float *o = out + (int64_t)(p0 + t) * rows + trow;
                    if (SWIGLU) {
                        const float g = tot[m][0][i] * s, up = tot[m][1][i] * s;
                        o[16 * hw + r16] = g / (1.0f + expf(-g)) * up;
                    } else {
                        o[nslot0 + r16] = tot[m][0][i] * s;
                        o[nslot1 + r16] = tot[m][1][i] * s;
                    }
                }
            }
        }
    }
}

int mq_launch_q2_mma_pf(int swiglu, const void *experts, int64_t expert_bytes, int64_t mat_off,
                        int rows, int kblocks, const int32_t *units_hdr, const int4 *units,
                        int max_units, const int32_t *perm, int topk, const void *xdig,
                        const uint32_t *xsum, const float *xscale, float *out, int n_cu,
                        hipStream_t st) {
    const int stiles = rows / (swiglu ? 32 : 64) / 4;
    int64_t want = (int64_t)max_units * stiles;
    int64_t cap = (int64_t)n_cu * 2;
    const int grid = (int)(want < cap ? want : cap);
    if (grid <= 0) return MOE_Q2_OK;
    if (swiglu)
        hipLaunchKernelGGL((k_q2_mma_pf<true, PF_MF>), dim3(grid), dim3(512), 0, st,
                           (const uint8_t *)experts, expert_bytes, mat_off, rows, kblocks, units_hdr,
                           units, perm, topk, (const mq_u32x4 *)xdig, xsum, xscale, out);
    else
        hipLaunchKernelGGL((k_q2_mma_pf<false, PF_MF>), dim3(grid), dim3(512), 0, st,
                           (const uint8_t *)experts, expert_bytes, mat_off, rows, kblocks, units_hdr,
                           units, perm, topk, (const mq_u32x4 *)xdig, xsum, xscale, out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
