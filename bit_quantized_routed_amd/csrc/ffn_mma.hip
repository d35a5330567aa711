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
// The decode kernel (k_q2_mma) and the prefill kernel (k_q2_mma_pf) differ in
// how they tile tokens and stage operands; both are described at their
// definitions below.
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
// sc2 = sc in both 16-bit halves; every byte product is at most 3 * 15, so one
// packed 16-bit multiply scales four bytes without carries.
typedef uint16_t mq_u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int32_t mq_mul_bytes(uint32_t x, uint32_t sc2) {
    return __builtin_bit_cast(int32_t, __builtin_bit_cast(mq_u16x2, x) * __builtin_bit_cast(mq_u16x2, sc2));
}

__device__ __forceinline__ mq_i32x4 mq_codes_x_scale(uint32_t cw, uint32_t sc) {
    const uint32_t sc2 = sc * 0x00010001u;
    mq_i32x4 b;
    b[0] = mq_mul_bytes(cw & 0x03030303u, sc2);
    b[1] = mq_mul_bytes((cw >> 2) & 0x03030303u, sc2);
    b[2] = mq_mul_bytes((cw >> 4) & 0x03030303u, sc2);
    b[3] = mq_mul_bytes((cw >> 6) & 0x03030303u, sc2);
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

// One block column of a 64-row tile is 64 * 84 = 5376 contiguous bytes = 336 uint4;
// a wave moves it with 6 16-byte loads per lane.  The sixth load of lanes 16..63
// repeats the last uint4 and lands in padding (the LDS slice holds 384 uint4), so
// no load or store is predicated.
struct mq_bcol { mq_u32x4 a, b, c, d, e, f; };

__device__ __forceinline__ void mq_bcol_load(const mq_u32x4 *__restrict__ src, int lane, mq_bcol &v) {
    v.a = src[lane];
    v.b = src[lane + 64];
    v.c = src[lane + 128];
    v.d = src[lane + 192];
    v.e = src[lane + 256];
    v.f = src[min(lane + 320, 335)];
}

__device__ __forceinline__ void mq_bcol_store(mq_u32x4 *__restrict__ dst, int lane, const mq_bcol &v) {
    dst[lane] = v.a;
    dst[lane + 64] = v.b;
    dst[lane + 128] = v.c;
    dst[lane + 192] = v.d;
    dst[lane + 256] = v.e;
    dst[lane + 320] = v.f;
}

// Activation operands of one block column for the lane's token: digits of groups
// 4kk + q4 (hi, lo), the two bf16 planes of the group sums 4q4 .. 4q4+3, and the
// row's scale.  Lanes without a token read an all-zero activation row.
struct mq_acol { mq_i32x4 hi[4], lo[4]; mq_s16x4 sh, sl; float sc; };

__device__ __forceinline__ void mq_acol_load(const mq_u32x4 *__restrict__ xd, const uint32_t *__restrict__ xs,
                                             const float *__restrict__ xsc, int cb, int q4, mq_acol &a) {
    a.sc = *xsc;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int g = cb * 16 + 4 * kk + q4;
        a.hi[kk] = __builtin_bit_cast(mq_i32x4, xd[2 * g]);
        a.lo[kk] = __builtin_bit_cast(mq_i32x4, xd[2 * g + 1]);
    }
    const uint32_t *p = xs + cb * 16;
    a.sh = __builtin_bit_cast(mq_s16x4, *(const uint2 *)(p + 2 * q4));
    a.sl = __builtin_bit_cast(mq_s16x4, *(const uint2 *)(p + 8 + 2 * q4));
}

// One 64-row block column from the wave's LDS slice into the 4 N fragments:
// integer products of both activation digits on the i8 matrix cores, the min
// term on the bf16 matrix cores, and the per-block fold with d and dmin.
__device__ __forceinline__ void mq_mma_column(const uint32_t *__restrict__ my, int r16, int q4,
                                              const mq_acol &a, mq_f32x4 (&tot)[4]) {
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
        const uint32_t *blk = my + (16 * nf + r16) * MQ_BLOCK_DWORDS;
        mq_i32x4 ih = {0, 0, 0, 0}, il = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint32_t cw = blk[4 + 4 * kk + q4];
            const uint32_t sc = (blk[kk] >> (8 * q4)) & 0xFu;
            const mq_i32x4 b = mq_codes_x_scale(cw, sc);
            ih = __builtin_amdgcn_mfma_i32_16x16x64_i8(a.hi[kk], b, ih, 0, 0, 0);
            il = __builtin_amdgcn_mfma_i32_16x16x64_i8(a.lo[kk], b, il, 0, 0, 0);
        }
        const mq_s16x4 bm = mq_mins_bf16(blk[q4]);
        mq_f32x4 am = {0.f, 0.f, 0.f, 0.f};
        am = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.sh, bm, am, 0, 0, 0);
        am = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.sl, bm, am, 0, 0, 0);
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

// Where a work unit's operands live, per lane: its weight tile and the lane's
// activation row (digits, group sums, scale).
struct mq_cursor {
    const mq_u32x4 *w;
    const mq_u32x4 *xd;
    const uint32_t *xs;
    const float *xsc;
    int p0, nt, r0;
};

#define MQ_DEC_PASSES 6
#define MQ_DEC_MAX_UNITS (16 * MQ_DEC_PASSES)    // work units per work-group

// Work unit = (touched expert, 64-row tile of the tiled layout, up to 16 slots);
// work-group g takes units g, g + grid, ... (at most MQ_DEC_MAX_UNITS of them).
// Per work-group (4 waves): wave w takes block columns w, w+4, ... of the tile for
// all 64 rows (4 N fragments).  Each wave streams its own block columns (5376
// contiguous bytes each) HBM -> registers one column ahead, together with the
// activation digits of that column (two register sets used alternately), and
// copies the weights to its private LDS slice.  The four waves' partial sums are
// added in a fixed order at the end of each unit.
//
// The stream runs across work units: the last column of a unit prefetches the
// first column of the work-group's next unit.  The work-group's unit records and
// per-token activation rows are gathered into LDS once, up front, so no memory
// load inside the stream depends on another one; every load is unconditional
// (padding tokens read an all-zero activation row, padding outputs go to a
// discard row).  The compiler's memory waits then only ever wait for the oldest
// column in flight, never drain the prefetch.
template <bool SWIGLU>
__global__ void __launch_bounds__(256) k_q2_mma(const uint8_t *__restrict__ experts, int64_t expert_bytes,
                                                int64_t mat_off, int rows, int kblocks,
                                                const int32_t *__restrict__ units_hdr,
                                                const int4 *__restrict__ units,
                                                const int32_t *__restrict__ perm, int topk, int zrow,
                                                int trash_row, const mq_u32x4 *__restrict__ xdig,
                                                const uint32_t *__restrict__ xsum,
                                                const float *__restrict__ xscale,
                                                float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) mq_u32x4 stage[4][384];   // one slice per wave
    __shared__ float red[4][16][64];
    __shared__ int4 t_unit[MQ_DEC_MAX_UNITS];                          // expert, p0, nt, r0
    __shared__ int t_row[MQ_DEC_MAX_UNITS][16];                        // activation row per token
    constexpr int ROW_TILE = SWIGLU ? 32 : 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, q4 = lane >> 4;
    const int tiles = rows / ROW_TILE;
    const int nwu = units_hdr[0] * tiles;
    const int G = kblocks * 16;                  // groups per activation row
    const int64_t tile_bytes = (int64_t)kblocks * 64 * MQ_BLOCK_BYTES;
    const int ncol = wv < kblocks ? (kblocks - wv + 3) / 4 : 0;   // this wave's columns per unit
    const int gsz = (int)gridDim.x;
    if ((int)blockIdx.x >= nwu) return;
    const int nj = (nwu - (int)blockIdx.x + gsz - 1) / gsz;      // units of this work-group
    mq_u32x4 *my = stage[wv];
    const uint32_t *myd = (const uint32_t *)my;

    // gather: thread (j, r) = (tid / 16 + 16 p, tid % 16)
    {
        const int r = tid & 15;
        int4 un[MQ_DEC_PASSES];
        int sl[MQ_DEC_PASSES];
#pragma unroll
        for (int p = 0; p < MQ_DEC_PASSES; ++p) {
            const int j = (tid >> 4) + 16 * p;
            un[p] = make_int4(0, 0, 1, 0);
            if (j < nj) un[p] = units[((int)blockIdx.x + j * gsz) / tiles];
        }
#pragma unroll
        for (int p = 0; p < MQ_DEC_PASSES; ++p) {
            const int j = (tid >> 4) + 16 * p;
            sl[p] = un[p].y + (r < un[p].z ? r : 0);
            if (SWIGLU && j < nj) sl[p] = perm[sl[p]];
        }
#pragma unroll
        for (int p = 0; p < MQ_DEC_PASSES; ++p) {
            const int j = (tid >> 4) + 16 * p;
            if (j < nj) {
                t_row[j][r] = r < un[p].z ? (SWIGLU ? sl[p] / topk : sl[p]) : zrow;
                if (r == 0) {
                    const int wu = (int)blockIdx.x + j * gsz;
                    t_unit[j] = make_int4(un[p].x, un[p].y, un[p].z, (wu - (wu / tiles) * tiles) * ROW_TILE);
                }
            }
        }
    }
    __syncthreads();

    auto open = [&](mq_cursor &c, int j) {
        const int4 t = t_unit[j];
        const int e = __builtin_amdgcn_readfirstlane(t.x);
        c.p0 = __builtin_amdgcn_readfirstlane(t.y);
        c.nt = __builtin_amdgcn_readfirstlane(t.z);
        c.r0 = __builtin_amdgcn_readfirstlane(t.w);
        c.w = (const mq_u32x4 *)(experts + (int64_t)e * expert_bytes + mat_off +
                                 (int64_t)(c.r0 / ROW_TILE) * tile_bytes);
        const int arow = t_row[j][r16];
        c.xd = xdig + (int64_t)arow * G * 2;
        c.xs = xsum + (int64_t)arow * G;
        c.xsc = xscale + arow;
    };
    // reduction of one finished unit and its stores; sc = the lane's row scale
    auto finish = [&](const mq_cursor &c, const mq_f32x4 (&tot)[4], float sc) {
        // D layout: lane l, element i -> token 4*(l/16) + i, row slot 16*nf + l%16
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wv][4 * nf + i][lane] = tot[nf][i];
        __syncthreads();
        if (SWIGLU) {
            // thread -> output row j (0..31), tokens t0 and t0 + 8
            const int j = tid & 31, t0 = tid >> 5;
            const int nfg = j >> 4, rr = j & 15;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int t = t0 + 8 * h;
                const int src = 16 * (t >> 2) + rr, i = t & 3;
                const float g = (red[0][4 * nfg + i][src] + red[1][4 * nfg + i][src]) +
                                (red[2][4 * nfg + i][src] + red[3][4 * nfg + i][src]);
                const float up = (red[0][4 * (nfg + 2) + i][src] + red[1][4 * (nfg + 2) + i][src]) +
                                 (red[2][4 * (nfg + 2) + i][src] + red[3][4 * (nfg + 2) + i][src]);
                const float st = __shfl(sc, t, 64);
                const float gs = g * st, us = up * st;
                out[(int64_t)(t < c.nt ? c.p0 + t : trash_row) * rows + c.r0 + j] =
                    gs / (1.0f + expf(-gs)) * us;
            }
        } else {
            // thread -> output row slot j (0..63), tokens t0, t0 + 4, t0 + 8, t0 + 12
            const int j = tid & 63, t0 = tid >> 6;
            const int nfj = j >> 4, rr = j & 15;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int t = t0 + 4 * h;
                const int src = 16 * (t >> 2) + rr, i = t & 3;
                const float v = (red[0][4 * nfj + i][src] + red[1][4 * nfj + i][src]) +
                                (red[2][4 * nfj + i][src] + red[3][4 * nfj + i][src]);
                out[(int64_t)(t < c.nt ? c.p0 + t : trash_row) * rows + c.r0 + j] = v * __shfl(sc, t, 64);
            }
        }
        __syncthreads();
    };

    mq_cursor cur;
    open(cur, 0);
    mq_f32x4 tot[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) tot[nf] = (mq_f32x4){0.f, 0.f, 0.f, 0.f};

    if (ncol == 0) {
        // fewer than 4 block columns: this wave only joins the reductions
        for (int j = 0; j < nj; ++j) {
            open(cur, j);
            finish(cur, tot, *cur.xsc);
        }
        return;
    }

    mq_bcol wb;
    mq_acol aA, aB;
    mq_bcol_load(cur.w + (int64_t)wv * 336, lane, wb);
    mq_acol_load(cur.xd, cur.xs, cur.xsc, wv, q4, aA);
    int i = 0, j = 0;
    // one block column; returns false when the stream has ended
    auto step = [&](const mq_acol &acur, mq_acol &anext) -> bool {
        mq_bcol_store(my, lane, wb);
        // the item after this one: the next column of this unit, or the first
        // column of the next unit (past the end: this column again, L2 hits whose
        // values are never used)
        mq_cursor nxt;
        const bool more = j + 1 < nj;
        open(nxt, more ? j + 1 : j);
        const bool last = i + 1 == ncol;
        const int cb = wv + 4 * i;
        const int cn = last ? (more ? wv : cb) : cb + 4;
        mq_bcol_load((last ? nxt.w : cur.w) + (int64_t)cn * 336, lane, wb);
        mq_acol_load(last ? nxt.xd : cur.xd, last ? nxt.xs : cur.xs, last ? nxt.xsc : cur.xsc, cn, q4, anext);
        mq_mma_column(myd, r16, q4, acur, tot);
        if (!last) {
            ++i;
            return true;
        }
        finish(cur, tot, acur.sc);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) tot[nf] = (mq_f32x4){0.f, 0.f, 0.f, 0.f};
        cur = nxt;
        i = 0;
        return ++j < nj;
    };
    while (step(aA, aB) && step(aB, aA)) {
    }
}

// ------------------------------------------------------------------ activation digits
// Per row: s = 2^(e - 14) with max|x| in (2^(e-1), 2^e] (1 for an all-zero row);
// a = rint(x / s) (|a| <= 2^14), hi = floor((a + 128) / 256), lo = a - 256 hi.
// xdig[row][group][digit] = 16 bytes, byte b of dword s = digit of element 4b + s;
// xsum[row][block][plane][16] = bf16 planes of A_j = sum of the group's a (hi plane
// bf16(A_j), lo plane bf16(A_j - hi)).
// One work-group per row (row == nrows: the all-zero row read by padding tokens).
// Thread i holds groups i, i + 256, ... (at most PD_NG) in registers: one pass of
// loads, a work-group max, then the digits from the registers.
#define PD_NG 4
template <int SRC>  // 0: fp32 rows, 1: bf16 rows
__global__ void __launch_bounds__(256) k_prep_digits(const void *__restrict__ src, int nrows, int len,
                                                     int64_t src_ld, mq_u32x4 *__restrict__ xdig,
                                                     uint32_t *__restrict__ xsum,
                                                     float *__restrict__ scale) {
    __shared__ float wmax[4];
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const bool zero_row = row == nrows;
    const int G = len / 16;
    float v[PD_NG][16];
#pragma unroll
    for (int n = 0; n < PD_NG; ++n) {
        const int g = tid + 256 * n;
        if (zero_row || g >= G) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[n][i] = 0.0f;
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
    const float inv_s = amax > 0.0f ? ldexpf(1.0f, 14 - ex) : 1.0f;
    if (tid == 0) scale[row] = amax > 0.0f ? ldexpf(1.0f, ex - 14) : 1.0f;
    mq_u32x4 *xr = xdig + (int64_t)row * G * 2;
    uint16_t *sr = (uint16_t *)(xsum + (int64_t)row * G);       // G/16 blocks x 32 bf16
#pragma unroll
    for (int n = 0; n < PD_NG; ++n) {
        const int g = tid + 256 * n;
        if (g >= G) break;
        int a[16];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            a[i] = (int)rintf(v[n][i] * inv_s);
            sum += a[i];
        }
        mq_u32x4 hi, lo;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            uint32_t h = 0, l = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int x = a[4 * b + s4];
                const int dh = (x + 128) >> 8;
                const int dl = x - (dh << 8);
                h |= ((uint32_t)(dh & 0xFF)) << (8 * b);
                l |= ((uint32_t)(dl & 0xFF)) << (8 * b);
            }
            hi[s4] = h;
            lo[s4] = l;
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
    if (len / 16 > 256 * PD_NG) return MOE_Q2_EUNSUPPORTED;
    dim3 grid(nrows + 1);                        // nrows rows + the zero row
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
                     int max_units, const int32_t *perm, int topk, int zrow, int trash_row,
                     const void *xdig, const uint32_t *xsum, const float *xscale, float *out, int n_cu,
                     hipStream_t st) {
    const int tiles = rows / (swiglu ? 32 : 64);
    const int64_t want = (int64_t)max_units * tiles;
    // resident work-groups (2 per compute unit), but never more than
    // MQ_DEC_MAX_UNITS work units per work-group
    int64_t g = (int64_t)n_cu * 2;
    if (g > want) g = want;
    if (g * MQ_DEC_MAX_UNITS < want) g = (want + MQ_DEC_MAX_UNITS - 1) / MQ_DEC_MAX_UNITS;
    if (g > 0x7fffffff) return MOE_Q2_EUNSUPPORTED;
    const int grid = (int)g;
    if (grid <= 0) return MOE_Q2_OK;
    if (swiglu)
        hipLaunchKernelGGL(k_q2_mma<true>, dim3(grid), dim3(256), 0, st, (const uint8_t *)experts,
                           expert_bytes, mat_off, rows, kblocks, units_hdr, units, perm, topk, zrow,
                           trash_row, (const mq_u32x4 *)xdig, xsum, xscale, out);
    else
        hipLaunchKernelGGL(k_q2_mma<false>, dim3(grid), dim3(256), 0, st, (const uint8_t *)experts,
                           expert_bytes, mat_off, rows, kblocks, units_hdr, units, perm, topk, zrow,
                           trash_row, (const mq_u32x4 *)xdig, xsum, xscale, out);
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
