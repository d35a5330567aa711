// Decode path of the routed experts: Q2 weights x activations on the vector
// ALUs with fp32 accumulation.  One kernel serves both halves of the expert FFN:
//   SWIGLU: h[p, r] = silu(x_t . Wg[r]) * (x_t . Wu[r])   for the slots p of an expert
//   PLAIN : y[p, r] = h_p . Wd[r]
//
// Work unit = (touched expert, row tile, up to FD_TCH slots of that expert);
// the grid is persistent and strides over the unit x tile space (the unit count
// is produced on the device by the bucketing kernel).
//
// Per work-group (4 waves, one 64-row tile of the tiled expert layout: SWIGLU
// tiles pair 32 gate rows with the same 32 up rows): the K dimension is walked
// in chunks of 4 block columns.  A chunk is one contiguous 21 KB span, streamed
// HBM -> registers with 16-byte loads one chunk ahead of the compute and then
// copied to LDS; wave w decodes block column w of the chunk, lane l owns tile
// row l (its block sits at an odd 21-dword stride: conflict-free LDS reads).
// The activations of the unit's slots are wave-uniform and read as scalars.
//
// Dot product per 16-weight group (see prep.hip for the activation side): the
// code dword holds weights i and i+8 at bits 2i and 2i+16, so
//   (code & (3<<2p | 3<<(2p+16))) | 0x64006400
// is the fp16 pair (1024 + 4^p q_p, 1024 + 4^p q_{p+8}) for p = 0..4, and the
// same on code >> 10 gives pairs 5..7 with factors 1, 4, 16.  Eight
// v_dot2_f32_f16 against the pre-divided activations, started from -1024*sum(xq),
// leave sum_i q_i x_i / s; the group then adds sc_j * that and m_j * sum x / s,
// and each block folds in d and -dmin.  The four waves' partial sums are added
// in a fixed order (deterministic).
#include "common.h"
#include "kernels.h"

#define FD_ROWS 64

// Wave-uniform data read through the scalar unit (constant address space).
#define MQ_CONST __attribute__((address_space(4)))

__device__ __forceinline__ float mq_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(mq_half2, a), __builtin_bit_cast(mq_half2, b), c,
                                  false);
}

// v_and_or_b32 with all-VGPR operands (gfx9 VOP3 takes no 32-bit literal).
__device__ __forceinline__ uint32_t mq_and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
    return r;
}

// Decode one 84-byte block (lane's row) against NT activation rows whose group
// records start at xb[t] (8 dwords per group) and gb[t] (2 floats per group).
template <int NT>
__device__ __forceinline__ void mq_block_dot(const uint32_t *__restrict__ bl,
                                             const uint32_t *__restrict__ xq,
                                             const float *__restrict__ gs, const uint32_t (&xo)[FD_TCH],
                                             const uint32_t (&mask)[5], uint32_t magic,
                                             float (&tot)[FD_TCH]) {
    uint32_t sw[4], cw[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) sw[i] = bl[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) cw[i] = bl[4 + i];
    const uint32_t dd = bl[20];
    const float d = mq_h2f((uint16_t)(dd & 0xFFFFu));
    const float dmin = mq_h2f((uint16_t)(dd >> 16));
    float accB[NT], accM[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) { accB[t] = 0.0f; accM[t] = 0.0f; }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t scb = sw[q] & 0x0F0F0F0Fu, mb = (sw[q] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 4 * q + i;
            const float scj = (float)((scb >> (8 * i)) & 0xFFu);
            const float mj = (float)((mb >> (8 * i)) & 0xFFu);
            const uint32_t c0 = cw[j], c10 = cw[j] >> 10;
            uint32_t A[8];
#pragma unroll
            for (int p = 0; p < 5; ++p) A[p] = mq_and_or(c0, mask[p], magic);
#pragma unroll
            for (int p = 5; p < 8; ++p) A[p] = mq_and_or(c10, mask[p - 5], magic);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const MQ_CONST uint32_t *xr = (const MQ_CONST uint32_t *)(xq + xo[t] + 8 * j);
                const MQ_CONST float *gp = (const MQ_CONST float *)(gs + (xo[t] >> 2) + 2 * j);
                float S = gp[0];
#pragma unroll
                for (int p = 0; p < 8; ++p) S = mq_dot2(A[p], xr[p], S);
                accB[t] = fmaf(scj, S, accB[t]);
                accM[t] = fmaf(mj, gp[1], accM[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        tot[t] = fmaf(d, accB[t], tot[t]);
        tot[t] = fmaf(-dmin, accM[t], tot[t]);
    }
}

// Chunk = up to 4 block columns of one 64-row tile: nb * 64 * 84 bytes, contiguous
// in the tiled expert layout (nb * 336 uint4).  Each thread owns uint4 i = tid + 256 n
// (indices past the chunk re-read its last uint4, which keeps every load in bounds
// and the prefetch registers unconditionally written).
struct mq_pf6 { mq_u32x4 a, b, c, d, e, f; };
__device__ __forceinline__ void mq_chunk_load(const mq_u32x4 *__restrict__ src, int n16, int tid,
                                              mq_pf6 &pf) {
    pf.a = src[min(tid, n16 - 1)];
    pf.b = src[min(tid + 256, n16 - 1)];
    pf.c = src[min(tid + 512, n16 - 1)];
    pf.d = src[min(tid + 768, n16 - 1)];
    pf.e = src[min(tid + 1024, n16 - 1)];
    pf.f = src[min(tid + 1280, n16 - 1)];
}
__device__ __forceinline__ void mq_chunk_store(mq_u32x4 *__restrict__ dst, int n16, int tid,
                                               const mq_pf6 &pf) {
    if (n16 == 4 * 336) {          // full chunk: mq_u32x4 1280..1343 belong to wave 0 only
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

template <bool SWIGLU>
__global__ void __launch_bounds__(256) k_q2_dec(const uint8_t *__restrict__ experts,
                                                int64_t expert_bytes, int64_t mat_off, int rows,
                                                int kblocks, const int32_t *__restrict__ units_hdr,
                                                const int4 *__restrict__ units,
                                                const int32_t *__restrict__ perm, int topk,
                                                const uint32_t *__restrict__ xq,
                                                const float2 *__restrict__ gsum,
                                                const float *__restrict__ xscale,
                                                float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint32_t stage[4 * 64 * MQ_BLOCK_DWORDS];
    __shared__ float red[4][FD_TCH][FD_ROWS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, known uniform
    constexpr int ROW_TILE = SWIGLU ? 32 : 64;
    const int tiles = rows / ROW_TILE;
    const int U = units_hdr[0];
    const int G = kblocks * 16;
    const int nchunks = (kblocks + 3) >> 2;
    const int64_t tile_bytes = (int64_t)kblocks * 64 * MQ_BLOCK_BYTES;
    uint32_t mask[5];
#pragma unroll
    for (int p = 0; p < 5; ++p) mask[p] = __builtin_amdgcn_readfirstlane(0x00030003u << (2 * p)) + 0u * lane;
    const uint32_t magic = 0x64006400u + 0u * lane;

    for (int wu = blockIdx.x; wu < U * tiles; wu += gridDim.x) {
        const int u = wu / tiles, tile = wu - u * tiles;
        const int4 un = units[u];
        const int e = un.x, p0 = un.y, nt = un.z;
        const int r0 = tile * ROW_TILE;
        int arow[FD_TCH];
#pragma unroll
        for (int t = 0; t < FD_TCH; ++t) {
            const int p = p0 + (t < nt ? t : 0);
            arow[t] = __builtin_amdgcn_readfirstlane(SWIGLU ? perm[p] / topk : p);
        }
        const mq_u32x4 *tbase = (const mq_u32x4 *)(experts + (int64_t)e * expert_bytes + mat_off +
                                             (int64_t)tile * tile_bytes);
        float tot[FD_TCH];
#pragma unroll
        for (int t = 0; t < FD_TCH; ++t) tot[t] = 0.0f;

        mq_pf6 pf;
        mq_chunk_load(tbase, min(4, kblocks) * 336, tid, pf);
        for (int c = 0; c < nchunks; ++c) {
            const int nb = min(4, kblocks - 4 * c);
            __syncthreads();
            mq_chunk_store((mq_u32x4 *)stage, nb * 336, tid, pf);
            __syncthreads();
            if (c + 1 < nchunks)
                mq_chunk_load(tbase + (int64_t)(c + 1) * 4 * 336, min(4, kblocks - 4 * (c + 1)) * 336,
                              tid, pf);
            if (wv < nb) {
                const int cb = 4 * c + wv;
                const uint32_t *bl = stage + (wv * 64 + lane) * MQ_BLOCK_DWORDS;
                // per-token dword offset of group record (row, cb*16) in xq (gsum is at 1/4)
                uint32_t xo[FD_TCH];
#pragma unroll
                for (int t = 0; t < FD_TCH; ++t) xo[t] = (uint32_t)(arow[t] * G + cb * 16) * 8u;
                const float *gs = (const float *)gsum;
                switch (nt) {
                case 1: mq_block_dot<1>(bl, xq, gs, xo, mask, magic, tot); break;
                case 2: mq_block_dot<2>(bl, xq, gs, xo, mask, magic, tot); break;
                case 3: mq_block_dot<3>(bl, xq, gs, xo, mask, magic, tot); break;
                default: mq_block_dot<4>(bl, xq, gs, xo, mask, magic, tot); break;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < FD_TCH; ++t) red[wv][t][lane] = tot[t];
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int t = 0; t < FD_TCH; ++t) {
                if (t < nt) {
                    const float s = xscale[arow[t]];
                    const float v = ((red[0][t][lane] + red[1][t][lane]) +
                                     (red[2][t][lane] + red[3][t][lane])) * s;
                    if (SWIGLU) {
                        const float up = __shfl(v, (lane & 31) + 32, 64);
                        if (lane < 32) {
                            const float h = v / (1.0f + expf(-v)) * up;
                            out[(int64_t)(p0 + t) * rows + r0 + lane] = h;
                        }
                    } else {
                        out[(int64_t)(p0 + t) * rows + r0 + lane] = v;
                    }
                }
            }
        }
    }
}

int mq_launch_q2_dec(int swiglu, const void *experts, int64_t expert_bytes, int64_t mat_off,
                     int rows, int kblocks, const int32_t *units_hdr, const int4 *units,
                     int max_units, const int32_t *perm, int topk, const uint32_t *xq,
                     const float2 *gsum, const float *xscale, float *out, int n_cu, hipStream_t st) {
    const int tiles = rows / (swiglu ? 32 : 64);
    int64_t want = (int64_t)max_units * tiles;
    int64_t cap = (int64_t)n_cu * 8;
    const int grid = (int)(want < cap ? want : cap);
    if (grid <= 0) return MOE_Q2_OK;
    if (swiglu)
        hipLaunchKernelGGL(k_q2_dec<true>, dim3(grid), dim3(256), 0, st, (const uint8_t *)experts,
                           expert_bytes, mat_off, rows, kblocks, units_hdr, units, perm, topk, xq,
                           gsum, xscale, out);
    else
        hipLaunchKernelGGL(k_q2_dec<false>, dim3(grid), dim3(256), 0, st, (const uint8_t *)experts,
                           expert_bytes, mat_off, rows, kblocks, units_hdr, units, perm, topk, xq,
                           gsum, xscale, out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
