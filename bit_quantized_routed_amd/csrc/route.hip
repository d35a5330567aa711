// Routing: router logits, softmax top-K with renormalised gates, and the
// deterministic token-by-expert bucketing (histogram, exclusive scan, stable
// permutation, touched-expert work units).
#include "common.h"
#include "kernels.h"
#include "prep_rows.h"
#include "topk_dev.h"

// ---------------------------------------------------------------- logits
// One wave per (expert, token tile of RT_TT tokens); lanes stride the hidden
// dimension in float4 steps; fp32 FMA, then a butterfly sum across the wave.
#define RT_TT 8
template <bool BF16>
__global__ void __launch_bounds__(256) k_router_logits(const void *__restrict__ x,
                                                       const float *__restrict__ wr,
                                                       const float *__restrict__ bias, int T,
                                                       int H, int E, float *__restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t0 = blockIdx.y * RT_TT;
    if (e >= E) return;
    const int nt = min(RT_TT, T - t0);
    float acc[RT_TT];
#pragma unroll
    for (int t = 0; t < RT_TT; ++t) acc[t] = 0.0f;
    const float4 *w4 = (const float4 *)(wr + (int64_t)e * H);
    for (int c = lane; c < H / 4; c += 64) {
        const float4 w = w4[c];
#pragma unroll
        for (int t = 0; t < RT_TT; ++t) {
            if (t < nt) {
                float4 v;
                if (BF16) {
                    const uint2 b = ((const uint2 *)((const uint16_t *)x + (int64_t)(t0 + t) * H))[c];
                    v = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                                    __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
                } else {
                    v = ((const float4 *)((const float *)x + (int64_t)(t0 + t) * H))[c];
                }
                acc[t] = fmaf(w.x, v.x, acc[t]);
                acc[t] = fmaf(w.y, v.y, acc[t]);
                acc[t] = fmaf(w.z, v.z, acc[t]);
                acc[t] = fmaf(w.w, v.w, acc[t]);
            }
        }
    }
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int t = 0; t < RT_TT; ++t) {
        const float s = mq_wave_sum(acc[t]);
        if (lane == 0 && t < nt) logits[(int64_t)(t0 + t) * E + e] = s + b;
    }
}

// ---------------------------------------------------------------- logits on MFMA
// bf16 activations x fp32 router weights.  Each weight is split exactly into three
// bf16 terms w = hi + mid + lo by truncation: hi = the top 8 significant bits of w,
// mid = the top 8 of r = w - hi, lo = r - mid (both differences exact in fp32; r
// spans at most the 16 bit positions below hi's, so lo keeps at most 8 significant
// bits and is a bf16 value whenever it stays a normal number, i.e. for
// |w| >= 2^-102; below that what is lost is under 2^-126), so every product with a
// bf16 activation is exact in fp32 and the MFMA accumulates in fp32
// (v_mfma_f32_16x16x32_bf16, three per fragment pair).  Truncation takes one mask
// per term.
// Tile: 64 tokens x 64 experts per work-group, wave w owns experts 16w..16w+15
// and the 4 token fragments; fragments are loaded straight from global memory.
// Split-K partial logits go to P[split][T][E] (summed in order by top-K).
typedef __bf16 mq_bf16x8 __attribute__((ext_vector_type(8)));
typedef short mq_s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void mq_split3(const float (&w)[8], mq_s16x8 &hi, mq_s16x8 &mid, mq_s16x8 &lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t b = __float_as_uint(w[i]);
        const float r1 = w[i] - __uint_as_float(b & 0xFFFF0000u);
        const uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
        const float r2 = r1 - __uint_as_float(m);
        hi[i] = (short)(b >> 16);
        mid[i] = (short)(m >> 16);
        lo[i] = (short)(__float_as_uint(r2) >> 16);
    }
}

// The k range of a split is walked in chunks of RT_KC 32-wide steps whose weight
// and activation loads are all issued before the chunk's multiplies; MF = token
// fragments per work-group (1 for up to 16 tokens, else 4).
#define RT_KC 8
template <int MF>
__device__ __forceinline__ void mq_router_wg(const uint16_t *__restrict__ x, const float *__restrict__ wr,
                                             int T, int H, int E, int k_per_split, float *__restrict__ P,
                                             int bx, int by, int bz) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int e0 = bx * 64 + wv * 16, t0 = by * 16 * MF;
    const int split = bz;
    const int k0 = split * k_per_split, k1 = min(H, k0 + k_per_split);
    const int r16 = lane & 15, q = lane >> 4;
    const int e = e0 + r16;
    mq_f32x4 acc[MF];
#pragma unroll
    for (int i = 0; i < MF; ++i) acc[i] = (mq_f32x4){0.f, 0.f, 0.f, 0.f};
    const float *wrow = wr + (int64_t)min(e, E - 1) * H;
    for (int kc = k0; kc < k1; kc += 32 * RT_KC) {
        float4 w0[RT_KC], w1[RT_KC];
        mq_u32x4 a[RT_KC][MF];
#pragma unroll
        for (int s = 0; s < RT_KC; ++s) {
            const int kk = kc + 32 * s + 8 * q;
            const bool ok = kc + 32 * s < k1;
            w0[s] = ok ? *(const float4 *)(wrow + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
            w1[s] = ok ? *(const float4 *)(wrow + kk + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
                const int t = t0 + 16 * mf + r16;
                a[s][mf] = (ok && t < T) ? *(const mq_u32x4 *)(x + (int64_t)t * H + kk)
                                         : (mq_u32x4){0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int s = 0; s < RT_KC; ++s) {
            if (kc + 32 * s >= k1) break;
            float w[8] = {w0[s].x, w0[s].y, w0[s].z, w0[s].w, w1[s].x, w1[s].y, w1[s].z, w1[s].w};
            if (e >= E) {
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = 0.0f;
            }
            mq_s16x8 bh, bm, bl;
            mq_split3(w, bh, bm, bl);
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
                const mq_bf16x8 av = __builtin_bit_cast(mq_bf16x8, a[s][mf]);
                acc[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(mq_bf16x8, bh), acc[mf], 0, 0, 0);
                acc[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(mq_bf16x8, bm), acc[mf], 0, 0, 0);
                acc[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(mq_bf16x8, bl), acc[mf], 0, 0, 0);
            }
        }
    }
    float *Ps = P + (int64_t)split * T * E;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * mf + 4 * q + i;
            if (t < T && e < E) Ps[(int64_t)t * E + e] = acc[mf][i];
        }
}

// Batches of at most RT_SMALL_T tokens: one work-group per expert e over the
// whole hidden dimension (thread i takes the float4 columns i, i + 256, ...;
// fp32 FMA of the bf16 activations, loads of 8 columns issued together), wave
// sums, then the 4 wave sums added in wave order.  The logits are final
// (P[t][e], one split).
#define RT_SMALL_T 8
__device__ __forceinline__ void mq_router_small_wg(const uint16_t *__restrict__ x,
                                                   const float *__restrict__ wr, int T, int H, int E,
                                                   float *__restrict__ P, int e) {
    __shared__ float red[4][RT_SMALL_T];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int C = H >> 2;
    const float4 *w4 = (const float4 *)(wr + (int64_t)e * H);
    float acc[RT_SMALL_T];
#pragma unroll
    for (int t = 0; t < RT_SMALL_T; ++t) acc[t] = 0.0f;
    for (int c0 = 0; c0 < C; c0 += 256 * 8) {
        float4 w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = c0 + tid + 256 * j;
            w[j] = c < C ? w4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int t = 0; t < RT_SMALL_T; ++t) {
            if (t >= T) break;
            const uint2 *x4 = (const uint2 *)(x + (int64_t)t * H);
            uint2 b[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = c0 + tid + 256 * j;
                b[j] = c < C ? x4[c] : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                acc[t] = fmaf(w[j].x, __uint_as_float(b[j].x << 16), acc[t]);
                acc[t] = fmaf(w[j].y, __uint_as_float(b[j].x & 0xFFFF0000u), acc[t]);
                acc[t] = fmaf(w[j].z, __uint_as_float(b[j].y << 16), acc[t]);
                acc[t] = fmaf(w[j].w, __uint_as_float(b[j].y & 0xFFFF0000u), acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < RT_SMALL_T; ++t) {
        if (t >= T) break;
        const float v = mq_wave_sum(acc[t]);
        if (lane == 0) red[wv][t] = v;
    }
    __syncthreads();
    if (tid < T) P[(int64_t)tid * E + e] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// MF = 0: mq_router_small_wg, one work-group per expert
template <int MF>
__global__ void __launch_bounds__(256) k_router_mma(const uint16_t *__restrict__ x,
                                                    const float *__restrict__ wr, int T, int H, int E,
                                                    int k_per_split, float *__restrict__ P) {
    if constexpr (MF == 0)
        mq_router_small_wg(x, wr, T, H, E, P, blockIdx.x);
    else
        mq_router_wg<MF>(x, wr, T, H, E, k_per_split, P, blockIdx.x, blockIdx.y, blockIdx.z);
}

// One launch for the two consumers of the bf16 layer input: the router
// work-groups (gx * gy * gz of them, flattened) and then one work-group per row of
// activation digits (T rows + the zero row).
template <int MF, int ND>
__global__ void __launch_bounds__(256) k_router_prep(const uint16_t *__restrict__ x,
                                                     const float *__restrict__ wr, int T, int H, int E,
                                                     int k_per_split, float *__restrict__ P, int gx, int gy,
                                                     int gz, mq_u32x4 *__restrict__ xdig,
                                                     uint32_t *__restrict__ xsum, float *__restrict__ xscale) {
    const int nr = gx * gy * gz;
    const int b = blockIdx.x;
    if (b < nr) {
        if constexpr (MF == 0)
            mq_router_small_wg(x, wr, T, H, E, P, b);
        else
            mq_router_wg<MF>(x, wr, T, H, E, k_per_split, P, b % gx, (b / gx) % gy, b / (gx * gy));
    } else {
        mq_prep_digits_wg<1, ND>(x, nullptr, 1, 0, T, H, H, xdig, xsum, xscale, MqSharedRows{}, b - nr);
    }
}

int mq_launch_router_prep(const uint16_t *x, const float *wr, int T, int H, int E, int nsplit, float *P,
                          void *xdig, uint32_t *xsum, float *xscale, int nd, int tiles, hipStream_t st) {
    if (H / 16 > 256 * PD_NG) return MOE_Q2_EUNSUPPORTED;
    int kps = (H + nsplit - 1) / nsplit;
    kps = (kps + 31) / 32 * 32;
    const bool small = T <= RT_SMALL_T && !tiles;
    if (small && nsplit != 1) return MOE_Q2_EINVAL;
    const int gx = small ? E : (E + 63) / 64, gz = nsplit;
    const int gy = T <= 16 ? 1 : (T + 63) / 64;
    const int64_t grid = (int64_t)gx * gy * gz + T + 1;
    if (grid > 0x7fffffff) return MOE_Q2_EUNSUPPORTED;
#define MQ_RP_LAUNCH(MFV, NDV)                                                                              \
    hipLaunchKernelGGL((k_router_prep<MFV, NDV>), dim3((unsigned)grid), dim3(256), 0, st, x, wr, T, H, E, kps, \
                       P, gx, gy, gz, (mq_u32x4 *)xdig, xsum, xscale)
    const int mf = small ? 0 : (T <= 16 ? 1 : 4);
    switch (mf * 2 + (nd == 2 ? 1 : 0)) {
    case 0: MQ_RP_LAUNCH(0, 1); break;
    case 1: MQ_RP_LAUNCH(0, 2); break;
    case 2: MQ_RP_LAUNCH(1, 1); break;
    case 3: MQ_RP_LAUNCH(1, 2); break;
    case 8: MQ_RP_LAUNCH(4, 1); break;
    default: MQ_RP_LAUNCH(4, 2); break;
    }
#undef MQ_RP_LAUNCH
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_router_splits(int T, int H, int E) {
    if (T <= RT_SMALL_T) return 1;
    const int tiles = ((T + 63) / 64) * ((E + 63) / 64);
    int s = (512 + tiles - 1) / tiles;
    const int smax = H / 128;
    if (s > smax) s = smax;
    return s < 1 ? 1 : s;
}

int mq_router_splits_fixed(int H) {
    const int s = H / 448;               // 448-wide k ranges: 16 splits at H = 7168
    return s < 1 ? 1 : (s > 16 ? 16 : s);
}

int mq_launch_router_mma(const uint16_t *x, const float *wr, int T, int H, int E, int nsplit,
                         float *P, int tiles, hipStream_t st) {
    int kps = (H + nsplit - 1) / nsplit;
    kps = (kps + 31) / 32 * 32;
    if (T <= RT_SMALL_T && !tiles) {
        if (nsplit != 1) return MOE_Q2_EINVAL;
        hipLaunchKernelGGL(k_router_mma<0>, dim3(E), dim3(256), 0, st, x, wr, T, H, E, kps, P);
    } else if (T <= 16)
        hipLaunchKernelGGL(k_router_mma<1>, dim3((E + 63) / 64, 1, nsplit), dim3(256), 0, st, x, wr, T, H,
                           E, kps, P);
    else
        hipLaunchKernelGGL(k_router_mma<4>, dim3((E + 63) / 64, (T + 63) / 64, nsplit), dim3(256), 0, st,
                           x, wr, T, H, E, kps, P);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

// ---------------------------------------------------------------- top-K
// (selection and small-batch bucketing helpers in topk_dev.h)
__global__ void __launch_bounds__(256) k_topk(const float *__restrict__ logits, int nsplit,
                                              const float *__restrict__ bias, int T, int E, int K,
                                              int32_t *__restrict__ idx, float *__restrict__ gate,
                                              int32_t *__restrict__ trace_idx,
                                              float *__restrict__ trace_w) {
    __shared__ MqTopkLds L;
    mq_topk_token<256>(logits, nsplit, bias, T, E, K, blockIdx.x, true, threadIdx.x, L, idx, gate, trace_idx,
                       trace_w);
}

// ---------------------------------------------------------------- bucketing
// Single work-group.  counts by LDS atomics (commutative), offsets by a scan,
// and the stable position of slot s = t*K + k inside expert e's bucket as
//   offsets[e] + #{t' < t : e chosen by t'}
// read from a per-expert token bitmap (bits set with atomic OR, so the result
// does not depend on thread order).  Tokens are processed in chunks of BK_CH.
// Also emits the touched experts as work units of at most `unit_tokens` slots:
//   units[u] = (expert, first bucket position, slot count, 0), units_hdr[0] = U,
// records U .. fill_units - 1 all zero (slot count 0: no unit), and, when urow is
// given, the row table urow[u][i] = token of the unit's slot i (zrow past the
// slot count), so that a consumer finds its rows with one load indexed by u.
#define BK_CH 512
#define BK_THREADS 1024
// (run by a work-group of BK_THREADS threads; sm = mq_bucket_lds_bytes(E) of LDS)
__device__ void mq_bucket_wg(const int32_t *__restrict__ idx, int T, int K, int E, int unit_tokens,
                             int32_t *__restrict__ counts_out, int32_t *__restrict__ offsets_out,
                             int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                             int32_t *__restrict__ units_hdr, int4 *__restrict__ units, int fill_units,
                             int32_t *__restrict__ urow, int zrow, uint32_t *sm) {
    const int tid = threadIdx.x;
    const int W = BK_CH / 32;                 // bitmap words per expert
    int32_t *cnt = (int32_t *)sm;             // [E]
    int32_t *off = cnt + E;                   // [E + 1]
    int32_t *run = off + E + 1;               // [E]
    int32_t *scan = run + E;                  // [E + 1] (unit scan)
    uint32_t *bm = (uint32_t *)(scan + E + 1);// [E][W]
    const int S = T * K;

    for (int e = tid; e < E; e += BK_THREADS) { cnt[e] = 0; run[e] = 0; }
    __syncthreads();
    for (int s = tid; s < S; s += BK_THREADS) atomicAdd(&cnt[idx[s]], 1);
    __syncthreads();
    {   // exclusive scans of cnt[e] (-> off) and of the unit count per expert (-> scan)
        __shared__ int wsum[2][BK_THREADS / 64];
        const int lane = tid & 63, wv = tid >> 6;
        const int c = tid < E ? cnt[tid] : 0;
        int a = c, b = (c + unit_tokens - 1) / unit_tokens;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int pa = __shfl_up(a, o, 64), pb = __shfl_up(b, o, 64);
            if (lane >= o) { a += pa; b += pb; }
        }
        if (lane == 63) { wsum[0][wv] = a; wsum[1][wv] = b; }
        __syncthreads();
        int ba = 0, bb = 0;
        for (int w = 0; w < wv; ++w) { ba += wsum[0][w]; bb += wsum[1][w]; }
        if (tid < E) {
            off[tid] = ba + a - c;
            scan[tid] = bb + b - (c + unit_tokens - 1) / unit_tokens;
        }
        if (tid == BK_THREADS - 1) {
            off[E] = ba + a;
            scan[E] = bb + b;
            units_hdr[0] = bb + b;
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += BK_THREADS) {
        counts_out[e] = cnt[e];
        offsets_out[e] = off[e];
        const int n = cnt[e];
        for (int c = 0, u = scan[e]; c < n; c += unit_tokens, ++u) {
            units[u] = make_int4(e, off[e] + c, min(unit_tokens, n - c), 0);
            if (urow)
                for (int i = n - c; i < unit_tokens; ++i) urow[(int64_t)u * unit_tokens + i] = zrow;
        }
    }
    for (int u = scan[E] + tid; u < fill_units; u += BK_THREADS) units[u] = make_int4(0, 0, 0, 0);
    if (tid == 0) offsets_out[E] = off[E];

    for (int t0 = 0; t0 < T; t0 += BK_CH) {
        const int tn = min(BK_CH, T - t0);
        for (int i = tid; i < E * W; i += BK_THREADS) bm[i] = 0u;
        __syncthreads();
        for (int s = t0 * K + tid; s < (t0 + tn) * K; s += BK_THREADS) {
            const int tl = s / K - t0;
            atomicOr(&bm[idx[s] * W + (tl >> 5)], 1u << (tl & 31));
        }
        __syncthreads();
        for (int s = t0 * K + tid; s < (t0 + tn) * K; s += BK_THREADS) {
            const int e = idx[s];
            const int tl = s / K - t0;
            const uint32_t *row = bm + e * W;
            int r = 0;
            for (int w = 0; w < (tl >> 5); ++w) r += __popc(row[w]);
            r += __popc(row[tl >> 5] & ((1u << (tl & 31)) - 1u));
            const int pos = off[e] + run[e] + r;
            perm[pos] = s;
            inv[s] = pos;
            if (urow) {
                const int local = run[e] + r;
                urow[(int64_t)(scan[e] + local / unit_tokens) * unit_tokens + local % unit_tokens] = s / K;
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += BK_THREADS) {
            int c = 0;
            for (int w = 0; w < W; ++w) c += __popc(bm[e * W + w]);
            run[e] += c;
        }
        __syncthreads();
    }
}

__global__ void __launch_bounds__(BK_THREADS) k_bucket(const int32_t *__restrict__ idx, int T, int K,
                                                       int E, int unit_tokens,
                                                       int32_t *__restrict__ counts_out,
                                                       int32_t *__restrict__ offsets_out,
                                                       int32_t *__restrict__ perm,
                                                       int32_t *__restrict__ inv,
                                                       int32_t *__restrict__ units_hdr,
                                                       int4 *__restrict__ units, int fill_units,
                                                       int32_t *__restrict__ urow, int zrow) {
    extern __shared__ uint32_t sm[];
    mq_bucket_wg(idx, T, K, E, unit_tokens, counts_out, offsets_out, perm, inv, units_hdr, units, fill_units,
                 urow, zrow, sm);
}

// Large batches (prefill): the same bucketing in three launches over chunks of
// BKP_CH tokens.  (1) per chunk, the expert histogram (LDS atomics: commutative) into
// cnt[e][chunk]; (2) one work-group: per expert the exclusive prefix over the chunks
// in chunk order and the total, exclusive scans over the experts (offsets, unit
// starts), unit records, and cnt[e][chunk] = offsets[e] + that prefix, the chunk's
// first bucket position for e; (3) per chunk, slot s = t*K + k of expert e goes to
// cnt[e][chunk] + #{tokens t' < t of the chunk that chose e} (a per-expert token
// bitmap in LDS).  Same results as mq_bucket_wg.
#define BKP_CH 64
__global__ void __launch_bounds__(256) k_bucket_hist(const int32_t *__restrict__ idx, int T, int K, int E,
                                                     int C, int32_t *__restrict__ cnt) {
    extern __shared__ int32_t hc[];                 // [E]
    const int c = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) hc[e] = 0;
    __syncthreads();
    const int s0 = c * BKP_CH * K, s1 = min(T, (c + 1) * BKP_CH) * K;
    for (int q = s0 + tid; q < s1; q += 256) atomicAdd(&hc[idx[q]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += 256) cnt[(int64_t)e * C + c] = hc[e];
}

// (256 threads, so that it finds room on a compute unit next to a concurrent
// launch; thread i owns the ept = ceil(E / 256) experts ept * i .. ept * i + ept - 1,
// so that every thread has work for E <= 256 and the scan stays in expert order)
#define BKP_EPT 4
__global__ void __launch_bounds__(256) k_bucket_scan(int C, int E, int unit_tokens, int32_t *__restrict__ cnt,
                                                     int32_t *__restrict__ counts_out,
                                                     int32_t *__restrict__ offsets_out,
                                                     int32_t *__restrict__ units_hdr,
                                                     int4 *__restrict__ units, int fill_units) {
    __shared__ int wsum[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ept = (E + 255) / 256;
    int cn[BKP_EPT];
#pragma unroll
    for (int q = 0; q < BKP_EPT; ++q) {               // expert totals, 16 counts at once
        const int e = ept * tid + q;
        int c = 0;
        if (q < ept && e < E) {
            const int32_t *row = cnt + (int64_t)e * C;
            for (int k0 = 0; k0 < C; k0 += 16) {
                int v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = row[min(k0 + j, C - 1)];
#pragma unroll
                for (int j = 0; j < 16; ++j) c += k0 + j < C ? v[j] : 0;
            }
        }
        cn[q] = c;
    }
    int tc = 0, tu = 0;                               // this thread's slots and units
#pragma unroll
    for (int q = 0; q < BKP_EPT; ++q) { tc += cn[q]; tu += (cn[q] + unit_tokens - 1) / unit_tokens; }
    int a = tc, b = tu;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int pa = __shfl_up(a, o, 64), pb = __shfl_up(b, o, 64);
        if (lane >= o) { a += pa; b += pb; }
    }
    if (lane == 63) { wsum[0][wv] = a; wsum[1][wv] = b; }
    __syncthreads();
    int ba = 0, bb = 0;
    for (int w = 0; w < wv; ++w) { ba += wsum[0][w]; bb += wsum[1][w]; }
    int off = ba + a - tc, u = bb + b - tu;           // exclusive: first slot and unit of the thread
#pragma unroll
    for (int q = 0; q < BKP_EPT; ++q) {
        const int e = ept * tid + q, c = cn[q];
        if (q < ept && e < E) {
            counts_out[e] = c;
            offsets_out[e] = off;
            for (int k = 0; k < c; k += unit_tokens, ++u)
                units[u] = make_int4(e, off + k, min(unit_tokens, c - k), 0);
            // chunk bases: offset plus the exclusive prefix over the chunks (in chunk
            // order), 16 counts loaded before any is overwritten
            int32_t *row = cnt + (int64_t)e * C;
            int run = off;
            for (int k0 = 0; k0 < C; k0 += 16) {
                int v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = row[min(k0 + j, C - 1)];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (k0 + j < C) {
                        row[k0 + j] = run;
                        run += v[j];
                    }
            }
        }
        off += c;
    }
    if (tid == 255) {
        offsets_out[E] = ba + a;
        units_hdr[0] = bb + b;
    }
    const int U = wsum[1][0] + wsum[1][1] + wsum[1][2] + wsum[1][3];
    for (int q = U + tid; q < fill_units; q += 256) units[q] = make_int4(0, 0, 0, 0);
}

__global__ void __launch_bounds__(256) k_bucket_place(const int32_t *__restrict__ idx, int T, int K, int E,
                                                      int C, const int32_t *__restrict__ base,
                                                      int32_t *__restrict__ perm, int32_t *__restrict__ inv) {
    extern __shared__ uint32_t bm[];                // [E][BKP_CH / 32] token bitmaps
    constexpr int W = BKP_CH / 32;
    const int c = blockIdx.x, tid = threadIdx.x, t0 = c * BKP_CH;
    for (int i = tid; i < E * W; i += 256) bm[i] = 0u;
    __syncthreads();
    const int s0 = t0 * K, s1 = min(T, t0 + BKP_CH) * K;
    for (int q = s0 + tid; q < s1; q += 256) {
        const int tl = q / K - t0;
        atomicOr(&bm[idx[q] * W + (tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    for (int q = s0 + tid; q < s1; q += 256) {
        const int e = idx[q], tl = q / K - t0;
        const uint32_t *row = bm + e * W;
        int r = 0;
#pragma unroll
        for (int w = 0; w < W; ++w)
            if (w < (tl >> 5)) r += __popc(row[w]);
        r += __popc(row[tl >> 5] & ((1u << (tl & 31)) - 1u));
        const int pos = base[(int64_t)e * C + c] + r;
        perm[pos] = q;
        inv[q] = pos;
    }
}

int mq_bucket_chunks(int T) { return (T + BKP_CH - 1) / BKP_CH; }

int mq_launch_bucket_par(const int32_t *idx, int T, int K, int E, int unit_tokens, int32_t *counts,
                         int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *units_hdr, int4 *units,
                         int fill_units, int32_t *chunk, hipStream_t st) {
    if (E > 256 * BKP_EPT || T < 1) return MOE_Q2_EUNSUPPORTED;
    const int C = mq_bucket_chunks(T);
    hipLaunchKernelGGL(k_bucket_hist, dim3(C), dim3(256), (size_t)E * 4, st, idx, T, K, E, C, chunk);
    MQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(256), 0, st, C, E, unit_tokens, chunk, counts, offsets,
                       units_hdr, units, fill_units);
    MQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_bucket_place, dim3(C), dim3(256), (size_t)E * (BKP_CH / 32) * 4, st, idx, T, K, E, C,
                       chunk, perm, inv);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

size_t mq_bucket_lds_bytes(int E) {
    return (size_t)(4 * E + 2) * 4 + (size_t)E * (BK_CH / 32) * 4;
}

// Top-K and bucketing in one work-group, for batches of at most TB_TOKENS
// tokens: one group of 256 threads selects for each token, the selections stay
// in LDS, then the whole work-group buckets them.
#define TB_TOKENS (BK_THREADS / 256)
__global__ void __launch_bounds__(BK_THREADS) k_topk_bucket(const float *__restrict__ logits, int nsplit,
                                                            const float *__restrict__ bias, int T, int E,
                                                            int K, int32_t *__restrict__ idx,
                                                            float *__restrict__ gate,
                                                            int32_t *__restrict__ trace_idx,
                                                            float *__restrict__ trace_w, int unit_tokens,
                                                            int32_t *__restrict__ counts,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ perm,
                                                            int32_t *__restrict__ inv,
                                                            int32_t *__restrict__ units_hdr,
                                                            int4 *__restrict__ units, int fill_units,
                                                            int32_t *__restrict__ urow, int zrow) {
    __shared__ MqTopkLds L[TB_TOKENS];
    __shared__ int sidx[TB_TOKENS * 16];
    __shared__ int soff[BK_THREADS], sun[BK_THREADS];
    const int g = threadIdx.x >> 8, i = threadIdx.x & 255;
    mq_topk_token<256>(logits, nsplit, bias, T, E, K, g, g < T, i, L[g], idx, gate, trace_idx, trace_w);
    if (g < T && i < K) sidx[g * K + i] = L[g].se[i];
    __syncthreads();
    mq_bucket_small_wg<BK_THREADS>(sidx, T * K, E, unit_tokens, true, counts, offsets, perm, inv, units_hdr,
                                   units, fill_units, urow, K, zrow, soff, sun, nullptr, nullptr);
}

int mq_launch_topk_bucket(const float *logits, int nsplit, const float *bias, int T, int E, int K,
                          int32_t *idx, float *gate, int32_t *trace_idx, float *trace_w, int unit_tokens,
                          int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *units_hdr,
                          int4 *units, int fill_units, int32_t *urow, int zrow, hipStream_t st) {
    if (E > BK_THREADS || T > TB_TOKENS || K > 16) return MOE_Q2_EUNSUPPORTED;
    hipLaunchKernelGGL(k_topk_bucket, dim3(1), dim3(BK_THREADS), 0, st, logits, nsplit,
                       bias, T, E, K, idx, gate, trace_idx, trace_w, unit_tokens, counts, offsets, perm, inv,
                       units_hdr, units, fill_units, urow, zrow);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_router(const void *x, int bf16, const float *wr, const float *bias, int T, int H,
                     int E, float *logits, hipStream_t st) {
    dim3 grid((E + 3) / 4, (T + RT_TT - 1) / RT_TT);
    if (bf16)
        hipLaunchKernelGGL(k_router_logits<true>, grid, dim3(256), 0, st, x, wr, bias, T, H, E, logits);
    else
        hipLaunchKernelGGL(k_router_logits<false>, grid, dim3(256), 0, st, x, wr, bias, T, H, E, logits);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_topk(const float *logits, int nsplit, const float *bias, int T, int E, int K,
                   int32_t *idx, float *gate, int32_t *trace_idx, float *trace_w, hipStream_t st) {
    hipLaunchKernelGGL(k_topk, dim3(T), dim3(256), 0, st, logits, nsplit, bias, T, E, K,
                       idx, gate, trace_idx, trace_w);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_bucket(const int32_t *idx, int T, int K, int E, int unit_tokens, int32_t *counts,
                     int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *units_hdr,
                     int4 *units, int fill_units, int32_t *urow, int zrow, hipStream_t st) {
    const size_t lds = mq_bucket_lds_bytes(E);
    hipLaunchKernelGGL(k_bucket, dim3(1), dim3(BK_THREADS), lds, st, idx, T, K, E, unit_tokens,
                       counts, offsets, perm, inv, units_hdr, units, fill_units, urow, zrow);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
