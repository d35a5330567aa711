// Device helpers of the routing: the top-K selection of one token and the bucketing
// of a small batch held in LDS.  Shared by the top-K + bucketing launch and by the
// decode gate/up kernel, which routes batches of a few tokens itself.
#pragma once
#include "common.h"

// One work-group per token.  Every thread adds the split-K partial logits of up to
// two experts (fixed order) and the bias.  The selection order is value
// descending, ties to the lower expert index; it is the order of the 64-bit keys
// (order-preserving bits of the logit, then the complemented expert index), all
// distinct, so an expert's rank is the number of larger keys.  Two levels: each
// chunk of 64 experts ranks its own keys and keeps those of rank < K as
// candidates (every member of the overall top K is in its chunk's top K), then
// the candidates are ranked among themselves; an expert of the overall top K has
// the same rank there, every other candidate a rank >= K.  Gates are the softmax
// over the selected logits, which equals the full softmax renormalised over the
// selection.
__device__ __forceinline__ uint32_t mq_order_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);    // -0 -> +0: equal floats, equal keys
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int B>
__device__ __forceinline__ float mq_sum_partials(const float *__restrict__ p, int64_t stride, int nsplit) {
    float a = 0.0f;
    for (int sp = 0; sp < nsplit; sp += B) {
        float v[B];
#pragma unroll
        for (int i = 0; i < B; ++i) v[i] = p[(int64_t)min(sp + i, nsplit - 1) * stride];
#pragma unroll
        for (int i = 0; i < B; ++i) a = sp + i < nsplit ? a + v[i] : a;
    }
    return a;
}

// LDS of one token's selection (experts padded to a multiple of 64, at most 512)
struct MqTopkLds {
    __attribute__((aligned(16))) uint64_t key[512];
    __attribute__((aligned(16))) uint64_t cand[8 * 16];   // [chunk][local rank < K]
    float lg[512];
    float sv[16];
    int se[16];
};

// Number of keys of key[0..n) (n even, 16-byte aligned) above `my`.
__device__ __forceinline__ int mq_count_above(const uint64_t *key, int n, uint64_t my) {
    int r[8] = {0, 0, 0, 0, 0, 0, 0, 0};           // independent counters (short chains)
    int m = 0;
    for (; m + 16 <= n; m += 16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const ulonglong2 k2 = *(const ulonglong2 *)&key[m + 2 * j];
            r[j] += (k2.x > my ? 1 : 0) + (k2.y > my ? 1 : 0);
        }
    }
    for (; m < n; m += 2) r[0] += (key[m] > my ? 1 : 0) + (key[m + 1] > my ? 1 : 0);
    return ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
}

// Token t by NT threads (thread index i); valid false: only the barriers.
template <int NT>
__device__ __forceinline__ void mq_topk_token(const float *__restrict__ logits, int nsplit,
                                              const float *__restrict__ bias, int T, int E, int K, int t,
                                              bool valid, int i, MqTopkLds &L, int32_t *__restrict__ idx,
                                              float *__restrict__ gate, int32_t *__restrict__ trace_idx,
                                              float *__restrict__ trace_w) {
    static_assert(NT >= 128, "one thread per candidate slot");
    const int E64 = (E + 63) & ~63;
    const int ncand = (E64 >> 6) * K;
    if (valid && i < 128) L.cand[i] = 0;             // empty candidate slots
    for (int e = i; valid && e < E64; e += NT) {
        if (e >= E) {
            L.key[e] = 0;                             // below every real key
            continue;
        }
        const float *p = logits + (int64_t)t * E + e;
        const int64_t stride = (int64_t)T * E;
        const float be = bias ? bias[e] : 0.0f;     // loaded together with the partials
        // partials added in split order; a batch of them is loaded at once (the
        // indices are clamped so that every load is unconditional)
        const float a = (nsplit <= 8 ? mq_sum_partials<8>(p, stride, nsplit)
                                     : mq_sum_partials<64>(p, stride, nsplit)) + be;
        L.lg[e] = a;
        L.key[e] = ((uint64_t)mq_order_key(a) << 32) | (uint32_t)(0xFFFFu - e);
    }
    __syncthreads();
    for (int e = i; valid && e < E; e += NT) {       // rank inside the chunk
        const uint64_t my = L.key[e];
        const int c = e >> 6;
        const int r = mq_count_above(L.key + 64 * c, 64, my);
        if (r < K) L.cand[c * K + r] = my;
    }
    __syncthreads();
    if (valid && i < ncand) {                        // rank among the candidates
        const uint64_t my = L.cand[i];
        const int r = mq_count_above(L.cand, (ncand + 1) & ~1, my);
        if (my != 0 && r < K) {
            const int e = 0xFFFF - (int)(my & 0xFFFFu);
            L.sv[r] = L.lg[e];
            L.se[r] = e;
        }
    }
    __syncthreads();
    // softmax over the K selected (one wave), skipped when no output is asked for
    if (valid && i < 64 && (idx || gate || trace_idx || trace_w)) {
        const float mx = L.sv[0];
        const float pk = i < K ? expf(L.sv[i] - mx) : 0.0f;
        float z = pk;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
        if (i < K) {
            const int me = L.se[i];
            const float g = pk / z;
            if (idx) idx[t * K + i] = me;
            if (gate) gate[t * K + i] = g;
            if (trace_idx) trace_idx[t * K + i] = me;
            if (trace_w) trace_w[t * K + i] = g;
        }
    }
}

// Bucketing of a small batch whose selections sit in LDS (sidx[S], S <= 256), by a
// work-group of NTH >= E threads, same results as mq_bucket_wg: every expert counts
// its slots by a scan of sidx, the offsets and unit starts are exclusive scans over the experts, and slot s
// lands at offsets[e] + #{s' < s : sidx[s'] = e} (stable in slot order).  The
// offsets, unit starts (and counts, unit total when given) stay in LDS; the global
// outputs are written only when `write` is set.
template <int NTH>
__device__ __forceinline__ void mq_bucket_small_wg(const int *sidx, int S, int E, int unit_tokens, bool write,
                                                   int32_t *__restrict__ counts_out,
                                                   int32_t *__restrict__ offsets_out,
                                                   int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                   int32_t *__restrict__ units_hdr, int4 *__restrict__ units,
                                                   int fill_units, int32_t *__restrict__ urow, int K, int zrow,
                                                   int *soff, int *sun, int *scnt, int *sU) {
    __shared__ int wsum[2][NTH / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int c = 0;
    if (tid < E)
        for (int s = 0; s < S; ++s) c += sidx[s] == tid ? 1 : 0;
    const int nu = (c + unit_tokens - 1) / unit_tokens;
    int a = c, b = nu;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int pa = __shfl_up(a, o, 64), pb = __shfl_up(b, o, 64);
        if (lane >= o) { a += pa; b += pb; }
    }
    if (lane == 63) { wsum[0][wv] = a; wsum[1][wv] = b; }
    __syncthreads();
    int ba = 0, bb = 0;
    for (int w = 0; w < wv; ++w) { ba += wsum[0][w]; bb += wsum[1][w]; }
    const int off = ba + a - c, u0 = bb + b - nu;
    if (tid < E) {
        soff[tid] = off;
        sun[tid] = u0;
        if (scnt) scnt[tid] = c;
    }
    if (write && tid < E) {
        counts_out[tid] = c;
        offsets_out[tid] = off;
        for (int k = 0, u = u0; k < c; k += unit_tokens, ++u) {
            units[u] = make_int4(tid, off + k, min(unit_tokens, c - k), 0);
            if (urow)
                for (int i = c - k; i < unit_tokens; ++i) urow[(int64_t)u * unit_tokens + i] = zrow;
        }
    }
    if (tid == NTH - 1) {
        if (sU) *sU = bb + b;
        if (write) {
            offsets_out[E] = ba + a;
            units_hdr[0] = bb + b;
        }
    }
    if (write) {
        int U = 0;
        for (int w = 0; w < NTH / 64; ++w) U += wsum[1][w];
        for (int u = U + tid; u < fill_units; u += NTH) units[u] = make_int4(0, 0, 0, 0);
    }
    __syncthreads();
    if (write && tid < S) {
        const int e = sidx[tid];
        int r = 0;
        for (int s = 0; s < tid; ++s) r += sidx[s] == e ? 1 : 0;
        const int pos = soff[e] + r;
        perm[pos] = tid;
        inv[tid] = pos;
        if (urow) urow[(int64_t)(sun[e] + r / unit_tokens) * unit_tokens + r % unit_tokens] = tid / K;
    }
}

