// Setup-time kernels (not part of the layer): seeded synthetic inputs and the
// Q2 quantizer.
#include "common.h"

// ------------------------------------------------------------------ synthetic
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11, section 3): per round the counter words 0 and 2 are
// multiplied by two odd constants; the high halves, xored with words 1 and 3 and
// the round key, and the low halves form the next counter; the key is bumped by
// two Weyl constants between rounds.
__device__ __forceinline__ void mq_philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
        const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    }
}

// value(i) = float(sum of the eight 16-bit halves of Philox(i) - 262140) * scale
__global__ void k_synth_normal(uint64_t seed, uint64_t stream, uint64_t start, int64_t n,
                               float scale, int out_bf16, void *out) {
#pragma clang fp contract(off)
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        const uint64_t i = start + (uint64_t)j;
        uint32_t c[4] = {(uint32_t)i, (uint32_t)(i >> 32), (uint32_t)stream,
                         (uint32_t)(stream >> 32)};
        mq_philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
        int32_t s = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) s += (int32_t)(c[w] & 0xFFFFu) + (int32_t)(c[w] >> 16);
        const float v = __fmul_rn((float)(s - 262140), scale);
        if (out_bf16) ((uint16_t *)out)[j] = mq_f32_to_bf16(v);
        else ((float *)out)[j] = v;
    }
}

// ------------------------------------------------------------------ quantizer
// Least fp16 h with n*h >= t (t >= 0, n = 15 or 7): nearest fp16 of t/n, stepped one
// ulp up when n*h (exact in fp32) is still below t.
__device__ __forceinline__ uint16_t mq_f16_up(float t, float n = 15.0f) {
#pragma clang fp contract(off)
    const float q = __fdiv_rn(t, n);
    uint16_t h = __half_as_ushort(__float2half_rn(q));
    if (__fmul_rn(mq_h2f(h), n) < t) h = (uint16_t)(h + 1);
    return h;
}

// One wave per 256-weight block; lane l owns weights 4l..4l+3 (group l/4).
__global__ void __launch_bounds__(256) k_quantize(const float *__restrict__ w, int64_t n_blocks,
                                                  uint8_t *__restrict__ out) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (blk >= n_blocks) return;
    const float4 x4 = ((const float4 *)(w + blk * MQ_QK))[lane];
    float x[4] = {x4.x, x4.y, x4.z, x4.w};
    float lo = fminf(fminf(x[0], x[1]), fminf(x[2], x[3]));
    float hi = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    lo = fminf(lo, __shfl_xor(lo, 1, 64));
    lo = fminf(lo, __shfl_xor(lo, 2, 64));
    hi = fmaxf(hi, __shfl_xor(hi, 1, 64));
    hi = fmaxf(hi, __shfl_xor(hi, 2, 64));
    lo = fminf(0.0f, lo);
    const float neg_lo = __fsub_rn(0.0f, lo);
    const float M = mq_wave_max(neg_lo);
    const uint16_t dmin16 = mq_f16_up(M);
    const float dmin = mq_h2f(dmin16);
    float m = 0.0f;
    if (dmin > 0.0f) m = fminf(ceilf(__fdiv_rn(neg_lo, dmin)), 15.0f);
    const float o = __fmul_rn(dmin, m);
    const float s = __fdiv_rn(__fadd_rn(hi, o), 3.0f);
    const float S = mq_wave_max(s);
    const uint16_t d16 = mq_f16_up(S);
    const float d = mq_h2f(d16);
    float sc = 0.0f;
    if (d > 0.0f) sc = fminf(ceilf(__fdiv_rn(s, d)), 15.0f);
    const float step = __fmul_rn(d, sc);
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float q = 0.0f;
        if (step > 0.0f) q = fminf(fmaxf(rintf(__fdiv_rn(__fadd_rn(x[i], o), step)), 0.0f), 3.0f);
        byte |= ((uint32_t)q) << (2 * i);
    }
    uint8_t *ob = out + blk * MQ_BLOCK_BYTES;
    ob[16 + lane] = (uint8_t)byte;
    if ((lane & 3) == 0) ob[lane >> 2] = (uint8_t)((uint32_t)sc | ((uint32_t)m << 4));
    if (lane == 0) {
        const bool bad = !(isfinite(d) && isfinite(dmin));
        const uint16_t dd = bad ? (uint16_t)0x7C00 : d16, dm = bad ? (uint16_t)0x7C00 : dmin16;
        ob[80] = (uint8_t)dd; ob[81] = (uint8_t)(dd >> 8);
        ob[82] = (uint8_t)dm; ob[83] = (uint8_t)(dm >> 8);
    }
}

// The 4-bit sibling (148-byte block): the same coverage rule with 15 code steps and
// 3-bit group scales --
//   dmin = least fp16 >= max_j(0 - lo_j) / 15, m_j = ceil((0 - lo_j) / dmin), o_j = dmin m_j,
//   s_j = (hi_j + o_j) / 15, d = least fp16 >= max_j s_j / 7, sc_j = ceil(s_j / d),
//   q = clamp(rint((x + o_j) / (d sc_j)), 0, 15).
// One wave per block; lane l owns elements 4l..4l+3 of the block (group j = l / 4,
// elements 4b + s of the group with b = l % 4).
__global__ void __launch_bounds__(256) k_quantize_q4(const float *__restrict__ w, int64_t n_blocks,
                                                     uint8_t *__restrict__ out) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (blk >= n_blocks) return;
    const float4 x4 = ((const float4 *)(w + blk * MQ_QK))[lane];
    float x[4] = {x4.x, x4.y, x4.z, x4.w};
    float lo = fminf(fminf(x[0], x[1]), fminf(x[2], x[3]));
    float hi = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    lo = fminf(lo, __shfl_xor(lo, 1, 64));
    lo = fminf(lo, __shfl_xor(lo, 2, 64));
    hi = fmaxf(hi, __shfl_xor(hi, 1, 64));
    hi = fmaxf(hi, __shfl_xor(hi, 2, 64));
    lo = fminf(0.0f, lo);
    const float neg_lo = __fsub_rn(0.0f, lo);
    const uint16_t dmin16 = mq_f16_up(mq_wave_max(neg_lo), 15.0f);
    const float dmin = mq_h2f(dmin16);
    float m = 0.0f;
    if (dmin > 0.0f) m = fminf(ceilf(__fdiv_rn(neg_lo, dmin)), 15.0f);
    const float o = __fmul_rn(dmin, m);
    const float sj = __fdiv_rn(__fadd_rn(hi, o), 15.0f);
    const uint16_t d16 = mq_f16_up(mq_wave_max(sj), 7.0f);
    const float d = mq_h2f(d16);
    float sc = 0.0f;
    if (d > 0.0f) sc = fminf(ceilf(__fdiv_rn(sj, d)), 7.0f);
    const float step = __fmul_rn(d, sc);
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = 0.0f;
        if (step > 0.0f) v = fminf(fmaxf(rintf(__fdiv_rn(__fadd_rn(x[i], o), step)), 0.0f), 15.0f);
        q[i] = (uint32_t)v;
    }
    uint8_t *ob = out + blk * (4 * MQ_BD4);
    const int j = lane >> 2, b = lane & 3;
    ob[16 + 8 * j + b] = (uint8_t)(q[0] | (q[1] << 4));
    ob[16 + 8 * j + 4 + b] = (uint8_t)(q[2] | (q[3] << 4));
    if (b == 0) ob[j] = (uint8_t)((uint32_t)sc | ((uint32_t)m << 4));
    if (lane == 0) {
        const bool bad = !(isfinite(d) && isfinite(dmin));
        const uint16_t dd = bad ? (uint16_t)0x7C00 : d16, dm = bad ? (uint16_t)0x7C00 : dmin16;
        ob[144] = (uint8_t)dd; ob[145] = (uint8_t)(dd >> 8);
        ob[146] = (uint8_t)dm; ob[147] = (uint8_t)(dm >> 8);
    }
}

extern "C" int moe_q2_synth_normal(uint64_t seed, uint64_t stream_id, uint64_t start, int64_t n,
                                   float scale, int32_t out_dtype, void *out, void *stream) {
    if (n < 0 || (n > 0 && out == nullptr)) return MOE_Q2_EINVAL;
    if (out_dtype != MOE_Q2_F32 && out_dtype != MOE_Q2_BF16) return MOE_Q2_EINVAL;
    if (n == 0) return MOE_Q2_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_synth_normal, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       seed, stream_id, start, n, scale, out_dtype == MOE_Q2_BF16 ? 1 : 0, out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

static int mq_quantize_launch(const float *w, int64_t rows, int64_t k, void *blocks_out, void *stream, bool q4) {
    if (rows < 0 || k < 0 || k % MQ_QK) return MOE_Q2_EINVAL;
    if (k > 0 && rows > INT64_MAX / k) return MOE_Q2_EINVAL;
    const int64_t n_blocks = rows * (k / MQ_QK);
    if (n_blocks > 0 && (w == nullptr || blocks_out == nullptr)) return MOE_Q2_EINVAL;
    if (((uintptr_t)w & 15) != 0) return MOE_Q2_EINVAL;
    if (n_blocks == 0) return MOE_Q2_OK;
    const int64_t wgs = (n_blocks + 3) / 4;
    if (wgs > 0x7FFFFFFF) return MOE_Q2_EUNSUPPORTED;
    if (q4)
        hipLaunchKernelGGL(k_quantize_q4, dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream, w, n_blocks,
                           (uint8_t *)blocks_out);
    else
        hipLaunchKernelGGL(k_quantize, dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream, w, n_blocks,
                           (uint8_t *)blocks_out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

extern "C" int moe_q2_quantize(const float *w, int64_t rows, int64_t k, void *blocks_out, void *stream) {
    return mq_quantize_launch(w, rows, k, blocks_out, stream, false);
}

extern "C" int moe_q2_quantize_q4(const float *w, int64_t rows, int64_t k, void *blocks_out, void *stream) {
    return mq_quantize_launch(w, rows, k, blocks_out, stream, true);
}

// Tiled expert layout: out block o of the gate/up part is (tile t, column b, slot s)
// with o = (t * nbh + b) * 64 + s; slot s < 32 is gate row 32t + s, else up row
// 32t + s - 32.  Down part: o = (t * nbi + b) * 64 + s, row 64t + s.  Blocks of the
// gate/up part are bg dwords, of the down part bd dwords (21: 2-bit, 37: 4-bit).
__global__ void k_pack_expert(const uint32_t *__restrict__ gate, const uint32_t *__restrict__ up,
                              const uint32_t *__restrict__ down, int H, int I, int bg, int bd,
                              uint32_t *__restrict__ out) {
    const int nbh = H / MQ_QK, nbi = I / MQ_QK;
    const int64_t ngu = (int64_t)2 * I * nbh, ndn = (int64_t)H * nbi;
    const int64_t ndw_gu = ngu * bg, ndw = ndw_gu + ndn * bd;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < ndw;
         w += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t *src;
        int64_t sblk;
        int k, bdw;
        if (w < ndw_gu) {
            const int64_t o = w / bg;
            k = (int)(w - o * bg);
            bdw = bg;
            const int64_t s = o & 63, tb = o >> 6;
            const int64_t t = tb / nbh, b = tb - t * nbh;
            const int64_t row = 32 * t + (s & 31);
            src = s < 32 ? gate : up;
            sblk = row * nbh + b;
        } else {
            const int64_t od = (w - ndw_gu) / bd;
            k = (int)(w - ndw_gu - od * bd);
            bdw = bd;
            const int64_t s = od & 63, tb = od >> 6;
            const int64_t t = tb / nbi, b = tb - t * nbi;
            src = down;
            sblk = (64 * t + s) * nbi + b;
        }
        out[w] = src[sblk * bdw + k];
    }
}

extern "C" int moe_q2_pack_expert(const void *gate, const void *up, const void *down, const moe_q2_shape *s,
                                  void *out, void *stream) {
    if (!gate || !up || !down || !out || !s) return MOE_Q2_EINVAL;
    const int hidden = s->hidden, inter = s->inter;
    if (hidden <= 0 || hidden % 256 || inter <= 0 || inter % 256) return MOE_Q2_EUNSUPPORTED;
    if (((uintptr_t)gate | (uintptr_t)up | (uintptr_t)down | (uintptr_t)out) & 3) return MOE_Q2_EINVAL;
    const int bg = (s->flags & MOE_Q2_GU_Q4) ? MQ_BD4 : MQ_BD2, bd = (s->flags & MOE_Q2_DOWN_Q4) ? MQ_BD4 : MQ_BD2;
    const int64_t nb = (int64_t)hidden / MQ_QK * inter;
    const int64_t ndw = 2 * nb * bg + nb * bd;
    int64_t grid = (ndw + 255) / 256;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(k_pack_expert, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint32_t *)gate, (const uint32_t *)up, (const uint32_t *)down, hidden, inter, bg, bd,
                       (uint32_t *)out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
