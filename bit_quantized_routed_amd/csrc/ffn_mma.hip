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
// pairs), A = hi and A = lo digits.  The min term is a 16-long product per block
// of m_j (exact in bf16) with A_j split into two bf16 planes, both planes in one
// K = 32 product on v_mfma_f32_16x16x32_bf16 (the planes as the two halves of K, m_j
// repeated).  Each block then folds d and dmin into an fp32 accumulator.
//
// MFMA roles: M = 16 of the unit's tokens (one fragment), N = 16 weight rows,
// K = the reduction dimension.  Operand byte order inside a lane's 16-byte K slice
// follows the code dword: byte b of dword s is weight 4b + s of the group (the
// activation digits are stored in the same order).
//
// Two weight codecs share the arithmetic (the block's dwords: scale/min bytes 0..3,
// codes, d|dmin last): the 2-bit block of 21 dwords (q in 0..3, sc_j 4 bits, one code
// dword per group) and its 4-bit sibling of 37 dwords (q in 0..15, sc_j 3 bits so
// that q*sc <= 105 stays an int8; two code dwords per group: byte b of the first
// holds elements 4b (low nibble) and 4b + 1, of the second 4b + 2 and 4b + 3, so the
// expanded operands keep the byte order above).  Two activation formats: two int8
// digits of 15-bit values (ND = 2) or one int8 digit (Q8, ND = 1), in which case the
// hi chains are absent.
//
// The decode kernel (k_q2_mma) and the prefill kernel (k_q2_mma_pf) differ in
// how they tile tokens and stage operands; both are described at their
// definitions below.
#include "common.h"
#include <hip/hip_ext.h>
#include <type_traits>
#include "kernels.h"
#include "prep_rows.h"
#include "topk_dev.h"
#include "timeline.h"

typedef int32_t mq_i32x4 __attribute__((ext_vector_type(4)));
typedef short mq_s16x4 __attribute__((ext_vector_type(4)));

// A launch whose start and end, when timing events are given, are recorded by the
// kernel's own dispatch (hipExtLaunchKernelGGL), so their difference is the kernel's
// duration with no extra packets around it; without events a plain launch.  Under
// stream capture the events are recorded around a plain launch instead.
static bool mq_capturing(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}
#define MQ_LAUNCH_TIMED(ev0, ev1, kernel, grid, block, shm, stream, ...)                       \
    do {                                                                                       \
        if (((ev0) || (ev1)) && !mq_capturing(stream)) {                                       \
            hipExtLaunchKernelGGL(kernel, grid, block, shm, stream, ev0, ev1, 0, __VA_ARGS__); \
        } else {                                                                               \
            hipError_t e_ = (ev0) ? hipEventRecord(ev0, stream) : hipSuccess;                \
            if (e_ != hipSuccess) return mq_fail_hip(e_);                                      \
            hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);                 \
            e_ = (ev1) ? hipEventRecord(ev1, stream) : hipSuccess;                             \
            if (e_ != hipSuccess) return mq_fail_hip(e_);                                      \
        }                                                                                      \
    } while (0)

// Nothing to launch: the timing events still get recorded (an empty interval).
static int mq_mark_empty(hipEvent_t ev0, hipEvent_t ev1, hipStream_t st) {
    hipError_t e = ev0 ? hipEventRecord(ev0, st) : hipSuccess;
    if (e == hipSuccess && ev1) e = hipEventRecord(ev1, st);
    return e == hipSuccess ? MOE_Q2_OK : mq_fail_hip(e);
}

// q*sc for the 16 weights of one group: dword s holds weights s, s+4, s+8, s+12.
// Every byte product is at most 3 * 15, so one packed 16-bit multiply (the scale
// broadcast to both halves by the operand select) scales four bytes without carries.
typedef uint16_t mq_u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int32_t mq_mul_bytes(uint32_t x, uint16_t sc) {
    // both 16-bit halves times the same scalar (a broadcast operand, no splat op)
    return __builtin_bit_cast(int32_t, __builtin_bit_cast(mq_u16x2, x) * (mq_u16x2){sc, sc});
}

__device__ __forceinline__ mq_i32x4 mq_codes_x_scale(uint32_t cw, uint32_t sc) {
    const uint16_t s = (uint16_t)sc;
    mq_i32x4 b;
    b[0] = mq_mul_bytes(cw & 0x03030303u, s);
    b[1] = mq_mul_bytes((cw >> 2) & 0x03030303u, s);
    b[2] = mq_mul_bytes((cw >> 4) & 0x03030303u, s);
    b[3] = mq_mul_bytes((cw >> 6) & 0x03030303u, s);
    return b;
}

// q*sc of the 4-bit codec: code dwords c0 (elements 4b, 4b + 1 in byte b) and c1
// (4b + 2, 4b + 3); every byte product is at most 15 * 7.
__device__ __forceinline__ mq_i32x4 mq_codes4_x_scale(uint32_t c0, uint32_t c1, uint32_t sc) {
    const uint16_t s = (uint16_t)sc;
    mq_i32x4 b;
    b[0] = mq_mul_bytes(c0 & 0x0F0F0F0Fu, s);
    b[1] = mq_mul_bytes((c0 >> 4) & 0x0F0F0F0Fu, s);
    b[2] = mq_mul_bytes(c1 & 0x0F0F0F0Fu, s);
    b[3] = mq_mul_bytes((c1 >> 4) & 0x0F0F0F0Fu, s);
    return b;
}

// q*sc operand of group g (g = 4 kk + q4) of the block at `blk` (BD dwords).
template <int BD>
__device__ __forceinline__ mq_i32x4 mq_group_operand(const uint32_t *blk, int g, int kk, int q4) {
    if constexpr (BD == MQ_BD2) {
        return mq_codes_x_scale(blk[4 + g], __builtin_amdgcn_ubfe(blk[kk], 8 * q4, 4));
    } else {
        return mq_codes4_x_scale(blk[4 + 2 * g], blk[5 + 2 * g], __builtin_amdgcn_ubfe(blk[kk], 8 * q4, 3));
    }
}

// m_j of 4 consecutive groups (one scale dword) as 4 bf16 (exact small integers).
__device__ __forceinline__ mq_s16x4 mq_mins_bf16(uint32_t swd) {
    uint32_t m = (swd >> 4) & 0x0F0F0F0Fu;
    // m kept whole (opaque to the combiner, which would otherwise turn each byte into
    // its own 4-bit field extract): the byte conversions then read its bytes directly
    asm("" : "+v"(m));
    mq_s16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (short)(__float_as_uint((float)((m >> (8 * i)) & 0xFFu)) >> 16);
    return r;
}

typedef __bf16 mq_bf16x8 __attribute__((ext_vector_type(8)));

// The min-term sums of one block for a lane's token and row: sums = the lane's group
// sums of 4 groups as two bf16 planes (hi in elements 0..3, lo in 4..7), bm = m_j of
// the same 4 groups; each m_j meets both planes of its group, all 16 groups over the
// lanes' K slices, in one K = 32 product.
__device__ __forceinline__ mq_f32x4 mq_min_term(mq_u32x4 sums, mq_s16x4 bm) {
    const uint2 b = __builtin_bit_cast(uint2, bm);
    const mq_u32x4 bb = {b.x, b.y, b.x, b.y};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mq_bf16x8, sums),
                                                  __builtin_bit_cast(mq_bf16x8, bb),
                                                  (mq_f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// One block column of a 64-row tile is 64 * 4 * BD contiguous bytes = 16 BD uint4
// (2-bit: 5376 bytes, 336 uint4; 4-bit: 9472 bytes, 592 uint4); a wave moves it with
// NLD = ceil(BD / 4) 16-byte loads per lane.  The last load of the lanes past the end
// repeats the last uint4 and lands in padding (the LDS slice holds 64 NLD uint4), so
// no load or store is predicated.
template <int BD>
struct mq_bcol {
    static constexpr int NLD = (BD + 3) / 4, N = 16 * BD;
    mq_u32x4 v[NLD];
};

// The loads name the global address space: a generic (flat) load also counts against
// the LDS counter, so every LDS wait of the column would wait for this prefetch of
// the next column too.  (Expert bytes are device memory or pinned host memory, both
// global.)  They are non-temporal: a weight column is read once per work-group, so it
// should not displace the activation operands and partial sums that other work-groups
// re-read from the caches.
template <int BD>
__device__ __forceinline__ void mq_bcol_load(const mq_u32x4 *__restrict__ src_, int lane, mq_bcol<BD> &c) {
    typedef const __attribute__((address_space(1))) mq_u32x4 *gvec;
    const gvec src = (gvec)src_;
    constexpr int NLD = mq_bcol<BD>::NLD;
#pragma unroll
    for (int i = 0; i < NLD - 1; ++i) c.v[i] = __builtin_nontemporal_load(&src[lane + 64 * i]);
    c.v[NLD - 1] = __builtin_nontemporal_load(&src[min(lane + 64 * (NLD - 1), mq_bcol<BD>::N - 1)]);
}

template <int BD>
__device__ __forceinline__ void mq_bcol_store(mq_u32x4 *__restrict__ dst, int lane, const mq_bcol<BD> &c) {
#pragma unroll
    for (int i = 0; i < mq_bcol<BD>::NLD; ++i) dst[lane + 64 * i] = c.v[i];
}

// Activation operands of one block column for one MFMA lane (token l % 16, group
// quad q4 = l / 16): digits of groups 4kk + q4 (hi, lo; lo only for one digit) and
// the two bf16 planes of the group sums 4q4 .. 4q4+3 (hi plane in the first two
// dwords of s, lo plane in the last two).
struct mq_acol { mq_i32x4 hi[4], lo[4]; mq_u32x4 s; };

// One 64-row block column from the wave's LDS slice into the 4 N fragments:
// integer products of the activation digits on the i8 matrix cores, the min
// term on the bf16 matrix cores, and the per-block fold with d and dmin -- of all
// 4 of each lane's token rows, or (one = true, a wave-uniform flag: a unit of one
// slot) only of the first, the others being padding whose sums are never stored.
template <int ND, int BD>
__device__ __forceinline__ void mq_mma_column(const uint32_t *__restrict__ my, int r16, int q4,
                                              const mq_acol &a, mq_f32x4 (&tot)[4], bool one) {
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
        const uint32_t *blk = my + (16 * nf + r16) * BD;
        mq_i32x4 ih = {0, 0, 0, 0}, il = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const mq_i32x4 b = mq_group_operand<BD>(blk, 4 * kk + q4, kk, q4);
            if (ND == 2) ih = __builtin_amdgcn_mfma_i32_16x16x64_i8(a.hi[kk], b, ih, 0, 0, 0);
            il = __builtin_amdgcn_mfma_i32_16x16x64_i8(a.lo[kk], b, il, 0, 0, 0);
        }
        const mq_f32x4 am = mq_min_term(a.s, mq_mins_bf16(blk[q4]));
        const uint32_t dd = blk[BD - 1];
        const float d = mq_h2f((uint16_t)(dd & 0xFFFFu));
        const float dmin = mq_h2f((uint16_t)(dd >> 16));
        tot[nf][0] = fmaf(d, (float)(ND == 2 ? (ih[0] << 8) + il[0] : il[0]), fmaf(-dmin, am[0], tot[nf][0]));
        if (!one) {
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                const float qv = (float)(ND == 2 ? (ih[i] << 8) + il[i] : il[i]);
                tot[nf][i] = fmaf(d, qv, fmaf(-dmin, am[i], tot[nf][i]));
            }
        }
    }
}

// Work unit = (touched expert's unit of up to 16 slots, group of 4 consecutive row
// tiles, k-split s).  Wave w streams tile 4g + w -- 64 rows, all 4 N fragments --
// over block columns [s * cps, (s + 1) * cps) and owns those rows' sums, so no
// reduction across waves is needed; the 4 waves step through the columns
// together and share one copy of each column's activation operands (16 tokens x
// 16 groups: two 16-byte digit vectors per lane and MFMA step, plus the group-sum
// planes), which the work-group loads cooperatively into LDS already arranged in
// MFMA lane order (one 16-byte LDS read per operand, lane-contiguous).  A wave's
// weight column (5376 contiguous bytes) goes through registers into its private
// LDS slice.  Both are prefetched one column ahead; the activation buffer is
// double-buffered, so one barrier per column suffices.
//
// Outputs are per-split partial sums, scaled by the token's activation scale:
//   GU  : gate rows -> out0[s][slot][row], up rows -> out1[s][slot][row]
//   down: out0[s][slot][row]
// Padding tokens (beyond the unit's count) read the all-zero activation row zrow
// and write to the discard row trash_row.
#define DM_AITEMS(ND) (256 * (ND) + 64)   // digit vectors + 64 sum vectors per column

// ------------------------------------------------------------------ dense rows
// The shared expert's bf16 rows for up to 255 tokens, in the same launch as the
// routed experts (work-groups appended to the grid), so the two overlap without a
// second stream.  Work-group = (block of 4 * 16 NF rows, k-split); wave w takes
// rows 16 NF w .. +16 NF - 1 of the block over the split's k range in steps of 32
// on v_mfma_f32_16x16x32_bf16 (B: 16 bytes of a weight row per lane, A: 16 bytes
// of a token row; with A2 also the token row's low bf16 plane), tokens in chunks
// of up to 64 (MF fragments of 16).  Operands come straight from global memory,
// two k-steps in flight (register ping-pong, unconditional clamped loads).  Token
// rows beyond T read row T - 1 and are never stored.  Outputs are per-split
// partial sums: row r < half -> out0[s][t][r], else out1[s][t][r - half].
struct MqDense {
    const uint16_t *w;       // [rows][K] bf16, row-major
    const uint16_t *x;       // [T][K] bf16
    const uint16_t *xlo;     // [T][K] bf16 low plane (A2) or null
    float *out0, *out1;
    int T, rows, K, half, nsplit, kps, out_ld, grid;
    int64_t split_stride;
};

// XL: the activation planes come from LDS (xl: hi plane of the one token over
// [k0, k1), the lo plane after it) instead of global memory.
template <int NF, int MF, bool A2, bool XL>
__device__ __forceinline__ void mq_dense_chunk(const MqDense &d, int row0, int k0, int k1, int t0, int ks,
                                               int lane, const uint16_t *xl) {
    typedef const __attribute__((address_space(1))) mq_u32x4 *gvec;
    typedef const __attribute__((address_space(1))) char *gbyte;
    const int r16 = lane & 15, q4 = lane >> 4;
    // per-lane 32-bit byte offsets from uniform bases (scalar base + vector offset
    // addressing; nothing per stage is kept in vector registers)
    uint32_t wo[NF], xo[MF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) wo[nf] = (uint32_t)(((row0 + 16 * nf + r16) * d.K + 8 * q4) * 2);
#pragma unroll
    for (int m = 0; m < MF; ++m) {
        const int tok = min(t0 + 16 * m + r16, d.T - 1);
        xo[m] = (uint32_t)((tok * d.K + 8 * q4) * 2);
    }
    mq_f32x4 acc[NF][MF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int m = 0; m < MF; ++m) acc[nf][m] = (mq_f32x4){0.f, 0.f, 0.f, 0.f};
    // ring of D stages of 32 k each in registers: loads run D stages ahead of the
    // multiplies (deep enough that the weight stream is not latency-bound at one
    // work-group per compute unit); D is what about 130 registers hold next to the
    // accumulators, so the kernel keeps the occupancy of its routed path
    constexpr int PER = NF + MF * (A2 ? 2 : 1);
    constexpr int DR = (130 - 4 * NF * MF) / (4 * PER);
    constexpr int D = DR > 8 ? 8 : (DR < 2 ? 2 : DR);
    mq_u32x4 b[D][NF], a[D][MF], l[D][MF];
    // an opaque copy of the weight base: the stage addresses are then formed here,
    // not hoisted out of the token-chunk loop into registers held across it
    const uint16_t *wbase = d.w;
    asm volatile("" : "+s"(wbase));
    auto load = [&](int s, int k) {
        const gbyte wb = (gbyte)(wbase + k), xb = (gbyte)(d.x + k), lb = (gbyte)((A2 ? d.xlo : d.x) + k);
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) b[s][nf] = *(gvec)(wb + wo[nf]);
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            if (XL) {
                const uint16_t *xp = xl + (k - k0) + 8 * q4;
                a[s][m] = *(const mq_u32x4 *)xp;
                if (A2) l[s][m] = *(const mq_u32x4 *)(xp + (k1 - k0));
            } else {
                a[s][m] = *(gvec)(xb + xo[m]);
                if (A2) l[s][m] = *(gvec)(lb + xo[m]);
            }
        }
    };
    auto mma = [&](int s) {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
            for (int m = 0; m < MF; ++m) {
                acc[nf][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mq_bf16x8, a[s][m]),
                                                                     __builtin_bit_cast(mq_bf16x8, b[s][nf]),
                                                                     acc[nf][m], 0, 0, 0);
                if (A2)
                    acc[nf][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mq_bf16x8, l[s][m]),
                                                                         __builtin_bit_cast(mq_bf16x8, b[s][nf]),
                                                                         acc[nf][m], 0, 0, 0);
            }
    };
    // stage j covers k0 + 32 j; slot s holds stage i + s of the block starting at i.
    // Loads past the last stage are clamped to it (in bounds; those slots are not
    // multiplied), so every load is unconditional.
    const int nst = (k1 - k0) >> 5;
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, k0 + 32 * min(s, nst - 1));
    int i = 0;
    for (; i + D < nst; i += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            mma(s);
            load(s, k0 + 32 * min(i + D + s, nst - 1));
            // keep each slot's reload after its multiply: the slot's registers are reused
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // last block: the slots past the last stage multiply a zero activation
#pragma unroll
    for (int s = 0; s < D; ++s) {
        const bool live = s < nst - i;
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            a[s][m] = live ? a[s][m] : (mq_u32x4){0u, 0u, 0u, 0u};
            if (A2) l[s][m] = live ? l[s][m] : (mq_u32x4){0u, 0u, 0u, 0u};
        }
        mma(s);
    }
    // D layout: lane l, element i -> token 4*(l/16) + i of fragment m, row 16*nf + l%16
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * m + 4 * q4 + i;
            if (t < d.T) {
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                    const int r = row0 + 16 * nf + r16;
                    float *o = r < d.half ? d.out0 + (int64_t)ks * d.split_stride + (int64_t)t * d.out_ld + r
                                          : d.out1 + (int64_t)ks * d.split_stride + (int64_t)t * d.out_ld +
                                                (r - d.half);
                    *o = acc[nf][m][i];
                }
            }
        }
}

template <int NF, bool A2>
__device__ __forceinline__ void mq_dense_wg(const MqDense &d, int wg, int wv, int lane) {
    const int rblocks = d.rows / (64 * NF);
    const int rb = wg % rblocks, ks = wg / rblocks;
    const int k0 = ks * d.kps, k1 = min(d.K, k0 + d.kps);
    if (k0 >= k1) return;
    const int row0 = rb * 64 * NF + wv * 16 * NF;
    for (int t0 = 0; t0 < d.T; t0 += 64) {
        const int nt = d.T - t0;
        if (nt > 48)
            mq_dense_chunk<NF, 4, A2, false>(d, row0, k0, k1, t0, ks, lane, nullptr);
        else if (nt > 32)
            mq_dense_chunk<NF, 3, A2, false>(d, row0, k0, k1, t0, ks, lane, nullptr);
        else if (nt > 16)
            mq_dense_chunk<NF, 2, A2, false>(d, row0, k0, k1, t0, ks, lane, nullptr);
        else
            mq_dense_chunk<NF, 1, A2, false>(d, row0, k0, k1, t0, ks, lane, nullptr);
    }
}

// Shared rows of a one-token down launch: h = silu(sum_s g[s][k]) * sum_s u[s][k]
// (splits added in order, 16 loads in flight) over the work-group's k range, as
// two bf16 planes in LDS (hi = bf16(h), lo = bf16(h - hi)) -- the arithmetic of the
// digit preparation launch's shared rows -- then the dense rows read them there.
__device__ __forceinline__ void mq_dense_wg_prep(const MqDense &d, const MqDownPrep &pp, int wg, int wv,
                                                 int lane, uint16_t *hl) {
    const int rblocks = d.rows / (64 * 2);
    const int rb = wg % rblocks, ks = wg / rblocks;
    const int k0 = ks * d.kps, k1 = min(d.K, k0 + d.kps);
    if (k0 >= k1) return;
    const int n = k1 - k0, tid = threadIdx.x;
    for (int k = tid; k < n; k += 256) {
        float g = 0.0f, u = 0.0f;
        for (int sp0 = 0; sp0 < pp.snsplit; sp0 += 16) {
            float gv[16], uv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t so = (int64_t)min(sp0 + j, pp.snsplit - 1) * pp.sstride + k0 + k;
                gv[j] = pp.sg[so];
                uv[j] = pp.su[so];
            }
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (sp0 + j < pp.snsplit) {
                    g += gv[j];
                    u += uv[j];
                }
        }
        const float h = g / (1.0f + expf(-g)) * u;
        const uint16_t hb = mq_f32_to_bf16(h);
        hl[k] = hb;
        hl[n + k] = mq_f32_to_bf16(h - mq_bf16_to_f32(hb));
    }
    __syncthreads();
    mq_dense_chunk<2, 1, true, true>(d, rb * 128 + wv * 32, k0, k1, 0, ks, lane, hl);
}

// The slot row `row` of a one-token down launch: h = silu(sum_s g[s][row]) *
// sum_s u[s][row] (splits in order), its power-of-two scale, digits and group sums,
// laid out as one row of the digit preparation's output (xr: [group][digit] 16-byte
// vectors, xs: [block][quad][plane][4] bf16), the same arithmetic.  Thread i takes
// elements 8 i .. 8 i + 7 (half a group; the two halves are joined by a lane swap).
template <int ND>
__device__ __forceinline__ void mq_row_prep_lds(const MqDownPrep &pp, int row, mq_u32x4 *xr, uint16_t *xs,
                                                float *rsc, float *wmax, int tid) {
    const int G = pp.len / 16;
    const int e0 = 8 * tid;
    const bool on = e0 < pp.len;
    float v[8];
    {
        float gs[8], us[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { gs[i] = 0.0f; us[i] = 0.0f; }
        for (int sp = 0; sp < pp.nsplit; sp += 4) {
            float4 a[4][2], b[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t off = (int64_t)min(sp + j, pp.nsplit - 1) * pp.split_stride + (int64_t)row * pp.len +
                                    min(e0, pp.len - 8);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    a[j][i] = ((const float4 *)(pp.g + off))[i];
                    b[j][i] = ((const float4 *)(pp.u + off))[i];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (sp + j < pp.nsplit) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        gs[4 * i] += a[j][i].x; gs[4 * i + 1] += a[j][i].y;
                        gs[4 * i + 2] += a[j][i].z; gs[4 * i + 3] += a[j][i].w;
                        us[4 * i] += b[j][i].x; us[4 * i + 1] += b[j][i].y;
                        us[4 * i + 2] += b[j][i].z; us[4 * i + 3] += b[j][i].w;
                    }
                }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = on ? gs[i] / (1.0f + expf(-gs[i])) * us[i] : 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = mq_wave_max(amax);
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    int ex = 0;
    if (amax > 0.0f) frexpf(amax, &ex);
    const float inv_s = amax > 0.0f ? ldexpf(1.0f, MQ_ACT_BITS(ND) - ex) : 1.0f;
    if (tid == 0) *rsc = amax > 0.0f ? ldexpf(1.0f, ex - MQ_ACT_BITS(ND)) : 1.0f;
    // this half group's bytes of the digit dwords: dword s4 holds the digits of the
    // elements 4 b + s4 of the group, so elements 0..7 fill bytes 0, 1 and elements
    // 8..15 bytes 2, 3 of every dword
    const int half = tid & 1, g = tid >> 1;
    uint32_t hp[4], lp[4];
    int sum = 0;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        uint32_t h = 0, l = 0;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int x = mq_quant_act<ND>(v[4 * b + s4] * 1.0f, inv_s);
            sum += x;
            const int dh = ND == 2 ? (x + 128) >> 8 : 0;
            const int dl = x - (dh << 8);
            h |= ((uint32_t)(dh & 0xFF)) << (8 * (2 * half + b));
            l |= ((uint32_t)(dl & 0xFF)) << (8 * (2 * half + b));
        }
        hp[s4] = h;
        lp[s4] = l;
    }
    mq_u32x4 hi, lo;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        hi[s4] = hp[s4] | (uint32_t)__shfl_xor((int)hp[s4], 1, 64);
        lo[s4] = lp[s4] | (uint32_t)__shfl_xor((int)lp[s4], 1, 64);
    }
    sum += __shfl_xor(sum, 1, 64);
    if (on && half == 0 && g < G) {
        if (ND == 2) {
            xr[2 * g] = hi;
            xr[2 * g + 1] = lo;
        } else {
            xr[g] = lo;
        }
        const float fs = (float)sum;                           // exact: |sum| <= 2^18
        const uint16_t bh = mq_f32_to_bf16(fs);
        const uint16_t bl = mq_f32_to_bf16(fs - mq_bf16_to_f32(bh));
        const int blk = g >> 4, j = g & 15;
        xs[blk * 32 + (j >> 2) * 8 + (j & 3)] = bh;
        xs[blk * 32 + (j >> 2) * 8 + 4 + (j & 3)] = bl;
    }
    __syncthreads();
}

// Rows per work-group of the dense path and its k-split: about 256 work-groups.
void mq_dense_split(int rows, int K, int nf, int *nsplit, int *kps) {
    const int rblocks = rows / (64 * nf);
    int s = 256 / (rblocks > 0 ? rblocks : 1);
    if (s > K / 64) s = K / 64;
    if (s < 1) s = 1;
    int k = (K + s - 1) / s;
    k = (k + 63) / 64 * 64;
    *kps = k;
    *nsplit = (K + k - 1) / k;
}

// LDS of the in-launch routing (it aliases the weight slices, which are not in use
// until the routing is done)
struct MqRouteLds {
    MqTopkLds L;
    int sidx[MQ_TOPK_BUCKET_MAX_T * 16];
    int soff[MQ_ROUTE_MAX_E], sun[MQ_ROUTE_MAX_E], scnt[MQ_ROUTE_MAX_E];
    int sU;
    int4 unit;
    int rows[MMA_TCH];
};

// Unit u of the batch -- (expert, first bucket position, slot count, chunk of the
// expert's slots) -- and, for threads below 16, the token of its slot tid (the zero
// row past the count): the batch's top-K selection and bucketing done in LDS by the
// same functions as the top-K + bucketing launch.  Work-group 0 also writes the
// routing outputs.  256 threads.
__device__ __forceinline__ int4 mq_route_unit(const MqRoute &rt, int u, MqRouteLds &R, int tid, int &urv) {
    const bool w0 = blockIdx.x == 0;
    const int S = rt.T * rt.K;
    if (rt.T == 1 && !w0) {
        // one token: every selected expert is a unit of one slot, in expert order, so
        // unit u is the selection of rank u by expert index (slot u, token 0)
        mq_topk_token<256>(rt.logits, 1, rt.bias, 1, rt.E, rt.K, 0, true, tid, R.L, nullptr, nullptr, nullptr,
                           nullptr);
        if (tid == 0) R.unit = make_int4(0, 0, 0, 0);
        __syncthreads();
        if (tid < rt.K) {
            const int e = R.L.se[tid];
            int r = 0;
            for (int q = 0; q < rt.K; ++q) r += R.L.se[q] < e ? 1 : 0;
            if (r == u) R.unit = make_int4(e, u, 1, 0);
        }
        __syncthreads();
        urv = tid == 0 ? 0 : rt.zrow;
        return R.unit;
    }
    for (int t = 0; t < rt.T; ++t) {
        mq_topk_token<256>(rt.logits, 1, rt.bias, rt.T, rt.E, rt.K, t, true, tid, R.L, w0 ? rt.idx : nullptr,
                           w0 ? rt.gate : nullptr, w0 ? rt.trace_idx : nullptr, w0 ? rt.trace_w : nullptr);
        // the selection of token t is final here; the next token's first writes to
        // it come two barriers later
        if (tid < rt.K) R.sidx[t * rt.K + tid] = R.L.se[tid];
    }
    __syncthreads();
    mq_bucket_small_wg<256>(R.sidx, S, rt.E, MMA_TCH, w0, rt.counts, rt.offsets, rt.perm, rt.inv, rt.units_hdr,
                            rt.units, rt.fill_units, rt.urow, rt.K, rt.zrow, R.soff, R.sun, R.scnt, &R.sU);
    if (tid == 0) R.unit = make_int4(0, 0, 0, 0);
    __syncthreads();
    if (tid < rt.E) {
        const int c = R.scnt[tid], u0 = R.sun[tid];
        if (u >= u0 && u < u0 + (c + MMA_TCH - 1) / MMA_TCH) {
            const int k = u - u0;
            R.unit = make_int4(tid, R.soff[tid] + MMA_TCH * k, min(MMA_TCH, c - MMA_TCH * k), k);
        }
    }
    __syncthreads();
    const int4 un = R.unit;
    if (tid < S && un.z > 0 && R.sidx[tid] == un.x) {    // slots of the unit's expert, in slot order
        int r = 0;
        for (int q = 0; q < tid; ++q) r += R.sidx[q] == un.x ? 1 : 0;
        r -= MMA_TCH * un.w;
        if (r >= 0 && r < MMA_TCH) R.rows[r] = tid / rt.K;
    }
    __syncthreads();
    urv = tid < un.z ? R.rows[tid] : rt.zrow;
    return un;
}

template <bool GU, int ND, int BD, bool MERGE>
__global__ void __launch_bounds__(256, MERGE && BD == MQ_BD2 ? 3 : 1) k_q2_mma(const uint8_t *__restrict__ experts, int64_t expert_bytes,
                                                int64_t mat_off, int tiles, int kblocks, int nsplit,
                                                int cps, int seg, const int4 *__restrict__ units,
                                                const int32_t *__restrict__ urow, int zrow,
                                                int trash_row, const mq_u32x4 *__restrict__ xdig,
                                                const uint32_t *__restrict__ xsum,
                                                const float *__restrict__ xscale, float *__restrict__ out0,
                                                float *__restrict__ out1, int out_ld, int64_t split_stride,
                                                int q2_grid, const MqDense dn, const MqRoute rt,
                                                int route_on, const MqDownPrep pp, int prep_on,
                                                const uint64_t *__restrict__ eptr) {
    constexpr int NLD = mq_bcol<BD>::NLD, NA = DM_AITEMS(ND), NIT = (NA + 255) / 256;
    __shared__ __attribute__((aligned(16))) mq_u32x4 sW[4][64 * NLD];      // weight slices, one per wave
    static_assert(sizeof(MqRouteLds) <= sizeof(sW), "routing LDS fits the weight slices");
    static_assert(MQ_DOWN_PREP_SHARED_BYTES <= sizeof(sW), "shared SwiGLU planes fit the weight slices");
    __shared__ __attribute__((aligned(16))) mq_u32x4 sA[2][NA];            // activation operands
    __shared__ int s_row[16];
    __shared__ float s_sc[16];
    // one-token down launch: the unit's activation row prepared here
    __shared__ __attribute__((aligned(16))) mq_u32x4 s_xr[ND * MQ_DOWN_PREP_MAX_LEN / 16];
    __shared__ __attribute__((aligned(16))) uint16_t s_xs[MQ_DOWN_PREP_MAX_LEN / 256 * 32];
    __shared__ float s_rsc, s_wmax[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, q4 = lane >> 4;
    MQ_TL(GU, 0, mq_tl_now());
    MQ_TL(GU, 3, mq_tl_hw());
    if ((int)blockIdx.x >= q2_grid) {
        // appended work-groups: the shared expert's dense rows
        MQ_TL(GU, 4, 1);
        if (GU)
            mq_dense_wg<4, false>(dn, (int)blockIdx.x - q2_grid, wv, lane);
        else if (prep_on)
            mq_dense_wg_prep(dn, pp, (int)blockIdx.x - q2_grid, wv, lane, (uint16_t *)&sW[0][0]);
        else
            mq_dense_wg<2, true>(dn, (int)blockIdx.x - q2_grid, wv, lane);
        MQ_TL_END(GU);
        return;
    }
    const int groups = tiles >> 2;
    const int tg = blockIdx.x % groups;
    const int rest = blockIdx.x / groups;
    const int ks = rest % nsplit, u = rest / nsplit;
    const int c0 = ks * cps, c1 = min(kblocks, c0 + cps);
    MQ_TL_NO_WORK(GU, c0 >= c1);
    if (c0 >= c1) return;
    // the unit and (gate/up) its row table: routed here, or two independent loads
    // (nothing else waits on global memory before the first activation loads)
    int4 un;
    int urv = 0;
    if (GU && route_on) {
        un = mq_route_unit(rt, u, *reinterpret_cast<MqRouteLds *>(&sW[0][0]), tid, urv);
    } else {
        un = units[u];
        urv = GU && tid < 16 ? urow[(int64_t)u * 16 + tid] : 0;
    }
    const int p0 = un.y, nt = un.z;
    MQ_TL_NO_WORK(GU, nt == 0);
    if (nt == 0) return;                                 // past the last unit
    // the expert's bytes: resident, or where an expert cache's plan put it
    const uint8_t *eb = eptr ? (const uint8_t *)eptr[un.x] : experts + (int64_t)un.x * expert_bytes;
    const int tile = 4 * tg + wv;
    const int G = kblocks * 16;
    const int64_t tile_bytes = (int64_t)kblocks * 64 * BD * 4;
    const mq_u32x4 *tb = (const mq_u32x4 *)(eb + mat_off + (int64_t)tile * tile_bytes);
    mq_bcol<BD> wb;
    mq_bcol_load<BD>(tb + (int64_t)c0 * (16 * BD), lane, wb);   // weights first: needs only the unit
    const bool lrow = !GU && prep_on;                    // activations from the row prepared here
    if (lrow) mq_row_prep_lds<ND>(pp, p0, s_xr, s_xs, &s_rsc, s_wmax, tid);
    float scv = 0.0f;                                    // row scale, to LDS in the loop
    if (tid < 16) {
        const int ar = tid < nt ? (GU ? urv : p0 + tid) : zrow;
        s_row[tid] = ar;
        scv = lrow ? (tid < nt ? s_rsc : 1.0f) : xscale[ar];
    }
    __syncthreads();
    // this thread's activation items (NIT), one per LDS slot so that a wave's
    // stores are lane-contiguous (the last ones clamped: duplicate writes of
    // identical data).  Slot i < 256 ND = (kk * ND + digit) * 64 + lane holds the digit
    // vector of MFMA step kk for lane (token l % 16, group 4 kk + l / 16); slot
    // 256 ND + l the group-sum vector of lane l (token l % 16, quad l / 16).
    // global address space stated explicitly: a generic (flat) load would also count
    // against the LDS counter and make every LDS wait in the column wait for it
    typedef const __attribute__((address_space(1))) mq_u32x4 *gvec;
    gvec asrc[NIT];
    const mq_u32x4 *lsrc[NIT];                           // (row prepared here) LDS source, null: zero
    int aslot[NIT], astep[NIT];
#pragma unroll
    for (int n = 0; n < NIT; ++n) {
        const int it = min(tid + 256 * n, NA - 1);
        if (it < 256 * ND) {
            const int l = it & 63, d = (it >> 6) % ND, kk = it / (64 * ND);
            const int tk = l & 15, g = 4 * kk + (l >> 4);
            asrc[n] = (gvec)(xdig + (int64_t)s_row[tk] * G * ND + g * ND + d);
            lsrc[n] = tk < nt ? s_xr + g * ND + d : nullptr;
            aslot[n] = it;
            astep[n] = 16 * ND;
        } else {
            const int l = it - 256 * ND;
            asrc[n] = (gvec)((const mq_u32x4 *)(xsum + (int64_t)s_row[l & 15] * G) + (l >> 4));
            lsrc[n] = (l & 15) < nt ? (const mq_u32x4 *)s_xs + (l >> 4) : nullptr;
            aslot[n] = it;
            astep[n] = 4;
        }
    }
    const mq_u32x4 z4 = {0u, 0u, 0u, 0u};
    auto aload = [&](int n, int c) {
        return lrow ? (lsrc[n] ? lsrc[n][c * astep[n]] : z4) : asrc[n][c * astep[n]];
    };
    mq_u32x4 ab[NIT];
#pragma unroll
    for (int n = 0; n < NIT; ++n) ab[n] = aload(n, c0);

    mq_f32x4 tot[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) tot[nf] = (mq_f32x4){0.f, 0.f, 0.f, 0.f};
    // D layout: lane l, element i -> token 4*(l/16) + i, row slot 16*nf + l%16
    auto store = [&](int kso) {
        float *o0 = out0 + (int64_t)kso * split_stride;
        float *o1 = GU ? out1 + (int64_t)kso * split_stride : nullptr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * q4 + i;
            const float sc = s_sc[t];
            const int64_t orow = (int64_t)(t < nt ? p0 + t : trash_row) * out_ld;
#pragma unroll
            for (int nf = 0; nf < 4; ++nf) {
                const float v = tot[nf][i] * sc;
                if (GU) {
                    // slots 0..31: gate rows 32*tile + slot; 32..63: up rows 32*tile + slot - 32
                    float *o = nf < 2 ? o0 : o1;
                    o[orow + 32 * tile + 16 * (nf & 1) + r16] = v;
                } else {
                    o0[orow + 64 * tile + 16 * nf + r16] = v;
                }
            }
        }
    };
    const uint32_t *myd = (const uint32_t *)sW[wv];
    const bool one = __builtin_amdgcn_readfirstlane(nt) == 1;
    int buf = 0;
    // MERGE: one work-group walks the ranges of several splits and stores each split's
    // sums, started from zero, where its range ends: the same values as one
    // work-group per split (a separate instantiation: the extra loop level costs
    // registers)
    MQ_TL(GU, 1, mq_tl_now());
    const int sl = MERGE ? seg : c1 - c0;
    for (int cs = c0; cs < c1; cs += sl) {
    const int ce = min(c1, cs + sl);
    for (int c = cs; c < ce; ++c) {
        if (tid < 16) s_sc[tid] = scv;
        mq_bcol_store<BD>(sW[wv], lane, wb);
#pragma unroll
        for (int n = 0; n < NIT; ++n) sA[buf][aslot[n]] = ab[n];
        // the registers are free again: the next column's loads go out before the
        // barrier, so its latency overlaps the wait for the other waves
        if (c + 1 < c1) {
            mq_bcol_load<BD>(tb + (int64_t)(c + 1) * (16 * BD), lane, wb);
#pragma unroll
            for (int n = 0; n < NIT; ++n) ab[n] = aload(n, c + 1);
        }
        __syncthreads();
        mq_acol a;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (ND == 2) a.hi[kk] = __builtin_bit_cast(mq_i32x4, sA[buf][(kk * 2) * 64 + lane]);
            a.lo[kk] = __builtin_bit_cast(mq_i32x4, sA[buf][(kk * ND + ND - 1) * 64 + lane]);
        }
        a.s = sA[buf][256 * ND + lane];
        mq_mma_column<ND, BD>(myd, r16, q4, a, tot, one);
        buf ^= 1;
    }
    store(MERGE ? cs / seg : ks);
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) tot[nf] = (mq_f32x4){0.f, 0.f, 0.f, 0.f};
    }
    MQ_TL_END(GU);
}
#ifdef MQ_WG_TIMELINE
__device__ unsigned long long mq_tl_buf[2][MQ_TL_MAX_WG][MQ_TL_SLOTS];

extern "C" int moe_q2_timeline_read(void *host, size_t bytes) {
    if (!host || bytes != sizeof(mq_tl_buf)) return MOE_Q2_EINVAL;
    const hipError_t e = hipMemcpyFromSymbol(host, HIP_SYMBOL(mq_tl_buf), sizeof(mq_tl_buf), 0,
                                             hipMemcpyDeviceToHost);
    return e == hipSuccess ? MOE_Q2_OK : mq_fail_hip(e);
}

extern "C" int moe_q2_timeline_clear(void) {
    static unsigned long long zero[2][MQ_TL_MAX_WG][MQ_TL_SLOTS];
    const hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(mq_tl_buf), zero, sizeof(zero), 0, hipMemcpyHostToDevice);
    return e == hipSuccess ? MOE_Q2_OK : mq_fail_hip(e);
}
#endif

// Split count along the reduction for the decode kernel: enough work-groups for
// one resident round at three per compute unit of a 256-CU device, at most
// max_split, and at least 2 block columns per split.
void mq_dec_split(int max_units, int tiles, int kblocks, int max_split, int *nsplit, int *cps) {
    const int64_t wgs = (int64_t)max_units * (tiles / 4);
    int s = (int)(768 / (wgs > 0 ? wgs : 1));
    const int smax = kblocks / 2 > 1 ? kblocks / 2 : 1;
    if (s > smax) s = smax;
    if (s > max_split) s = max_split;
    if (s < 1) s = 1;
    const int c = (kblocks + s - 1) / s;
    *cps = c;
    *nsplit = (kblocks + c - 1) / c;
}

int mq_launch_q2_mma(int gu, const MqFormat &fmt, const void *experts, int64_t expert_bytes, int64_t mat_off,
                     int tiles, int kblocks, const int4 *units, int max_units, int split_units, int max_split,
                     int merge,
                     const int32_t *urow, int zrow, int trash_row, const void *xdig,
                     const uint32_t *xsum, const float *xscale, float *out0, float *out1, int out_ld,
                     int64_t split_stride, const MqDenseSpec *dense, const MqRoute *route,
                     const MqDownPrep *prep, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (tiles % 4) return MOE_Q2_EUNSUPPORTED;
    if ((fmt.nd != 1 && fmt.nd != 2) || (fmt.bd != MQ_BD2 && fmt.bd != MQ_BD4)) return MOE_Q2_EINVAL;
    if (gu && !urow) return MOE_Q2_EINVAL;
    if (route && (!gu || route->T < 1 || route->T > MQ_TOPK_BUCKET_MAX_T || route->E > MQ_ROUTE_MAX_E ||
                  route->K > 16 || route->K < 1))
        return MOE_Q2_EINVAL;
    const MqRoute rt = route ? *route : MqRoute{};
    const int route_on = route ? 1 : 0;
    if (prep && (gu || prep->len > MQ_DOWN_PREP_MAX_LEN || prep->len != kblocks * MQ_QK || prep->nsplit < 1 ||
                 (dense && (dense->T != 1 || !prep->sg || prep->snsplit < 1))))
        return MOE_Q2_EINVAL;
    const MqDownPrep pp = prep ? *prep : MqDownPrep{};
    const int prep_on = prep ? 1 : 0;
    int nsplit = 1, cps = kblocks;
    if (max_split < 1) return MOE_Q2_EINVAL;
    mq_dec_split(split_units, tiles, kblocks, max_split, &nsplit, &cps);
    // merge: one work-group per unit and tile group walks all nsplit ranges and stores
    // each range's partial sums (the outputs of nsplit work-groups, with fewer of them)
    const int seg = cps;
    if (merge) {
        nsplit = 1;
        cps = kblocks;
    }
    const int64_t q2_grid = (int64_t)max_units * nsplit * (tiles / 4);
    MqDense dn = {};
    int64_t dgrid = 0;
    if (dense) {
        const int nf = gu ? 4 : 2;
        if (dense->rows % (64 * nf) || dense->K % 64 || dense->T < 1) return MOE_Q2_EUNSUPPORTED;
        dn.w = dense->w;
        dn.x = dense->x;
        dn.xlo = dense->xlo;
        dn.out0 = dense->out0;
        dn.out1 = dense->out1;
        dn.T = dense->T;
        dn.rows = dense->rows;
        dn.K = dense->K;
        dn.half = dense->half;
        dn.out_ld = dense->out_ld;
        dn.split_stride = dense->split_stride;
        mq_dense_split(dense->rows, dense->K, nf, &dn.nsplit, &dn.kps);
        // (the in-launch shared SwiGLU holds 2 x kps bf16 in the weight-slice LDS)
        // (the host decides the in-launch preparation against the same limit before enqueuing)
        if (prep && 4 * dn.kps > MQ_DOWN_PREP_SHARED_BYTES) return MOE_Q2_EUNSUPPORTED;
        if (dn.nsplit != dense->nsplit) return MOE_Q2_EINVAL;       // workspace sized for another split
        dgrid = (int64_t)(dense->rows / (64 * nf)) * dn.nsplit;
        dn.grid = (int)dgrid;
    }
    const int64_t grid = q2_grid + dgrid;
    if (grid <= 0) return mq_mark_empty(ev0, ev1, st);
    if (grid > 0x7fffffff) return MOE_Q2_EUNSUPPORTED;
#define MQ_Q2_MMA_LAUNCH1(GUV, NDV, BDV, MV)                                                             \
    MQ_LAUNCH_TIMED(ev0, ev1, (k_q2_mma<GUV, NDV, BDV, MV>), dim3((unsigned)grid), dim3(256), 0, st,      \
                    (const uint8_t *)experts, expert_bytes, mat_off, tiles, kblocks, nsplit, cps, seg, units, urow, \
                    zrow, trash_row, (const mq_u32x4 *)xdig, xsum, xscale, out0, out1, out_ld, split_stride,  \
                    (int)q2_grid, dn, rt, route_on, pp, prep_on, fmt.eptr)
#define MQ_Q2_MMA_LAUNCH(GUV, NDV, BDV)                                                                  \
    do {                                                                                                 \
        if (merge) MQ_Q2_MMA_LAUNCH1(GUV, NDV, BDV, true);                                              \
        else MQ_Q2_MMA_LAUNCH1(GUV, NDV, BDV, false);                                                    \
    } while (0)
    const int sel = (gu ? 4 : 0) + (fmt.nd == 2 ? 2 : 0) + (fmt.bd == MQ_BD4 ? 1 : 0);
    switch (sel) {
    case 0: MQ_Q2_MMA_LAUNCH(false, 1, MQ_BD2); break;
    case 1: MQ_Q2_MMA_LAUNCH(false, 1, MQ_BD4); break;
    case 2: MQ_Q2_MMA_LAUNCH(false, 2, MQ_BD2); break;
    case 3: MQ_Q2_MMA_LAUNCH(false, 2, MQ_BD4); break;
    case 4: MQ_Q2_MMA_LAUNCH(true, 1, MQ_BD2); break;
    case 5: MQ_Q2_MMA_LAUNCH(true, 1, MQ_BD4); break;
    case 6: MQ_Q2_MMA_LAUNCH(true, 2, MQ_BD2); break;
    default: MQ_Q2_MMA_LAUNCH(true, 2, MQ_BD4); break;
    }
#undef MQ_Q2_MMA_LAUNCH
#undef MQ_Q2_MMA_LAUNCH1
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

// ------------------------------------------------------------------ activation digits
// (row preparation in prep_rows.h)


template <int SRC, int ND>
__global__ void __launch_bounds__(256) k_prep_digits(const void *__restrict__ src,
                                                     const void *__restrict__ src2, int nsplit,
                                                     int64_t split_stride, int nrows, int len,
                                                     int64_t src_ld, mq_u32x4 *__restrict__ xdig,
                                                     uint32_t *__restrict__ xsum,
                                                     float *__restrict__ scale, const MqSharedRows sh) {
    mq_prep_digits_wg<SRC, ND>(src, src2, nsplit, split_stride, nrows, len, src_ld, xdig, xsum, scale, sh,
                               (int)blockIdx.x);
}

int mq_launch_prep_digits(const void *src, int src_bf16, int nrows, int len, int64_t src_ld,
                          void *xdig, uint32_t *xsum, float *scale, int nd, hipStream_t st) {
    if (nrows <= 0) return MOE_Q2_OK;
    if (len / 16 > 256 * PD_NG) return MOE_Q2_EUNSUPPORTED;
    dim3 grid(nrows + 1);                        // nrows rows + the zero row
#define MQ_PREP_LAUNCH(SRCV, NDV)                                                                         \
    hipLaunchKernelGGL((k_prep_digits<SRCV, NDV>), grid, dim3(256), 0, st, src, nullptr, 1, (int64_t)0, nrows, \
                       len, src_ld, (mq_u32x4 *)xdig, xsum, scale, MqSharedRows{})
    if (src_bf16) {
        if (nd == 2) MQ_PREP_LAUNCH(1, 2); else MQ_PREP_LAUNCH(1, 1);
    } else {
        if (nd == 2) MQ_PREP_LAUNCH(0, 2); else MQ_PREP_LAUNCH(0, 1);
    }
#undef MQ_PREP_LAUNCH
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_prep_swiglu_digits(const float *gate, const float *up, int nsplit, int64_t split_stride,
                                 int nrows, int len, int64_t src_ld, void *xdig, uint32_t *xsum,
                                 float *scale, const MqSharedSwiglu *shared, int nd, hipStream_t st) {
    if (nrows <= 0) return MOE_Q2_OK;
    if (len / 16 > 256 * PD_NG) return MOE_Q2_EUNSUPPORTED;
    MqSharedRows sh = {};
    int extra = 0;
    if (shared) {
        sh = MqSharedRows{shared->g, shared->u, shared->nsplit, shared->split_stride, shared->Is, shared->hi,
                          shared->lo};
        extra = shared->T * ((shared->Is + 255) / 256);
    }
    if (nd == 2)
        hipLaunchKernelGGL((k_prep_digits<2, 2>), dim3(nrows + 1 + extra), dim3(256), 0, st, (const void *)gate,
                           (const void *)up, nsplit, split_stride, nrows, len, src_ld, (mq_u32x4 *)xdig, xsum,
                           scale, sh);
    else
        hipLaunchKernelGGL((k_prep_digits<2, 1>), dim3(nrows + 1 + extra), dim3(256), 0, st, (const void *)gate,
                           (const void *)up, nsplit, split_stride, nrows, len, src_ld, (mq_u32x4 *)xdig, xsum,
                           scale, sh);
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
// unit's activation digits + group sums (576 B per token) are staged in LDS by
// direct global-to-LDS loads (16 bytes per lane, 1 KB per wave instruction), so a
// token's activations are read from memory once per 256 rows and no registers hold
// the staged data; the next column is loaded while the current one is multiplied.
// Within a column a wave expands its two fragments' q*sc operands once and then
// takes one token fragment at a time (four integer chains, the min term, the fold),
// so the accumulators of a single fragment are live: with the staging registers gone
// this leaves room for 5 token fragments, units of up to 80 slots (at about 64 slots
// per expert, 64-slot units would give half the experts a second pass over their
// weights for a few tokens).
//
// LDS layout: the two activation buffers, then the two weight buffers (a fragment's
// activation offset, at most 32 KB, is then a constant of the read instruction).
// Activations = [token][32 16-byte digit words] with word w of token t at position
// w ^ (t & 15), then [token][4 sum words] with word q at q ^ ((t & 15) >> 2); the
// XOR swizzles keep the 16 lanes that read one word of 16 different tokens on
// distinct banks.  Weights = the 4 tiles' column pieces in global order.
template <bool SWIGLU, int MF, int ND, int BD>
__global__ void __launch_bounds__(512) k_q2_mma_pf(const uint8_t *__restrict__ experts,
                                                   int64_t expert_bytes, int64_t mat_off, int rows,
                                                   int kblocks, const int32_t *__restrict__ units_hdr,
                                                   const int4 *__restrict__ units,
                                                   const int32_t *__restrict__ perm, int topk,
                                                   const mq_u32x4 *__restrict__ xdig,
                                                   const uint32_t *__restrict__ xsum,
                                                   const float *__restrict__ xscale,
                                                   float *__restrict__ out, const uint64_t *__restrict__ eptr) {
    constexpr int NTOK = 16 * MF;
    constexpr int WPT = 16 * ND;                        // 16-byte digit words per token and column
    constexpr int TPL = 64 / WPT;                       // tokens per 1 KB digit load
    constexpr int CV = 16 * BD;                         // uint4 per tile column (64 rows x BD dwords)
    constexpr int NWJ = 4 * CV / 64;                    // weight loads (1 KB each): BD
    constexpr int NDJ = NTOK / TPL;                     // digit loads
    constexpr int NSJ = NTOK * 4 / 64;                  // sum loads (16 tokens each)
    constexpr int NJ = NDJ + NSJ + NWJ;
    constexpr int JPW = (NJ + 7) / 8;                   // loads per wave (at most)
    constexpr int SUMS = NTOK * 4 * WPT;                // dword offset of the sum words
    static_assert(4 * CV % 64 == 0 && NTOK % 16 == 0, "load split");
    // one LDS array for all staging (weights, activations, token rows)
    constexpr int SB_SZ = NWJ * 256, SA_SZ = NTOK * (4 * WPT + 16), SB_OFF = 2 * SA_SZ;
    __shared__ __attribute__((aligned(16))) uint32_t smem[2 * SB_SZ + 2 * SA_SZ + 2 * NTOK];
    typedef __attribute__((address_space(1))) void gvoid;
    typedef __attribute__((address_space(3))) void lvoid;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, q4 = lane >> 4;
    const int tw = wv >> 1, hw = wv & 1;
    const int nslot0 = SWIGLU ? 16 * hw : 32 * hw;       // first fragment's slot
    const int nslot1 = SWIGLU ? 32 + 16 * hw : 32 * hw + 16;
    const int stiles = rows / (SWIGLU ? 32 : 64) / 4;
    const int U = units_hdr[0];
    const int64_t tile_bytes = (int64_t)kblocks * 64 * 4 * BD;
    const mq_i32x4 zi = {0, 0, 0, 0};
    const int sw = r16;                                  // digit word swizzle of this lane's token
    const int ssw = 4 * (q4 ^ (r16 >> 2));               // sum word position (dwords)
    // this lane's digit words of MFMA step kk (d = 0 hi, 1 lo; the one digit of Q8 at
    // d = 0) in its token's row of a buffer, in dwords; fragment m adds 16 * 4 WPT m
    // (a constant of the LDS read)
    int xo[4][ND];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int d = 0; d < ND; ++d) xo[kk][d] = r16 * 4 * WPT + 4 * ((ND * (4 * kk + q4) + d) ^ sw);

    // Work items blockIdx.x, + gridDim.x, ...  While an item runs, the next one's token
    // rows are loaded (into the other half of arow_b) and, in its last column, the next
    // item's first column is staged, so consecutive items run back to back.
    const int nitems = U * stiles;
    int wu = blockIdx.x;
    if (wu >= nitems) return;
    int *arow_b = (int *)(smem + 2 * SB_SZ + 2 * SA_SZ);   // [2][NTOK]
    // token row of slot i of a unit; slots past its count repeat the last token (their
    // sums are computed and never stored)
    auto token_row = [&](const int4 &v, int i) {
        const int slot = v.y + min(i, v.z - 1);
        return SWIGLU ? perm[slot] / topk : slot;
    };
    int4 un = units[wu / stiles];
    if (tid < NTOK) arow_b[tid] = token_row(un, tid);
    __syncthreads();
    // load j = wv + 8 n of a column: digits of tokens TPL j .. TPL j + TPL - 1 (j < NDJ), sums of
    // tokens 16 (j - NDJ) .. +15, or 1 KB of the 4 tiles' weight pieces; each lane's
    // byte offset from the column's base is fixed for the work item
    uint32_t voff[JPW];
    auto set_voff = [&](const int *arow) {
#pragma unroll
        for (int n = 0; n < JPW; ++n) {
            const int j = wv + 8 * n;
            uint32_t o = 0;
            if (j < NDJ) {
                const int t = TPL * j + lane / WPT, w = (lane % WPT) ^ (t & 15);
                o = (uint32_t)((arow[t] * kblocks * WPT + w) * 16);
            } else if (j < NDJ + NSJ) {
                const int q = 64 * (j - NDJ) + lane, t = q >> 2, w = (q & 3) ^ ((t & 15) >> 2);
                o = (uint32_t)((arow[t] * kblocks * 16 + 4 * w) * 4);
            } else if (j < NJ) {
                const int p = 64 * (j - NDJ - NSJ) + lane, tl = p / CV, w = p - tl * CV;
                o = (uint32_t)(tl * tile_bytes + w * 16);
            }
            voff[n] = o;
        }
    };
    // column b of the item at tbase into buffer buf; digit and sum loads only for the
    // first mfc token fragments (the rest are never read)
    auto dma = [&](int b, int buf, int mfc, const uint8_t *tbase) {
        const char *db = (const char *)xdig + (int64_t)b * (16 * WPT);
        const char *sb = (const char *)xsum + (int64_t)b * 64;
        const char *wb = (const char *)tbase + (int64_t)b * (16 * CV);
#pragma unroll
        for (int n = 0; n < JPW; ++n) {
            const int j = wv + 8 * n;
            if (j < NDJ) {
                if (j < (16 / TPL) * mfc)
                    __builtin_amdgcn_global_load_lds((gvoid *)(db + voff[n]), (lvoid *)(smem + buf * SA_SZ + 256 * j), 16, 0, 0);
            } else if (j < NDJ + NSJ) {
                if (j - NDJ < mfc)
                    __builtin_amdgcn_global_load_lds((gvoid *)(sb + voff[n]),
                                                     (lvoid *)(smem + buf * SA_SZ + SUMS + 256 * (j - NDJ)), 16, 0, 0);
            } else if (j < NJ) {
                __builtin_amdgcn_global_load_lds((gvoid *)(wb + voff[n]),
                                                 (lvoid *)(smem + SB_OFF + buf * SB_SZ + 256 * (j - NDJ - NSJ)), 16, 0, 0);
            }
        }
    };
    bool pre = false;                                    // the item's first column is staged
    int bpar = 0;                                        // buffer of the item's first column
    for (int k = 0; wu < nitems; wu += gridDim.x, ++k) {
        const int u = wu / stiles, st = wu - u * stiles;
        const int e = un.x, p0 = un.y, nt = un.z;
        const int *arow_s = arow_b + (k & 1) * NTOK;
        int *arow_n = arow_b + ((k + 1) & 1) * NTOK;
        const uint8_t *tb = (eptr ? (const uint8_t *)eptr[e] : experts + (int64_t)e * expert_bytes) + mat_off +
                            (int64_t)(4 * st) * tile_bytes;
        // the next item; from 3 columns on, its rows are written in column kblocks - 2
        // (every wave is past the previous item's outputs, which read that half, once
        // column 0's barrier is behind it) and its first column staged in the last one
        const int wn = wu + gridDim.x;
        const bool has_next = wn < nitems;
        const int4 unn = has_next ? units[wn / stiles] : make_int4(0, 0, 1, 0);
        const int stn = wn - (wn / stiles) * stiles;
        const uint8_t *tbn = (eptr && has_next ? (const uint8_t *)eptr[unn.x] : experts + (int64_t)unn.x * expert_bytes) +
                             mat_off + (int64_t)(4 * stn) * tile_bytes;
        const int mfcn = (unn.z + 15) >> 4;
        const bool chain = has_next && kblocks >= 3;
        const int nrow = has_next && tid < NTOK ? token_row(unn, tid) : 0;
        if (!pre) set_voff(arow_s);
        // MFC token fragments carry tokens (the rest of MF are skipped): one copy of the
        // column loop per count, so no fragment test sits in the loop
        auto run = [&](auto mfc_tag) {
            constexpr int MFC = decltype(mfc_tag)::value;
            mq_f32x4 tot[MFC][2];
#pragma unroll
            for (int m = 0; m < MFC; ++m) { tot[m][0] = (mq_f32x4){0.f, 0.f, 0.f, 0.f}; tot[m][1] = tot[m][0]; }
            // One barrier per column: the buffer loaded during step b (column b + 1, or the
            // next item's first column) was last read in step b - 1, which every wave
            // finished before that step's barrier; each wave waits for its own loads
            // before the barrier.
            if (!pre) {
                dma(0, bpar, MFC, tb);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            for (int b = 0; b < kblocks; ++b) {
                const int cur = (b + bpar) & 1;
                if (b + 1 < kblocks) dma(b + 1, cur ^ 1, MFC, tb);
                if (chain && b == kblocks - 2 && tid < NTOK) arow_n[tid] = nrow;
                if (chain && b == kblocks - 1) {
                    set_voff(arow_n);                    // this item's loads are all issued
                    dma(0, cur ^ 1, mfcn, tbn);
                }
                const uint32_t *blk0 = smem + SB_OFF + cur * SB_SZ + (tw * 64 + nslot0 + r16) * BD;
                const uint32_t *blk1 = smem + SB_OFF + cur * SB_SZ + (tw * 64 + nslot1 + r16) * BD;
                const uint32_t *sAc = smem + cur * SA_SZ;
                // both fragments' q*sc operands of the column, expanded once and kept
                // across the token fragments
                mq_i32x4 b0[4], b1[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    b0[kk] = mq_group_operand<BD>(blk0, 4 * kk + q4, kk, q4);
                    b1[kk] = mq_group_operand<BD>(blk1, 4 * kk + q4, kk, q4);
                }
                const mq_s16x4 bm0 = mq_mins_bf16(blk0[q4]), bm1 = mq_mins_bf16(blk1[q4]);
                const uint32_t dd0 = blk0[BD - 1], dd1 = blk1[BD - 1];
                const float d0 = mq_h2f((uint16_t)(dd0 & 0xFFFFu)), m0 = mq_h2f((uint16_t)(dd0 >> 16));
                const float d1 = mq_h2f((uint16_t)(dd1 & 0xFFFFu)), m1 = mq_h2f((uint16_t)(dd1 >> 16));
                // one token fragment at a time: its four integer chains, the min term, the
                // fold; the next fragment's activation operands are read from LDS ahead
                // (the first PK of the 4 MFMA steps of the next fragment: what the register
                // budget of two waves per SIMD allows without spills)
                constexpr int PK = 3;
                mq_i32x4 xa[2][PK][ND];
                auto xop = [&](int m, int kk, int d) {
                    return __builtin_bit_cast(mq_i32x4, *(const mq_u32x4 *)(sAc + xo[kk][d] + 16 * 4 * WPT * m));
                };
                auto xread = [&](int m, mq_i32x4 (&x)[PK][ND]) {
#pragma unroll
                    for (int kk = 0; kk < PK; ++kk)
#pragma unroll
                        for (int d = 0; d < ND; ++d) x[kk][d] = xop(m, kk, d);
                };
                xread(0, xa[0]);
#pragma unroll
                for (int m = 0; m < MFC; ++m) {
                    mq_i32x4 hi0 = zi, lo0, hi1 = zi, lo1;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        if (kk == PK && m + 1 < MFC) xread(m + 1, xa[(m + 1) & 1]);
                        const mq_i32x4 al = kk < PK ? xa[m & 1][kk][ND - 1] : xop(m, kk, ND - 1);
                        // the first step of each chain starts from zero (no accumulator to clear)
                        if (ND == 2) {
                            const mq_i32x4 ah = kk < PK ? xa[m & 1][kk][0] : xop(m, kk, 0);
                            hi0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah, b0[kk], kk ? hi0 : zi, 0, 0, 0);
                            lo0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, b0[kk], kk ? lo0 : zi, 0, 0, 0);
                            hi1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah, b1[kk], kk ? hi1 : zi, 0, 0, 0);
                            lo1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, b1[kk], kk ? lo1 : zi, 0, 0, 0);
                        } else {
                            lo0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, b0[kk], kk ? lo0 : zi, 0, 0, 0);
                            lo1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(al, b1[kk], kk ? lo1 : zi, 0, 0, 0);
                        }
                    }
                    const mq_u32x4 xv = *(const mq_u32x4 *)(sAc + SUMS + (16 * m + r16) * 16 + ssw);
                    const mq_f32x4 a0 = mq_min_term(xv, bm0), a1 = mq_min_term(xv, bm1);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int v0 = ND == 2 ? (hi0[i] << 8) + lo0[i] : lo0[i];
                        const int v1 = ND == 2 ? (hi1[i] << 8) + lo1[i] : lo1[i];
                        tot[m][0][i] = fmaf(d0, (float)v0, fmaf(-m0, a0[i], tot[m][0][i]));
                        tot[m][1][i] = fmaf(d1, (float)v1, fmaf(-m1, a1[i], tot[m][1][i]));
                    }
                }
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            // outputs: lane holds tokens 16m + 4*q4 + i of row slots (nslot0|nslot1) + r16
            const int trow = (4 * st + tw) * (SWIGLU ? 32 : 64);
#pragma unroll
            for (int m = 0; m < MFC; ++m) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * m + 4 * q4 + i;
                    if (t < nt) {
                        const float sc = xscale[arow_s[t]];
                        float *o = out + (int64_t)(p0 + t) * rows + trow;
                        if (SWIGLU) {
                            const float gt = tot[m][0][i] * sc, up = tot[m][1][i] * sc;
                            o[16 * hw + r16] = gt / (1.0f + expf(-gt)) * up;
                        } else {
                            o[nslot0 + r16] = tot[m][0][i] * sc;
                            o[nslot1 + r16] = tot[m][1][i] * sc;
                        }
                    }
                }
            }
        };
        const int mfa = (nt + 15) >> 4;                  // 1..MF, uniform
        static_assert(MF == 4 || MF == 5, "one loop copy per fragment count 1..MF");
        if constexpr (MF == 5) {
            if (mfa >= 5) run(std::integral_constant<int, 5>{});
            else if (mfa == 4) run(std::integral_constant<int, 4>{});
            else if (mfa == 3) run(std::integral_constant<int, 3>{});
            else if (mfa == 2) run(std::integral_constant<int, 2>{});
            else run(std::integral_constant<int, 1>{});
        } else {
            if (mfa >= 4) run(std::integral_constant<int, 4>{});
            else if (mfa == 3) run(std::integral_constant<int, 3>{});
            else if (mfa == 2) run(std::integral_constant<int, 2>{});
            else run(std::integral_constant<int, 1>{});
        }
        if (has_next && !chain) {                        // short items: the next rows here
            if (tid < NTOK) arow_n[tid] = nrow;
            __syncthreads();
        }
        pre = chain;
        bpar = (bpar + kblocks) & 1;
        un = unn;
    }
}


int mq_launch_q2_mma_pf(int swiglu, const MqFormat &fmt, const void *experts, int64_t expert_bytes,
                        int64_t mat_off, int rows, int kblocks, const int32_t *units_hdr, const int4 *units,
                        int max_units, const int32_t *perm, int topk, const void *xdig,
                        const uint32_t *xsum, const float *xscale, float *out, int n_cu, int mf,
                        hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if ((fmt.nd != 1 && fmt.nd != 2) || (fmt.bd != MQ_BD2 && fmt.bd != MQ_BD4)) return MOE_Q2_EINVAL;
    // fragments per unit (the bucketing's unit size / 16): 5, or 4 where the staging
    // of 4-bit weights with two-digit activations of 80 tokens would not fit in LDS
    if (mf != PF_MF && mf != 4) return MOE_Q2_EINVAL;
    if (mf == PF_MF && fmt.nd == 2 && fmt.bd == MQ_BD4) return MOE_Q2_EINVAL;
    const int stiles = rows / (swiglu ? 32 : 64) / 4;
    int64_t want = (int64_t)max_units * stiles;
    int64_t cap = (int64_t)n_cu;       // one persistent work-group per compute unit (LDS-bound)
    const int grid = (int)(want < cap ? want : cap);
    if (grid <= 0) return mq_mark_empty(ev0, ev1, st);
#define MQ_PF_LAUNCH(SW, MFV, NDV, BDV)                                                                 \
    MQ_LAUNCH_TIMED(ev0, ev1, (k_q2_mma_pf<SW, MFV, NDV, BDV>), dim3(grid), dim3(512), 0, st,             \
                    (const uint8_t *)experts, expert_bytes, mat_off, rows, kblocks, units_hdr, units, perm, \
                    topk, (const mq_u32x4 *)xdig, xsum, xscale, out, fmt.eptr)
#define MQ_PF_SW(MFV, NDV, BDV)                                                                         \
    do {                                                                                                 \
        if (swiglu) MQ_PF_LAUNCH(true, MFV, NDV, BDV);                                                   \
        else MQ_PF_LAUNCH(false, MFV, NDV, BDV);                                                         \
    } while (0)
    // instantiations: 80-slot units for every format but 4-bit weights with two
    // digits (64-slot units), and 64-slot units of the 2-bit kernels for a layer
    // whose other matrix is 4-bit (one bucketing serves both launches)
    if (mf == PF_MF) {
        if (fmt.nd == 2) MQ_PF_SW(PF_MF, 2, MQ_BD2);
        else if (fmt.bd == MQ_BD2) MQ_PF_SW(PF_MF, 1, MQ_BD2);
        else MQ_PF_SW(PF_MF, 1, MQ_BD4);
    } else {
        if (fmt.nd != 2) return MOE_Q2_EINVAL;
        if (fmt.bd == MQ_BD2) MQ_PF_SW(4, 2, MQ_BD2);
        else MQ_PF_SW(4, 2, MQ_BD4);
    }
#undef MQ_PF_SW
#undef MQ_PF_LAUNCH
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
