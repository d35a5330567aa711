// bf16 x bf16 -> fp32 GEMM on MFMA (v_mfma_f32_16x16x32_bf16), used for the
// full-precision shared expert:  P[split, m, n] = sum_{k in split} A[m, k] * B[n, k].
//
// A is [M, K] (activations, one or two bf16 planes: with two planes the kernel
// adds A_hi*B + A_lo*B, which carries an fp32 activation to ~16 bits), B is
// [N, K] (weights, row-major along K).  Split-K partial sums go to P and are
// reduced in a fixed order by the epilogue kernels (deterministic, no atomics).
//
// Tiles: BM = 16*MF*WM rows of A, BN = 16*NF*WN rows of B, BK wide; 4 waves
// arranged WM x WN, each owning MF x NF 16x16 accumulator fragments.  The next
// K tile is loaded into registers while the current one is multiplied.  LDS
// rows are padded by 8 bf16 (a 4-bank shift per row) so the 16-byte fragment
// reads of 16 lanes fall on distinct banks.  Fragment layout of the 16x16x32 instruction: lane l
// holds A[l%16][8*(l/16) .. +7] and B[l%16][8*(l/16) .. +7]; D lane l, element i
// is D[4*(l/16) + i][l%16].
#include "common.h"
#include "kernels.h"

typedef __bf16 mq_bf16x8 __attribute__((ext_vector_type(8)));

// SWI (one split, N = 2 Is: B rows 0..Is-1 gate, Is..2Is-1 up): each wave's NF
// fragments hold 8 NF gate columns and the same 8 NF up columns, so the epilogue
// writes h = silu(gate) * up as bf16 planes Hhi (and Hlo = bf16(h - hi) if given),
// [M][Is], with the arithmetic of k_swiglu_partials at one split.
template <int MF, int NF, int WM, int WN, int BK, bool A2, bool SWI>
__global__ void __launch_bounds__(256) k_gemm_bf16(const uint16_t *__restrict__ A,
                                                   const uint16_t *__restrict__ Alo, int lda,
                                                   const uint16_t *__restrict__ B, int ldb, int M,
                                                   int N, int K, int k_per_split,
                                                   float *__restrict__ P, uint16_t *__restrict__ Hhi,
                                                   uint16_t *__restrict__ Hlo) {
    constexpr int BM = 16 * MF * WM, BN = 16 * NF * WN;
    static_assert(!SWI || NF % 2 == 0, "gate and up fragments in pairs");
    constexpr int HN = 8 * NF;                       // (SWI) gate columns per wave
    constexpr int NPL = A2 ? 2 : 1;
    constexpr int AS = BK + 8;                       // padded LDS row (bf16 elements)
    constexpr int CPR = BK / 8;                      // 16-byte chunks per tile row
    constexpr int NA = (BM * CPR * NPL + 255) / 256; // A chunks per thread
    constexpr int NB = (BN * CPR + 255) / 256;       // B chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t sA[NPL][BM * AS];
    __shared__ __attribute__((aligned(16))) uint16_t sB[BN * AS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / WN, wn = wv % WN;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int Is = N / 2, g0 = blockIdx.x * (BN / 2);      // (SWI) first gate column
    // B row of LDS row r: plain n0 + r; SWI: wave w's rows are its HN gate rows, then
    // the same HN up rows (a negative value: past the matrix)
    auto brow = [&](int r) {
        if (!SWI) return n0 + r < N ? n0 + r : -1;
        const int w = r / (2 * HN), q = r - w * 2 * HN, h = q / HN, o = q - h * HN;
        const int g = g0 + w * HN + o;
        return g < Is ? h * Is + g : -1;
    };
    const int split = blockIdx.z;
    const int k0 = split * k_per_split;
    const int k1 = min(K, k0 + k_per_split);

    mq_f32x4 acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = (mq_f32x4){0.f, 0.f, 0.f, 0.f};

    mq_u32x4 ra[NA], rb[NB];
    auto load = [&](int k) {
#pragma unroll
        for (int n = 0; n < NA; ++n) {
            const int c = tid + 256 * n;
            ra[n] = (mq_u32x4){0u, 0u, 0u, 0u};
            if (c < BM * CPR * NPL) {
                const int pl = c / (BM * CPR), cc = c - pl * BM * CPR;
                const int r = cc / CPR, q = cc - r * CPR;
                if (m0 + r < M)
                    ra[n] = *(const mq_u32x4 *)((pl ? Alo : A) + (int64_t)(m0 + r) * lda + k + 8 * q);
            }
        }
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int c = tid + 256 * n;
            rb[n] = (mq_u32x4){0u, 0u, 0u, 0u};
            if (c < BN * CPR) {
                const int r = c / CPR, q = c - r * CPR;
                const int br = brow(r);
                if (br >= 0) rb[n] = *(const mq_u32x4 *)(B + (int64_t)br * ldb + k + 8 * q);
            }
        }
    };
    if (k0 < k1) load(k0);
    for (int k = k0; k < k1; k += BK) {
        __syncthreads();
#pragma unroll
        for (int n = 0; n < NA; ++n) {
            const int c = tid + 256 * n;
            if (c < BM * CPR * NPL) {
                const int pl = c / (BM * CPR), cc = c - pl * BM * CPR;
                const int r = cc / CPR, q = cc - r * CPR;
                *(mq_u32x4 *)(&sA[pl][r * AS + 8 * q]) = ra[n];
            }
        }
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int c = tid + 256 * n;
            if (c < BN * CPR) {
                const int r = c / CPR, q = c - r * CPR;
                *(mq_u32x4 *)(&sB[r * AS + 8 * q]) = rb[n];
            }
        }
        __syncthreads();
        if (k + BK < k1) load(k + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            mq_bf16x8 b[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j)
                b[j] = *(const mq_bf16x8 *)(&sB[((wn * NF + j) * 16 + (lane & 15)) * AS + kk +
                                                8 * (lane >> 4)]);
#pragma unroll
            for (int pl = 0; pl < NPL; ++pl) {
#pragma unroll
                for (int i = 0; i < MF; ++i) {
                    const mq_bf16x8 a = *(const mq_bf16x8 *)(&sA[pl][((wm * MF + i) * 16 + (lane & 15)) * AS +
                                                                     kk + 8 * (lane >> 4)]);
#pragma unroll
                    for (int j = 0; j < NF; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
                }
            }
        }
    }
    if (SWI) {
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int j = 0; j < NF / 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + (wm * MF + i) * 16 + 4 * (lane >> 4) + e;
                    const int g = g0 + wn * HN + j * 16 + (lane & 15);
                    if (m < M && g < Is) {
                        const float a = acc[i][j][e], c = acc[i][j + NF / 2][e];
                        const float h = a / (1.0f + expf(-a)) * c;
                        const uint16_t hb = mq_f32_to_bf16(h);
                        Hhi[(int64_t)m * Is + g] = hb;
                        if (Hlo) Hlo[(int64_t)m * Is + g] = mq_f32_to_bf16(h - mq_bf16_to_f32(hb));
                    }
                }
        return;
    }
    float *Pout = P + (int64_t)split * M * N;
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + (wm * MF + i) * 16 + 4 * (lane >> 4) + e;
                const int n = n0 + (wn * NF + j) * 16 + (lane & 15);
                if (m < M && n < N) Pout[(int64_t)m * N + n] = acc[i][j][e];
            }
}

// h[m, j] = silu(a) * c with a = sum_s P[s, m, j], c = sum_s P[s, m, Is + j];
// written as bf16 hi (and lo = bf16(h - hi) when requested).
__global__ void k_swiglu_partials(const float *__restrict__ P, int nsplit, int M, int Is,
                                  uint16_t *__restrict__ hi, uint16_t *__restrict__ lo) {
    const int64_t n = (int64_t)M * Is;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / Is, j = i - m * Is;
        float a = 0.f, c = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const float *Ps = P + (int64_t)s * M * 2 * Is + m * 2 * Is;
            a += Ps[j];
            c += Ps[Is + j];
        }
        const float h = a / (1.0f + expf(-a)) * c;
        const uint16_t hb = mq_f32_to_bf16(h);
        hi[i] = hb;
        if (lo) lo[i] = mq_f32_to_bf16(h - mq_bf16_to_f32(hb));
    }
}

// out[m, n] = sum_s P[s, m, n] (fixed order).
__global__ void k_sum_partials(const float *__restrict__ P, int nsplit, int64_t MN,
                               float *__restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = 0.f;
        for (int s = 0; s < nsplit; ++s) v += P[s * MN + i];
        out[i] = v;
    }
}

// Skinny (M <= 64) products stream B with 256-wide K tiles and split K so that
// at least ~2 work-groups per compute unit are in flight; wide products use
// 128 x 128 tiles with 64-wide K steps.
int mq_gemm_splits(int M, int N, int K, int n_cu) {
    if (M > 64) return 1;
    const int nt = (N + 63) / 64;
    int split = (2 * n_cu + nt - 1) / nt;
    const int kmax = K / 256;
    if (split > kmax) split = kmax;
    if (split < 1) split = 1;
    return split;
}

int mq_launch_gemm_bf16(const uint16_t *A, const uint16_t *Alo, int lda, const uint16_t *B, int ldb,
                        int M, int N, int K, int nsplit, float *P, hipStream_t st) {
    const int bk = M <= 64 ? 256 : 64;
    int kps = (K + nsplit - 1) / nsplit;
    kps = (kps + bk - 1) / bk * bk;
    const bool two = Alo != nullptr;
#define MQ_GEMM(MF, NF, WM, WN, BK, A2)                                                        \
    hipLaunchKernelGGL((k_gemm_bf16<MF, NF, WM, WN, BK, A2, false>),                           \
                       dim3((N + 16 * NF * WN - 1) / (16 * NF * WN),                            \
                            (M + 16 * MF * WM - 1) / (16 * MF * WM), nsplit),                  \
                       dim3(256), 0, st, A, Alo, lda, B, ldb, M, N, K, kps, P, nullptr, nullptr)
    if (M <= 16) {
        if (two) MQ_GEMM(1, 1, 1, 4, 256, true); else MQ_GEMM(1, 1, 1, 4, 256, false);
    } else if (M <= 32) {
        if (two) MQ_GEMM(2, 1, 1, 4, 256, true); else MQ_GEMM(2, 1, 1, 4, 256, false);
    } else if (M <= 64) {
        if (two) MQ_GEMM(4, 1, 1, 4, 256, true); else MQ_GEMM(4, 1, 1, 4, 256, false);
    } else {
        if (two) MQ_GEMM(4, 4, 2, 2, 64, true); else MQ_GEMM(4, 4, 2, 2, 64, false);
    }
#undef MQ_GEMM
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_gemm_bf16_swiglu(const uint16_t *A, const uint16_t *Alo, int lda, const uint16_t *B, int ldb,
                               int M, int Is, int K, uint16_t *hi, uint16_t *lo, hipStream_t st) {
    if (M <= 64 || K % 64) return MOE_Q2_EUNSUPPORTED;
    constexpr int MF = 4, NF = 4, WM = 2, WN = 2;
    const dim3 grid((Is + 8 * NF * WN - 1) / (8 * NF * WN), (M + 16 * MF * WM - 1) / (16 * MF * WM), 1);
    if (Alo)
        hipLaunchKernelGGL((k_gemm_bf16<MF, NF, WM, WN, 64, true, true>), grid, dim3(256), 0, st, A, Alo, lda,
                           B, ldb, M, 2 * Is, K, K, nullptr, hi, lo);
    else
        hipLaunchKernelGGL((k_gemm_bf16<MF, NF, WM, WN, 64, false, true>), grid, dim3(256), 0, st, A, Alo,
                           lda, B, ldb, M, 2 * Is, K, K, nullptr, hi, lo);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_swiglu_partials(const float *P, int nsplit, int M, int Is, uint16_t *hi, uint16_t *lo,
                              hipStream_t st) {
    const int64_t n = (int64_t)M * Is;
    const int grid = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_swiglu_partials, dim3(grid), dim3(256), 0, st, P, nsplit, M, Is, hi, lo);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

int mq_launch_sum_partials(const float *P, int nsplit, int64_t MN, float *out, hipStream_t st) {
    const int grid = (int)((MN + 255) / 256 < 4096 ? (MN + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_sum_partials, dim3(grid), dim3(256), 0, st, P, nsplit, MN, out);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
