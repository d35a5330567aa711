// Shared device helpers of the MoE-Q2 library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/moe_q2.h"

#define MQ_QK 256
#define MQ_GROUP 16
#define MQ_NGROUPS 16
#define MQ_BLOCK_BYTES 84
#define MQ_BLOCK_DWORDS 21
#define MQ_WAVE 64
// Block dwords of the two weight codecs: the 2-bit block (84 bytes) and its 4-bit
// sibling (148 bytes).
#define MQ_BD2 21
#define MQ_BD4 37

typedef _Float16 mq_half2 __attribute__((ext_vector_type(2)));
typedef short mq_bf16x2_raw __attribute__((ext_vector_type(2)));
typedef float mq_f32x4 __attribute__((ext_vector_type(4)));
// Native 128-bit vector (HIP's uint4 class copies through memcpy and can end up in
// scratch memory; this type stays in registers).
typedef uint32_t mq_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float mq_bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t mq_f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float mq_h2f(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

__device__ __forceinline__ float mq_wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MQ_WAVE);
    return v;
}

__device__ __forceinline__ float mq_wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MQ_WAVE));
    return v;
}

// Host-side launch check.
#define MQ_LAUNCH_CHECK()                                                      \
    do {                                                                       \
        hipError_t _e = hipGetLastError();                                     \
        if (_e != hipSuccess) return mq_fail_hip(_e);                          \
    } while (0)

int mq_fail_hip(hipError_t e);
