// Per-work-group timeline of the matrix-core decode launches: a diagnostic build
// only (compiled with -DMQ_WG_TIMELINE into libmoe_q2_timeline.so, never into the
// library itself, where every mark below compiles to nothing).
//
// Thread 0 of every work-group of the gate/up (kind 1) and down (kind 0) launches
// writes, for work-group index b < MQ_TL_MAX_WG, one record of MQ_TL_SLOTS
// 64-bit words into a device array, which the last launch of each kind overwrites:
//   0  entry time          1  time the column loop starts (its weights in flight)
//   2  end time            3  XCC id (bits 0..3) | hardware id register << 8
//   4  role: 0 routed unit, 1 shared-expert rows, 2 past the last unit (no work)
// Times are s_memrealtime ticks: the device's constant 100 MHz clock, the same on
// every compute unit.  moe_q2_timeline_read copies the array out and
// moe_q2_timeline_clear zeroes it (both synchronous, host-side only).
#pragma once

#define MQ_TL_SLOTS 8
#define MQ_TL_MAX_WG 16384

#ifdef MQ_WG_TIMELINE
extern __device__ unsigned long long mq_tl_buf[2][MQ_TL_MAX_WG][MQ_TL_SLOTS];

__device__ __forceinline__ unsigned long long mq_tl_now() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ unsigned long long mq_tl_hw() {
    unsigned x, h;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(h));
    return (unsigned long long)(x & 0xFu) | ((unsigned long long)h << 8);
}

// one word of this work-group's record (thread 0; vector stores only)
#define MQ_TL(kind, slot, value)                                                         \
    do {                                                                                \
        if (threadIdx.x == 0 && blockIdx.x < MQ_TL_MAX_WG)                              \
            mq_tl_buf[(kind)][blockIdx.x][(slot)] = (value);                            \
    } while (0)
// the end mark, once every wave of the work-group is done
#define MQ_TL_END(kind)                                                                  \
    do {                                                                                \
        __syncthreads();                                                                \
        MQ_TL(kind, 2, mq_tl_now());                                                    \
    } while (0)
// role and end of a work-group about to leave with no work (cond uniform)
#define MQ_TL_NO_WORK(kind, cond)                                                        \
    do {                                                                                \
        if (cond) {                                                                     \
            MQ_TL(kind, 4, 2);                                                          \
            MQ_TL(kind, 2, mq_tl_now());                                                \
        }                                                                               \
    } while (0)
#else
#define MQ_TL(kind, slot, value) do {} while (0)
#define MQ_TL_END(kind) do {} while (0)
#define MQ_TL_NO_WORK(kind, cond) do {} while (0)
#endif
// Every line of the kernel sources that names a timeline mark contains "MQ_TL", and the
// device array and accessors sit in one "#ifdef MQ_WG_TIMELINE" block: without them
// (and the include of this header) a source reads as the library compiles it.
