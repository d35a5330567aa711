// Budgeted HBM cache of routed experts streamed from host memory on misses
// ("DwarfStar (ds4)" (opensourcealternatives.to), section FAQ: routed experts come
// from slower storage through an in-memory cache; "DwarfStar 4" (aiany.app),
// section "What Sets It Apart": configurable expert-cache budgets).  The cache is
// planned and filled on the device, after the bucketing has counted the slots of
// every expert, so a cached layer needs no host round trip and stays capturable.
//
// Policy (least recently used, ties by index): a touched expert already resident
// keeps its slot (its stamp becomes the call's clock); the missing experts, in
// increasing key order, take the slots no touched expert uses, in increasing
// (stamp, slot index) order -- empty slots (stamp 0) first.  Missing experts beyond
// those slots (a call touching more experts than the budget holds) stay uncached:
// the routed kernels read them straight from host memory for this call.
//
// Frequency admission (policy MOE_Q2_CACHE_LRU_ADMIT): a missing expert takes the slot
// it is paired with only if the key the slot holds was touched by fewer calls than the
// missing one (an empty slot always); otherwise the slot keeps its key and stamp and
// the expert is read from host memory for this call.
//
// State (int32, device): [0] clock, [1] hits, [2] misses (both cumulative),
// [3] misses of the last call, [4] experts touched by the last call, [5] misses of
// the last call left uncached, [6] uncached misses (cumulative), [7] 0, then
// slot_key[n_slots] (-1: empty), slot_stamp[n_slots], key_slot[n_keys] (-1: absent),
// key_count[n_keys] (calls that touched the key, saturating at 2^31 - 1).
// The cumulative counters wrap modulo 2^32.  The clock never overflows: once it
// reaches MQ_CACHE_CLOCK_LIMIT, the next call first renumbers the used slots' stamps
// 1, 2, ... in their (stamp, slot index) order and restarts the clock at the number
// of used slots, which keeps every later decision of the policy unchanged.
#include "common.h"
#include "kernels.h"

#define MQ_CACHE_HDR 8
#define MQ_CACHE_THREADS 1024
#define MQ_CACHE_CLOCK_LIMIT (1 << 30)

__global__ void __launch_bounds__(256) k_cache_reset(int32_t *__restrict__ state, int n_slots, int n_keys) {
    const int64_t ks = MQ_CACHE_HDR + 2 * (int64_t)n_slots;                          // key_slot
    const int64_t n = ks + 2 * (int64_t)n_keys;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int32_t v = 0;
        if (i >= MQ_CACHE_HDR && i < MQ_CACHE_HDR + n_slots) v = -1;                 // slot_key
        if (i >= ks && i < ks + n_keys) v = -1;                                       // key_slot
        state[i] = v;                                                                 // stamps, counts: 0
    }
}

int mq_launch_cache_reset(int32_t *state, int n_slots, int n_keys, hipStream_t st) {
    const int64_t n = MQ_CACHE_HDR + 2 * (int64_t)n_slots + 2 * (int64_t)n_keys;
    int64_t grid = (n + 255) / 256;
    if (grid > 1024) grid = 1024;
    hipLaunchKernelGGL(k_cache_reset, dim3((unsigned)grid), dim3(256), 0, st, state, n_slots, n_keys);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

// One work-group.  counts: slots per expert of this call (E <= MQ_CACHE_THREADS);
// out: eptr[e], the address the routed kernels read touched expert e from (its slot
// in `slots`, or host + e * host_bytes for a miss left uncached), the list (expert,
// slot) of the misses to copy, in increasing expert order, and its length.
__global__ void __launch_bounds__(MQ_CACHE_THREADS) k_cache_plan(const int32_t *__restrict__ counts, int E,
                                                                int key_base, int32_t *__restrict__ state,
                                                                int n_slots, int n_keys,
                                                                const uint8_t *slots, int64_t slot_bytes,
                                                                const uint8_t *host, int64_t host_bytes,
                                                                uint64_t *__restrict__ eptr,
                                                                int2 *__restrict__ misses,
                                                                int32_t *__restrict__ n_miss, int policy) {
    __shared__ int32_t s_stamp[MOE_Q2_CACHE_MAX_SLOTS], s_key[MOE_Q2_CACHE_MAX_SLOTS];
    __shared__ int32_t s_miss[MQ_CACHE_THREADS], s_victim[MQ_CACHE_THREADS];
    __shared__ int32_t s_wsum[MQ_CACHE_THREADS / 64], s_hits, s_placed;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t *slot_key = state + MQ_CACHE_HDR;
    int32_t *slot_stamp = slot_key + n_slots;
    int32_t *key_slot = slot_stamp + n_slots;
    int32_t *key_count = key_slot + n_keys;
    int32_t clock0 = state[0];
    for (int s = tid; s < n_slots; s += MQ_CACHE_THREADS) {
        s_stamp[s] = slot_stamp[s];
        s_key[s] = slot_key[s];
    }
    if (tid == 0) {
        s_hits = 0;
        s_placed = 0;
    }
    s_victim[tid] = -1;
    __syncthreads();
    // 0. clock renumbering (see the state layout above); n_slots <= 2 * MQ_CACHE_THREADS
    if (clock0 >= MQ_CACHE_CLOCK_LIMIT) {
        int32_t nv[MOE_Q2_CACHE_MAX_SLOTS / MQ_CACHE_THREADS];
        int used = 0;
#pragma unroll
        for (int k = 0; k < MOE_Q2_CACHE_MAX_SLOTS / MQ_CACHE_THREADS; ++k) {
            const int s = tid + k * MQ_CACHE_THREADS;
            nv[k] = 0;
            if (s < n_slots && s_stamp[s] > 0) {
                const int32_t st = s_stamp[s];
                int rank = 0;
                for (int q = 0; q < n_slots; ++q) {
                    const int32_t sq = s_stamp[q];
                    rank += (sq > 0 && (sq < st || (sq == st && q < s))) ? 1 : 0;
                }
                nv[k] = rank + 1;
            }
        }
        for (int q = 0; q < n_slots; ++q) used += s_stamp[q] > 0 ? 1 : 0;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < MOE_Q2_CACHE_MAX_SLOTS / MQ_CACHE_THREADS; ++k) {
            const int s = tid + k * MQ_CACHE_THREADS;
            if (s < n_slots) s_stamp[s] = nv[k];
        }
        clock0 = used;
        __syncthreads();
    }
    const int32_t clock = clock0 + 1;
    // 1. hits keep their slot (stamped with this call's clock); misses are flagged.
    // (A state not made by moe_q2_cache_reset with this n_slots could hold a slot out
    // of range: it is read as a miss, and step 4 keeps every slot index in range, so
    // such misuse gives wrong results but no access outside the buffers.)
    int miss = 0;
    int32_t my_count = 0;                                // touches of this call's key (tid < E)
    if (tid < E) {
        int32_t sl = -1;
        if (counts[tid] > 0) {
            const int32_t kc = key_count[key_base + tid];
            my_count = kc < 0x7FFFFFFF ? kc + 1 : kc;    // this call's touch, saturating
            key_count[key_base + tid] = my_count;        // (only this thread's key)
            sl = key_slot[key_base + tid];
            if (sl >= n_slots) sl = -1;
            if (sl >= 0) {
                s_stamp[sl] = clock;
                atomicAdd(&s_hits, 1);                   // a count: commutative
            } else {
                miss = 1;
            }
        }
        eptr[tid] = (uint64_t)(sl >= 0 ? slots + (int64_t)sl * slot_bytes : host + (int64_t)tid * host_bytes);
    }
    // 2. rank of each miss among the misses, in expert order (work-group scan)
    int r = miss;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int p = __shfl_up(r, o, 64);
        if (lane >= o) r += p;
    }
    if (lane == 63) s_wsum[wv] = r;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wv; ++w) base += s_wsum[w];
    int nm = 0;
    for (int w = 0; w < MQ_CACHE_THREADS / 64; ++w) nm += s_wsum[w];
    s_miss[tid] = miss ? base + r - 1 : -1;
    // 3. the slots no touched expert uses, ranked by (stamp, slot index); the first
    // nm of them are the victims, victim i taken by the miss of rank i (misses of rank
    // at or past the number of such slots stay uncached)
    for (int s = tid; s < n_slots; s += MQ_CACHE_THREADS) {
        const int32_t st = s_stamp[s];
        if (st < clock) {
            int rank = 0;
            for (int q = 0; q < n_slots; ++q) {
                const int32_t sq = s_stamp[q];
                rank += (sq < st || (sq == st && q < s)) ? 1 : 0;
            }
            if (rank < nm) s_victim[rank] = s;
        }
    }
    __syncthreads();
    // 4. admission, evictions (the victims' old keys), then the new keys; all keys
    // distinct.  A victim's key is not touched by this call, so its count is the one
    // before the call (step 1 changed only touched keys' counts).
    const int free_slots = n_slots - s_hits;             // slots no touched expert uses
    const int nfill = min(nm, free_slots);
    const bool paired = tid < E && s_miss[tid] >= 0 && s_miss[tid] < nfill;
    int v = -1;
    bool place = false;
    if (paired) {
        v = s_victim[s_miss[tid]];                       // >= 0 for a state made by the reset
        const int32_t old = v >= 0 ? s_key[v] : -1;
        const bool known = old >= 0 && old < n_keys;
        place = v >= 0 && (policy != MOE_Q2_CACHE_LRU_ADMIT || !known || key_count[old] < my_count);
        if (place) {
            if (known) key_slot[old] = -1;
            atomicAdd(&s_placed, 1);                     // a count: commutative
        }
    }
    __syncthreads();
    if (paired) {
        const int i = s_miss[tid];
        if (place) {
            key_slot[key_base + tid] = v;
            s_key[v] = key_base + tid;
            s_stamp[v] = clock;
            eptr[tid] = (uint64_t)(slots + (int64_t)v * slot_bytes);
            misses[i] = make_int2(tid, v);
        } else {
            misses[i] = make_int2(tid, -1);              // not copied: read from host memory
        }
    }
    __syncthreads();
    for (int s = tid; s < n_slots; s += MQ_CACHE_THREADS) {
        slot_stamp[s] = s_stamp[s];
        slot_key[s] = s_key[s];
    }
    if (tid == 0) {
        uint32_t *cnt = (uint32_t *)state;               // cumulative counters wrap
        state[0] = clock;
        cnt[1] += (uint32_t)s_hits;
        cnt[2] += (uint32_t)nm;
        state[3] = nm;
        state[4] = s_hits + nm;
        state[5] = nm - s_placed;
        cnt[6] += (uint32_t)(nm - s_placed);
        *n_miss = nfill;                                 // list length (unplaced entries skipped)
    }
}

int mq_launch_cache_plan(const int32_t *counts, int E, int key_base, int32_t *state, int n_slots, int n_keys,
                         const void *slots, int64_t slot_bytes, const void *host, int64_t host_bytes,
                         uint64_t *eptr, int2 *misses, int32_t *n_miss, int policy, hipStream_t st) {
    if (E > MQ_CACHE_THREADS || n_slots > MOE_Q2_CACHE_MAX_SLOTS) return MOE_Q2_EUNSUPPORTED;
    hipLaunchKernelGGL(k_cache_plan, dim3(1), dim3(MQ_CACHE_THREADS), 0, st, counts, E, key_base, state, n_slots,
                       n_keys, (const uint8_t *)slots, slot_bytes, (const uint8_t *)host, host_bytes, eptr, misses,
                       n_miss, policy);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}

// The missed experts' bytes from host memory (read over the host link by the
// work-groups) into their slots: chunks of 4 KiB, miss-major, grid-strided, 16 bytes
// per thread and step; the miss count is read on the device.
#define MQ_FILL_CHUNK 4096
__global__ void __launch_bounds__(256) k_cache_fill(const uint8_t *__restrict__ host, int64_t expert_bytes,
                                                   uint8_t *__restrict__ slots, int64_t slot_bytes,
                                                   const int2 *__restrict__ misses,
                                                   const int32_t *__restrict__ n_miss) {
    const int64_t cpe = (expert_bytes + MQ_FILL_CHUNK - 1) / MQ_FILL_CHUNK;
    const int64_t total = (int64_t)(*n_miss) * cpe;
    for (int64_t c = blockIdx.x; c < total; c += gridDim.x) {
        const int64_t i = c / cpe, off = (c - i * cpe) * MQ_FILL_CHUNK + 16 * (int64_t)threadIdx.x;
        const int2 m = misses[i];
        if (off < expert_bytes && m.y >= 0) {
            const mq_u32x4 v = *(const mq_u32x4 *)(host + (int64_t)m.x * expert_bytes + off);
            *(mq_u32x4 *)(slots + (int64_t)m.y * slot_bytes + off) = v;
        }
    }
}

int mq_launch_cache_fill(const void *host, int64_t expert_bytes, void *slots, int64_t slot_bytes,
                         const int2 *misses, const int32_t *n_miss, int n_cu, hipStream_t st) {
    hipLaunchKernelGGL(k_cache_fill, dim3(2 * n_cu), dim3(256), 0, st, (const uint8_t *)host, expert_bytes,
                       (uint8_t *)slots, slot_bytes, misses, n_miss);
    MQ_LAUNCH_CHECK();
    return MOE_Q2_OK;
}
