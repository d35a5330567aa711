// Launchers of the device kernels (host side, internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define FD_TCH 4        // slots per work unit of the vector-ALU decode kernel
#define MMA_TCH 16      // slots per work unit of the matrix-core decode kernel
#define MQ_TOPK_BUCKET_MAX_T 4   // largest batch whose bucketing runs in the top-K launch
#define PF_MF 5         // token fragments per unit of the prefill kernel (4 for a layer
                        // with a 4-bit matrix and two-digit activations)

int mq_launch_router(const void *x, int bf16, const float *wr, const float *bias, int T, int H,
                     int E, float *logits, hipStream_t st);
int mq_launch_topk(const float *logits, int nsplit, const float *bias, int T, int E, int K,
                   int32_t *idx, float *gate, int32_t *trace_idx, float *trace_w, hipStream_t st);
int mq_router_splits(int T, int H, int E);
int mq_launch_router_mma(const uint16_t *x, const float *wr, int T, int H, int E, int nsplit,
                         float *P, int tiles, hipStream_t st);
// Split count of the router for a batch-invariant call: a function of H alone.
int mq_router_splits_fixed(int H);
int mq_launch_bucket(const int32_t *idx, int T, int K, int E, int unit_tokens, int32_t *counts,
                     int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *units_hdr,
                     int4 *units, int fill_units, int32_t *urow, int zrow, hipStream_t st);
size_t mq_bucket_lds_bytes(int E);
// Large batches: the same bucketing in three launches over chunks of tokens; chunk:
// workspace of mq_bucket_chunks(T) * E ints.  No row table (prefill and vector-ALU
// decode kernels read the permutation).
int mq_bucket_chunks(int T);
int mq_launch_bucket_par(const int32_t *idx, int T, int K, int E, int unit_tokens, int32_t *counts,
                         int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *units_hdr, int4 *units,
                         int fill_units, int32_t *chunk, hipStream_t st);
#define MQ_BUCKET_PAR_MIN_T 256   // batches from this size bucket in three launches (no row table)
// Top-K and bucketing in one work-group (T <= MQ_TOPK_BUCKET_MAX_T).
int mq_launch_topk_bucket(const float *logits, int nsplit, const float *bias, int T, int E, int K,
                          int32_t *idx, float *gate, int32_t *trace_idx, float *trace_w, int unit_tokens,
                          int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *units_hdr,
                          int4 *units, int fill_units, int32_t *urow, int zrow, hipStream_t st);
int mq_launch_prep(const void *src, int src_bf16, int nrows, int len, int64_t src_ld, uint32_t *xq,
                   float2 *gsum, float *scale, hipStream_t st);
int mq_launch_rmsnorm(const float *h, int T, int H, float eps, uint16_t *x, hipStream_t st);
int mq_launch_q2_dec(int swiglu, const void *experts, int64_t expert_bytes, int64_t mat_off,
                     int rows, int kblocks, const int32_t *units_hdr, const int4 *units,
                     int max_units, const int32_t *perm, int topk, const uint32_t *xq,
                     const float2 *gsum, const float *xscale, float *out, int n_cu, hipStream_t st);
// shared: the shared expert's output as sh_nsplit partial sums sh_stride floats apart
int mq_launch_combine(const float *y, int nsplit, int64_t split_stride, const int32_t *inv,
                      const float *gate, const float *shared, int sh_nsplit, int64_t sh_stride, int T, int H,
                      int K, int accumulate, float *out, hipStream_t st);
int mq_launch_split_bf16(const float *x, int64_t n, uint16_t *hi, uint16_t *lo, hipStream_t st);
int mq_gemm_splits(int M, int N, int K, int n_cu);
int mq_launch_gemm_bf16(const uint16_t *A, const uint16_t *Alo, int lda, const uint16_t *B, int ldb,
                        int M, int N, int K, int nsplit, float *P, hipStream_t st);
// One split, more than 64 rows: the gate/up product with the SwiGLU in its epilogue
// (h as bf16 planes [M][Is]; lo optional), no partial sums.
int mq_launch_gemm_bf16_swiglu(const uint16_t *A, const uint16_t *Alo, int lda, const uint16_t *B, int ldb,
                               int M, int Is, int K, uint16_t *hi, uint16_t *lo, hipStream_t st);
int mq_launch_swiglu_partials(const float *P, int nsplit, int M, int Is, uint16_t *hi, uint16_t *lo,
                              hipStream_t st);
int mq_launch_sum_partials(const float *P, int nsplit, int64_t MN, float *out, hipStream_t st);
// Router (bf16 layer input) and the layer input's activation digits in one launch.
// tiles: force the MFMA split-K tiles (no one-work-group-per-expert router for few
// tokens), so that every batch size takes the same per-token summation order.
int mq_launch_router_prep(const uint16_t *x, const float *wr, int T, int H, int E, int nsplit, float *P,
                          void *xdig, uint32_t *xsum, float *xscale, int nd, int tiles, hipStream_t st);
// nd: activation digits (2: 15-bit, 1: Q8)
int mq_launch_prep_digits(const void *src, int src_bf16, int nrows, int len, int64_t src_ld,
                          void *xdig, uint32_t *xsum, float *scale, int nd, hipStream_t st);
// Optional shared-expert rows of the same launch: SwiGLU of the dense split partials
// g/u [nsplit][T][Is] into two bf16 planes hi/lo [T][Is].
struct MqSharedSwiglu {
    const float *g, *u;
    int nsplit;
    int64_t split_stride;
    int Is, T;
    uint16_t *hi, *lo;
};
int mq_launch_prep_swiglu_digits(const float *gate, const float *up, int nsplit, int64_t split_stride,
                                 int nrows, int len, int64_t src_ld, void *xdig, uint32_t *xsum,
                                 float *scale, const MqSharedSwiglu *shared, int nd, hipStream_t st);
// Decode kernel: split count along the reduction (shared by the workspace sizing).
// Gate/up splits are summed by the intermediate preparation, down splits by the
// combine; a split is taken only while the launch stays within about 768 resident
// work-groups (in practice: down splits in two for batches of a token or two, whose
// few work-groups are otherwise latency-bound).
#define MQ_DEC_SPLIT_GU 4
#define MQ_DEC_SPLIT_D 2
// Batch-invariant calls keep the splits of a one-token batch at every batch size, so
// their limits weigh the batched calls (a speculative-verification pass) against the
// one-token call: gate/up at most 2, down unsplit.
#define MQ_DEC_SPLIT_GU_BI 2
#define MQ_DEC_SPLIT_D_BI 1
void mq_dec_split(int max_units, int tiles, int kblocks, int max_split, int *nsplit, int *cps);
// zrow: index of the all-zero activation row (written by the digit preparation after
// the real rows); trash_row: an output row that absorbs padding-token writes; outputs
// are per-split partial sums split_stride floats apart (gu: gate -> out0, up -> out1).
// Optional dense rows (the shared expert) appended to a decode launch: bf16 weights
// [rows][K], bf16 activations [T][K] (+ low plane), per-split partial outputs
// (rows below `half` -> out0, the rest -> out1, split_stride floats apart).
struct MqDenseSpec {
    const uint16_t *w, *x, *xlo;
    float *out0, *out1;
    int T, rows, K, half, out_ld, nsplit;
    int64_t split_stride;
};
void mq_dense_split(int rows, int K, int nf, int *nsplit, int *kps);
// Routing done inside the decode gate/up launch (batches of at most
// MQ_TOPK_BUCKET_MAX_T tokens, E <= MQ_ROUTE_MAX_E, K <= 16): every routed
// work-group selects and buckets the batch from the final logits in LDS and takes
// its unit from there; work-group 0 writes the routing outputs (the same arrays the
// top-K + bucketing launch writes) for the later launches.
#define MQ_ROUTE_MAX_E 256
struct MqRoute {
    const float *logits, *bias;
    int T, E, K;
    int32_t *idx;
    float *gate;
    int32_t *trace_idx;
    float *trace_w;
    int32_t *counts, *offsets, *perm, *inv, *units_hdr;
    int4 *units;
    int fill_units;
    int32_t *urow;
    int zrow;
};
// One-token batches: the down launch prepares its own activations instead of reading
// the digit preparation launch's output -- the SwiGLU of the gate/up split partials
// of its unit's slot row (digits, group sums, scale: the same arithmetic) and, for
// the appended shared rows, the shared SwiGLU of the dense partials over the
// work-group's k range (two bf16 planes).  len <= MQ_DOWN_PREP_MAX_LEN.
#define MQ_DOWN_PREP_MAX_LEN 2048
#define MQ_DOWN_PREP_SHARED_BYTES (4 * 384 * 16)   // LDS of the shared SwiGLU planes (the weight slices)
struct MqDownPrep {
    const float *g, *u;        // routed gate/up split partials [nsplit][rows][len]
    int nsplit, len;
    int64_t split_stride;
    const float *sg, *su;      // shared dense partials [snsplit][1][Is] (or null)
    int snsplit;
    int64_t sstride;
};
// ev0 / ev1 (optional, both or neither): timing events recorded by the kernel's own
// dispatch (start and end of the kernel; both recorded on the stream when nothing is
// launched).
// units: max_units records, those past the last unit with slot count 0; urow (gate/up):
// the [max_units][16] row table of the bucketing; down reads the rows of its slots.
// route (gate/up only, optional): route in the launch instead of reading units/urow.
// Format of one routed launch: activation digits (2: 15-bit, 1: Q8), weight block
// dwords (21: 2-bit codec, 37: 4-bit sibling) and the optional table of expert
// addresses written by an expert cache's plan (null: expert e at
// experts + e * expert_bytes; else at eptr[e], a cache slot or host memory).
struct MqFormat {
    int nd, bd;
    const uint64_t *eptr;
};
// split_units: the unit count the k-split policy is computed for (max_units, or a
// fixed count when the split must not depend on the batch); max_split its limit.  merge: one work-group
// walks the k ranges of all splits and stores each range's partials (bit-identical
// to one work-group per split; for a fixed split on a batch large enough to fill
// the device without splitting).
int mq_launch_q2_mma(int gu, const MqFormat &fmt, const void *experts, int64_t expert_bytes, int64_t mat_off,
                     int tiles, int kblocks, const int4 *units, int max_units, int split_units, int max_split, int merge,
                     const int32_t *urow, int zrow, int trash_row, const void *xdig,
                     const uint32_t *xsum, const float *xscale, float *out0, float *out1, int out_ld,
                     int64_t split_stride, const MqDenseSpec *dense, const MqRoute *route,
                     const MqDownPrep *prep, hipStream_t st, hipEvent_t ev0 = nullptr,
                     hipEvent_t ev1 = nullptr);
int mq_launch_q2_mma_pf(int swiglu, const MqFormat &fmt, const void *experts, int64_t expert_bytes,
                        int64_t mat_off, int rows, int kblocks, const int32_t *units_hdr, const int4 *units,
                        int max_units, const int32_t *perm, int topk, const void *xdig,
                        const uint32_t *xsum, const float *xscale, float *out, int n_cu, int mf,
                        hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// Expert cache (cache.hip): state reset, the plan of one call (eslot, miss list) and
// the copy of the missed experts from host memory into their slots.
int mq_launch_cache_reset(int32_t *state, int n_slots, int n_keys, hipStream_t st);
// eptr: the address of every touched expert for the routed kernels (its slot, or
// host + e * host_bytes for a miss left uncached).
int mq_launch_cache_plan(const int32_t *counts, int E, int key_base, int32_t *state, int n_slots, int n_keys,
                         const void *slots, int64_t slot_bytes, const void *host, int64_t host_bytes,
                         uint64_t *eptr, int2 *misses, int32_t *n_miss, int policy, hipStream_t st);
int mq_launch_cache_fill(const void *host, int64_t expert_bytes, void *slots, int64_t slot_bytes,
                         const int2 *misses, const int32_t *n_miss, int n_cu, hipStream_t st);
