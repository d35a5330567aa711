/* moe_q2.h -- C ABI of the 2-bit routed-expert MoE layer for MI355X (gfx950).
 *
 * The layer (ds4 README mirror, section "Model Weights": only the routed MoE
 * experts are stored at 2 bits, as asymmetric super-block quants; shared
 * experts, projections and routing keep full precision), DeepSeek-style:
 *
 *   logits  l[t,e] = x[t,:] . router_w[e,:] (+ router_b[e])           fp32
 *   top-K   S_t = the K largest l[t,.], descending (ties: lower e)
 *   gates   g[t,k] = softmax(l[t,.])[S_t,k] / sum_{j in S_t} softmax(l[t,.])[j]
 *   expert  FFN_e(x) = (silu(x.Wg_e^T) * (x.Wu_e^T)) . Wd_e^T
 *   out[t]  = FFN_shared(x[t]) + sum_k g[t,k] * FFN_{S_t,k}(x[t])
 *
 * run for micro-batched decode (many sessions, a few tokens per expert) and for
 * prefill (many tokens per expert) -- the ds4 README mirror, section "So, what
 * can I do with this software?", serves both from one multi-session server.
 *
 * Q2 super-block (84 bytes, 256 weights, 2.625 bits/weight; the pages name the
 * Q2_K family, this byte order is this library's own):
 *   bytes  0..15  group j (weights 16j..16j+15): low nibble scale sc_j, high nibble min m_j
 *   bytes 16..79  2-bit codes, weight i in byte 16 + i/4 at bit 2*(i%4)
 *   bytes 80..81  d    (fp16)        bytes 82..83  dmin (fp16)
 *   w_i = d * sc_j * q_i - dmin * m_j
 * Blocks run along each matrix's reduction dimension.
 *
 * Q4 sibling block (148 bytes, 256 weights, 4.625 bits/weight; this library's own
 * higher-precision member of the family, for the per-layer and per-matrix format mixes
 * of the ds4 README mirror, section "Model Weights": q2 with the last expert layers at
 * q4; routed gate/up and down at different precisions):
 *   bytes   0..15  group j: bits 0..2 scale sc_j (0..7; bit 3 reserved, ignored), high nibble min m_j
 *   bytes  16..143 4-bit codes, group j in bytes 16 + 8j .. 16 + 8j + 7: element 4b + s of
 *                  the group (b, s in 0..3) in byte 16 + 8j + 4 (s / 2) + b, low nibble for
 *                  even s, high nibble for odd s
 *   bytes 144..145 d (fp16)       bytes 146..147 dmin (fp16)
 *   w_i = d * sc_j * q_i - dmin * m_j,  q_i in 0..15
 * A routed expert's gate/up and down matrices each take the format its shape's flags
 * give (MOE_Q2_GU_Q4, MOE_Q2_DOWN_Q4), in the same tiled layout with 148-byte blocks.
 *
 * Routed expert layout (row tiles, so that a run of block columns of 64 rows is
 * one contiguous span and streams from HBM with plain 16-byte loads):
 *   gate/up: I/32 tiles; tile t = block columns b = 0..H/256-1 of 64 rows, slots
 *            0..31 = gate rows 32t.., slots 32..63 = up rows 32t..  ([t][b][slot][84 B])
 *   down:    H/64 tiles; tile t = block columns b = 0..I/256-1 of down rows 64t..64t+63
 *   expert = gate/up tiles, then down tiles; experts back to back.
 * moe_q2_pack_expert builds it from row-major matrices.
 *
 * Conventions for every entry point:
 *   - pointers marked "device" must be device memory of the current HIP device;
 *     the caller owns every buffer; moe_q2_forward allocates no memory;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *     is asynchronous: a device fault surfaces at the caller's next sync.  The
 *     work that needs only the layer input (the routed experts' activation
 *     preparation and the shared expert) runs as a concurrent branch:
 *     moe_q2_forward forks it onto an internal stream with an event recorded on
 *     `stream` and joins it back with events before the routed experts and the
 *     combine, so the caller sees ordinary stream-ordered semantics (and the
 *     fork/join is legal under graph capture; a call that fails after the fork
 *     still joins the branch into `stream` before it returns).  The internal
 *     stream and its three events are the library's only state: created by the
 *     first such call on a device, kept until the process ends; calls from
 *     several host threads on one device enqueue one at a time.  The one-token
 *     and micro-batch decode path with a bf16 layer input never uses them, and
 *     MOE_Q2_SERIAL keeps every launch on `stream` and touches no internal state;
 *   - arguments are validated before anything is enqueued; a non-zero status
 *     means nothing was enqueued (except MOE_Q2_EHIP, raised when a launch
 *     fails, after which earlier launches of the same call may have run);
 *   - no C++ exception and no abort crosses this interface.
 */
#ifndef MOE_Q2_H
#define MOE_Q2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_Q2_OK = 0,
    MOE_Q2_EINVAL = -1,        /* null pointer, bad size, misaligned buffer, x==out misuse */
    MOE_Q2_EUNSUPPORTED = -2,  /* shape outside the supported envelope */
    MOE_Q2_EWORKSPACE = -3,    /* workspace missing or smaller than moe_q2_workspace_size */
    MOE_Q2_EHIP = -4           /* a HIP call failed; see moe_q2_last_hip_error */
} moe_q2_status;

/* activation dtypes */
enum { MOE_Q2_F32 = 0, MOE_Q2_BF16 = 1 };

/* moe_q2_shape.flags */
enum {
    MOE_Q2_PATH_AUTO = 0,      /* decode kernels below MOE_Q2_PREFILL_MIN_TOKENS tokens, else prefill */
    MOE_Q2_PATH_DECODE = 1,    /* force the decode kernels (up to 16 slots per work unit) */
    MOE_Q2_PATH_PREFILL = 2,   /* force the prefill kernels (up to 80 slots per work unit; 64
                                  when a 4-bit matrix meets the default 15-bit activations) */
    MOE_Q2_PRE_RMSNORM = 4,    /* x is the fp32 residual stream h; the layer input is
                                  bf16(h / sqrt(mean(h^2) + rms_eps)) (unit gain) */
    MOE_Q2_RESIDUAL_ADD = 8,   /* out += layer(...) instead of out = layer(...) */
    MOE_Q2_DECODE_VALU = 16,   /* decode path: routed experts on the vector-ALU dot-product
                                  kernel instead of the integer matrix-core kernel */
    MOE_Q2_SERIAL = 32,        /* run every launch on `stream` (no internal stream) */
    MOE_Q2_BATCH_INVARIANT = 64,
                               /* every token's outputs, routing and gates are bit-identical
                                  whatever the batch it is in (1 .. MOE_Q2_MAX_TOKENS tokens):
                                  one set of kernels and one summation order per token for every
                                  batch size (decode kernels, router split and reduction splits
                                  fixed by the shape: gate/up at most 2 k-splits, down unsplit;
                                  the ds4 README mirror, section "DSpark
                                  Speculative Decoding", notes that batched verification groups
                                  floating point differently from one-token decode).  Needs a
                                  bf16 (or PRE_RMSNORM) layer input when there is a shared
                                  expert; not with PATH_PREFILL (EINVAL) or DECODE_VALU */
    MOE_Q2_ACT_Q8 = 128,       /* Q8 activations for the routed experts (ds4 README mirror,
                                  section "Model Weights": decode uses Q8 activations): per row
                                  a = clamp(rint(v / s), -127, 127), s = 2^(e - 7) with max|v| in
                                  [2^(e-1), 2^e), for the layer input and the SwiGLU output; one
                                  int8 digit instead of the default two (15-bit values).  Router
                                  and shared expert unchanged.  Not with DECODE_VALU */
    MOE_Q2_GU_Q4 = 256,        /* routed gate/up matrices in the 4-bit sibling format (below) */
    MOE_Q2_DOWN_Q4 = 512       /* routed down matrix in the 4-bit sibling format.  Either Q4
                                  flag with DECODE_VALU: EUNSUPPORTED */
};
#define MOE_Q2_PREFILL_MIN_TOKENS 256
/* Token envelope of one call.  n_tokens <= MOE_Q2_MAX_TOKENS, and the activation
 * rows the routed kernels address with 32-bit byte offsets must stay below 2^31 bytes:
 * (n_tokens + 1) * 2 * hidden <= INT32_MAX and (n_tokens * topk + 1) * 2 * inter <=
 * INT32_MAX.  Larger batches are rejected with MOE_Q2_EUNSUPPORTED before anything
 * is enqueued; the caller splits them into several calls (tokens are independent). */
#define MOE_Q2_MAX_TOKENS 65535

typedef struct {
    int32_t hidden;        /* H: multiple of 256, <= 16384 */
    int32_t inter;         /* I: routed expert intermediate size, multiple of 256, <= 16384 */
    int32_t n_experts;     /* E: 1..512 */
    int32_t shared_inter;  /* Is: shared expert intermediate, multiple of 256, or 0 = none */
    int32_t act_dtype;     /* MOE_Q2_F32 or MOE_Q2_BF16 (ignored under PRE_RMSNORM: x is fp32) */
    int32_t flags;         /* MOE_Q2_PATH_* | MOE_Q2_PRE_RMSNORM | MOE_Q2_RESIDUAL_ADD |
                              MOE_Q2_DECODE_VALU | MOE_Q2_SERIAL | MOE_Q2_BATCH_INVARIANT |
                              MOE_Q2_ACT_Q8 | MOE_Q2_GU_Q4 | MOE_Q2_DOWN_Q4 */
    float   rms_eps;       /* used under MOE_Q2_PRE_RMSNORM */
} moe_q2_shape;

/* Optional device outputs of the routing and bucketing (each pointer nullable).
 * Slot s = t*K + k; bucket order sorts slots by (expert, token).
 * events: nullable host array of 2 * MOE_Q2_N_PHASES hipEvent_t created by the caller;
 * when set, each non-null events[2i] / events[2i+1] is recorded on the stream before /
 * after phase i (phases that do not run record both events back to back; the
 * activation-preparation and shared-expert phases are recorded on the stream
 * they run on). */
typedef struct {
    int32_t *topk_idx;     /* [T, K]  selected experts, descending logit */
    float   *topk_w;       /* [T, K]  renormalised gate weights */
    int32_t *counts;       /* [E]     slots per expert */
    int32_t *offsets;      /* [E + 1] exclusive prefix sum of counts */
    int32_t *perm;         /* [T * K] slot at each bucket position */
    void   **events;       /* [2 * MOE_Q2_N_PHASES] hipEvent_t, nullable */
} moe_q2_trace;

/* Phases of moe_q2_forward (for moe_q2_trace.events); PREP_X and SHARED run on the
 * concurrent branch, the others in this order on the calling stream. */
enum {
    MOE_Q2_PH_RMSNORM = 0,      /* RMSNorm of the residual stream -> bf16 */
    MOE_Q2_PH_ROUTER,           /* router logits */
    MOE_Q2_PH_TOPK,             /* softmax top-K */
    MOE_Q2_PH_BUCKET,           /* histogram, scan, stable permutation, work units */
    MOE_Q2_PH_PREP_X,           /* activation preparation for the routed experts */
    MOE_Q2_PH_GATE_UP,          /* routed Q2 gate/up + SwiGLU */
    MOE_Q2_PH_PREP_H,           /* intermediate preparation */
    MOE_Q2_PH_DOWN,             /* routed Q2 down projection */
    MOE_Q2_PH_SHARED,           /* shared expert (bf16 MFMA) */
    MOE_Q2_PH_COMBINE,          /* weighted combine (+ residual) */
    MOE_Q2_PH_CACHE,            /* expert cache: plan and fill of the missed experts */
    MOE_Q2_N_PHASES
};

/* Bytes of one 84-byte super-block. */
size_t moe_q2_block_bytes(void);

/* Bytes of one Q4 sibling block (148). */
size_t moe_q2_q4_block_bytes(void);

/* Bytes of one routed expert: gate and up (2 * H * I / 256 blocks) and down (H * I / 256
 * blocks), each in the format the shape's flags give; 0 for an invalid shape. */
size_t moe_q2_expert_bytes(const moe_q2_shape *s);

/* Device workspace needed by moe_q2_forward for n_tokens tokens and top-K topk.
 * Returns MOE_Q2_OK and writes *bytes, or an error status for an invalid shape. */
int moe_q2_workspace_size(const moe_q2_shape *s, int32_t n_tokens, int32_t topk,
                          size_t *bytes);

/* How moe_q2_forward runs a shape (host only, nothing is enqueued): the path and
 * routed kernels it picks, whether the shared expert rides in the routed launches,
 * whether the concurrent branch uses the internal stream, and the reduction splits.
 * Returns MOE_Q2_OK and fills *plan, or the status moe_q2_workspace_size returns. */
typedef struct {
    int32_t path;            /* MOE_Q2_PATH_DECODE or MOE_Q2_PATH_PREFILL */
    int32_t routed_kernel;   /* 0 matrix-core decode, 1 vector-ALU decode, 2 matrix-core prefill */
    int32_t shared_fused;    /* 1: shared-expert rows appended to the routed decode launches */
    int32_t side_branch;     /* 1: activation preparation and shared expert on the internal stream */
    int32_t split_gate_up;   /* reduction splits of the routed gate/up and down launches */
    int32_t split_down;
    int32_t router_splits;   /* split-K partial logits of the router */
    int32_t merged;          /* bit 0 / bit 1: the gate/up / down splits are walked by one
                                work-group each (batch-invariant mode on a batch that fills the
                                device unsplit; the same partial sums as one work-group per split) */
    size_t  workspace_bytes;
} moe_q2_plan;
int moe_q2_describe(const moe_q2_shape *s, int32_t n_tokens, int32_t topk, moe_q2_plan *plan);

/* One MoE layer for n_tokens tokens.
 *   x          device [T, H], act_dtype (fp32 under PRE_RMSNORM); 16-byte aligned
 *   router_w   device [E, H] fp32 row-major
 *   experts_q2 device, E experts back to back in the tiled layout above (each
 *              3 * H * I / 256 blocks: 84 bytes, or 148 for the matrices the Q4 flags
 *              name; moe_q2_expert_bytes); 16-byte aligned
 *   shared_w   device bf16 gate [Is, H], up [Is, H], down [H, Is] back to back;
 *              NULL iff shared_inter == 0
 *   topk       K, 1 <= K <= min(E, 16)
 *   out        device [T, H] fp32; written (or accumulated under RESIDUAL_ADD).
 *              out may equal x only under PRE_RMSNORM | RESIDUAL_ADD (residual stream
 *              updated in place); any other overlap is EINVAL.
 *   router_b   device [E] fp32, added to the logits before softmax; nullable
 *   workspace  device scratch of at least moe_q2_workspace_size bytes, 256-byte aligned
 *   trace      host struct of nullable device pointers; nullable
 * n_tokens == 0 is a no-op returning MOE_Q2_OK. */
int moe_q2_forward(const void *x, const float *router_w, const void *experts_q2,
                   const uint16_t *shared_w, int32_t topk, float *out,
                   const moe_q2_shape *s, int32_t n_tokens, const float *router_b,
                   void *workspace, size_t workspace_bytes, const moe_q2_trace *trace,
                   void *stream);

/* Budgeted HBM cache of routed experts whose home is host memory ("DwarfStar (ds4)"
 * (opensourcealternatives.to), section FAQ: routed experts stream from slower storage
 * through an in-memory cache on misses; "DwarfStar 4" (aiany.app), section "What Sets
 * It Apart": configurable expert-cache budgets).  The budget is n_slots expert slots of
 * HBM; a call's touched experts are looked up by key (key_base + expert index, so
 * several layers can share one cache), the missing ones are copied from host memory
 * into slots chosen least-recently-used (ties by slot index; empty slots first), and
 * the routed kernels read every expert from its slot.  Planning and copying run on the
 * device after the bucketing: no host synchronisation, capturable in a HIP graph.
 * The caller owns every buffer; calls that share a cache must be ordered on one stream.
 * Policy MOE_Q2_CACHE_LRU: missing experts (in key order) take the slots this call
 * does not use in least-recently-used order.  MOE_Q2_CACHE_LRU_ADMIT adds frequency
 * admission: a missing expert takes its slot only if the key the slot holds was touched
 * by fewer calls (empty slots always); otherwise it is read from host memory for this
 * call and the slot keeps its key -- frequently used experts stay resident under a
 * skewed routing.
 * state (int32, device): [0] call clock, [1] hits, [2] misses (cumulative), [3] misses and
 * [4] touched experts of the last call, [5] misses of the last call read from host
 * memory uncached, [6] such misses (cumulative), [7] 0, then slot_key[n_slots] (-1:
 * empty), slot_stamp[n_slots] (clock of the last call that used the slot, 0: empty),
 * key_slot[n_keys] (-1: absent), key_count[n_keys] (calls that touched the key,
 * saturating at 2^31 - 1).  Cumulative counters wrap modulo 2^32; when the clock
 * reaches 2^30 the next call renumbers the used slots' stamps 1, 2, ... in their
 * (stamp, slot index) order and restarts the clock there, so the policy never sees an
 * overflow and its decisions do not change. */
#define MOE_Q2_CACHE_MAX_SLOTS 2048
enum { MOE_Q2_CACHE_LRU = 0, MOE_Q2_CACHE_LRU_ADMIT = 1 };
typedef struct {
    void    *slots;       /* device, n_slots * slot_bytes, 16-byte aligned: the budget */
    int64_t  slot_bytes;  /* >= moe_q2_expert_bytes of every layer using the cache, multiple of 16 */
    int32_t  n_slots;     /* 1 .. MOE_Q2_CACHE_MAX_SLOTS */
    int32_t  n_keys;      /* valid keys 0 .. n_keys - 1 */
    int32_t *state;       /* device, moe_q2_cache_state_bytes(n_slots, n_keys) bytes */
    int32_t  policy;      /* MOE_Q2_CACHE_LRU or MOE_Q2_CACHE_LRU_ADMIT */
    int32_t  reserved;    /* 0 */
} moe_q2_cache;

/* Bytes of a cache's state; 0 for n_slots or n_keys out of range. */
size_t moe_q2_cache_state_bytes(int32_t n_slots, int32_t n_keys);

/* Empties the cache (writes its initial state with a kernel on `stream`). */
int moe_q2_cache_reset(const moe_q2_cache *cache, void *stream);

/* moe_q2_forward with the routed experts in host memory behind `cache`:
 *   host_experts  the layer's E experts back to back (moe_q2_expert_bytes(s) each, the
 *                 tiled layout), in pinned host memory (hipHostMalloc, or a pinned torch
 *                 tensor); checked with hipPointerGetAttributes, EINVAL for other memory
 *   key_base      the layer's first key: expert e has key key_base + e (key_base >= 0,
 *                 key_base + E <= n_keys)
 * A call that touches more missing experts than the slots its hits leave free caches
 * the first ones (in key order) and reads the rest straight from host memory for that
 * call.  Not with MOE_Q2_DECODE_VALU.  The results are those of moe_q2_forward on the
 * same experts resident in HBM, bit for bit.  The workspace is moe_q2_workspace_size's. */
int moe_q2_forward_cached(const void *x, const float *router_w, const void *host_experts, int32_t key_base,
                          const moe_q2_cache *cache, const uint16_t *shared_w, int32_t topk, float *out,
                          const moe_q2_shape *s, int32_t n_tokens, const float *router_b,
                          void *workspace, size_t workspace_bytes, const moe_q2_trace *trace, void *stream);

/* moe_q2_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer, the same kernels and results, without the workspace arguments.  The
 * workspace is a fixed array of MOE_Q2_NOALLOC_MAX_BYTES per device inside the
 * library's device code (allocated when the library's code is loaded on a device,
 * held until the process ends; its address is looked up once per device).  A call
 * whose moe_q2_workspace_size exceeds it returns MOE_Q2_EUNSUPPORTED before anything
 * is enqueued (128 MiB holds decode batches up to about 150 tokens of the
 * DeepSeek-class shape: hidden 7168, 256 experts, top-8, intermediate 2048).
 * Every launch stays on `stream` (as under MOE_Q2_SERIAL: no internal stream is
 * created) and no memory is allocated or freed.  All calls on one device share the
 * array and it keeps the last call's contents: calls that overlap in time on one
 * device (several streams or host threads) race and must be ordered by the caller;
 * no call needs any of it to start at zero. */
#define MOE_Q2_NOALLOC_MAX_BYTES (128u << 20)
int moe_q2_forward_noalloc(const void *x, const float *router_w, const void *experts_q2,
                           const uint16_t *shared_w, int32_t topk, float *out,
                           const moe_q2_shape *s, int32_t n_tokens, const float *router_b,
                           const moe_q2_trace *trace, void *stream);

/* Quantize a row-major fp32 matrix w [rows, k] (device, 16-byte aligned; k a multiple
 * of 256, so every row is k / 256 blocks along its reduction dimension) into
 * rows * k / 256 84-byte blocks (device, row-major: block b of row r at index
 * r * k / 256 + b) with the coverage round-to-nearest rule, all steps in IEEE fp32:
 *   lo_j = min(0, min x), hi_j = max x per group; dmin = least fp16 >= max_j(0-lo_j)/15;
 *   m_j = ceil((0-lo_j)/dmin); o_j = dmin*m_j; s_j = (hi_j+o_j)/3;
 *   d = least fp16 >= max_j s_j/15; sc_j = ceil(s_j/d); q = clamp(rint((x+o_j)/(d*sc_j)),0,3).
 * Setup helper, not part of the layer.  Blocks whose scale would overflow fp16 are
 * written with d = dmin = +inf. */
int moe_q2_quantize(const float *w, int64_t rows, int64_t k, void *blocks_out, void *stream);

/* moe_q2_quantize for the Q4 sibling format: rows * k / 256 148-byte blocks, by the
 * same coverage rule with 15 code steps and 3-bit group scales (all steps IEEE fp32):
 *   dmin = least fp16 >= max_j(0-lo_j)/15; m_j = ceil((0-lo_j)/dmin); o_j = dmin*m_j;
 *   s_j = (hi_j+o_j)/15; d = least fp16 >= max_j s_j/7; sc_j = ceil(s_j/d);
 *   q = clamp(rint((x+o_j)/(d*sc_j)),0,15).  Setup helper, not part of the layer. */
int moe_q2_quantize_q4(const float *w, int64_t rows, int64_t k, void *blocks_out, void *stream);

/* Pack one routed expert from row-major block matrices (device): gate [I rows x H/256
 * blocks], up [I x H/256], down [H x I/256], each in the format s->flags give
 * (MOE_Q2_GU_Q4 / MOE_Q2_DOWN_Q4) -> out (device, moe_q2_expert_bytes(s) bytes) in the
 * tiled layout above; 4-byte aligned buffers.  Setup helper, not part of the layer. */
int moe_q2_pack_expert(const void *gate, const void *up, const void *down, const moe_q2_shape *s,
                       void *out, void *stream);

/* Seeded synthetic inputs for tests and benchmarks (not part of the layer):
 * value j = float(S(start + j) - 262140) * scale, where S(i) is the sum of the eight
 * 16-bit halves of Philox4x32-10 (Salmon et al., SC'11) on counter
 * (i_lo, i_hi, stream_lo, stream_hi) under key (seed_lo, seed_hi).  out_dtype
 * MOE_Q2_F32 writes fp32, MOE_Q2_BF16 writes the fp32 value rounded to bf16 (nearest even). */
int moe_q2_synth_normal(uint64_t seed, uint64_t stream_id, uint64_t start, int64_t n,
                        float scale, int32_t out_dtype, void *out, void *stream);

/* Static description of a status code. */
const char *moe_q2_status_string(int status);

/* hipError_t of the last failing HIP call made by this library on this thread. */
int moe_q2_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_Q2_H */
