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
 *     fork/join is legal under graph capture).  The internal stream and its
 *     three events are created by the first call on a device and kept until
 *     the process ends; calls from several host threads on one device enqueue
 *     one at a time.  MOE_Q2_SERIAL keeps every launch on `stream` and touches
 *     no internal state;
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
    MOE_Q2_PATH_PREFILL = 2,   /* force the prefill kernels (up to 64 slots per work unit) */
    MOE_Q2_PRE_RMSNORM = 4,    /* x is the fp32 residual stream h; the layer input is
                                  bf16(h / sqrt(mean(h^2) + rms_eps)) (unit gain) */
    MOE_Q2_RESIDUAL_ADD = 8,   /* out += layer(...) instead of out = layer(...) */
    MOE_Q2_DECODE_VALU = 16,   /* decode path: routed experts on the vector-ALU dot-product
                                  kernel instead of the integer matrix-core kernel */
    MOE_Q2_SERIAL = 32         /* run every launch on `stream` (no internal stream) */
};
#define MOE_Q2_PREFILL_MIN_TOKENS 256

typedef struct {
    int32_t hidden;        /* H: multiple of 256, <= 16384 */
    int32_t inter;         /* I: routed expert intermediate size, multiple of 256, <= 16384 */
    int32_t n_experts;     /* E: 1..512 */
    int32_t shared_inter;  /* Is: shared expert intermediate, multiple of 256, or 0 = none */
    int32_t act_dtype;     /* MOE_Q2_F32 or MOE_Q2_BF16 (ignored under PRE_RMSNORM: x is fp32) */
    int32_t flags;         /* MOE_Q2_PATH_* | MOE_Q2_PRE_RMSNORM | MOE_Q2_RESIDUAL_ADD |
                              MOE_Q2_DECODE_VALU | MOE_Q2_SERIAL */
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
    MOE_Q2_N_PHASES
};

/* Bytes of one 84-byte super-block. */
size_t moe_q2_block_bytes(void);

/* Bytes of one routed expert: 3 * H * I / 256 blocks (gate, up, down). */
size_t moe_q2_expert_bytes(const moe_q2_shape *s);

/* Device workspace needed by moe_q2_forward for n_tokens tokens and top-K topk.
 * Returns MOE_Q2_OK and writes *bytes, or an error status for an invalid shape. */
int moe_q2_workspace_size(const moe_q2_shape *s, int32_t n_tokens, int32_t topk,
                          size_t *bytes);

/* One MoE layer for n_tokens tokens.
 *   x          device [T, H], act_dtype (fp32 under PRE_RMSNORM); 16-byte aligned
 *   router_w   device [E, H] fp32 row-major
 *   experts_q2 device, E experts back to back in the tiled layout above (each
 *              3 * H * I / 256 blocks of 84 bytes); 16-byte aligned
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

/* Quantize n_blocks * 256 fp32 weights (device, contiguous; every 256 consecutive
 * values form one block) into n_blocks 84-byte blocks (device) with the coverage
 * round-to-nearest rule, all steps in IEEE fp32:
 *   lo_j = min(0, min x), hi_j = max x per group; dmin = least fp16 >= max_j(0-lo_j)/15;
 *   m_j = ceil((0-lo_j)/dmin); o_j = dmin*m_j; s_j = (hi_j+o_j)/3;
 *   d = least fp16 >= max_j s_j/15; sc_j = ceil(s_j/d); q = clamp(rint((x+o_j)/(d*sc_j)),0,3).
 * Setup helper, not part of the layer.  Blocks whose scale would overflow fp16 are
 * written with d = dmin = +inf. */
int moe_q2_quantize(const float *w, int64_t n_blocks, void *blocks_out, void *stream);

/* Pack one routed expert from row-major Q2 matrices (device): gate [I rows x H/256
 * blocks], up [I x H/256], down [H x I/256] -> out (device, moe_q2_expert_bytes bytes)
 * in the tiled layout above.  Setup helper, not part of the layer. */
int moe_q2_pack_expert(const void *gate, const void *up, const void *down, int32_t hidden,
                       int32_t inter, void *out, void *stream);

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
