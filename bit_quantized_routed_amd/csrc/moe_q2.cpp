// Host side of the MoE-Q2 C ABI: validation, workspace carving, path choice and
// stream-ordered launches.  No allocation, no host synchronisation.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

static thread_local int g_last_hip_error = 0;

int mq_fail_hip(hipError_t e) {
    g_last_hip_error = (int)e;
    return MOE_Q2_EHIP;
}

extern "C" int moe_q2_last_hip_error(void) { return g_last_hip_error; }

extern "C" const char *moe_q2_status_string(int status) {
    switch (status) {
    case MOE_Q2_OK: return "ok";
    case MOE_Q2_EINVAL: return "invalid argument";
    case MOE_Q2_EUNSUPPORTED: return "unsupported shape or option";
    case MOE_Q2_EWORKSPACE: return "workspace missing or too small";
    case MOE_Q2_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

extern "C" size_t moe_q2_block_bytes(void) { return MQ_BLOCK_BYTES; }

extern "C" size_t moe_q2_q4_block_bytes(void) { return 4 * MQ_BD4; }

// Block bytes of the gate/up and of the down matrices of a shape's routed experts.
static size_t gu_block_bytes(const moe_q2_shape *s) { return s->flags & MOE_Q2_GU_Q4 ? 4 * MQ_BD4 : 4 * MQ_BD2; }
static size_t down_block_bytes(const moe_q2_shape *s) { return s->flags & MOE_Q2_DOWN_Q4 ? 4 * MQ_BD4 : 4 * MQ_BD2; }

static bool shape_ok(const moe_q2_shape *s) {
    if (!s) return false;
    if (s->hidden <= 0 || s->hidden % 256 || s->hidden > 16384) return false;
    if (s->inter <= 0 || s->inter % 256 || s->inter > 16384) return false;
    if (s->n_experts < 1 || s->n_experts > 512) return false;
    if (s->shared_inter < 0 || s->shared_inter % 256 || s->shared_inter > 16384) return false;
    return true;
}

extern "C" size_t moe_q2_expert_bytes(const moe_q2_shape *s) {
    if (!shape_ok(s)) return 0;
    const size_t blocks = (size_t)s->hidden * s->inter / MQ_QK;
    return 2 * blocks * gu_block_bytes(s) + blocks * down_block_bytes(s);
}

namespace {
struct Workspace {
    size_t total = 0;
    size_t logits, idx, gate, counts, offsets, perm, inv, units_hdr, units, urow = 0, bchunk = 0, xbf, xq, xg, xs, h,
        hq, hg, hs, y, xlo, sp, shi, slo, ysh, eslot, misses, nmiss;
    int max_units = 0, split_gu = 1, split_d = 1, rsplit = 1;
    int nd = 2;                 // activation digits: 2 (15-bit) or 1 (Q8)
    bool bi = false;            // batch-invariant: splits and router fixed by the shape
    int split_units = 0;        // unit count the decode k-split policy is computed for
    // routed path and, for the matrix-core decode kernels, their reduction splits
    bool prefill = false, valu = false;
    // prefill token fragments per unit (units of 16 pf_mf slots, one bucketing for both
    // launches): 4 when a 4-bit matrix meets two-digit activations (LDS), else 5
    int pf_mf = PF_MF;
    int dec_units = 0, dsplit_gu = 1, dsplit_d = 1, max_split_gu = 1, max_split_d = 1;
    // batch-invariant on a batch that fills the device unsplit: one work-group walks
    // all of a fixed split's k ranges (same partials, fewer work-groups)
    bool merge_gu = false, merge_d = false;
    // shared expert fused into the matrix-core decode launches (bf16 layer input)
    bool fused = false, prep_in_down = false;
    int fsplit_gu = 1, fsplit_d = 1;
    size_t fgu = 0, fd = 0;
};

// Upper bound on the work units of a bucketing with `tch` slots per unit.
int units_bound(size_t S, size_t E, int tch) {
    return (int)((S + tch - 1) / tch + (S < E ? S : E));
}

size_t take(size_t &cursor, size_t bytes) {
    const size_t at = cursor;
    cursor += (bytes + 255) & ~(size_t)255;
    return at;
}

Workspace carve(const moe_q2_shape *s, int T, int K) {
    Workspace w;
    const size_t H = s->hidden, I = s->inter, E = s->n_experts;
    const size_t S = (size_t)T * K;
    size_t c = 0;
    // work units: at most ceil(S / tch) + min(E, S) for either kernel's unit size
    w.max_units = units_bound(S, E, FD_TCH);
    w.bi = (s->flags & MOE_Q2_BATCH_INVARIANT) != 0;
    w.nd = (s->flags & MOE_Q2_ACT_Q8) ? 1 : 2;
    const bool q4 = (s->flags & (MOE_Q2_GU_Q4 | MOE_Q2_DOWN_Q4)) != 0;
    // a batch-invariant call keeps one set of kernels for every batch size
    w.prefill = !w.bi &&
                ((s->flags & MOE_Q2_PATH_PREFILL) ||
                 (!(s->flags & MOE_Q2_PATH_DECODE) && T >= MOE_Q2_PREFILL_MIN_TOKENS));
    w.valu = !w.prefill && (s->flags & MOE_Q2_DECODE_VALU) != 0;
    if (q4 && w.nd == 2) w.pf_mf = 4;
    int cps = 0;
    if (!w.prefill && !w.valu) {
        w.dec_units = units_bound(S, E, MMA_TCH);
        // batch-invariant: the splits of a one-token batch (under the batch-invariant
        // limits), whatever the batch
        w.split_units = w.bi ? units_bound((size_t)K, E, MMA_TCH) : w.dec_units;
        w.max_split_gu = w.bi ? MQ_DEC_SPLIT_GU_BI : MQ_DEC_SPLIT_GU;
        w.max_split_d = w.bi ? MQ_DEC_SPLIT_D_BI : MQ_DEC_SPLIT_D;
        mq_dec_split(w.split_units, (int)(I / 32), (int)(H / MQ_QK), w.max_split_gu, &w.dsplit_gu, &cps);
        mq_dec_split(w.split_units, (int)(H / 64), (int)(I / MQ_QK), w.max_split_d, &w.dsplit_d, &cps);
        if (w.bi) {
            int own = 1;
            mq_dec_split(w.dec_units, (int)(I / 32), (int)(H / MQ_QK), w.max_split_gu, &own, &cps);
            w.merge_gu = own == 1 && w.dsplit_gu > 1;
            mq_dec_split(w.dec_units, (int)(H / 64), (int)(I / MQ_QK), w.max_split_d, &own, &cps);
            w.merge_d = own == 1 && w.dsplit_d > 1;
        }
    }
    w.rsplit = w.bi ? mq_router_splits_fixed((int)H) : mq_router_splits(T, (int)H, (int)E);
    w.logits = take(c, (size_t)w.rsplit * T * E * 4);
    w.idx = take(c, S * 4);
    w.gate = take(c, S * 4);
    w.counts = take(c, E * 4);
    w.offsets = take(c, (E + 1) * 4);
    w.perm = take(c, S * 4);
    w.inv = take(c, S * 4);
    w.units_hdr = take(c, 16);
    // expert cache of a call (moe_q2_forward_cached): slot per expert, miss list
    w.eslot = take(c, E * 8);
    w.misses = take(c, E * 8);
    w.nmiss = take(c, 16);
    w.units = take(c, (size_t)w.max_units * 16);
    if (w.dec_units) w.urow = take(c, (size_t)w.dec_units * MMA_TCH * 4);   // row table of the units
    if (T >= MQ_BUCKET_PAR_MIN_T)                   // per-chunk expert counts of the large-batch bucketing
        w.bchunk = take(c, (size_t)mq_bucket_chunks(T) * E * 4);
    // activation buffers hold one extra row: the all-zero row that padding tokens
    // of the decode kernels read; h and y one extra row that absorbs their writes
    w.xbf = take(c, (size_t)T * H * 2);
    w.xq = take(c, (size_t)(T + 1) * H * w.nd);  // fp16 pairs, or the int8 digits
    w.xg = take(c, (size_t)(T + 1) * (H / 16) * 8);
    w.xs = take(c, (size_t)(T + 1) * 4);
    // h: the intermediate (S + 1 rows), or for the matrix-core decode kernels the
    // gate and up split partial sums; y: the routed outputs, or their split partials
    w.h = take(c, (w.prefill || w.valu ? 1 : 2 * (size_t)w.dsplit_gu) * (S + 1) * I * 4);
    w.hq = take(c, (S + 1) * I * w.nd);
    w.hg = take(c, (S + 1) * (I / 16) * 8);
    w.hs = take(c, (S + 1) * 4);
    w.y = take(c, (size_t)w.dsplit_d * (S + 1) * H * 4);
    const size_t Is = s->shared_inter;
    const bool in_bf16 = (s->flags & MOE_Q2_PRE_RMSNORM) || s->act_dtype == MOE_Q2_BF16;
    w.fused = Is > 0 && !w.prefill && !w.valu && in_bf16;
    if (w.fused) {
        // dense partial sums of the shared expert: gate and up [split][T][Is], down [split][T][H]
        int kps = 0;
        mq_dense_split((int)(2 * Is), (int)H, 4, &w.fsplit_gu, &kps);
        mq_dense_split((int)H, (int)Is, 2, &w.fsplit_d, &kps);
        // one token: the down launch prepares its own activations when its LDS holds
        // the shared SwiGLU planes of a work-group's k range (2 x kps bf16)
        w.prep_in_down = T == 1 && I <= MQ_DOWN_PREP_MAX_LEN && 4 * (size_t)kps <= MQ_DOWN_PREP_SHARED_BYTES;
        w.fgu = take(c, (size_t)w.fsplit_gu * T * 2 * Is * 4);
        w.fd = take(c, (size_t)w.fsplit_d * T * H * 4);
        w.shi = take(c, (size_t)T * Is * 2);
        w.slo = take(c, (size_t)T * Is * 2);
    } else if (Is) {
        // split-K policy fixed at 256 compute units so the size does not depend on the device
        w.split_gu = mq_gemm_splits(T, (int)(2 * Is), (int)H, 256);
        w.split_d = mq_gemm_splits(T, (int)H, (int)Is, 256);
        const size_t pgu = (size_t)w.split_gu * T * 2 * Is, pd = (size_t)w.split_d * T * H;
        w.xlo = take(c, (size_t)T * H * 2);
        w.sp = take(c, (pgu > pd ? pgu : pd) * 4);
        w.shi = take(c, (size_t)T * Is * 2);
        w.slo = take(c, (size_t)T * Is * 2);
        if (w.split_d > 1) w.ysh = take(c, (size_t)T * H * 4);
    }
    w.total = c;
    return w;
}

int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}
}  // namespace

static const int KNOWN_FLAGS = MOE_Q2_PATH_DECODE | MOE_Q2_PATH_PREFILL | MOE_Q2_PRE_RMSNORM |
                               MOE_Q2_RESIDUAL_ADD | MOE_Q2_DECODE_VALU | MOE_Q2_SERIAL |
                               MOE_Q2_BATCH_INVARIANT | MOE_Q2_ACT_Q8 | MOE_Q2_GU_Q4 | MOE_Q2_DOWN_Q4;

namespace {
// Joins the concurrent branch back into the calling stream when a call returns
// after the fork without having joined it (an enqueue failed): the caller's stream
// then still depends on everything the call put on the internal stream, so a
// captured graph stays connected and no work is left running unobserved.
struct SideJoin {
    hipEvent_t join = nullptr;
    hipStream_t st = nullptr, sst = nullptr;
    bool pending = false;
    ~SideJoin() {
        if (pending && hipEventRecord(join, sst) == hipSuccess) (void)hipStreamWaitEvent(st, join, 0);
    }
};

// The concurrent branch (activation preparation + shared expert): one internal
// stream and fork / prep / join events per device, created on first use and kept
// for the process.  `mu`
// makes the enqueue of one forward call atomic with respect to other host
// threads, so each join waited on is the one its own call recorded.
struct SideBranch {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, prep = nullptr, join = nullptr;
    bool ready = false;
    std::mutex mu;
};
SideBranch g_side[64];
std::mutex g_side_init;

SideBranch *side_branch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    SideBranch &b = g_side[dev];
    std::lock_guard<std::mutex> g(g_side_init);
    if (!b.ready) {
        if (!b.s && hipStreamCreateWithFlags(&b.s, hipStreamNonBlocking) != hipSuccess) {
            b.s = nullptr;
            return nullptr;
        }
        if (!b.fork && hipEventCreateWithFlags(&b.fork, hipEventDisableTiming) != hipSuccess) {
            b.fork = nullptr;
            return nullptr;
        }
        if (!b.prep && hipEventCreateWithFlags(&b.prep, hipEventDisableTiming) != hipSuccess) {
            b.prep = nullptr;
            return nullptr;
        }
        if (!b.join && hipEventCreateWithFlags(&b.join, hipEventDisableTiming) != hipSuccess) {
            b.join = nullptr;
            return nullptr;
        }
        b.ready = true;
    }
    return &b;
}
}  // namespace

static int check_common(const moe_q2_shape *s, int32_t n_tokens, int32_t topk) {
    if (!s) return MOE_Q2_EINVAL;
    if (!shape_ok(s)) return MOE_Q2_EUNSUPPORTED;
    if (n_tokens < 0) return MOE_Q2_EINVAL;
    if (topk < 1 || topk > 16 || topk > s->n_experts) return MOE_Q2_EINVAL;
    // the token grid of the combine and the 32-bit byte offsets of the activation
    // rows (layer input: T + 1 rows of 2 H bytes; intermediate: T K + 1 rows of 2 I)
    const int64_t T = n_tokens;
    if (T > MOE_Q2_MAX_TOKENS) return MOE_Q2_EUNSUPPORTED;
    if ((T + 1) * 2 * s->hidden > INT32_MAX || (T * topk + 1) * 2 * s->inter > INT32_MAX)
        return MOE_Q2_EUNSUPPORTED;
    if (s->flags & ~KNOWN_FLAGS) return MOE_Q2_EINVAL;
    if ((s->flags & MOE_Q2_PATH_DECODE) && (s->flags & MOE_Q2_PATH_PREFILL)) return MOE_Q2_EINVAL;
    if (!(s->flags & MOE_Q2_PRE_RMSNORM) && s->act_dtype != MOE_Q2_F32 && s->act_dtype != MOE_Q2_BF16)
        return MOE_Q2_EINVAL;
    if ((s->flags & MOE_Q2_PRE_RMSNORM) && !(s->rms_eps >= 0.0f && s->rms_eps < 1e30f))
        return MOE_Q2_EINVAL;
    // combinations of the options
    const int f = s->flags;
    const bool bi = f & MOE_Q2_BATCH_INVARIANT, q8 = f & MOE_Q2_ACT_Q8;
    const bool q4 = f & (MOE_Q2_GU_Q4 | MOE_Q2_DOWN_Q4), valu = f & MOE_Q2_DECODE_VALU;
    if (bi && (f & MOE_Q2_PATH_PREFILL)) return MOE_Q2_EINVAL;     // one kernel set for every batch
    if (valu && (bi || q8 || q4)) return MOE_Q2_EUNSUPPORTED;       // the vector-ALU kernel: 2-bit, 15-bit
    const bool in_bf16 = (f & MOE_Q2_PRE_RMSNORM) || s->act_dtype == MOE_Q2_BF16;
    if (bi && s->shared_inter > 0 && !in_bf16) return MOE_Q2_EUNSUPPORTED;   // shared expert on split GEMMs
    return MOE_Q2_OK;
}

extern "C" int moe_q2_workspace_size(const moe_q2_shape *s, int32_t n_tokens, int32_t topk,
                                     size_t *bytes) {
    if (!bytes) return MOE_Q2_EINVAL;
    const int rc = check_common(s, n_tokens, topk);
    if (rc) return rc;
    *bytes = carve(s, n_tokens, topk).total;
    return MOE_Q2_OK;
}

extern "C" int moe_q2_describe(const moe_q2_shape *s, int32_t n_tokens, int32_t topk, moe_q2_plan *plan) {
    if (!plan) return MOE_Q2_EINVAL;
    const int rc = check_common(s, n_tokens, topk);
    if (rc) return rc;
    const Workspace w = carve(s, n_tokens, topk);
    moe_q2_plan p = {};
    p.path = w.prefill ? MOE_Q2_PATH_PREFILL : MOE_Q2_PATH_DECODE;
    p.routed_kernel = w.prefill ? 2 : (w.valu ? 1 : 0);
    p.shared_fused = w.fused ? 1 : 0;
    p.side_branch = (!(s->flags & MOE_Q2_SERIAL) && !w.fused) ? 1 : 0;
    p.split_gate_up = w.prefill || w.valu ? 1 : w.dsplit_gu;
    p.split_down = w.prefill || w.valu ? 1 : w.dsplit_d;
    p.router_splits = w.rsplit;
    p.merged = (w.merge_gu ? 1 : 0) | (w.merge_d ? 2 : 0);
    p.workspace_bytes = w.total;
    *plan = p;
    return MOE_Q2_OK;
}

static bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

// Argument checks of a forward call that need no workspace (no HIP call).
static int check_forward(const void *x, const float *router_w, const void *experts_q2, const uint16_t *shared_w,
                         int32_t topk, const float *out, const moe_q2_shape *s, int32_t n_tokens) {
    const int rc = check_common(s, n_tokens, topk);
    if (rc) return rc;
    if (!x || !router_w || !experts_q2 || !out) return MOE_Q2_EINVAL;
    if ((s->shared_inter > 0) != (shared_w != nullptr)) return MOE_Q2_EINVAL;
    if (((uintptr_t)x & 15) || ((uintptr_t)experts_q2 & 15) || ((uintptr_t)out & 15) ||
        ((uintptr_t)router_w & 15) || ((uintptr_t)shared_w & 15))
        return MOE_Q2_EINVAL;
    const bool rms = (s->flags & MOE_Q2_PRE_RMSNORM) != 0;
    const bool accum = (s->flags & MOE_Q2_RESIDUAL_ADD) != 0;
    const size_t xbytes = (size_t)n_tokens * s->hidden * ((rms || s->act_dtype == MOE_Q2_F32) ? 4 : 2);
    if (ranges_overlap(x, xbytes, out, (size_t)n_tokens * s->hidden * 4)) {
        if (!(x == (const void *)out && rms && accum)) return MOE_Q2_EINVAL;
    }
    return MOE_Q2_OK;
}

// The layer on a caller's workspace.  serial: keep every launch on `stream` (no
// internal stream), whatever the flags say.
// An expert-cache call: the layer's experts in host memory, its first key, the cache.
struct CacheCall {
    const void *host;
    int key_base;
    const moe_q2_cache *c;
};

// cache: nullable; with it, experts_q2 is the host copy and the routed kernels read
// the cache's slots.
static int forward_impl(const void *x, const float *router_w, const void *experts_q2, const uint16_t *shared_w,
                        int32_t topk, float *out, const moe_q2_shape *s, int32_t n_tokens,
                        const float *router_b, void *workspace, size_t workspace_bytes,
                        const moe_q2_trace *trace, void *stream, bool serial, const CacheCall *cache) {
    int rc = check_forward(x, router_w, experts_q2, shared_w, topk, out, s, n_tokens);
    if (rc) return rc;
    const bool rms = (s->flags & MOE_Q2_PRE_RMSNORM) != 0;
    const bool accum = (s->flags & MOE_Q2_RESIDUAL_ADD) != 0;
    const int T = n_tokens, K = topk, H = s->hidden, I = s->inter, E = s->n_experts;
    if (T == 0) return MOE_Q2_OK;
    const Workspace w = carve(s, T, K);
    if (!workspace || workspace_bytes < w.total) return MOE_Q2_EWORKSPACE;
    if ((uintptr_t)workspace & 255) return MOE_Q2_EINVAL;
    const bool prefill = w.prefill;

    hipStream_t st = (hipStream_t)stream;
    hipEvent_t *ev = trace && trace->events ? (hipEvent_t *)trace->events : nullptr;
    auto mark_on = [&](int phase, int end, hipStream_t on) -> int {
        if (!ev || !ev[2 * phase + end]) return MOE_Q2_OK;
        const hipError_t e = hipEventRecord(ev[2 * phase + end], on);
        return e == hipSuccess ? MOE_Q2_OK : mq_fail_hip(e);
    };
    auto mark = [&](int phase, int end) -> int { return mark_on(phase, end, st); };
#define MQ_PHASE(ph, call)                                                                 \
    do {                                                                                   \
        if ((rc = mark(ph, 0))) return rc;                                                 \
        if ((rc = (call))) return rc;                                                      \
        if ((rc = mark(ph, 1))) return rc;                                                 \
    } while (0)
    // the routed-expert kernels take their phase's events into the launch itself
    auto evk = [&](int phase, int end) -> hipEvent_t { return ev ? ev[2 * phase + end] : nullptr; };
    char *ws = (char *)workspace;
    float *logits = (float *)(ws + w.logits);
    int32_t *idx = (int32_t *)(ws + w.idx);
    float *gate = (float *)(ws + w.gate);
    int32_t *counts = trace && trace->counts ? trace->counts : (int32_t *)(ws + w.counts);
    int32_t *offsets = trace && trace->offsets ? trace->offsets : (int32_t *)(ws + w.offsets);
    int32_t *perm = trace && trace->perm ? trace->perm : (int32_t *)(ws + w.perm);
    int32_t *inv = (int32_t *)(ws + w.inv);
    int32_t *units_hdr = (int32_t *)(ws + w.units_hdr);
    int4 *units = (int4 *)(ws + w.units);
    // matrix-core decode: unit records padded to the grid's unit count, row table
    const bool dec_mma = w.dec_units > 0;
    int32_t *urow = dec_mma ? (int32_t *)(ws + w.urow) : nullptr;
    const int fill_units = dec_mma ? w.dec_units : 0;

    // layer input
    const void *xin = x;
    int xin_bf16 = s->act_dtype == MOE_Q2_BF16;
    if (rms) {
        uint16_t *xbf = (uint16_t *)(ws + w.xbf);
        MQ_PHASE(MOE_Q2_PH_RMSNORM, mq_launch_rmsnorm((const float *)x, T, H, s->rms_eps, xbf, st));
        xin = xbf;
        xin_bf16 = 1;
    }
    // The matrix-core decode path with a bf16 layer input runs the shared expert
    // inside the routed launches (appended dense work-groups), all on `stream`.
    // Otherwise the work that depends on the layer input only -- the routed
    // experts' activation preparation and the shared expert (full-precision bf16
    // weights on MFMA, weight 1) -- runs as a branch concurrent with the routing
    // (forked here; the routed experts wait for the preparation, the combine for
    // the whole branch) unless MOE_Q2_SERIAL is set.
    const bool valu = w.valu;
    float *ysh = nullptr;
    int ysh_split = 1;
    int64_t ysh_stride = 0;
    SideBranch *side = nullptr;
    std::unique_lock<std::mutex> side_lock;
    SideJoin side_join;                  // declared after the lock: runs before the unlock
    hipStream_t sst = st;
    if (!serial && !(s->flags & MOE_Q2_SERIAL) && !w.fused) {
        side = side_branch();
        if (side) {
            side_lock = std::unique_lock<std::mutex>(side->mu);
            hipError_t e = hipEventRecord(side->fork, st);
            if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
            if (e != hipSuccess) return mq_fail_hip(e);
            sst = side->s;
            side_join.join = side->join;
            side_join.st = st;
            side_join.sst = sst;
            side_join.pending = true;
        }
    }
    uint32_t *xq = (uint32_t *)(ws + w.xq);
    float2 *xg = (float2 *)(ws + w.xg);
    float *xs = (float *)(ws + w.xs);
    // on one stream with a bf16 input, the router launch also prepares the digits
    const bool prep_in_router = !side && !valu && xin_bf16;
    if ((rc = mark_on(MOE_Q2_PH_PREP_X, 0, sst))) return rc;
    if (valu)
        rc = mq_launch_prep(xin, xin_bf16, T, H, H, xq, xg, xs, sst);
    else if (!prep_in_router)
        rc = mq_launch_prep_digits(xin, xin_bf16, T, H, H, xq, (uint32_t *)xg, xs, w.nd, sst);
    if (rc) return rc;
    if ((rc = mark_on(MOE_Q2_PH_PREP_X, 1, sst))) return rc;
    if (side) {
        const hipError_t e = hipEventRecord(side->prep, sst);
        if (e != hipSuccess) return mq_fail_hip(e);
    }
    if ((rc = mark_on(MOE_Q2_PH_SHARED, 0, sst))) return rc;
    if (s->shared_inter > 0 && !w.fused) {
        const int Is = s->shared_inter;
        const uint16_t *xa = (const uint16_t *)xin, *xa_lo = nullptr;
        if (!xin_bf16) {
            uint16_t *hi = (uint16_t *)(ws + w.xbf), *lo = (uint16_t *)(ws + w.xlo);
            if ((rc = mq_launch_split_bf16((const float *)xin, (int64_t)T * H, hi, lo, sst))) return rc;
            xa = hi;
            xa_lo = lo;
        }
        float *P = (float *)(ws + w.sp);
        uint16_t *shi = (uint16_t *)(ws + w.shi), *slo = (uint16_t *)(ws + w.slo);
        if (w.split_gu == 1 && T > 64) {                // SwiGLU in the product's epilogue
            if ((rc = mq_launch_gemm_bf16_swiglu(xa, xa_lo, H, shared_w, H, T, Is, H, shi, slo, sst)))
                return rc;
        } else {
            if ((rc = mq_launch_gemm_bf16(xa, xa_lo, H, shared_w, H, T, 2 * Is, H, w.split_gu, P, sst)))
                return rc;
            if ((rc = mq_launch_swiglu_partials(P, w.split_gu, T, Is, shi, slo, sst))) return rc;
        }
        if ((rc = mq_launch_gemm_bf16(shi, slo, Is, shared_w + (size_t)2 * Is * H, Is, T, H, Is,
                                      w.split_d, P, sst)))
            return rc;
        if (w.split_d == 1) {
            ysh = P;                                     // one split: the product is the sum
        } else {
            ysh = (float *)(ws + w.ysh);
            if ((rc = mq_launch_sum_partials(P, w.split_d, (int64_t)T * H, ysh, sst))) return rc;
        }
    }
    if ((rc = mark_on(MOE_Q2_PH_SHARED, 1, sst))) return rc;
    if (side) {
        const hipError_t e = hipEventRecord(side->join, sst);
        if (e != hipSuccess) return mq_fail_hip(e);
    }

    // routing
    // bf16 activations: MFMA router (split-K partials); fp32 activations: vector-ALU router
    int nsplit = 1;
    if (xin_bf16 && prep_in_router) {
        nsplit = w.rsplit;
        MQ_PHASE(MOE_Q2_PH_ROUTER, mq_launch_router_prep((const uint16_t *)xin, router_w, T, H, E, nsplit,
                                                         logits, xq, (uint32_t *)xg, xs, w.nd, w.bi ? 1 : 0, st));
    } else if (xin_bf16) {
        nsplit = w.rsplit;
        MQ_PHASE(MOE_Q2_PH_ROUTER, mq_launch_router_mma((const uint16_t *)xin, router_w, T, H, E, nsplit,
                                                        logits, w.bi ? 1 : 0, st));
    } else {
        MQ_PHASE(MOE_Q2_PH_ROUTER, mq_launch_router(xin, 0, router_w, nullptr, T, H, E, logits, st));
    }
    // few tokens: the bucketing runs in the top-K launch (its phase then reads zero),
    // or, on the matrix-core decode path, inside the gate/up launch (both phases zero)
    const int tch = valu ? FD_TCH : (prefill ? 16 * w.pf_mf : MMA_TCH);
    const bool route_in_gu = !cache && !valu && !prefill && nsplit == 1 && T <= MQ_TOPK_BUCKET_MAX_T &&
                             E <= MQ_ROUTE_MAX_E && K <= 16;
    MqRoute rt = {};
    if (route_in_gu) {
        rt = MqRoute{logits, router_b, T, (int)E, K, idx, gate, trace ? trace->topk_idx : nullptr,
                     trace ? trace->topk_w : nullptr, counts, offsets, perm, inv, units_hdr, units, fill_units,
                     urow, T};
        MQ_PHASE(MOE_Q2_PH_TOPK, MOE_Q2_OK);
        MQ_PHASE(MOE_Q2_PH_BUCKET, MOE_Q2_OK);
    } else if (T <= MQ_TOPK_BUCKET_MAX_T) {
        MQ_PHASE(MOE_Q2_PH_TOPK, mq_launch_topk_bucket(logits, nsplit, router_b, T, E, K, idx, gate,
                                                       trace ? trace->topk_idx : nullptr,
                                                       trace ? trace->topk_w : nullptr, tch, counts,
                                                       offsets, perm, inv, units_hdr, units, fill_units,
                                                       urow, T, st));
        MQ_PHASE(MOE_Q2_PH_BUCKET, MOE_Q2_OK);
    } else {
        MQ_PHASE(MOE_Q2_PH_TOPK, mq_launch_topk(logits, nsplit, router_b, T, E, K, idx, gate,
                                                trace ? trace->topk_idx : nullptr,
                                                trace ? trace->topk_w : nullptr, st));
        if (!urow && T >= MQ_BUCKET_PAR_MIN_T)
            MQ_PHASE(MOE_Q2_PH_BUCKET, mq_launch_bucket_par(idx, T, K, E, tch, counts, offsets, perm, inv,
                                                            units_hdr, units, fill_units,
                                                            (int32_t *)(ws + w.bchunk), st));
        else
            MQ_PHASE(MOE_Q2_PH_BUCKET, mq_launch_bucket(idx, T, K, E, tch, counts, offsets, perm, inv,
                                                        units_hdr, units, fill_units, urow, T, st));
    }
    if (side) {
        const hipError_t e = hipStreamWaitEvent(st, side->prep, 0);
        if (e != hipSuccess) return mq_fail_hip(e);
    }
    // routed experts
    const int ncu = device_cus();
    const int64_t ebytes = (int64_t)moe_q2_expert_bytes(s);
    // expert cache: plan the call from the bucketing's counts, copy the misses from
    // host memory, then read every routed expert from its slot
    const uint64_t *eptr = nullptr;
    if (cache) {
        uint64_t *ep = (uint64_t *)(ws + w.eslot);
        int32_t *nm = (int32_t *)(ws + w.nmiss);
        int2 *ml = (int2 *)(ws + w.misses);
        MQ_PHASE(MOE_Q2_PH_CACHE, (rc = mq_launch_cache_plan(counts, E, cache->key_base, cache->c->state,
                                                             cache->c->n_slots, cache->c->n_keys, cache->c->slots,
                                                             cache->c->slot_bytes, cache->host, ebytes, ep, ml, nm,
                                                             cache->c->policy, st))
                                      ? rc
                                      : mq_launch_cache_fill(cache->host, ebytes, cache->c->slots,
                                                             cache->c->slot_bytes, ml, nm, ncu, st));
        eptr = ep;
    } else if ((rc = mark(MOE_Q2_PH_CACHE, 0)) || (rc = mark(MOE_Q2_PH_CACHE, 1))) {
        return rc;
    }
    const int64_t mat_gu = (int64_t)I * (H / MQ_QK) * (int64_t)gu_block_bytes(s);   // bytes of gate (or up)
    const MqFormat fgu = {w.nd, (s->flags & MOE_Q2_GU_Q4) ? MQ_BD4 : MQ_BD2, eptr};
    const MqFormat fdn = {w.nd, (s->flags & MOE_Q2_DOWN_Q4) ? MQ_BD4 : MQ_BD2, eptr};
    float *h = (float *)(ws + w.h);
    float *y = (float *)(ws + w.y);
    uint32_t *hq = (uint32_t *)(ws + w.hq);
    float2 *hg = (float2 *)(ws + w.hg);
    float *hsc = (float *)(ws + w.hs);
    if (valu) {
        MQ_PHASE(MOE_Q2_PH_GATE_UP, mq_launch_q2_dec(1, experts_q2, ebytes, 0, I, H / MQ_QK, units_hdr,
                                                     units, w.max_units, perm, K, xq, xg, xs, h, ncu, st));
        MQ_PHASE(MOE_Q2_PH_PREP_H, mq_launch_prep(h, 0, T * K, I, I, hq, hg, hsc, st));
        MQ_PHASE(MOE_Q2_PH_DOWN, mq_launch_q2_dec(0, experts_q2, ebytes, 2 * mat_gu, H, I / MQ_QK, units_hdr,
                                                  units, w.max_units, perm, K, hq, hg, hsc, y, ncu, st));
    } else if (prefill) {
        if ((rc = mq_launch_q2_mma_pf(1, fgu, experts_q2, ebytes, 0, I, H / MQ_QK, units_hdr, units, w.max_units,
                                      perm, K, xq, (const uint32_t *)xg, xs, h, ncu, w.pf_mf, st,
                                      evk(MOE_Q2_PH_GATE_UP, 0), evk(MOE_Q2_PH_GATE_UP, 1))))
            return rc;
        MQ_PHASE(MOE_Q2_PH_PREP_H, mq_launch_prep_digits(h, 0, T * K, I, I, hq, (uint32_t *)hg, hsc, w.nd, st));
        if ((rc = mq_launch_q2_mma_pf(0, fdn, experts_q2, ebytes, 2 * mat_gu, H, I / MQ_QK, units_hdr, units,
                                      w.max_units, perm, K, hq, (const uint32_t *)hg, hsc, y, ncu, w.pf_mf, st,
                                      evk(MOE_Q2_PH_DOWN, 0), evk(MOE_Q2_PH_DOWN, 1))))
            return rc;
    } else {
        // split partial sums: gate and up [dsplit_gu][S + 1][I], y [dsplit_d][S + 1][H]
        const int S = T * K;
        const int64_t gstride = (int64_t)(S + 1) * I, ystride = (int64_t)(S + 1) * H;
        float *gp = h, *up = h + (int64_t)w.dsplit_gu * gstride;
        MqDenseSpec dgu = {}, dd = {};
        MqSharedSwiglu shs = {};
        if (w.fused) {
            // shared expert rows in the same launches; its outputs are dense partials
            const int Is = s->shared_inter;
            float *fg = (float *)(ws + w.fgu);
            float *fu = fg + (int64_t)w.fsplit_gu * T * Is;
            uint16_t *shi = (uint16_t *)(ws + w.shi), *slo = (uint16_t *)(ws + w.slo);
            dgu = MqDenseSpec{shared_w, (const uint16_t *)xin, nullptr, fg, fu, T, 2 * Is, H, Is, Is,
                              w.fsplit_gu, (int64_t)T * Is};
            shs = MqSharedSwiglu{fg, fu, w.fsplit_gu, (int64_t)T * Is, Is, T, shi, slo};
            ysh = (float *)(ws + w.fd);
            ysh_split = w.fsplit_d;
            ysh_stride = (int64_t)T * H;
            dd = MqDenseSpec{shared_w + (size_t)2 * Is * H, shi, slo, ysh, ysh, T, H, Is, H, H, w.fsplit_d,
                             ysh_stride};
        }
        if ((rc = mq_launch_q2_mma(1, fgu, experts_q2, ebytes, 0, I / 32, H / MQ_QK, units, w.dec_units,
                                   w.split_units, w.max_split_gu, w.merge_gu ? 1 : 0, urow, T, S,
                                   xq, (const uint32_t *)xg, xs, gp, up, I, gstride, w.fused ? &dgu : nullptr,
                                   route_in_gu ? &rt : nullptr, nullptr, st, evk(MOE_Q2_PH_GATE_UP, 0),
                                   evk(MOE_Q2_PH_GATE_UP, 1))))
            return rc;
        // one token (shared expert fused): the down launch prepares its own activations
        const bool prep_in_down = w.prep_in_down;
        MqDownPrep dp = {};
        if (prep_in_down) {
            dp = MqDownPrep{gp, up, w.dsplit_gu, (int)I, gstride, shs.g, shs.u, shs.nsplit, shs.split_stride};
            MQ_PHASE(MOE_Q2_PH_PREP_H, MOE_Q2_OK);
        } else {
            MQ_PHASE(MOE_Q2_PH_PREP_H, mq_launch_prep_swiglu_digits(gp, up, w.dsplit_gu, gstride, S, I, I, hq,
                                                                    (uint32_t *)hg, hsc, w.fused ? &shs : nullptr,
                                                                    w.nd, st));
        }
        if ((rc = mq_launch_q2_mma(0, fdn, experts_q2, ebytes, 2 * mat_gu, H / 64, I / MQ_QK, units,
                                   w.dec_units, w.split_units, w.max_split_d, w.merge_d ? 1 : 0, nullptr, S, S, hq, (const uint32_t *)hg, hsc, y, nullptr, H, ystride,
                                   w.fused ? &dd : nullptr, nullptr, prep_in_down ? &dp : nullptr, st,
                                   evk(MOE_Q2_PH_DOWN, 0), evk(MOE_Q2_PH_DOWN, 1))))
            return rc;
    }
    const int ysplit = (prefill || valu) ? 1 : w.dsplit_d;
    const int64_t ystride = (int64_t)(T * K + 1) * H;
    if (side) {
        const hipError_t e = hipStreamWaitEvent(st, side->join, 0);
        if (e != hipSuccess) return mq_fail_hip(e);
        side_join.pending = false;
    }
    MQ_PHASE(MOE_Q2_PH_COMBINE, mq_launch_combine(y, ysplit, ystride, inv, gate, ysh, ysh_split, ysh_stride, T,
                                                  H, K, accum ? 1 : 0, out, st));
    if (!rms && ev) {
        if ((rc = mark(MOE_Q2_PH_RMSNORM, 0)) || (rc = mark(MOE_Q2_PH_RMSNORM, 1))) return rc;
    }
    return MOE_Q2_OK;
#undef MQ_PHASE
}

extern "C" int moe_q2_forward(const void *x, const float *router_w, const void *experts_q2,
                              const uint16_t *shared_w, int32_t topk, float *out,
                              const moe_q2_shape *s, int32_t n_tokens, const float *router_b,
                              void *workspace, size_t workspace_bytes, const moe_q2_trace *trace,
                              void *stream) {
    return forward_impl(x, router_w, experts_q2, shared_w, topk, out, s, n_tokens, router_b, workspace,
                        workspace_bytes, trace, stream, false, nullptr);
}

// ------------------------------------------------------------------ expert cache
extern "C" size_t moe_q2_cache_state_bytes(int32_t n_slots, int32_t n_keys) {
    if (n_slots < 1 || n_slots > MOE_Q2_CACHE_MAX_SLOTS || n_keys < 1 || n_keys > (1 << 28)) return 0;
    return (size_t)4 * (8 + 2 * (size_t)n_slots + 2 * (size_t)n_keys);
}

static int check_cache(const moe_q2_cache *c) {
    if (!c || !c->slots || !c->state) return MOE_Q2_EINVAL;
    if (!moe_q2_cache_state_bytes(c->n_slots, c->n_keys)) return MOE_Q2_EINVAL;
    if (c->slot_bytes <= 0 || (c->slot_bytes & 15) || ((uintptr_t)c->slots & 15) || ((uintptr_t)c->state & 3))
        return MOE_Q2_EINVAL;
    if ((c->policy != MOE_Q2_CACHE_LRU && c->policy != MOE_Q2_CACHE_LRU_ADMIT) || c->reserved != 0)
        return MOE_Q2_EINVAL;
    return MOE_Q2_OK;
}

extern "C" int moe_q2_cache_reset(const moe_q2_cache *cache, void *stream) {
    const int rc = check_cache(cache);
    if (rc) return rc;
    return mq_launch_cache_reset(cache->state, cache->n_slots, cache->n_keys, (hipStream_t)stream);
}

extern "C" int moe_q2_forward_cached(const void *x, const float *router_w, const void *host_experts,
                                     int32_t key_base, const moe_q2_cache *cache, const uint16_t *shared_w,
                                     int32_t topk, float *out, const moe_q2_shape *s, int32_t n_tokens,
                                     const float *router_b, void *workspace, size_t workspace_bytes,
                                     const moe_q2_trace *trace, void *stream) {
    int rc = check_forward(x, router_w, host_experts, shared_w, topk, out, s, n_tokens);
    if (rc) return rc;
    if ((rc = check_cache(cache))) return rc;
    if (s->flags & MOE_Q2_DECODE_VALU) return MOE_Q2_EUNSUPPORTED;
    const int64_t E = s->n_experts;
    if (key_base < 0 || key_base + E > cache->n_keys) return MOE_Q2_EINVAL;
    if (cache->slot_bytes < (int64_t)moe_q2_expert_bytes(s)) return MOE_Q2_EINVAL;
    if (n_tokens == 0) return MOE_Q2_OK;
    // the host copy must be pinned memory the device can read (a host query; pageable
    // memory would fault the kernels that read it)
    hipPointerAttribute_t pa;
    if (hipPointerGetAttributes(&pa, host_experts) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_Q2_EINVAL;
    }
    if (pa.type != hipMemoryTypeHost || !pa.devicePointer) return MOE_Q2_EINVAL;
    const CacheCall cc = {pa.devicePointer, key_base, cache};
    return forward_impl(x, router_w, host_experts, shared_w, topk, out, s, n_tokens, router_b, workspace,
                        workspace_bytes, trace, stream, false, &cc);
}

// ------------------------------------------------------------------ no-allocation entry point
// The workspace of moe_q2_forward_noalloc: one fixed array per device, part of the
// library's device code object (allocated when the module is loaded on a device and
// held until the process ends).  In host code `scratch` only names the symbol; its
// device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[MOE_Q2_NOALLOC_MAX_BYTES];

namespace {
struct ScratchAddr {
    void *ptr = nullptr;
    bool ready = false;
};
ScratchAddr g_scratch[64];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up once per device (with that
// device current) and kept.
int scratch_address(void **p) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return mq_fail_hip(e);
    if (dev < 0 || dev >= 64) return MOE_Q2_EUNSUPPORTED;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    ScratchAddr &a = g_scratch[dev];
    if (!a.ready) {
        void *q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return mq_fail_hip(e);
        if (!q || ((uintptr_t)q & 255)) return MOE_Q2_EHIP;
        a.ptr = q;
        a.ready = true;
    }
    *p = a.ptr;
    return MOE_Q2_OK;
}
}  // namespace

extern "C" int moe_q2_forward_noalloc(const void *x, const float *router_w, const void *experts_q2,
                                      const uint16_t *shared_w, int32_t topk, float *out,
                                      const moe_q2_shape *s, int32_t n_tokens, const float *router_b,
                                      const moe_q2_trace *trace, void *stream) {
    int rc = check_forward(x, router_w, experts_q2, shared_w, topk, out, s, n_tokens);
    if (rc) return rc;
    if (n_tokens == 0) return MOE_Q2_OK;
    if (carve(s, n_tokens, topk).total > (size_t)MOE_Q2_NOALLOC_MAX_BYTES) return MOE_Q2_EUNSUPPORTED;
    void *ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return forward_impl(x, router_w, experts_q2, shared_w, topk, out, s, n_tokens, router_b, ws,
                        (size_t)MOE_Q2_NOALLOC_MAX_BYTES, trace, stream, true, nullptr);
}
