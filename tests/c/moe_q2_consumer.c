/* A plain C consumer of the library's C ABI (include/moe_q2.h): no C++, no torch.
 *
 *   moe_q2_consumer <dir>
 *
 * reads one layer's inputs from <dir> (meta.txt: "H I E K Is act flags T eps has_bias",
 * then the raw arrays x.bin, router_w.bin, experts.bin, shared.bin (if Is > 0),
 * router_b.bin (if has_bias)), copies them to device memory it allocates with the HIP
 * runtime, sizes and allocates the workspace, runs moe_q2_forward on the default
 * stream with a routing trace, and writes out.bin (fp32 [T, H]) and idx.bin (int32
 * [T, K]).  It also checks that invalid arguments come back as statuses before
 * anything runs.  Exit status 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/moe_q2.h"

static void *read_file(const char *dir, const char *name, size_t want) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    void *p = malloc(want ? want : 1);
    if (!p || fread(p, 1, want, f) != want) { fprintf(stderr, "short read %s\n", path); exit(2); }
    fclose(f);
    return p;
}

static void write_file(const char *dir, const char *name, const void *p, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, n, f) != n) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(f);
}

#define HIPCHECK(call)                                                                    \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
            return 3;                                                                     \
        }                                                                                 \
    } while (0)

static void *to_device(const void *host, size_t n) {
    void *d = NULL;
    if (hipMalloc(&d, n ? n : 1) != hipSuccess) { fprintf(stderr, "hipMalloc failed\n"); exit(3); }
    if (n && hipMemcpy(d, host, n, hipMemcpyHostToDevice) != hipSuccess) { fprintf(stderr, "copy failed\n"); exit(3); }
    return d;
}

int main(int argc, char **argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s <dir>\n", argv[0]); return 1; }
    const char *dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE *mf = fopen(path, "r");
    int H, I, E, K, Is, act, flags, T, has_bias;
    float eps;
    if (!mf || fscanf(mf, "%d %d %d %d %d %d %d %d %f %d", &H, &I, &E, &K, &Is, &act, &flags, &T, &eps,
                      &has_bias) != 10) {
        fprintf(stderr, "bad meta.txt\n");
        return 1;
    }
    fclose(mf);
    moe_q2_shape s;
    memset(&s, 0, sizeof s);
    s.hidden = H; s.inter = I; s.n_experts = E; s.shared_inter = Is;
    s.act_dtype = act; s.flags = flags; s.rms_eps = eps;

    const size_t xb = (size_t)T * H * ((flags & MOE_Q2_PRE_RMSNORM) || act == MOE_Q2_F32 ? 4 : 2);
    const size_t eb = moe_q2_expert_bytes(&s) * (size_t)E;
    const size_t sb = (size_t)3 * Is * H * 2;
    if (!eb) { fprintf(stderr, "moe_q2_expert_bytes: invalid shape\n"); return 1; }
    void *x = read_file(dir, "x.bin", xb);
    void *rw = read_file(dir, "router_w.bin", (size_t)E * H * 4);
    void *ex = read_file(dir, "experts.bin", eb);
    void *sh = Is ? read_file(dir, "shared.bin", sb) : NULL;
    void *rb = has_bias ? read_file(dir, "router_b.bin", (size_t)E * 4) : NULL;

    void *dx = to_device(x, xb), *drw = to_device(rw, (size_t)E * H * 4), *dex = to_device(ex, eb);
    void *dsh = Is ? to_device(sh, sb) : NULL, *drb = has_bias ? to_device(rb, (size_t)E * 4) : NULL;
    float *dout = NULL;
    int32_t *didx = NULL;
    HIPCHECK(hipMalloc((void **)&dout, (size_t)T * H * 4));
    HIPCHECK(hipMalloc((void **)&didx, (size_t)T * K * 4));
    if (flags & MOE_Q2_RESIDUAL_ADD) HIPCHECK(hipMemset(dout, 0, (size_t)T * H * 4));

    /* invalid arguments: statuses, nothing enqueued */
    size_t ws_bytes = 0;
    int rc = moe_q2_workspace_size(&s, T, 0, &ws_bytes);
    if (rc != MOE_Q2_EINVAL) { fprintf(stderr, "topk 0 gave %d\n", rc); return 4; }
    printf("topk 0: %s\n", moe_q2_status_string(rc));
    moe_q2_shape bad = s;
    bad.hidden = H + 1;
    rc = moe_q2_workspace_size(&bad, T, K, &ws_bytes);
    if (rc != MOE_Q2_EUNSUPPORTED) { fprintf(stderr, "hidden %d gave %d\n", H + 1, rc); return 4; }
    printf("hidden %d: %s\n", H + 1, moe_q2_status_string(rc));
    rc = moe_q2_forward(dx, (const float *)drw, dex, (const uint16_t *)dsh, K, dout, &s, T,
                        (const float *)drb, NULL, 0, NULL, NULL);
    if (rc != MOE_Q2_EWORKSPACE) { fprintf(stderr, "no workspace gave %d\n", rc); return 4; }
    printf("no workspace: %s\n", moe_q2_status_string(rc));

    /* the layer */
    rc = moe_q2_workspace_size(&s, T, K, &ws_bytes);
    if (rc) { fprintf(stderr, "workspace_size: %s\n", moe_q2_status_string(rc)); return 4; }
    moe_q2_plan plan;
    rc = moe_q2_describe(&s, T, K, &plan);
    if (rc) { fprintf(stderr, "describe: %s\n", moe_q2_status_string(rc)); return 4; }
    printf("plan: path %d kernel %d shared_fused %d splits %d/%d router_splits %d workspace %zu\n", plan.path,
           plan.routed_kernel, plan.shared_fused, plan.split_gate_up, plan.split_down, plan.router_splits,
           plan.workspace_bytes);
    void *dws = NULL;
    HIPCHECK(hipMalloc(&dws, ws_bytes));
    moe_q2_trace tr;
    memset(&tr, 0, sizeof tr);
    tr.topk_idx = didx;
    rc = moe_q2_forward(dx, (const float *)drw, dex, (const uint16_t *)dsh, K, dout, &s, T, (const float *)drb,
                        dws, ws_bytes, &tr, NULL);
    if (rc) { fprintf(stderr, "forward: %s (hip %d)\n", moe_q2_status_string(rc), moe_q2_last_hip_error()); return 5; }
    HIPCHECK(hipDeviceSynchronize());
    float *out = (float *)malloc((size_t)T * H * 4);
    int32_t *idx = (int32_t *)malloc((size_t)T * K * 4);
    HIPCHECK(hipMemcpy(out, dout, (size_t)T * H * 4, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(idx, didx, (size_t)T * K * 4, hipMemcpyDeviceToHost));
    write_file(dir, "out.bin", out, (size_t)T * H * 4);
    write_file(dir, "idx.bin", idx, (size_t)T * K * 4);
    printf("forward: ok, %d tokens\n", T);
    hipFree(dws); hipFree(dout); hipFree(didx); hipFree(dx); hipFree(drw); hipFree(dex);
    if (dsh) hipFree(dsh);
    if (drb) hipFree(drb);
    free(x); free(rw); free(ex); free(sh); free(rb); free(out); free(idx);
    return 0;
}
