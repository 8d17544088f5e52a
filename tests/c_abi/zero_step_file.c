/*
 * zero_step_file -- drives owned-shard steps through the C ABI of
 * include/zero_dp.h from plain C (no Python, no torch): device memory from
 * the HIP runtime, every other operation a zero_* call.
 *
 * The step is the fused ZeRO-DP owned-partition update: the Nd ranks' fp16
 * gradient slices of the owned window are summed, unscaled and checked for
 * inf/NaN, mixed-precision Adam/AdamW updates the fp32 master, momentum and
 * variance, and the updated fp16 parameters land in the all-gather buffer
 * at the window's offset (upskillscore "ZeRO: partitioning training state
 * across GPUs", section "How it works"; trishampatil "Forward/Backward Under
 * ZeRO-3").  A step whose gradients overflow is skipped on the device.
 *
 *   usage: zero_step_file IN OUT [step|noalloc]
 *
 * IN (little-endian, as written by the test that runs this program):
 *   char[8] "ZDPSTEP1"
 *   int64 n, ag_len, ag_off        window length, all-gather buffer length, window offset
 *   int32 nd, steps
 *   double L, lr, beta1, beta2, eps, weight_decay
 *   float master0[n]               initial fp32 master
 *   uint16 ag0[ag_len]             initial all-gather buffer (fp16 bits)
 *   steps x uint16 slices[nd][n]   each step's gradient slices (fp16 bits)
 * OUT:
 *   char[8] "ZDPOUT01"
 *   per step: int32 cur, t, overflow, 0; double sumsq; int64 skipped;
 *             float master[n], exp_avg[n], exp_avg_sq[n] (the committed set);
 *             uint16 ag[ag_len] (the whole all-gather buffer)
 *
 * The initial window is filled by zero_emit_fp16 from master0 (over ag0's
 * window).  "noalloc" takes each step with zero_adam_step_noalloc instead
 * of zero_adam_step and its workspace.  Exit status 0 on success, 1 on a
 * failed call (the message names it), 2 on bad usage or input.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_dp.h"

static void die(const char* what, const char* msg) {
    fprintf(stderr, "zero_step_file: %s: %s\n", what, msg);
    exit(1);
}

static void hip_ok(hipError_t e, const char* what) {
    if (e != hipSuccess) die(what, hipGetErrorString(e));
}

static void zero_ok(int rc, const char* what) {
    if (rc != ZERO_OK) {
        char msg[256];
        snprintf(msg, sizeof msg, "%s (status %d, hip error %d)", zero_strerror(rc), rc, zero_last_hip_error());
        die(what, msg);
    }
}

static void read_all(FILE* f, void* dst, size_t bytes) {
    if (bytes != 0 && fread(dst, 1, bytes, f) != bytes) {
        fprintf(stderr, "zero_step_file: input ends early\n");
        exit(2);
    }
}

static void write_all(FILE* f, const void* src, size_t bytes) {
    if (bytes != 0 && fwrite(src, 1, bytes, f) != bytes) die("write", "output write failed");
}

static void* host_alloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (p == NULL) die("malloc", "out of host memory");
    return p;
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    hip_ok(hipMalloc(&p, bytes ? bytes : 16), "hipMalloc");
    return p;
}

int main(int argc, char** argv) {
    if (argc < 3 || argc > 4 || (argc == 4 && strcmp(argv[3], "step") != 0 && strcmp(argv[3], "noalloc") != 0)) {
        fprintf(stderr, "usage: zero_step_file IN OUT [step|noalloc]\n");
        return 2;
    }
    const int noalloc = argc == 4 && strcmp(argv[3], "noalloc") == 0;
    if (zero_abi_version() != ZERO_DP_ABI_VERSION) die("zero_abi_version", "library and header disagree");

    FILE* in = fopen(argv[1], "rb");
    if (in == NULL) {
        fprintf(stderr, "zero_step_file: %s: cannot open\n", argv[1]);
        return 2;
    }
    char magic[8];
    int64_t n, ag_len, ag_off;
    int32_t nd, steps;
    double L, lr, beta1, beta2, eps, wd;
    read_all(in, magic, 8);
    read_all(in, &n, 8);
    read_all(in, &ag_len, 8);
    read_all(in, &ag_off, 8);
    read_all(in, &nd, 4);
    read_all(in, &steps, 4);
    read_all(in, &L, 8);
    read_all(in, &lr, 8);
    read_all(in, &beta1, 8);
    read_all(in, &beta2, 8);
    read_all(in, &eps, 8);
    read_all(in, &wd, 8);
    if (memcmp(magic, "ZDPSTEP1", 8) != 0 || n < 0 || n > (INT64_C(1) << 32) || nd < 1 || nd > 4096 ||
        steps < 0 || ag_off < 0 || ag_len < ag_off + n || ag_len > (INT64_C(1) << 33)) {
        fprintf(stderr, "zero_step_file: bad input header\n");
        return 2;
    }

    /* slice k of the owned window at base + k * stride + 8: a stride and an
       offset that are multiples of 8 elements, as the ABI requires */
    const int64_t stride = (n + 7) / 8 * 8 + 16;
    const int64_t elem_off = 8;
    const size_t fbytes = (size_t)n * sizeof(float);
    float* master0 = host_alloc(fbytes);
    uint16_t* ag_host = host_alloc((size_t)ag_len * 2);
    uint16_t* sl_host = host_alloc((size_t)nd * (size_t)stride * 2);
    float* state_host = host_alloc(3 * fbytes);
    memset(sl_host, 0, (size_t)nd * (size_t)stride * 2);
    read_all(in, master0, fbytes);
    read_all(in, ag_host, (size_t)ag_len * 2);

    hipStream_t stream;
    hip_ok(hipStreamCreate(&stream), "hipStreamCreate");
    zero_adam_state st;
    for (int s = 0; s < 2; ++s) {
        st.master[s] = dev_alloc(fbytes);
        st.exp_avg[s] = dev_alloc(fbytes);
        st.exp_avg_sq[s] = dev_alloc(fbytes);
    }
    st.ctl = dev_alloc(sizeof(zero_step_ctl));
    uint16_t* ag = dev_alloc((size_t)ag_len * 2);
    uint16_t* slices = dev_alloc((size_t)nd * (size_t)stride * 2);
    void* workspace = NULL;
    if (!noalloc) {
        const int64_t wsb = zero_workspace_bytes();
        workspace = dev_alloc((size_t)wsb);
        hip_ok(hipMemset(workspace, 0, (size_t)wsb), "hipMemset(workspace)");
    }

    /* committed set 0 = master0 with zero moments; t = 0 */
    zero_step_ctl ctl;
    zero_ctl_init(&ctl, L);
    hip_ok(hipMemcpy(st.master[0], master0, fbytes, hipMemcpyHostToDevice), "hipMemcpy(master)");
    hip_ok(hipMemset(st.exp_avg[0], 0, fbytes), "hipMemset(exp_avg)");
    hip_ok(hipMemset(st.exp_avg_sq[0], 0, fbytes), "hipMemset(exp_avg_sq)");
    hip_ok(hipMemcpy(st.ctl, &ctl, sizeof ctl, hipMemcpyHostToDevice), "hipMemcpy(ctl)");
    hip_ok(hipMemcpy(ag, ag_host, (size_t)ag_len * 2, hipMemcpyHostToDevice), "hipMemcpy(allgather)");
    zero_ok(zero_emit_fp16(st.master[0], n, ag, ag_off, stream), "zero_emit_fp16");

    zero_grad_src src;
    memset(&src, 0, sizeof src);
    src.base = slices;
    src.slice_stride = stride;
    src.elem_off = elem_off;
    src.n = n;
    src.nd = nd;
    src.loss_scale = L;
    zero_adam_hp hp;
    memset(&hp, 0, sizeof hp);
    hp.lr = lr;
    hp.beta1 = beta1;
    hp.beta2 = beta2;
    hp.eps = eps;
    hp.weight_decay = wd;

    FILE* out = fopen(argv[2], "wb");
    if (out == NULL) die(argv[2], "cannot open");
    write_all(out, "ZDPOUT01", 8);
    for (int32_t step = 0; step < steps; ++step) {
        for (int32_t k = 0; k < nd; ++k) read_all(in, sl_host + (size_t)k * (size_t)stride + elem_off, (size_t)n * 2);
        hip_ok(hipMemcpyAsync(slices, sl_host, (size_t)nd * (size_t)stride * 2, hipMemcpyHostToDevice, stream),
               "hipMemcpyAsync(slices)");
        if (noalloc)
            zero_ok(zero_adam_step_noalloc(&src, &st, &hp, ag, ag_off, stream), "zero_adam_step_noalloc");
        else
            zero_ok(zero_adam_step(&src, &st, &hp, ag, ag_off, workspace, stream), "zero_adam_step");
        hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize");
        hip_ok(hipMemcpy(&ctl, st.ctl, sizeof ctl, hipMemcpyDeviceToHost), "hipMemcpy(ctl)");
        const int c = ctl.cur;
        if (c != 0 && c != 1) die("control block", "cur is neither 0 nor 1");
        hip_ok(hipMemcpy(state_host, st.master[c], fbytes, hipMemcpyDeviceToHost), "hipMemcpy(master)");
        hip_ok(hipMemcpy(state_host + n, st.exp_avg[c], fbytes, hipMemcpyDeviceToHost), "hipMemcpy(exp_avg)");
        hip_ok(hipMemcpy(state_host + 2 * n, st.exp_avg_sq[c], fbytes, hipMemcpyDeviceToHost),
               "hipMemcpy(exp_avg_sq)");
        hip_ok(hipMemcpy(ag_host, ag, (size_t)ag_len * 2, hipMemcpyDeviceToHost), "hipMemcpy(allgather)");
        const int32_t head[4] = {ctl.cur, ctl.t, ctl.overflow, 0};
        write_all(out, head, sizeof head);
        write_all(out, &ctl.sumsq, 8);
        write_all(out, &ctl.skipped, 8);
        write_all(out, state_host, 3 * fbytes);
        write_all(out, ag_host, (size_t)ag_len * 2);
    }
    if (fclose(out) != 0) die(argv[2], "close failed");
    fclose(in);

    for (int s = 0; s < 2; ++s) {
        hip_ok(hipFree(st.master[s]), "hipFree");
        hip_ok(hipFree(st.exp_avg[s]), "hipFree");
        hip_ok(hipFree(st.exp_avg_sq[s]), "hipFree");
    }
    hip_ok(hipFree(st.ctl), "hipFree");
    hip_ok(hipFree(ag), "hipFree");
    hip_ok(hipFree(slices), "hipFree");
    if (workspace != NULL) hip_ok(hipFree(workspace), "hipFree");
    hip_ok(hipStreamDestroy(stream), "hipStreamDestroy");
    free(master0);
    free(ag_host);
    free(sl_host);
    free(state_host);
    return 0;
}
