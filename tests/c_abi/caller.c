/*
 * A plain C99 caller of the apexw C ABI: no C++, no Python, no torch.
 *
 *   caller host            state/workspace sizes and argument errors only
 *                          (no GPU needed); prints key=value lines
 *   caller gpu OUT FMT N   allocates with the HIP C runtime API, runs N
 *                          steps of a small mixed-dtype list in state format
 *                          FMT (0 fp32, 1 bf16, 2 8-bit) and writes the
 *                          inputs and results to OUT for the test to check
 *                          against the oracle
 *
 * Inputs come from a fixed xorshift generator in this file: uniform draws
 * scaled like the workloads (theta within 0.02, g within 1e-3), their bit
 * patterns written to OUT as they are uploaded.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "apexw.h"

#define N_T 4

static const int64_t NUMEL[N_T] = {1000, 4096, 77, 2560};
static const int32_t PDT[N_T] = {APEXW_F32, APEXW_BF16, APEXW_F32, APEXW_BF16};
static const int32_t GDT[N_T] = {APEXW_F32, APEXW_F32, APEXW_BF16, APEXW_BF16};
static const int32_t GROUP[N_T] = {0, 1, 0, 1};

static int host_mode(void) {
    size_t sb = 0, wb = 0;
    int rc = apexw_state_bytes(N_T, NUMEL, APEXW_STATE_Q8, &sb);
    printf("state_bytes_q8_rc=%d\nstate_bytes_q8=%zu\n", rc, sb);
    rc = apexw_state_bytes(N_T, NUMEL, APEXW_STATE_F32, &sb);
    printf("state_bytes_f32_rc=%d\nstate_bytes_f32=%zu\n", rc, sb);
    rc = apexw_workspace_bytes(N_T, NUMEL, &wb);
    printf("workspace_rc=%d\nworkspace_bytes=%zu\n", rc, wb);
    rc = apexw_state_bytes(N_T, NUMEL, 7, &sb);
    printf("bad_fmt_rc=%d\n", rc);
    printf("bad_fmt_msg=%s\n", apexw_last_error());
    rc = apexw_destroy(NULL);
    printf("null_destroy_rc=%d\n", rc);
    return 0;
}

/* ---------------------------------------------------------------- GPU */

#define HIPCHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); return 2; } } while (0)
#define APCHECK(x) do { int r_ = (x); if (r_ != APEXW_OK) { \
    fprintf(stderr, "%s: %d %s\n", #x, r_, apexw_last_error()); return 3; } } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 32);
}
static float uniform_pm(float scale) {            /* uniform in (-scale, scale) */
    return ((float)(next_u32() >> 8) * (1.0f / 16777216.0f) * 2.0f - 1.0f) * scale;
}
static uint16_t to_bf16_trunc(float f) {          /* inputs only: any bf16 will do */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static size_t elem_size(int32_t dt) { return dt == APEXW_F32 ? 4 : 2; }

static void fill(void *host, int64_t n, int32_t dt, float scale) {
    for (int64_t i = 0; i < n; ++i) {
        float x = uniform_pm(scale);
        if (dt == APEXW_F32) ((float *)host)[i] = x;
        else ((uint16_t *)host)[i] = to_bf16_trunc(x);
    }
}

static int gpu_mode(const char *out_path, int fmt, int steps) {
    FILE *out = fopen(out_path, "wb");
    if (!out) { perror(out_path); return 1; }
    void *params[N_T], *grads[N_T], *host_p[N_T], *host_g[N_T];
    size_t sb = 0, wb = 0;
    APCHECK(apexw_state_bytes(N_T, NUMEL, fmt, &sb));
    APCHECK(apexw_workspace_bytes(N_T, NUMEL, &wb));
    void *state = NULL, *ws = NULL;
    HIPCHECK(hipMalloc(&state, sb));
    HIPCHECK(hipMalloc(&ws, wb));
    for (int i = 0; i < N_T; ++i) {
        const size_t pb = (size_t)NUMEL[i] * elem_size(PDT[i]);
        const size_t gb = (size_t)NUMEL[i] * elem_size(GDT[i]);
        host_p[i] = malloc(pb);
        host_g[i] = malloc(gb);
        fill(host_p[i], NUMEL[i], PDT[i], 0.02f);
        HIPCHECK(hipMalloc(&params[i], pb));
        HIPCHECK(hipMalloc(&grads[i], gb));
        HIPCHECK(hipMemcpy(params[i], host_p[i], pb, hipMemcpyHostToDevice));
        fwrite(host_p[i], 1, pb, out);                       /* initial theta */
    }
    apexw_t h = NULL;
    APCHECK(apexw_create(N_T, NUMEL, PDT, GDT, GROUP, 2, fmt, state, sb, ws, wb, NULL, &h));
    const apexw_group groups[2] = {{1e-3, 0.9, 0.999, 1e-8, 0.01}, {3e-3, 0.8, 0.99, 1e-6, 0.0}};
    for (int k = 0; k < steps; ++k) {
        for (int i = 0; i < N_T; ++i) {
            const size_t gb = (size_t)NUMEL[i] * elem_size(GDT[i]);
            fill(host_g[i], NUMEL[i], GDT[i], 1e-3f);
            HIPCHECK(hipMemcpy(grads[i], host_g[i], gb, hipMemcpyHostToDevice));
            fwrite(host_g[i], 1, gb, out);                   /* grads of step k */
        }
        APCHECK(apexw_step(h, groups, 2, params, (const void *const *)grads, NULL, NULL));
    }
    HIPCHECK(hipDeviceSynchronize());
    for (int i = 0; i < N_T; ++i) {                          /* final theta */
        const size_t pb = (size_t)NUMEL[i] * elem_size(PDT[i]);
        HIPCHECK(hipMemcpy(host_p[i], params[i], pb, hipMemcpyDeviceToHost));
        fwrite(host_p[i], 1, pb, out);
    }
    void *blob = malloc(sb);                                 /* whole state buffer */
    HIPCHECK(hipMemcpy(blob, state, sb, hipMemcpyDeviceToHost));
    fwrite(blob, 1, sb, out);
    int32_t t[N_T];
    APCHECK(apexw_read_steps(h, t, NULL));
    fwrite(t, 4, N_T, out);
    APCHECK(apexw_destroy(h));
    fclose(out);
    for (int i = 0; i < N_T; ++i) {
        HIPCHECK(hipFree(params[i]));
        HIPCHECK(hipFree(grads[i]));
        free(host_p[i]);
        free(host_g[i]);
    }
    HIPCHECK(hipFree(state));
    HIPCHECK(hipFree(ws));
    free(blob);
    printf("ok steps=%d fmt=%d state_bytes=%zu\n", steps, fmt, sb);
    return 0;
}

int main(int argc, char **argv) {
    if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_mode();
    if (argc >= 5 && strcmp(argv[1], "gpu") == 0)
        return gpu_mode(argv[2], atoi(argv[3]), atoi(argv[4]));
    fprintf(stderr, "usage: caller host | caller gpu OUT FMT STEPS\n");
    return 1;
}
