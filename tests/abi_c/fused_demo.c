/* The whole boundary from plain C on the GPU, without Python or torch:
 * arrms_create -> arrms_fused -> arrms_destroy on device buffers allocated with
 * hipMalloc, the outputs checked against the CPU oracle (liboracle.so, test
 * infrastructure), then a C loop of back-to-back calls timed with HIP events;
 * then the no-allocation entry point on the same inputs, whose outputs must equal
 * arrms_fused's bit for bit, and its own timed loop.
 *
 * usage: fused_demo W T H [timed_calls]
 * Inputs: seeded normals / uniforms from libsynth.so, cut to BF16 by keeping the
 * upper 16 bits (any BF16 pattern is a valid input).  Prints what it checks and
 * one "timing" line; exits 0 when every check passes. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "arrms.h"

/* oracle (test infrastructure) and the seeded input generator */
int oracle_fused(int W, int T, int H, const uint16_t* const* x, const uint16_t* residual, const uint16_t* weight,
                 float eps, uint16_t* reduced, uint16_t* residual_out, uint16_t* norm_out, float* inv_rms);
void synth_normal(uint64_t seed, uint64_t tag, double sigma, int64_t n, float* out, uint64_t outlier_tag,
                  double outlier_p, double outlier_scale);
void synth_uniform(uint64_t seed, uint64_t tag, double lo, double hi, int64_t n, float* out);

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));                     \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

static void to_bf16_bits(const float* f, uint16_t* out, size_t n) {
    size_t i;
    for (i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &f[i], 4);
        out[i] = (uint16_t)(u >> 16);
    }
}

static float bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* position of a BF16 pattern on the ordered line of values (for step distances) */
static long ordered(uint16_t b) { return (b & 0x8000) ? -(long)(b & 0x7fff) : (long)(b & 0x7fff); }

int main(int argc, char** argv) {
    if (argc < 4) {
        printf("usage: %s W T H [timed_calls]\n", argv[0]);
        return 2;
    }
    const int W = atoi(argv[1]), T = atoi(argv[2]), H = atoi(argv[3]);
    const int calls = argc > 4 ? atoi(argv[4]) : 2000;
    const float eps = 1e-6f;
    if (W < 1 || W > ARRMS_MAX_WORLD || T < 1 || H < 1 || H > ARRMS_MAX_HIDDEN || calls < 1) {
        printf("bad arguments\n");
        return 2;
    }
    const size_t n = (size_t)T * (size_t)H;
    float* f = (float*)malloc(n * sizeof(float));
    uint16_t* hx = (uint16_t*)malloc((size_t)W * n * 2);
    uint16_t* hres = (uint16_t*)malloc(n * 2);
    uint16_t* hw = (uint16_t*)malloc((size_t)H * 2);
    uint16_t* ro = (uint16_t*)malloc(n * 2);
    uint16_t* no = (uint16_t*)malloc(n * 2);
    uint16_t* ref_ro = (uint16_t*)malloc(n * 2);
    uint16_t* ref_no = (uint16_t*)malloc(n * 2);
    if (!f || !hx || !hres || !hw || !ro || !no || !ref_ro || !ref_no) {
        printf("FAIL host allocation\n");
        return 1;
    }
    int r;
    for (r = 0; r < W; ++r) {
        synth_normal(7, (uint64_t)r, 1.0, (int64_t)n, f, 2000 + (uint64_t)r, 0.0, 1.0);
        to_bf16_bits(f, hx + (size_t)r * n, n);
    }
    synth_normal(7, 1000, 1.0, (int64_t)n, f, 0, 0.0, 1.0);
    to_bf16_bits(f, hres, n);
    synth_uniform(7, 1001, 0.5, 1.5, H, f);
    to_bf16_bits(f, hw, (size_t)H);

    void* dx[ARRMS_MAX_WORLD];
    void *dres, *dw, *dro, *dno;
    for (r = 0; r < W; ++r) {
        HIP_OK(hipMalloc(&dx[r], n * 2));
        HIP_OK(hipMemcpy(dx[r], hx + (size_t)r * n, n * 2, hipMemcpyHostToDevice));
    }
    HIP_OK(hipMalloc(&dres, n * 2));
    HIP_OK(hipMalloc(&dw, (size_t)H * 2));
    HIP_OK(hipMalloc(&dro, n * 2));
    HIP_OK(hipMalloc(&dno, n * 2));
    HIP_OK(hipMemcpy(dres, hres, n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dw, hw, (size_t)H * 2, hipMemcpyHostToDevice));

    arrms_handle_t h = NULL;
    int rc = arrms_create(&h, 0, W, T, H);
    if (rc != ARRMS_OK) {
        printf("FAIL arrms_create: %s\n", arrms_status_string(rc));
        return 1;
    }
    arrms_plan_t plan;
    rc = arrms_query_plan(h, (const void* const*)dx, W, T, H, dres, dw, eps, dro, dno, &plan);
    printf("plan: variant %d grid %d block %d kernels %d\n", plan.variant, plan.grid, plan.block, plan.kernels);
    rc = arrms_fused(h, (const void* const*)dx, W, T, H, dres, dw, eps, dro, dno, NULL);
    if (rc != ARRMS_OK) {
        printf("FAIL arrms_fused: %s (HIP error %d)\n", arrms_status_string(rc), arrms_last_hip_error(h));
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(ro, dro, n * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(no, dno, n * 2, hipMemcpyDeviceToHost));

    const uint16_t* xs[ARRMS_MAX_WORLD];
    for (r = 0; r < W; ++r) xs[r] = hx + (size_t)r * n;
    if (oracle_fused(W, T, H, xs, hres, hw, eps, NULL, ref_ro, ref_no, NULL) != 0) {
        printf("FAIL oracle rejected the arguments\n");
        return 1;
    }
    size_t i, ro_bad = 0, no_diff = 0;
    long max_steps = 0;
    double max_abs = 0.0;
    for (i = 0; i < n; ++i) {
        if (ro[i] != ref_ro[i]) ++ro_bad;
        if (no[i] != ref_no[i]) {
            long d = labs(ordered(no[i]) - ordered(ref_no[i]));
            double e = fabs((double)bf16_value(no[i]) - (double)bf16_value(ref_no[i]));
            ++no_diff;
            if (d > max_steps) max_steps = d;
            if (e > max_abs) max_abs = e;
        }
    }
    const int pass = ro_bad == 0 && max_steps <= 2 && max_abs <= 0.03125;
    printf("%s residual_out mismatches %zu of %zu; norm_out not bit-identical %zu (max %ld steps, %g)\n",
           pass ? "ok  " : "FAIL", ro_bad, n, no_diff, max_steps, max_abs);

    /* back-to-back calls from C on the null stream, same buffers */
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    int k;
    for (k = 0; k < 50; ++k) arrms_fused(h, (const void* const*)dx, W, T, H, dres, dw, eps, dro, dno, NULL);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipEventRecord(e0, NULL));
    for (k = 0; k < calls; ++k) {
        rc = arrms_fused(h, (const void* const*)dx, W, T, H, dres, dw, eps, dro, dno, NULL);
        if (rc != ARRMS_OK) {
            printf("FAIL arrms_fused in the timed loop: %s\n", arrms_status_string(rc));
            return 1;
        }
    }
    HIP_OK(hipEventRecord(e1, NULL));
    HIP_OK(hipEventSynchronize(e1));
    float ms = 0.0f;
    HIP_OK(hipEventElapsedTime(&ms, e0, e1));
    const double us = 1e3 * ms / calls;
    const double bytes = 2.0 * T * H * (W + 3) + 2.0 * H;
    printf("timing: W=%d T=%d H=%d, %d back-to-back calls from C (same buffers): %.2f us/call, %.1f GB/s\n", W, T,
           H, calls, us, bytes / (us * 1e-6) / 1e9);

    /* the no-allocation entry point (current device, no handle): same bits as arrms_fused */
    HIP_OK(hipMemset(dro, 0, n * 2));
    HIP_OK(hipMemset(dno, 0, n * 2));
    HIP_OK(hipDeviceSynchronize());
    rc = arrms_fused_noalloc((const void* const*)dx, W, T, H, dres, dw, eps, dro, dno, NULL);
    if (rc != ARRMS_OK) {
        printf("FAIL arrms_fused_noalloc: %s\n", arrms_status_string(rc));
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    uint16_t* ro2 = (uint16_t*)malloc(n * 2);
    uint16_t* no2 = (uint16_t*)malloc(n * 2);
    if (!ro2 || !no2) {
        printf("FAIL host allocation\n");
        return 1;
    }
    HIP_OK(hipMemcpy(ro2, dro, n * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(no2, dno, n * 2, hipMemcpyDeviceToHost));
    const int same = memcmp(ro2, ro, n * 2) == 0 && memcmp(no2, no, n * 2) == 0;
    printf("%s arrms_fused_noalloc outputs %s arrms_fused's\n", same ? "ok  " : "FAIL",
           same ? "bit-identical to" : "differ from");
    free(ro2), free(no2);
    HIP_OK(hipEventRecord(e0, NULL));
    for (k = 0; k < calls; ++k) {
        rc = arrms_fused_noalloc((const void* const*)dx, W, T, H, dres, dw, eps, dro, dno, NULL);
        if (rc != ARRMS_OK) {
            printf("FAIL arrms_fused_noalloc in the timed loop: %s\n", arrms_status_string(rc));
            return 1;
        }
    }
    HIP_OK(hipEventRecord(e1, NULL));
    HIP_OK(hipEventSynchronize(e1));
    HIP_OK(hipEventElapsedTime(&ms, e0, e1));
    printf("timing: arrms_fused_noalloc, %d back-to-back calls from C: %.2f us/call\n", calls, 1e3 * ms / calls);

    HIP_OK(hipEventDestroy(e0));
    HIP_OK(hipEventDestroy(e1));
    rc = arrms_destroy(h);
    for (r = 0; r < W; ++r) HIP_OK(hipFree(dx[r]));
    HIP_OK(hipFree(dres));
    HIP_OK(hipFree(dw));
    HIP_OK(hipFree(dro));
    HIP_OK(hipFree(dno));
    free(f), free(hx), free(hres), free(hw), free(ro), free(no), free(ref_ro), free(ref_no);
    return (pass && same && rc == ARRMS_OK) ? 0 : 1;
}
