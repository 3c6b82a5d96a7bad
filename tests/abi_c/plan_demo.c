/* A plain C99 caller of the library's host-only entry points: proves that
 * include/arrms.h is a C header (no C++ constructs) and that the shared library
 * links from C.  Prints one line per check; exits non-zero on a failure.  No
 * GPU is needed: arrms_plan and arrms_status_string do no HIP calls. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "arrms.h"

static int failures = 0;
#define CHECK(cond, what)                               \
    do {                                                \
        if (cond) {                                     \
            printf("ok   %s\n", what);                  \
        } else {                                        \
            printf("FAIL %s\n", what);                  \
            ++failures;                                 \
        }                                               \
    } while (0)

int main(void) {
    const uintptr_t base = (uintptr_t)1 << 40;
    const uintptr_t step = (uintptr_t)1 << 28;
    const void* partials[4];
    arrms_plan_t p;
    int r, rc;
    for (r = 0; r < 4; ++r) partials[r] = (const void*)(base + (uintptr_t)r * step);
    const void* residual = (const void*)(base + 4 * step);
    const void* weight = (const void*)(base + 5 * step);
    void* residual_out = (void*)(base + 6 * step);
    void* norm_out = (void*)(base + 7 * step);

    CHECK(strcmp(arrms_status_string(ARRMS_OK), "ok") == 0, "status string");

    rc = arrms_plan(256, ARRMS_VARIANT_AUTO, NULL, 8, 4096, 2048, partials, 4, 4096, 2048, residual, weight,
                    1e-6f, residual_out, norm_out, &p);
    CHECK(rc == ARRMS_OK && p.variant == ARRMS_VARIANT_ROW && p.kernels == 1, "prefill plan is the row variant");
    printf("     grid %d block %d vec_per_thread %d threads_per_row %d xcd_chunk %d\n", p.grid, p.block,
           p.vec_per_thread, p.threads_per_row, p.xcd_chunk);

    rc = arrms_plan(256, ARRMS_VARIANT_AUTO, NULL, 8, 4096, 2048, partials, 4, 37, 2047, residual, weight, 1e-6f,
                    residual_out, norm_out, &p);
    CHECK(rc == ARRMS_OK && p.variant == ARRMS_VARIANT_SCALAR, "odd H takes the element-wise variant");

    rc = arrms_plan(256, ARRMS_VARIANT_AUTO, NULL, 8, 4096, 2048, partials, 4, 16, 2048, residual, weight, -1.0f,
                    residual_out, norm_out, &p);
    CHECK(rc == ARRMS_ERR_INVALID_ARG, "negative eps is rejected");

    rc = arrms_plan(256, ARRMS_VARIANT_AUTO, NULL, 8, 4096, 2048, partials, 4, 16, 2048, residual, weight, 1e-6f,
                    (void*)partials[2], norm_out, &p);
    CHECK(rc == ARRMS_ERR_INVALID_ARG, "an output aliasing a partial is rejected");

    {
        arrms_tuning_t t;
        memset(&t, 0, sizeof t);
        t.splith_max_tokens = -1;
        t.xcd_chunk = -1;
        t.vec_per_thread = 2;
        rc = arrms_plan(256, ARRMS_VARIANT_ROW, &t, 8, 4096, 2048, partials, 4, 100, 2048, residual, weight, 1e-6f,
                        residual_out, norm_out, &p);
        CHECK(rc == ARRMS_OK && p.vec_per_thread == 2, "tuning override reaches the plan");
    }

    rc = arrms_plan_reduce(256, NULL, 8, 4096, 2048, partials, 4, 4096, 2048, residual_out, &p);
    CHECK(rc == ARRMS_OK && p.variant == ARRMS_VARIANT_REDUCE, "rank-sum plan");

    CHECK(arrms_destroy(NULL) == ARRMS_OK, "destroy(NULL) is a no-op");
    CHECK(arrms_fused(NULL, partials, 4, 1, 2048, residual, weight, 1e-6f, residual_out, norm_out, NULL) ==
              ARRMS_ERR_INVALID_ARG,
          "a call without a handle is rejected before any HIP call");
    return failures ? 1 : 0;
}
