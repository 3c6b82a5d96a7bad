/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer, on random
 * small shapes and bit patterns (NaN, infinities, subnormals included), with every
 * buffer exactly its stated size: any read or write past a buffer, or any undefined
 * operation, aborts.  Exit status 0 and no sanitizer report = pass. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fused_rows(int W, int T, int H, const uint16_t* const* x, const uint16_t* residual,
                      const uint16_t* weight, float eps, uint16_t* reduced, uint16_t* residual_out,
                      uint16_t* norm_out, float* inv_rms, int row_begin, int row_end);

static uint64_t state = 0x13198A2E03707344ull;
static uint64_t next(void) { /* SplitMix64 */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main(void) {
    for (int it = 0; it < 3000; ++it) {
        const int W = 1 + (int)(next() % 16), T = (int)(next() % 6), H = 1 + (int)(next() % 70);
        const size_t n = (size_t)T * H;
        uint16_t* x[16];
        for (int r = 0; r < W; ++r) {
            x[r] = malloc(n * 2 + 1);
            for (size_t i = 0; i < n; ++i) x[r][i] = (uint16_t)next();
        }
        uint16_t* res = malloc(n * 2 + 1);
        uint16_t* w = malloc((size_t)H * 2);
        uint16_t* red = malloc(n * 2 + 1);
        uint16_t* ro = malloc(n * 2 + 1);
        uint16_t* no = malloc(n * 2 + 1);
        float* inv = malloc((size_t)T * 4 + 1);
        for (size_t i = 0; i < n; ++i) res[i] = (uint16_t)next();
        for (int h = 0; h < H; ++h) w[h] = (uint16_t)next();
        const float eps = (next() % 2) ? 0.0f : 1e-6f;
        const int b = T ? (int)(next() % (T + 1)) : 0;
        const int e = b + (T > b ? (int)(next() % (T - b + 1)) : 0);
        if (oracle_fused_rows(W, T, H, (const uint16_t* const*)x, res, w, eps, red, ro, no, inv, b, e) != 0) {
            fprintf(stderr, "oracle rejected valid arguments\n");
            return 1;
        }
        if (oracle_fused_rows(W, T, H, (const uint16_t* const*)x, res, w, eps, red, ro, no, inv, 0, T + 1) == 0) {
            fprintf(stderr, "oracle accepted a row range past T\n");
            return 1;
        }
        for (int r = 0; r < W; ++r) free(x[r]);
        free(res); free(w); free(red); free(ro); free(no); free(inv);
    }
    printf("oracle fuzz ok\n");
    return 0;
}
