/*
 * CPU oracle for the fused rank-sum + residual add + RMSNorm operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code with the GPU library and is not a fallback for it.
 *
 * What it computes: the contract of the page "[TLERaw] Add NVSHMEM allreduce
 * RMSNorm tutorial" (FlagTree PR #1122), section Summary, restated in section
 * Implementation 3 ("Residual + RMSNorm epilogue"):
 *
 *     reduced      = sum over the W rank partials of x
 *     residual_out = reduced + residual
 *     norm_out     = RMSNorm(residual_out, weight, eps)
 *
 * on BF16 [T][H] token rows (section Correctness: BF16, hidden size 2048).
 * The page fixes neither the rounding points nor the reduction order; the
 * readings taken here (each one stated at the step it governs) are:
 *
 *   1. every BF16 input is widened exactly to binary32;
 *   2. the rank sum runs in binary32, round to nearest even, in rank order
 *      0, 1, ..., W-1 starting from x_0 (not from +0);
 *   3. `reduced` is a BF16 tensor between the collective and the epilogue
 *      (the page's collective is a BF16 collective, Implementation 1), so the
 *      binary32 sum is rounded once to BF16;
 *   4. residual_out = BF16(f32(reduced) + f32(residual));
 *   5. RMSNorm's input is the BF16 residual_out; the mean of squares over the
 *      H elements of the row is accumulated in binary64 (at least the FP32
 *      accumulation the page asks for), sequentially in h;
 *   6. eps sits inside the square root: inv = 1 / sqrt(mean + eps), taken in
 *      binary64 and rounded once to binary32;
 *   7. norm_out = BF16((f32(residual_out) * inv) * f32(weight)): normalise,
 *      then scale by the weight, each product rounded to binary32.
 *
 * No fast-math, no FMA contraction (built with -ffp-contract=off), SSE2
 * scalar arithmetic, denormals kept: each operation is one IEEE-754
 * operation in the stated format.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* BF16 bit pattern -> binary32: the BF16 bits are the top half of the binary32 bits (exact). */
static float widen(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * binary32 -> BF16, round to nearest, ties to even, from the definition: keep
 * the upper 16 bits, then compare the 16 dropped bits with one half of the
 * last kept place.  Above one half, or exactly one half with an odd kept
 * part, the kept part goes up by one (a carry into the exponent is the
 * correct result, and turns the largest finite values into infinity).
 * A NaN stays a NaN, made quiet.
 */
static uint16_t round_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

uint16_t oracle_round_bf16(float f) { return round_bf16(f); }

/* Same, from a binary32 bit pattern (a signalling NaN reaches the rounding unchanged). */
uint16_t oracle_round_bf16_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return round_bf16(f);
}
float oracle_widen_bf16(uint16_t b) { return widen(b); }

/*
 * Rows [row_begin, row_end) of the operator.
 *   x[r]          : W pointers, each BF16 [T][H] row-major (row stride H)
 *   residual      : BF16 [T][H]
 *   weight        : BF16 [H]
 *   reduced       : BF16 [T][H] output, may be NULL
 *   residual_out  : BF16 [T][H] output
 *   norm_out      : BF16 [T][H] output
 *   inv_rms       : binary32 [T] output (the per-row 1/RMS), may be NULL
 * Returns 0, or -1 on a bad argument.
 */
int oracle_fused_rows(int W, int T, int H, const uint16_t* const* x, const uint16_t* residual,
                      const uint16_t* weight, float eps, uint16_t* reduced, uint16_t* residual_out,
                      uint16_t* norm_out, float* inv_rms, int row_begin, int row_end) {
    if (W < 1 || T < 0 || H < 1 || row_begin < 0 || row_end > T || row_begin > row_end) return -1;
    for (int t = row_begin; t < row_end; ++t) {
        const size_t row = (size_t)t * (size_t)H;
        double sum_sq = 0.0;
        for (int h = 0; h < H; ++h) {
            /* steps 1-3: binary32 rank sum in rank order, then one rounding to BF16 */
            float acc = widen(x[0][row + h]);
            for (int r = 1; r < W; ++r) acc = acc + widen(x[r][row + h]);
            const uint16_t red = round_bf16(acc);
            if (reduced) reduced[row + h] = red;
            /* step 4: residual add in binary32, rounded to BF16 */
            const uint16_t ro = round_bf16(widen(red) + widen(residual[row + h]));
            residual_out[row + h] = ro;
            /* step 5: square (exact in binary64) and accumulate in order */
            const double v = (double)widen(ro);
            sum_sq = sum_sq + v * v;
        }
        /* step 6: one binary64 reciprocal square root, rounded once to binary32 */
        const double mean_sq = sum_sq / (double)H;
        const float inv = (float)(1.0 / sqrt(mean_sq + (double)eps));
        if (inv_rms) inv_rms[t] = inv;
        /* step 7: normalise, then scale by the weight */
        for (int h = 0; h < H; ++h) {
            const float normed = widen(residual_out[row + h]) * inv;
            const float scaled = normed * widen(weight[h]);
            norm_out[row + h] = round_bf16(scaled);
        }
    }
    return 0;
}

/* All T rows. */
int oracle_fused(int W, int T, int H, const uint16_t* const* x, const uint16_t* residual,
                 const uint16_t* weight, float eps, uint16_t* reduced, uint16_t* residual_out,
                 uint16_t* norm_out, float* inv_rms) {
    return oracle_fused_rows(W, T, H, x, residual, weight, eps, reduced, residual_out, norm_out,
                             inv_rms, 0, T);
}
