// Host-only fuzz of the library's argument validation and launch planning
// (arrms_plan, arrms_plan_reduce), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The kernel launchers are replaced by stubs: the
// planner never launches.  Pointers are fake integers; they are compared, never
// dereferenced.  Exit status 0 and no sanitizer report = pass.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "arrms.h"
#include "arrms_internal.h"

namespace arrms {
hipError_t launch_row(const Args&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_splith(const Args&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_scalar(const Args&, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_reduce(const Args&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace arrms

static uint64_t state = 0x243F6A8885A308D3ull;
static uint64_t next() {  // SplitMix64
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int pick(const int* v, int n) { return v[next() % n]; }

static int fail(const char* what, int i) {
    fprintf(stderr, "check failed: %s (iteration %d)\n", what, i);
    return 1;
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 200000;
    const int worlds[] = {-1, 0, 1, 2, 3, 4, 5, 8, 9, 12, 16, 17};
    const int tokens[] = {-5, 0, 1, 2, 3, 16, 17, 64, 255, 256, 1000, 4096, 16383, 100000, 1 << 24, 0x7fffffff};
    const int hiddens[] = {-1, 0, 1, 3, 8, 64, 128, 1000, 1001, 2048, 5120, 8192, 16384, 16392, 24576, 65536, 65537};
    const int tvpt[] = {0, 0, 0, 1, 2, 3, 4, 8};
    const int ttpr[] = {0, 0, 0, 16, 32, 48, 64, 128, 256, 320, 512, 1024, 2048};
    const int tblk[] = {0, 0, 64, 100, 256, 1024, 2048};
    const int tspl[] = {-2, -1, -1, 0, 8, 100000};
    const int txcd[] = {-2, -1, -1, 0, 1, 7, 64, 1 << 29};
    const int offs[] = {0, 0, 0, 0, 2, 1, 16, 8};
    for (int i = 0; i < iters; ++i) {
        const int W = pick(worlds, 12), T = pick(tokens, 16), H = pick(hiddens, 17);
        const int maxw = 1 + (int)(next() % 16), maxh = 1 + (int)(next() % 65536);
        const int maxt = (next() % 4) ? (int)(next() % 20000) : 0x7fffffff;
        const int cu = (next() % 8) ? 256 : (int)(next() % 300);
        const int trpb[] = {0, 0, 0, 1, 2, 3, 4, 8, 64, 128};
        const int tse[] = {0, 0, 1, 2, 4, 3};
        const int tro[] = {0, 0, 0, 1, 2, 3, -1};
        const int tpl[] = {0, 0, 0, 1, 2, 3, -1};
        arrms_tuning_t tun = {pick(tvpt, 8), pick(ttpr, 13), pick(tblk, 7), pick(tspl, 6), pick(txcd, 8), pick(trpb, 10),
                              pick(tse, 6), pick(tro, 7), pick(tpl, 7)};
        const arrms_tuning_t* tp = (next() % 3) ? &tun : nullptr;
        const int variant = (int)(next() % 6) - 1;
        const uintptr_t base = 0x7f0000000000ull;
        const uintptr_t step = 1ull << 36;
        const void* parts[17];
        for (int r = 0; r < 17; ++r) parts[r] = (const void*)(base + r * step + pick(offs, 8));
        const void* res = (const void*)(base + 20 * step + pick(offs, 8));
        const void* w = (const void*)(base + 21 * step);
        void* ro = (next() % 10) ? (void*)(base + 22 * step) : (void*)res;
        void* no = (void*)(base + 23 * step + pick(offs, 8));
        const float eps = (next() % 10) ? 1e-6f : -1.0f;
        arrms_plan_t p;
        const int rc = arrms_plan(cu, variant, tp, maxw, maxt, maxh, parts, W, T, H, res, w, eps, ro, no, &p);
        if (rc == ARRMS_OK && T > 0 && p.grid > 0) {
            if (p.blocks > p.grid || p.block < 64 || p.block > 1024 || p.block % 64) return fail("shape", i);
            if ((long long)p.grid * p.block > 0xffffffffLL) return fail("grid limit", i);
            if (p.variant == ARRMS_VARIANT_ROW) {
                if ((long)p.blocks * p.rows_per_block < T) return fail("row cover", i);
                if ((long)p.threads_per_row * p.vec_per_thread < H / 8) return fail("row width", i);
                if (p.block != p.threads_per_row * p.rows_per_block) return fail("row block", i);
            } else if (p.variant == ARRMS_VARIANT_SPLITH) {
                if ((long)p.chunks_per_row * p.block * p.vec_per_thread < H / 8) return fail("split cover", i);
                if (p.blocks != T * p.chunks_per_row) return fail("split blocks", i);
                if (p.chunks_per_row > (((maxh + 7) / 8 + 63) / 64)) return fail("workspace", i);
            } else if (p.variant == ARRMS_VARIANT_SCALAR) {
                if (p.blocks != T) return fail("scalar blocks", i);
                const int e = p.elems_per_load;
                if (!(e == 1 || e == 2 || e == 4) || H % e) return fail("scalar load width", i);
                uintptr_t any = (uintptr_t)res | (uintptr_t)w | (uintptr_t)ro | (uintptr_t)no;
                for (int r = 0; r < W; ++r) any |= (uintptr_t)parts[r];
                if (any & (uintptr_t)(2 * e - 1)) return fail("scalar load alignment", i);
                const bool tuned_block = tp && tp->threads_per_row >= 64;
                if (!tuned_block && (long)p.block * 8 < H && p.block != 256) return fail("scalar span", i);
                if (!tuned_block && (long)p.block * 8 >= H && (long)(p.block - 64) * 8 >= H)
                    return fail("scalar lanes", i);
                if (p.block > 1024) return fail("scalar block", i);
            } else {
                return fail("variant", i);
            }
            if (p.xcd_chunk && p.grid % (8 * p.xcd_chunk)) return fail("xcd grid", i);
            // residual_out store policy: split-H always write-back (read back by its second
            // kernel); row and scalar streaming unless tuned to write-back
            int want = tp && tp->residual_out_store == 2;
            if (p.variant == ARRMS_VARIANT_SPLITH) want = 1;
            if (p.residual_out_cached != want) return fail("residual_out store policy", i);
            // the rank loop: always for the scalar kernel beyond 8 ranks; for 6-8 ranks only on
            // power-of-two workgroups with at least 8 rows per CU; never for the other variants
            if (p.variant == ARRMS_VARIANT_SCALAR && W > 8 && !p.rank_loop) return fail("fused rank loop", i);
            const bool pow2_block = p.block == 256 || p.block == 512 || p.block == 1024;
            if (p.rank_loop && (p.variant != ARRMS_VARIANT_SCALAR ||
                                (W <= 8 && (W < 6 || (long long)T < 8LL * cu ||
                                            !(pow2_block || (W == 8 && p.block >= 512))))))
                return fail("fused rank loop shape", i);
            // preloaded arguments: only kernels with a flat twin (row, or scalar without the rank
            // loop, W <= 8); never when tuned off; always when tuned on; else from 16 MiB per call
            const bool twin = W <= 8 && (p.variant == ARRMS_VARIANT_ROW ||
                                         (p.variant == ARRMS_VARIANT_SCALAR && !p.rank_loop));
            const long long bytes = 2LL * T * H * (W + 3) + 2LL * H;
            const int mode = tp ? tp->kernarg_preload : 0;
            const int want_pl = twin && (mode == 2 || (mode == 0 && bytes >= (16LL << 20)));
            if (p.kernarg_preload != want_pl) return fail("fused kernarg preload", i);
        }
        if (rc == ARRMS_OK && tp && (tp->residual_out_store < 0 || tp->residual_out_store > 2 || tp->scalar_elems == 3 ||
                                     tp->kernarg_preload < 0 || tp->kernarg_preload > 2))
            return fail("invalid tuning accepted", i);
        // The no-allocation entry point's plan (automatic, no tuning, absolute limits):
        // every plan it accepts keeps the split-H workspace index, row * chunks + chunk
        // for row < T, inside its static scratch.
        arrms_plan_t q;
        const int rcs = arrms_plan(cu > 0 ? cu : 1, ARRMS_VARIANT_AUTO, nullptr, ARRMS_MAX_WORLD, 0x7fffffff,
                                   ARRMS_MAX_HIDDEN, parts, W, T, H, res, w, eps, ro, no, &q);
        if (rcs == ARRMS_OK && T > 0 && q.grid > 0 &&
            arrms::splith_workspace_fits(q, T, ARRMS_NOALLOC_SCRATCH_DOUBLES)) {
            if (q.variant == ARRMS_VARIANT_SPLITH &&
                ((long long)q.blocks > ARRMS_NOALLOC_SCRATCH_DOUBLES || q.blocks != T * q.chunks_per_row))
                return fail("static scratch bound", i);
        }
        if (rcs == ARRMS_OK && T > 0 && q.variant == ARRMS_VARIANT_SPLITH &&
            (long long)T * q.chunks_per_row > ARRMS_NOALLOC_SCRATCH_DOUBLES &&
            arrms::splith_workspace_fits(q, T, ARRMS_NOALLOC_SCRATCH_DOUBLES))
            return fail("static scratch accepted", i);
        const int rc2 = arrms_plan_reduce(cu, tp, maxw, maxt, maxh, parts, W, T, H, no, &p);
        if (rc2 == ARRMS_OK && T > 0 && p.grid > 0) {
            const long long count = (long long)T * H;
            if ((long long)p.grid * p.block > 0xffffffffLL) return fail("reduce grid limit", i);
            const int e = p.elems_per_load;
            if (!(e == 1 || e == 2 || e == 4 || e == 8)) return fail("reduce load width", i);
            if ((p.variant == ARRMS_VARIANT_REDUCE) != (e == 8)) return fail("reduce variant", i);
            if (p.variant != ARRMS_VARIANT_REDUCE && p.variant != ARRMS_VARIANT_REDUCE_SCALAR)
                return fail("reduce variant kind", i);
            if (p.rank_loop != (W >= 6 && (long long)p.blocks >= 8LL * cu)) return fail("reduce rank loop", i);
            const int rmode = tp ? tp->kernarg_preload : 0;
            const int rwant = W <= 8 && !p.rank_loop &&
                              (rmode == 2 || (rmode == 0 && 2LL * count * (W + 1) >= (16LL << 20)));
            if (p.kernarg_preload != rwant) return fail("reduce kernarg preload", i);
            // every pointer has the same offset modulo 2E bytes, and the groups cover the elements
            int e2 = 0, head = -1;
            arrms::reduce_alignment(parts, W, no, count, e, &e2, &head);
            if (e2 != e || head < 0 || head >= e || head > count) return fail("reduce alignment", i);
            // (a head cut short by a tiny count leaves no groups, so nothing to align)
            for (int r = 0; r < W && head < count; ++r)
                if ((((uintptr_t)parts[r] + 2u * head) | ((uintptr_t)no + 2u * head)) & (uintptr_t)(2 * e - 1))
                    return fail("reduce aligned start", i);
            const long long per_block = 256LL * (e == 8 ? p.vec_per_thread : 8 / e);
            if ((long long)p.blocks * per_block < (count - head) / e) return fail("reduce cover", i);
        }
    }
    printf("plan fuzz ok: %d iterations\n", iters);
    return 0;
}
