// C ABI of the fused rank-partial sum + residual add + RMSNorm library
// (declared in include/arrms.h): handle lifecycle, argument validation,
// variant selection and launch on the caller's stream.
//
// The page "[TLERaw] Add NVSHMEM allreduce RMSNorm tutorial" (FlagTree PR #1122),
// section Implementation 4, gives its host side an init / workspace / cleanup
// life cycle behind a C ABI; here the one-time work (device query, workspace
// allocation, reading the variant override) happens in
// arrms_create only, and arrms_fused does no allocation and no synchronisation.
#include "arrms.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "arrms_internal.h"

struct arrms_ctx {
    int device;
    int cu_count;
    int max_world;
    int max_tokens;
    int max_hidden;
    int variant;  // forced variant, ARRMS_VARIANT_AUTO for per-shape choice
    bool has_tuning;
    arrms_tuning_t tuning;
    int ws_chunks;  // chunks per row the workspace holds
    double* ws;
    int last_hip_error;
};

namespace {

// Smallest split-H chunk: one wave of 16-byte vectors (512 BF16 elements).
constexpr int kMinChunkVec = 64;
// Largest (W + 2) * vectors-per-lane the row variant keeps in registers.
constexpr int kMaxLiveVectors = 40;
// Traffic of one automatic XCD run of the row variant.
constexpr long kXcdRunBytes = 3L << 20;
// Vectors per lane of the rank-sum-only kernel (measured on MI355X at W=2/4/8,
// T=4096, H=2048: one vector per lane with ~3 MiB XCD runs is fastest, e.g.
// 5.6 TB/s at W=4 against 5.1 TB/s with four vectors per lane).
constexpr int kReduceAutoVpt = 1;
// Rows with less traffic than this never use split-H automatically.
constexpr long kSplitMinRowBytes = 144L << 10;
// Store policy of residual_out in the row and scalar kernels: streaming
// (non-temporal) stores unless tuned.  Measured on MI355X with back-to-back calls
// rotating over 4.5 GB of buffers, write-back stores were 3-9 % slower on most
// shapes (W = 1..16, H = 1024..16384, T = 1024..16384) and at most 2 % faster on a
// few small ones; with a rotation of only 0.7 GB (partly served by the Infinity
// Cache) they were 2-9 % faster up to 128 MiB of residual_out per call.  So
// write-back stores pay only where the call's data is cache-resident; the tuning
// field selects them for such callers.

int chunks_capacity(int max_hidden) {
    const int nvec = (max_hidden + 7) / 8;
    return (nvec + kMinChunkVec - 1) / kMinChunkVec;
}

// Register-array extent of the rank loop: specialised W, else the generic 16.
int world_extent(int world) { return (world <= 8 || world == 16) ? world : arrms::kMaxWorld; }

// Must match the __launch_bounds__ of the row kernels.
int row_max_threads(int world, int vpt) {
    if (world_extent(world) > 8) return vpt == 1 ? 512 : 256;
    return vpt == 1 ? 1024 : (vpt <= 4 ? 512 : 256);
}

// Smallest power of two >= n, at least 16 (16 and 32 are sub-wave row groups).
int pow2_threads(int n) {
    int t = 16;
    while (t < n) t *= 2;
    return t;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a);
    const uintptr_t y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool valid_tuning(const arrms_tuning_t* t) {
    if (!t) return true;
    const int v = t->vec_per_thread;
    if (!(v == 0 || v == 1 || v == 2 || v == 4 || v == 8)) return false;
    const int r = t->threads_per_row;
    if (!(r == 0 || r == 16 || r == 32 || (r > 0 && r % 64 == 0 && r <= 1024))) return false;
    const int b = t->splith_block;
    if (!(b == 0 || (b > 0 && b % 64 == 0 && b <= 1024))) return false;
    if (t->splith_max_tokens < -1) return false;
    if (t->xcd_chunk < -1) return false;
    const int rp = t->rows_per_block;
    if (rp < 0 || rp > 64 || (rp & (rp - 1))) return false;
    const int se = t->scalar_elems;
    if (!(se == 0 || se == 1 || se == 2 || se == 4)) return false;
    if (t->residual_out_store < 0 || t->residual_out_store > 2) return false;
    if (t->kernarg_preload < 0 || t->kernarg_preload > 2) return false;
    return true;
}

// Write-back (1) or streaming (0) stores for residual_out in the row and scalar kernels.
int residual_out_cached(const arrms_tuning_t* t) { return t && t->residual_out_store == 2; }

// Launch shape of a vector-variant plan whose logical workgroup count is
// p->blocks.  The XCD mapping keeps runs of K consecutive blocks on one XCD
// (see logical_block in the kernels); K is clamped to blocks / 8 rounded up,
// so the grid pads p->blocks by less than 8K.
void finish_vector_plan(const arrms_tuning_t* t, arrms_plan_t* p, int auto_chunk) {
    long k = (t && t->xcd_chunk >= 0) ? t->xcd_chunk : auto_chunk;
    const long whole = (p->blocks + 7L) / 8;
    if (k > whole) k = whole;
    const long grid = k ? (p->blocks + 8 * k - 1) / (8 * k) * (8 * k) : p->blocks;
    if (grid > 0x7fffffffL) k = 0;  // keep the launch within the grid-size limit
    p->xcd_chunk = static_cast<int>(k);
    p->grid = k ? static_cast<int>(grid) : p->blocks;
}

// Row variant plan; returns ARRMS_ERR_UNSUPPORTED when the shape or the
// tuning overrides do not fit the row kernels.
//
// Automatic lane layout (measured on MI355X, W=4 H=2048, W=8 H=5120 and
// H=8192): row groups of a power-of-two lane count do better than exact fits
// (a 5-wave group for H=5120 loses about 4% to an 8-wave group with idle
// lanes), and the best groups hold 256 to 512 lanes.  So: the fewest vectors
// per lane whose power-of-two row group is at most 512 lanes.
int plan_row(int cu_count, int world, int tokens, int hidden, const arrms_tuning_t* t, arrms_plan_t* p) {
    const int nvec = hidden / 8;
    const int we = world_extent(world);
    int best_vpt = 0, best_tpr = 0;
    for (int vpt = 1; vpt <= 8; vpt *= 2) {
        if (t && t->vec_per_thread && t->vec_per_thread != vpt) continue;
        if ((we + 2) * vpt > kMaxLiveVectors) continue;
        int tpr = pow2_threads((nvec + vpt - 1) / vpt);
        if (t && t->threads_per_row) tpr = t->threads_per_row;
        if (tpr > row_max_threads(world, vpt) || static_cast<long>(tpr) * vpt < nvec) continue;
        if (!best_vpt || (best_tpr > 512 && tpr < best_tpr)) {
            best_vpt = vpt;
            best_tpr = tpr;
        }
    }
    if (!best_vpt) return ARRMS_ERR_UNSUPPORTED;
    // One rank (no rank sum, W = 1): at one vector per input a lane keeps only 32
    // bytes of HBM reads in flight, too few at full occupancy to cover the memory
    // latency.  Rows of 512..2048 elements therefore take four vectors per lane in
    // sub-wave row groups, when that still leaves two workgroups per compute unit
    // (measured on MI355X at H = 512, 1024, 2048 and T = 2048..16384: 4-14 % faster;
    // with fewer workgroups it is slower, and at W >= 2 it wins and loses by shape).
    // Two ranks (48 bytes in flight per lane) gain the same way, but only while the
    // four-vector workgroups fit in one round on the CUs: capped at four per CU (these
    // instances hold 5-6 workgroups per CU) they measured 4-13 % faster at
    // H = 512..2048 and T = 2048..16384 and never slower; past the cap a second,
    // partial round made them up to 12 % slower.  Three ranks won at some of these
    // shapes and lost up to 4 % at others, and W >= 4 loses (8 % at W=4 H=2048
    // T=4096), so they keep one vector per lane.
    // A tuned lane layout or row count per workgroup is taken as given: the
    // four-vector layout is an automatic choice only.
    const bool layout_tuned = t && (t->vec_per_thread || t->threads_per_row || t->rows_per_block);
    if (!layout_tuned && world <= 2 && nvec >= 64 && nvec <= 256) {
        const int tpr4 = pow2_threads((nvec + 3) / 4);
        const long blocks4 = (static_cast<long>(tokens) + 256 / tpr4 - 1) / (256 / tpr4);
        const bool fits = world == 1 || blocks4 <= 4L * cu_count;
        if (blocks4 >= 2L * cu_count && fits) {
            best_vpt = 4;
            best_tpr = tpr4;
        }
    }
    int rpb = best_tpr < 256 ? 256 / best_tpr : 1;
    while (rpb > 1 && best_tpr * rpb > row_max_threads(world, best_vpt)) rpb /= 2;
    if (t && t->rows_per_block) {
        rpb = t->rows_per_block;
        if (best_tpr * rpb > row_max_threads(world, best_vpt) || (best_tpr * rpb) % 64) return ARRMS_ERR_UNSUPPORTED;
    }
    p->variant = ARRMS_VARIANT_ROW;
    p->vec_per_thread = best_vpt;
    p->threads_per_row = best_tpr;
    p->rows_per_block = rpb;
    p->chunks_per_row = 1;
    p->block = best_tpr * rpb;
    p->blocks = static_cast<int>((static_cast<long>(tokens) + rpb - 1) / rpb);
    p->kernels = 1;
    p->residual_out_cached = residual_out_cached(t);
    // Automatic XCD runs: about 3 MiB of traffic per run, a power of two of
    // blocks (measured best: 64 blocks at W=4 H=2048, 16 at W=8 H=5120/8192);
    // small grids keep the hardware order.
    int k = 0;
    if (p->blocks >= 64) {
        const long block_bytes = 2L * rpb * (world + 3) * hidden;
        k = 1;
        while (2L * k * block_bytes <= kXcdRunBytes) k *= 2;
    }
    finish_vector_plan(t, p, k);
    return ARRMS_OK;
}

// Split-H plan.  Aims at about two workgroups per compute unit over the whole
// call, with chunks of at least one wave of vectors.
int plan_splith(int cu_count, int max_hidden, int world, int tokens, int hidden,
                const arrms_tuning_t* t, arrms_plan_t* p) {
    const int nvec = hidden / 8;
    const int cap = chunks_capacity(max_hidden);
    int vpt = (t && t->vec_per_thread) ? t->vec_per_thread : 1;
    const int max_block = world_extent(world) > 8 ? 512 : 1024;  // split-H __launch_bounds__
    if (vpt > 2) return ARRMS_ERR_UNSUPPORTED;
    if (world_extent(world) > 8 && vpt > 1) return ARRMS_ERR_UNSUPPORTED;
    int block;
    if (t && t->splith_block) {
        block = t->splith_block;
    } else {
        const long want_wgs = 2L * cu_count;
        long chunks = (want_wgs + tokens - 1) / tokens;
        const long max_chunks = (nvec + kMinChunkVec - 1) / kMinChunkVec;
        if (chunks > max_chunks) chunks = max_chunks;
        if (chunks < 1) chunks = 1;
        const long chunk_vec = (nvec + chunks - 1) / chunks;
        block = static_cast<int>((chunk_vec + vpt - 1) / vpt);
        block = (block + 63) / 64 * 64;
        if (block > max_block) {
            vpt = (world_extent(world) > 8) ? 1 : 2;
            block = static_cast<int>((chunk_vec + vpt - 1) / vpt);
            block = (block + 63) / 64 * 64;
            if (block > max_block) block = max_block;
        }
    }
    if (block > max_block) return ARRMS_ERR_UNSUPPORTED;
    const int chunk_vec = block * vpt;
    const int chunks = (nvec + chunk_vec - 1) / chunk_vec;
    if (chunks > cap) return ARRMS_ERR_UNSUPPORTED;
    if (static_cast<long>(tokens) * chunks > 0x7ffffff0L) return ARRMS_ERR_UNSUPPORTED;
    p->variant = ARRMS_VARIANT_SPLITH;
    p->vec_per_thread = vpt;
    p->threads_per_row = block;
    p->rows_per_block = 1;
    p->chunks_per_row = chunks;
    p->block = block;
    p->blocks = tokens * chunks;
    p->kernels = 2;
    p->residual_out_cached = 1;  // the second kernel reads residual_out back
    finish_vector_plan(t, p, 0);
    return ARRMS_OK;
}

// Scalar plan: one row per workgroup, 8 elements per lane per span: enough whole
// waves to cover the row in one span, at most 1024 lanes (the kernels'
// __launch_bounds__); a longer row runs on 256 lanes.  More than 8 ranks, or
// rank_loop, take the generic instance, which adds the ranks after x_0 one load
// round at a time.  Loads are `elems` BF16
// elements wide (the widest that H and every pointer's alignment allow, at most
// the tuned width).  XCD runs as in the row variant (about 3 MiB of traffic per run).
// The kernel aligns its lanes to 128-byte lines by rotating a one-span row, so a
// row takes no lanes beyond its own length.
void plan_scalar(int world, int tokens, int hidden, int elems, const arrms_tuning_t* t, arrms_plan_t* p,
                 bool rank_loop = false) {
    const int max_block = 1024;
    int block = ((hidden + 7) / 8 + 63) / 64 * 64;
    // A row longer than one span of the largest workgroup takes several spans anyway;
    // 4-wave workgroups run them 9-13 % faster than the largest ones (measured on
    // MI355X at W=4 and W=1 with H=16383, and W=16 with H=5119).
    if (block > max_block) block = 256;
    if (t && t->threads_per_row >= 64) block = t->threads_per_row;  // tuned: a multiple of 64
    if (block > max_block) block = max_block;
    if (t && t->scalar_elems && t->scalar_elems < elems) elems = t->scalar_elems;
    p->variant = ARRMS_VARIANT_SCALAR;
    p->vec_per_thread = 0;
    p->threads_per_row = block;
    p->rows_per_block = 1;
    p->chunks_per_row = 1;
    p->block = block;
    p->blocks = tokens;
    p->kernels = 1;
    p->elems_per_load = elems;
    p->residual_out_cached = residual_out_cached(t);
    p->rank_loop = world > 8 || rank_loop;  // the generic instance adds ranks 1.. one at a time
    int k = 0;
    if (p->blocks >= 64) {
        const long row_bytes = 2L * (world + 3) * hidden;
        k = 1;
        while (2L * k * row_bytes <= kXcdRunBytes) k *= 2;
    }
    finish_vector_plan(t, p, k);
}

// More than 8 ranks: the automatic choice takes the scalar kernel for rows of one
// span (H <= 8192 on its 1024 lanes) once there are enough rows to overlap its rank
// loop.  That kernel keeps only x_0, the residual and the weight in registers and adds
// the other ranks one load round at a time, so it runs many more workgroups per CU
// than the row kernel holding all 9-16 ranks; per row it pays one memory round trip
// per rank.  Measured on MI355X (4.5 GB rotation) against the row kernel: 8-30 %
// faster from T = 1024 at W = 9, 10, 12 and H = 2048-4096 (the generic 9-15-rank row
// kernel), and 7-10 % faster from T = 2048 at W = 16 (its own row instance), but
// 8 % slower at W = 16 T = 1024 and 1.3-2.3x slower at T <= 512.  Rows of 4104-8192
// elements, which would otherwise take split-H, gain 13-38 % (W = 12, 16 at H = 6144,
// 8192); longer rows, on several spans, measured even, so they keep their plan; a
// tuned lane layout keeps the row kernel.
bool many_ranks_scalar(int cu_count, int world, int tokens, int hidden, const arrms_tuning_t* t) {
    if (world <= 8 || hidden > 8 * 1024) return false;
    if (t && (t->vec_per_thread || t->threads_per_row || t->rows_per_block)) return false;
    const long long min_rows = static_cast<long long>(world == 16 ? 8 : 4) * cu_count;
    return tokens >= min_rows;
}

// Six to eight ranks: the rank loop also beats the row kernel, by 2-6 % (W = 6, 7, 8 at
// H = 2048, 4096, 8192, T >= 2048, measured on MI355X), but only on workgroups of 256,
// 512 or 1024 lanes: those divide a CU's 32 wave slots, which the rank loop needs full
// to cover its round trips.  With 384-896 lanes it lost 1-7 %, and below 8 rows per CU
// 10 % (W=8 H=2048 T=1024).  W <= 5 measured even or slower.
bool mid_ranks_rank_loop(int cu_count, int world, int tokens, int hidden, const arrms_tuning_t* t) {
    if (world < 6 || world > 8) return false;
    if (t && (t->vec_per_thread || t->threads_per_row || t->rows_per_block || t->scalar_elems)) return false;
    const int lanes = ((hidden + 7) / 8 + 63) / 64 * 64;
    if (lanes != 256 && lanes != 512 && lanes != 1024) return false;
    return tokens >= 8LL * cu_count;
}

// Rows the 16-byte kernels cannot take, with eight ranks: the rank loop instead of the
// specialised 8-rank scalar instance once a row takes 512 lanes or more.  That instance
// holds all eight ranks' loads (94 VGPRs at 2-byte loads: one 1024-lane workgroup per
// CU), the rank loop 45 at most.  Measured on MI355X (separately allocated tensors,
// 4.5 GB rotation): H = 8191 68.9 -> 78.1 %, H = 5119 65.3 -> 71.6 %, H = 4095 +2.6 %;
// on 256 lanes (H = 2047) 2 % slower, and at 6 or 7 ranks 1-4 % slower, so those keep
// the specialised instance.
bool odd_rows_rank_loop(int cu_count, int world, int tokens, int hidden, const arrms_tuning_t* t) {
    if (world != 8) return false;
    if (t && (t->threads_per_row || t->scalar_elems)) return false;
    const int lanes = ((hidden + 7) / 8 + 63) / 64 * 64;
    return lanes >= 512 && lanes <= 1024 && tokens >= 8LL * cu_count;
}

// Rows whose stride is not a multiple of 128 bytes (H % 64 != 0, H % 8 == 0): row r
// starts at byte 2*r*H mod 128 of a line, so the row kernel's wave instructions
// straddle two cache lines in most rows, while the scalar kernel rotates its lanes
// onto whole lines (8-byte loads here).  Measured on MI355X (4.5 GB rotation,
// interleaved runs) for rows of one span: from 256 lanes (H > 1536) and 16 rows per
// CU the scalar kernel is even or faster, 2-6 % at W = 2-8 (H = 2040, 3000, 5000, 6000, 8136) and 15-18 % at W = 1
// (four vectors per lane in the row kernel), except -1.3 % at W = 4 H = 7000; with 8
// rows per CU W = 1 lost 4 %.  Shorter rows gain only at one rank with 64 rows per CU
// (7-22 % at H = 520-1032; even or 2 % slower with 16-32), and lose 5-15 % at W = 4,
// where the row kernel packs several rows per workgroup.  A tuned lane layout keeps the
// row kernel.
bool line_offset_rows_scalar(int cu_count, int world, int tokens, int hidden, const arrms_tuning_t* t) {
    if (hidden % 64 == 0 || hidden > 8 * 1024) return false;
    if (t && (t->vec_per_thread || t->threads_per_row || t->rows_per_block)) return false;
    const int lanes = ((hidden + 7) / 8 + 63) / 64 * 64;
    if (lanes >= 256) return tokens >= 16LL * cu_count;
    return world == 1 && tokens >= 64LL * cu_count;
}

// Widest load, in BF16 elements, that H and the OR of all pointer addresses allow.
int scalar_elems(int hidden, uintptr_t any) {
    if (hidden % 4 == 0 && (any & 7u) == 0) return 4;
    if (hidden % 2 == 0 && (any & 3u) == 0) return 2;
    return 1;
}

// Automatic crossover to split-H, measured on MI355X with HIP-graph replay (GPU
// time per call) on ten shapes with 110-350 KiB of traffic per row: below about
// 144 KiB per row (W=4 H=8192, W=8 H=5120 and 6144, W=2 H=12288) split-H at best
// ties the one-kernel row variant at T=1 and loses 10-20 % from T=8 on; above it,
// split-H wins while T stays below a crossover that grows with the row (about 64
// rows at 160 KiB, about 100 at 176-224 KiB, between 128 and 192 at 350 KiB).
// Rule: split while T <= (cu/4) * (row KiB - 128) / 32, capped at cu/2.  With 256
// CUs that is 64 rows at 160 KiB, 96 at 176 KiB and the cap of 128 from 192 KiB
// up; the cap stays below the measured crossover of the longest rows, where the
// row kernel is the safe side.  Rows under 144 KiB never split automatically.
int auto_splith_max_tokens(int cu_count, int world, int hidden) {
    const long row_bytes = 2L * (world + 3) * hidden;
    if (row_bytes < kSplitMinRowBytes) return 0;
    long t = (cu_count / 4) * (row_bytes - (128L << 10)) / (32L << 10);
    if (t > cu_count / 2) t = cu_count / 2;
    return static_cast<int>(t);
}

}  // namespace

extern "C" {

const char* arrms_status_string(int status) {
    switch (status) {
        case ARRMS_OK: return "ok";
        case ARRMS_ERR_INVALID_ARG: return "invalid argument";
        case ARRMS_ERR_UNSUPPORTED: return "unsupported shape or variant";
        case ARRMS_ERR_HIP: return "HIP runtime error";
        case ARRMS_ERR_OOM: return "out of device memory";
        case ARRMS_ERR_SCRATCH: return "request exceeds the static scratch of the no-allocation entry point";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// A launch's grid in work-items (workgroups x lanes) is a 32-bit quantity on this
// GPU; larger requests are refused at planning time rather than by the runtime.
int check_grid(int rc, arrms_plan_t* plan) {
    if (rc == ARRMS_OK && static_cast<long long>(plan->grid) * plan->block > 0xffffffffLL) {
        memset(plan, 0, sizeof *plan);
        return ARRMS_ERR_UNSUPPORTED;
    }
    return rc;
}

int plan_fused(int cu_count, int variant, const arrms_tuning_t* tuning, int max_world, int max_tokens,
               int max_hidden, const void* const* partials, int world, int tokens, int hidden,
               const void* residual, const void* weight, float eps, const void* residual_out,
               const void* norm_out, arrms_plan_t* plan) {
    if (!plan) return ARRMS_ERR_INVALID_ARG;
    memset(plan, 0, sizeof *plan);
    if (cu_count < 1 || max_world < 1 || max_world > ARRMS_MAX_WORLD || max_tokens < 0 ||
        max_hidden < 1 || max_hidden > ARRMS_MAX_HIDDEN)
        return ARRMS_ERR_INVALID_ARG;
    if (variant < ARRMS_VARIANT_AUTO || variant > ARRMS_VARIANT_SCALAR) return ARRMS_ERR_INVALID_ARG;
    if (!valid_tuning(tuning)) return ARRMS_ERR_INVALID_ARG;
    if (world < 1 || world > max_world) return ARRMS_ERR_INVALID_ARG;
    if (tokens < 0 || tokens > max_tokens) return ARRMS_ERR_INVALID_ARG;
    if (hidden < 1 || hidden > max_hidden) return ARRMS_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || !isfinite(eps)) return ARRMS_ERR_INVALID_ARG;
    if (tokens == 0) return ARRMS_OK;  // nothing to do, nothing enqueued

    if (!partials || !residual || !weight || !residual_out || !norm_out) return ARRMS_ERR_INVALID_ARG;
    for (int r = 0; r < world; ++r)
        if (!partials[r]) return ARRMS_ERR_INVALID_ARG;

    // BF16 element alignment of every pointer.
    uintptr_t any = reinterpret_cast<uintptr_t>(residual) | reinterpret_cast<uintptr_t>(weight) |
                    reinterpret_cast<uintptr_t>(residual_out) | reinterpret_cast<uintptr_t>(norm_out);
    for (int r = 0; r < world; ++r) any |= reinterpret_cast<uintptr_t>(partials[r]);
    if (any & 1u) return ARRMS_ERR_INVALID_ARG;

    // Aliasing: outputs overlap nothing, except residual_out == residual exactly.
    const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden) * 2;
    const size_t nw = static_cast<size_t>(hidden) * 2;
    if (overlap(residual_out, n, norm_out, n)) return ARRMS_ERR_INVALID_ARG;
    if (residual_out != residual && overlap(residual_out, n, residual, n)) return ARRMS_ERR_INVALID_ARG;
    if (overlap(norm_out, n, residual, n)) return ARRMS_ERR_INVALID_ARG;
    if (overlap(residual_out, n, weight, nw) || overlap(norm_out, n, weight, nw)) return ARRMS_ERR_INVALID_ARG;
    for (int r = 0; r < world; ++r)
        if (overlap(residual_out, n, partials[r], n) || overlap(norm_out, n, partials[r], n))
            return ARRMS_ERR_INVALID_ARG;

    const bool vector_ok = (hidden % 8 == 0) && ((any & 15u) == 0);
    const int elems = scalar_elems(hidden, any);
    switch (variant) {
        case ARRMS_VARIANT_SCALAR:
            plan_scalar(world, tokens, hidden, elems, tuning, plan);
            return ARRMS_OK;
        case ARRMS_VARIANT_ROW:
            if (!vector_ok || hidden > ARRMS_ROW_MAX_HIDDEN) return ARRMS_ERR_UNSUPPORTED;
            return plan_row(cu_count, world, tokens, hidden, tuning, plan);
        case ARRMS_VARIANT_SPLITH:
            if (!vector_ok) return ARRMS_ERR_UNSUPPORTED;
            return plan_splith(cu_count, max_hidden, world, tokens, hidden, tuning, plan);
        default:
            break;
    }
    if (!vector_ok) {
        plan_scalar(world, tokens, hidden, elems, tuning, plan, odd_rows_rank_loop(cu_count, world, tokens, hidden,
                                                                                    tuning));
        return ARRMS_OK;
    }
    int split_max = (tuning && tuning->splith_max_tokens >= 0) ? tuning->splith_max_tokens
                                                              : auto_splith_max_tokens(cu_count, world, hidden);
    // More than 8 ranks, rows of one scalar span, enough rows: the scalar kernel.
    if (tokens > split_max && many_ranks_scalar(cu_count, world, tokens, hidden, tuning)) {
        plan_scalar(world, tokens, hidden, elems, tuning, plan);
        return ARRMS_OK;
    }
    // Six to eight ranks on power-of-two workgroups, enough rows: its rank loop.
    if (tokens > split_max && mid_ranks_rank_loop(cu_count, world, tokens, hidden, tuning)) {
        plan_scalar(world, tokens, hidden, elems, tuning, plan, true);
        return ARRMS_OK;
    }
    // Rows that start inside a 128-byte line, enough rows: the scalar kernel's rotated lanes.
    if (tokens > split_max && line_offset_rows_scalar(cu_count, world, tokens, hidden, tuning)) {
        plan_scalar(world, tokens, hidden, elems, tuning, plan);
        return ARRMS_OK;
    }
    // The automatic choice always finds a plan: tuning overrides that no vector
    // kernel can honour end in the scalar kernel (same results).
    if (hidden > ARRMS_ROW_MAX_HIDDEN || tokens <= split_max) {
        if (plan_splith(cu_count, max_hidden, world, tokens, hidden, tuning, plan) == ARRMS_OK) return ARRMS_OK;
        memset(plan, 0, sizeof *plan);
    }
    if (hidden <= ARRMS_ROW_MAX_HIDDEN && plan_row(cu_count, world, tokens, hidden, tuning, plan) == ARRMS_OK)
        return ARRMS_OK;
    // A row the row kernels cannot hold in registers: split it, else take the scalar kernel.
    memset(plan, 0, sizeof *plan);
    if (plan_splith(cu_count, max_hidden, world, tokens, hidden, tuning, plan) == ARRMS_OK) return ARRMS_OK;
    memset(plan, 0, sizeof *plan);
    plan_scalar(world, tokens, hidden, elems, tuning, plan);
    return ARRMS_OK;
}

int plan_reduce(int cu_count, const arrms_tuning_t* tuning, int max_world, int max_tokens, int max_hidden,
                const void* const* partials, int world, int tokens, int hidden, const void* reduced,
                arrms_plan_t* plan) {
    if (!plan) return ARRMS_ERR_INVALID_ARG;
    memset(plan, 0, sizeof *plan);
    if (cu_count < 1 || max_world < 1 || max_world > ARRMS_MAX_WORLD || max_tokens < 0 || max_hidden < 1 ||
        max_hidden > ARRMS_MAX_HIDDEN)
        return ARRMS_ERR_INVALID_ARG;
    if (!valid_tuning(tuning)) return ARRMS_ERR_INVALID_ARG;
    if (world < 1 || world > max_world) return ARRMS_ERR_INVALID_ARG;
    if (tokens < 0 || tokens > max_tokens) return ARRMS_ERR_INVALID_ARG;
    if (hidden < 1 || hidden > max_hidden) return ARRMS_ERR_INVALID_ARG;
    if (tokens == 0) return ARRMS_OK;
    if (!partials || !reduced) return ARRMS_ERR_INVALID_ARG;
    uintptr_t any = reinterpret_cast<uintptr_t>(reduced);
    for (int r = 0; r < world; ++r) {
        if (!partials[r]) return ARRMS_ERR_INVALID_ARG;
        any |= reinterpret_cast<uintptr_t>(partials[r]);
    }
    if (any & 1u) return ARRMS_ERR_INVALID_ARG;
    const long long count = static_cast<long long>(tokens) * hidden;
    const size_t n = static_cast<size_t>(count) * 2;
    // The output may be exactly one of the partials (each element is read before it is written).
    for (int r = 0; r < world; ++r)
        if (reduced != partials[r] && overlap(reduced, n, partials[r], n)) return ARRMS_ERR_INVALID_ARG;
    plan->kernels = 1;
    plan->rows_per_block = 1;
    plan->chunks_per_row = 1;
    plan->block = 256;
    plan->threads_per_row = 256;
    // Load width: the widest at which every pointer has the same offset (the first
    // few elements up to the aligned start are summed element-wise); tuning may cap it.
    int elems = 8, head = 0;
    arrms::reduce_alignment(partials, world, reduced, count, (tuning && tuning->scalar_elems) ? tuning->scalar_elems : 8,
                            &elems, &head);
    int vpt = 1;
    if (elems == 8) {
        vpt = kReduceAutoVpt;
        if (tuning && tuning->vec_per_thread) vpt = tuning->vec_per_thread;
        if (world > 8) {
            if (tuning && tuning->vec_per_thread > 1) return ARRMS_ERR_UNSUPPORTED;
            vpt = 1;
        }
        if (vpt > 4) return ARRMS_ERR_UNSUPPORTED;
    }
    // lanes move 16 bytes per partial per step whatever the width: groups per lane
    const int groups_per_lane = elems == 8 ? vpt : 8 / elems;
    const long long ngroups = (count - head) / elems;
    const long long per_block = 256LL * groups_per_lane;
    long long blocks = (ngroups + per_block - 1) / per_block;
    if (blocks < 1) blocks = 1;
    if (blocks > 0x7ffffff0LL) return ARRMS_ERR_UNSUPPORTED;
    plan->variant = elems == 8 ? ARRMS_VARIANT_REDUCE : ARRMS_VARIANT_REDUCE_SCALAR;
    plan->vec_per_thread = elems == 8 ? vpt : 0;
    plan->elems_per_load = elems;
    plan->blocks = static_cast<int>(blocks);
    // Six ranks or more: add them one load round at a time once every CU has at least 8
    // workgroups (measured on MI355X, 4.5 GB rotation: W = 9-16 4-11 % faster from 8
    // workgroups per CU, 80.9 % of HBM peak at W=16 T=4096 H=2048; W = 6 and 8 3-5 %
    // faster; W = 5 even, W = 4 up to 5 % slower; at 4 workgroups per CU 10 % slower and
    // at 1 per CU 1.8x, where the workgroups cannot cover the loop's round trips).
    plan->rank_loop = world >= 6 && blocks >= 8LL * cu_count;
    int k = 0;
    if (plan->blocks >= 64) {
        const long block_bytes = 2L * elems * per_block * (world + 1);
        k = 1;
        while (2L * k * block_bytes <= kXcdRunBytes) k *= 2;
    }
    finish_vector_plan(tuning, plan, k);
    return ARRMS_OK;
}

// Kernels with preloaded arguments (plan field kernarg_preload): their waves start
// without fetching the argument block from memory.  Measured on MI355X (W=4 H=2048,
// rotating buffers, the two interleaved): T = 1024 5 % faster, T = 4096 1.8 %
// (20.5 against 20.9 us), T = 16384 0.3 %; in HIP-graph replay T = 1 and 64 4-6 %
// faster.  Their flat argument list costs the host 0.2 us more per launch, and in
// some processes about 1 us more (back-to-back calls from C at T = 1 and 16 took
// 3.5-3.8 us instead of 2.5-2.7), so they serve only calls whose GPU time hides the
// launch: at least 16 MiB of traffic (about 5 us per call at W=4 H=2048).  Only row, scalar and
// rank-sum kernels specialised on W <= 8 have such twins (not split-H, which serves
// decode sizes, nor the rank loop's generic kernels, which carry 16 pointers).
constexpr long long kPreloadMinBytes = 16LL << 20;

void choose_preload(const arrms_tuning_t* t, bool has_twin, long long bytes, arrms_plan_t* p) {
    const int mode = t ? t->kernarg_preload : 0;
    p->kernarg_preload = has_twin && (mode == 2 || (mode == 0 && bytes >= kPreloadMinBytes)) ? 1 : 0;
}

}  // namespace

namespace arrms {

hipError_t launch_fused(const arrms_plan_t& p, const void* const* partials, int world, int tokens, int hidden,
                        const void* residual, const void* weight, float eps, void* residual_out, void* norm_out,
                        double* ws, hipStream_t stream) {
    Args a;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < world; ++r) a.x.p[r] = partials[r];
    a.residual = residual;
    a.weight = weight;
    a.residual_out = residual_out;
    a.norm_out = norm_out;
    a.ws = ws;
    a.hidden_d = static_cast<double>(hidden);
    a.eps = eps;
    a.world = world;
    a.tokens = tokens;
    a.hidden = hidden;
    a.nvec = hidden / 8;
    a.threads_per_row = p.threads_per_row;
    a.rows_per_block = p.rows_per_block;
    a.chunks = p.chunks_per_row;
    a.chunk_vec = p.block * p.vec_per_thread;
    a.blocks = p.blocks;
    a.xcd_chunk = p.xcd_chunk;
    a.elems_per_load = p.elems_per_load;
    a.ro_cached = p.residual_out_cached;
    a.rank_loop = p.rank_loop;
    a.preload = p.kernarg_preload;
    switch (p.variant) {
        case ARRMS_VARIANT_ROW: return launch_row(a, p.vec_per_thread, p.grid, p.block, stream);
        case ARRMS_VARIANT_SPLITH: return launch_splith(a, p.vec_per_thread, p.grid, p.block, stream);
        case ARRMS_VARIANT_SCALAR: return launch_scalar(a, p.grid, p.block, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace arrms

extern "C" {

int arrms_plan(int cu_count, int variant, const arrms_tuning_t* tuning, int max_world, int max_tokens,
               int max_hidden, const void* const* partials, int world, int tokens, int hidden,
               const void* residual, const void* weight, float eps, const void* residual_out,
               const void* norm_out, arrms_plan_t* plan) {
    const int rc = check_grid(plan_fused(cu_count, variant, tuning, max_world, max_tokens, max_hidden, partials,
                                         world, tokens, hidden, residual, weight, eps, residual_out, norm_out, plan),
                              plan);
    if (rc == ARRMS_OK && plan->grid > 0) {
        const bool twin = world <= 8 && (plan->variant == ARRMS_VARIANT_ROW ||
                                         (plan->variant == ARRMS_VARIANT_SCALAR && !plan->rank_loop));
        choose_preload(tuning, twin, 2LL * tokens * hidden * (world + 3) + 2LL * hidden, plan);
    }
    return rc;
}

int arrms_plan_reduce(int cu_count, const arrms_tuning_t* tuning, int max_world, int max_tokens, int max_hidden,
                      const void* const* partials, int world, int tokens, int hidden, const void* reduced,
                      arrms_plan_t* plan) {
    const int rc = check_grid(plan_reduce(cu_count, tuning, max_world, max_tokens, max_hidden, partials, world,
                                          tokens, hidden, reduced, plan),
                              plan);
    if (rc == ARRMS_OK && plan->grid > 0)
        choose_preload(tuning, world <= 8 && !plan->rank_loop, 2LL * tokens * hidden * (world + 1), plan);
    return rc;
}

int arrms_reduce(arrms_handle_t h, const void* const* partials, int world, int tokens, int hidden, void* reduced,
                 hipStream_t stream) {
    if (!h) return ARRMS_ERR_INVALID_ARG;
    arrms_plan_t p;
    const int rc = arrms_plan_reduce(h->cu_count, h->has_tuning ? &h->tuning : nullptr, h->max_world, h->max_tokens,
                                     h->max_hidden, partials, world, tokens, hidden, reduced, &p);
    if (rc != ARRMS_OK || p.grid == 0) return rc;
    // the pointers advanced to their first element aligned for the planned load width
    const long long count = static_cast<long long>(tokens) * hidden;
    int elems = 0, head = 0;
    arrms::reduce_alignment(partials, world, reduced, count, p.elems_per_load, &elems, &head);
    arrms::Args a;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < world; ++r) a.x.p[r] = static_cast<const uint16_t*>(partials[r]) + head;
    a.reduced = static_cast<uint16_t*>(reduced) + head;
    a.world = world;
    a.tokens = tokens;
    a.hidden = hidden;
    a.count = count - head;
    a.head = head;
    a.elems_per_load = elems;
    a.rank_loop = p.rank_loop;
    a.preload = p.kernarg_preload;
    a.blocks = p.blocks;
    a.xcd_chunk = p.xcd_chunk;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != h->device && hipSetDevice(h->device) != hipSuccess) {
        h->last_hip_error = static_cast<int>(hipErrorInvalidDevice);
        return ARRMS_ERR_HIP;
    }
    const hipError_t e = arrms::launch_reduce(a, p.vec_per_thread, p.grid, p.block, stream);
    if (prev >= 0 && prev != h->device) (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        h->last_hip_error = static_cast<int>(e);
        (void)hipGetLastError();  // reported through the status and arrms_last_hip_error
        return ARRMS_ERR_HIP;
    }
    return ARRMS_OK;
}

int arrms_create(arrms_handle_t* out, int device, int max_world, int max_tokens, int max_hidden) {
    if (!out) return ARRMS_ERR_INVALID_ARG;
    *out = nullptr;
    if (max_world < 1 || max_world > ARRMS_MAX_WORLD || max_tokens < 0 || max_hidden < 1 ||
        max_hidden > ARRMS_MAX_HIDDEN || device < 0)
        return ARRMS_ERR_INVALID_ARG;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count) return ARRMS_ERR_HIP;
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cu < 1)
        return ARRMS_ERR_HIP;

    arrms_ctx* h = new (std::nothrow) arrms_ctx();
    if (!h) return ARRMS_ERR_OOM;
    h->device = device;
    h->cu_count = cu;
    h->max_world = max_world;
    h->max_tokens = max_tokens;
    h->max_hidden = max_hidden;
    h->variant = ARRMS_VARIANT_AUTO;
    h->ws_chunks = chunks_capacity(max_hidden);

    const char* force = getenv("ARRMS_FORCE_VARIANT");
    if (force) {
        if (!strcmp(force, "row")) h->variant = ARRMS_VARIANT_ROW;
        else if (!strcmp(force, "splith")) h->variant = ARRMS_VARIANT_SPLITH;
        else if (!strcmp(force, "scalar")) h->variant = ARRMS_VARIANT_SCALAR;
    }

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (hipSetDevice(device) != hipSuccess) {
        delete h;
        return ARRMS_ERR_HIP;
    }
    int rc = ARRMS_OK;
    const size_t rows = max_tokens > 0 ? static_cast<size_t>(max_tokens) : 1;
    const hipError_t e = hipMalloc(reinterpret_cast<void**>(&h->ws), rows * h->ws_chunks * sizeof(double));
    if (e != hipSuccess) {
        rc = (e == hipErrorOutOfMemory) ? ARRMS_ERR_OOM : ARRMS_ERR_HIP;
        (void)hipGetLastError();  // reported here; leave no stale error for the caller's next launch check
    }
    if (rc != ARRMS_OK) {
        if (h->ws) (void)hipFree(h->ws);
        delete h;
        h = nullptr;
    }
    if (prev >= 0 && prev != device) (void)hipSetDevice(prev);
    *out = h;
    return rc;
}

int arrms_destroy(arrms_handle_t h) {
    if (!h) return ARRMS_OK;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    (void)hipSetDevice(h->device);
    int rc = ARRMS_OK;
    if (h->ws && hipFree(h->ws) != hipSuccess) rc = ARRMS_ERR_HIP;
    if (prev >= 0 && prev != h->device) (void)hipSetDevice(prev);
    delete h;
    return rc;
}

int arrms_last_hip_error(arrms_handle_t h) { return h ? h->last_hip_error : -1; }

int arrms_set_variant(arrms_handle_t h, int variant) {
    if (!h || variant < ARRMS_VARIANT_AUTO || variant > ARRMS_VARIANT_SCALAR) return ARRMS_ERR_INVALID_ARG;
    h->variant = variant;
    return ARRMS_OK;
}

int arrms_set_tuning(arrms_handle_t h, const arrms_tuning_t* tuning) {
    if (!h || !valid_tuning(tuning)) return ARRMS_ERR_INVALID_ARG;
    h->has_tuning = tuning != nullptr;
    if (tuning) h->tuning = *tuning;
    return ARRMS_OK;
}

int arrms_query_plan(arrms_handle_t h, const void* const* partials, int world, int tokens, int hidden,
                     const void* residual, const void* weight, float eps, const void* residual_out,
                     const void* norm_out, arrms_plan_t* plan) {
    if (!h) {
        if (plan) memset(plan, 0, sizeof *plan);
        return ARRMS_ERR_INVALID_ARG;
    }
    return arrms_plan(h->cu_count, h->variant, h->has_tuning ? &h->tuning : nullptr, h->max_world,
                      h->max_tokens, h->max_hidden, partials, world, tokens, hidden, residual, weight, eps,
                      residual_out, norm_out, plan);
}

int arrms_fused(arrms_handle_t h, const void* const* partials, int world, int tokens, int hidden,
                const void* residual, const void* weight, float eps, void* residual_out, void* norm_out,
                hipStream_t stream) {
    arrms_plan_t p;
    const int rc = arrms_query_plan(h, partials, world, tokens, hidden, residual, weight, eps, residual_out,
                                    norm_out, &p);
    if (rc != ARRMS_OK || p.grid == 0) return rc;
    // The handle's workspace holds max_tokens rows of the most chunks any call can plan.
    if (!arrms::splith_workspace_fits(p, tokens, static_cast<long long>(h->max_tokens > 0 ? h->max_tokens : 1) *
                                                     h->ws_chunks))
        return ARRMS_ERR_UNSUPPORTED;

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != h->device && hipSetDevice(h->device) != hipSuccess) {
        h->last_hip_error = static_cast<int>(hipErrorInvalidDevice);
        return ARRMS_ERR_HIP;
    }
    const hipError_t e = arrms::launch_fused(p, partials, world, tokens, hidden, residual, weight, eps, residual_out,
                                             norm_out, h->ws, stream);
    if (prev >= 0 && prev != h->device) (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        h->last_hip_error = static_cast<int>(e);
        (void)hipGetLastError();  // reported through the status and arrms_last_hip_error
        return ARRMS_ERR_HIP;
    }
    return ARRMS_OK;
}

}  // extern "C"
