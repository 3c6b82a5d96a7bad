// gfx950 kernels for the fused rank-partial sum + residual add + RMSNorm.
//
// Operation: the contract of the page "[TLERaw] Add NVSHMEM allreduce RMSNorm
// tutorial" (FlagTree PR #1122), section Summary and section Implementation 3:
// reduced = sum of the W rank partials, residual_out = reduced + residual,
// norm_out = RMSNorm(residual_out, weight, eps), on BF16 token rows.  Token rows
// go to independent workgroups (section Implementation 2, Row-parallel
// execution).  The page's one-CTA-per-row mapping is only approximate there,
// which leaves room for the split-H variant (several workgroups per row, for
// few rows) and for sub-wave row groups (several rows per wave, for small H).
//
// Every variant performs the same IEEE operations per element:
//   binary32 rank sum in rank order 0..W-1 starting from x_0, rounded once to BF16;
//   binary32 residual add, rounded to BF16 (residual_out);
//   binary64 sum of the exact squares of residual_out over the row;
//   inv = (float)(1 / sqrt(sum / H + eps)) in binary64 (correctly rounded divide
//   and square root, one rounding to binary32);
//   norm_out = BF16((residual_out * inv) * weight), two binary32 products.
// Only the association order of the binary64 sum of squares differs between
// variants (and from a sequential sum); see the note at seg_sum.
//
// The operation is bound by HBM bandwidth (about 0.6 flop per byte at W=4), so
// there is no matrix-core work: the kernels are built around 16-byte coalesced
// vector loads issued all at once per lane, registers that keep residual_out
// between the two passes over a row, and cross-lane (DPP) reductions.
#include <hip/hip_runtime.h>

#include "arrms_device.h"

namespace arrms {
namespace {

using namespace dev;

// ---------------------------------------------------------------- row variant
// threads_per_row lanes own one token row (16 or 32 lanes: several rows per
// wave; a multiple of 64: one or more whole waves per row), rows_per_block rows
// per workgroup.  Lane l handles vectors l, l + tpr, ..., l + (VPT-1)*tpr of the
// row, so at each step a wave reads 1 KiB of contiguous memory per input.  All
// (W + 2) * VPT loads of a lane are issued before any arithmetic; residual_out
// stays in registers for the second pass.  Both outputs are written with
// streaming stores, or residual_out with write-back stores when RC is set (a
// tuning choice that pays only where the call's data stays cache-resident).
// Largest workgroup of a row kernel; the host planner uses the same table.
template <int W, int VPT>
constexpr int row_max_threads() {
    return (W == 0 || W > 8) ? (VPT == 1 ? 512 : 256) : (VPT == 1 ? 1024 : (VPT <= 4 ? 512 : 256));
}

// The flat argument list of the row and scalar twins (FlatFusedArgs on the host),
// and the argument block rebuilt from it.
#define ARRMS_FLAT_FUSED_PARAMS                                                                              \
    int tokens, int xcd_chunk, uint32_t shape, float eps, const void* residual, const void* x0, const void* x1, \
        const void* x2, const void* x3, const void* x4, const void* x5, const void* x6, const void* x7,          \
        const void* weight, void* residual_out, void* norm_out
#define ARRMS_FLAT_FUSED_NAMES \
    tokens, xcd_chunk, shape, eps, residual, x0, x1, x2, x3, x4, x5, x6, x7, weight, residual_out, norm_out

template <class K, int W>
__device__ __forceinline__ K fused_block(ARRMS_FLAT_FUSED_PARAMS) {
    const void* const x[8] = {x0, x1, x2, x3, x4, x5, x6, x7};
    K a;
#pragma unroll
    for (int r = 0; r < W; ++r) a.x.p[r] = x[r];
    a.residual = residual;
    a.weight = weight;
    a.residual_out = residual_out;
    a.norm_out = norm_out;
    a.eps = eps;
    a.tokens = tokens;
    a.xcd_chunk = xcd_chunk;
    a.shape = shape;
    return a;
}

template <int W, int VPT, bool RC>
__device__ __forceinline__ void row_body(const RowArgs<(W > 0 ? W : kMaxWorld)>& a) {
    constexpr int WA = W > 0 ? W : kMaxWorld;
    const int world = W > 0 ? W : static_cast<int>((a.shape >> 26) & 31u);
    const int nvec = static_cast<int>(a.shape & 0xffffu);
    const int tpr = static_cast<int>((a.shape >> 16) & 127u) * 16;
    const int rpb_log2 = static_cast<int>((a.shape >> 23) & 7u);
    const int blocks = static_cast<int>((static_cast<unsigned>(a.tokens) + (1u << rpb_log2) - 1u) >> rpb_log2);
    const int block = logical_block(a.xcd_chunk, blocks);
    if (block < 0) return;  // padding workgroup of the XCD mapping (whole workgroup)
    const int tid = threadIdx.x;
    const int row_in_block = tid / tpr;
    const int lane = tid - row_in_block * tpr;
    const long long row = (static_cast<long long>(block) << rpb_log2) + row_in_block;
    const bool row_ok = row < a.tokens;
    const size_t base = static_cast<size_t>(row_ok ? row : 0) * static_cast<size_t>(nvec);

    bool ok[VPT];
    u32x4 xv[VPT][WA];
    u32x4 rv[VPT];
    u32x4 wv[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * tpr;
        ok[k] = row_ok && v < nvec;
        if (ok[k]) {
#pragma unroll
            for (int r = 0; r < WA; ++r)
                if (W > 0 || r < world) xv[k][r] = ld4_stream(a.x.p[r], base + v);
            rv[k] = ld4_stream(a.residual, base + v);
            wv[k] = ld4(a.weight, v);
        }
    }

    double ss = 0.0;
    u32x4 ro[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        if (ok[k]) {
            ro[k] = residual_vec<W>(xv[k], world, rv[k], ss);
            if constexpr (RC) {
                st4(a.residual_out, base + lane + k * tpr, ro[k]);
            } else {
                st4_stream(a.residual_out, base + lane + k * tpr, ro[k]);
            }
        }
    }

    ss = seg_sum(ss, tpr < 64 ? tpr : 64);
    if (tpr > 64) {
        // Cross-wave combine through LDS, in wave order (deterministic).
        __shared__ double wave_ss[16];
        if ((tid & 63) == 0) wave_ss[tid >> 6] = ss;
        __syncthreads();
        const int first = (row_in_block * tpr) >> 6;
        const int waves = tpr >> 6;
        double t = wave_ss[first];
        for (int i = 1; i < waves; ++i) t = t + wave_ss[first + i];
        ss = t;
    }
    const float inv = inv_rms(ss, static_cast<double>(nvec * 8), a.eps);

#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (ok[k]) st4_stream(a.norm_out, base + lane + k * tpr, norm_vec(ro[k], inv, wv[k]));
}

template <int W, int VPT, bool RC>
__global__ void __launch_bounds__((row_max_threads<W, VPT>())) row_kernel(const RowArgs<(W > 0 ? W : kMaxWorld)> a) {
    row_body<W, VPT, RC>(a);
}

// The same kernel for W <= 8 with the flat argument list, its leading dwords
// preloaded into scalar registers.
template <int W, int VPT, bool RC>
__global__ void __launch_bounds__((row_max_threads<W, VPT>())) row_kernel_flat(ARRMS_FLAT_FUSED_PARAMS) {
    static_assert(W >= 1 && W <= 8, "flat argument lists carry at most 8 partials");
    row_body<W, VPT, RC>(fused_block<RowArgs<W>, W>(ARRMS_FLAT_FUSED_NAMES));
}

// ------------------------------------------------------------ split-H variant
// For few rows: row t is cut into `chunks` chunks of chunk_vec vectors and each
// chunk gets a workgroup, in two kernels launched back to back on the stream.
// Phase 1: rank sum, residual add and residual_out store for the chunk; the
// chunk's binary64 sum of squares goes to ws[t][chunk].  Phase 2: each chunk's
// workgroup adds ws[t][0..chunks-1] in chunk order (every workgroup of a row
// gets the same bits), computes 1/RMS, re-reads its residual_out chunk and
// writes norm_out.  The kernel boundary orders phase 1's stores before phase
// 2's loads on every XCD; a single-kernel hand-off between workgroups would
// need a device-scope release per workgroup, which writes back the XCD's whole
// L2 and costs far more than the second launch.  No workgroup ever waits for
// another, and the workspace needs no reset between calls.
template <int W>
constexpr int splith_max_threads() { return (W == 0 || W > 8) ? 512 : 1024; }

template <int W, int VPT>
__global__ void __launch_bounds__(splith_max_threads<W>())
    splith_partial_kernel(const SplitPartialArgs<(W > 0 ? W : kMaxWorld)> a) {
    constexpr int WA = W > 0 ? W : kMaxWorld;
    const int world = W > 0 ? W : static_cast<int>((a.shape >> 16) & 31u);
    const int chunks = static_cast<int>(a.shape & 0xffffu);
    const int nvec = static_cast<int>(a.vec & 0xffffu);
    const int chunk_vec = static_cast<int>(a.vec >> 16);
    const int block = logical_block(a.xcd_chunk, a.blocks);
    if (block < 0) return;
    const int row = block / chunks;
    const int chunk = block - row * chunks;
    const int tid = threadIdx.x;
    const int nthreads = chunk_vec / VPT;  // the workgroup size
    const int v0 = chunk * chunk_vec;
    const int v1 = min(nvec, v0 + chunk_vec);
    const size_t base = static_cast<size_t>(row) * static_cast<size_t>(nvec);

    bool ok[VPT];
    u32x4 xv[VPT][WA];
    u32x4 rv[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = v0 + tid + k * nthreads;
        ok[k] = v < v1;
        if (ok[k]) {
#pragma unroll
            for (int r = 0; r < WA; ++r)
                if (W > 0 || r < world) xv[k][r] = ld4_stream(a.x.p[r], base + v);
            rv[k] = ld4_stream(a.residual, base + v);
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        if (ok[k]) {
            const u32x4 ro = residual_vec<W>(xv[k], world, rv[k], ss);
            st4(a.residual_out, base + v0 + tid + k * nthreads, ro);  // re-read by phase 2: keep cached
        }
    }

    __shared__ double wave_ss[16];
    ss = seg_sum(ss, 64);
    if ((tid & 63) == 0) wave_ss[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) {
        double t = wave_ss[0];
        for (int i = 1; i < (nthreads >> 6); ++i) t = t + wave_ss[i];
        a.ws[static_cast<size_t>(row) * chunks + chunk] = t;
    }
}

__global__ void __launch_bounds__(1024) splith_norm_kernel(const SplitNormArgs a) {
    const int chunks = static_cast<int>(a.shape & 0xffffu);
    const int nthreads = static_cast<int>(a.shape >> 16);
    const int nvec = static_cast<int>(a.vec & 0xffffu);
    const int chunk_vec = static_cast<int>(a.vec >> 16);
    const int block = logical_block(a.xcd_chunk, a.blocks);
    if (block < 0) return;
    const int row = block / chunks;
    const int chunk = block - row * chunks;
    const int tid = threadIdx.x;
    const int v0 = chunk * chunk_vec;
    const int v1 = min(nvec, v0 + chunk_vec);
    const size_t base = static_cast<size_t>(row) * static_cast<size_t>(nvec);
    const double* part = a.ws + static_cast<size_t>(row) * chunks;
    double total = part[0];
    for (int c = 1; c < chunks; ++c) total = total + part[c];
    const float inv = inv_rms(total, static_cast<double>(nvec * 8), a.eps);
    for (int v = v0 + tid; v < v1; v += nthreads)
        st4_stream(a.norm_out, base + v, norm_vec(ld4(a.residual_out, base + v), inv, ld4(a.weight, v)));
}

// -------------------------------------------------------------- scalar variant
// Rows that the 16-byte kernels cannot take (H % 8 != 0, or a pointer not 16-byte
// aligned); rows whose stride is not a multiple of 128 bytes (H % 64 != 0), which
// the planner gives it where its line rotation (below) measured faster; and,
// through the generic instance's rank loop (W = 0: only x_0 loaded up front, the
// other ranks added one load round at a time), calls with many ranks.  Loads are E
// BF16 elements wide (E = 4, 2 or 1: 8-, 4- or 2-byte loads), the widest that H and
// the alignment of every pointer allow.  One row per workgroup of n lanes
// (n <= 1024), XCD runs as in the row variant.  The row is walked in spans of
// kScalarSpan * n elements; in a span lane l owns the E-element groups l, l + n, ..., l + (8 / E - 1) * n, so each
// load instruction of a wave covers 128 * E contiguous bytes and a lane moves 16
// bytes per input per span, as in the row variant.
//
// Every access goes through a buffer resource spanning one row of its tensor (the
// weight's whole H elements), so the hardware's range check does the masking: a
// group index before or past the row loads zeros, which add nothing to the sum of
// squares, and stores nothing.  No index is clamped, no store is under a branch,
// and one 32-bit byte offset per group serves every tensor: at 2-byte loads this
// kernel's time follows its instruction count, and 64-bit per-tensor addresses,
// clamps and store branches cost it more than the memory traffic.  All loads of a
// span are issued before its arithmetic.  When the row fits one span,
// residual_out stays in registers for the second pass; otherwise the second pass
// re-reads it (each group is read back by the lane that stored it).
//
// A row whose start is not on a 128-byte line (H % 64 != 0, or a pointer offset)
// would make every wave instruction straddle two lines.  So the lanes' group indexes are
// moved back by the row's offset within its line of the first partial (`shift`
// groups); the wave instructions then cover whole lines of every tensor aligned
// like that partial.  A row that fits one span is rotated: index i takes group
// (i - shift) mod span, a one-to-one map of the span, so the last `shift` groups
// go to the first lanes and only wave 0's first instruction touches two lines (the
// row's first and last); the row needs no lanes beyond its own length.  (Extra
// lanes for the shift cost more than the straddling: 5-wave workgroups on rows of
// 2048 elements were 18 % slower than 4-wave ones on MI355X.)  A longer row is
// shifted instead: index i takes group i - shift over ng + shift indexes, and the
// indexes before the row start fall outside its range.  Since shift < 64 <= n, only
// a lane's first group of the first span can wrap or fall before the row.
constexpr int kScalarSpan = 8;

// Largest workgroup of a scalar kernel (the host planner uses the same limit).  The
// generic-W instance holds only x_0's loads (its rank loop adds the others one round
// at a time), so it fits 1024 lanes as the specialised ones do.
template <int W>
constexpr int scalar_max_threads() { return 1024; }

template <int W, int E, bool RC>
__device__ __forceinline__ void scalar_body(const ScalarArgs<(W > 0 ? W : kMaxWorld)>& a) {
    typedef typename Group<E>::T G;
    typedef Buf<E> B;
    constexpr int S = kScalarSpan / E;  // groups per lane per input in a span
    constexpr int WL = W > 0 ? W : 1;   // ranks whose loads a span keeps in registers
    const int world = W > 0 ? W : static_cast<int>((a.shape >> 22) & 31u);
    const int row = logical_block(a.xcd_chunk, a.tokens);
    if (row < 0) return;  // padding workgroup of the XCD mapping (whole workgroup)
    const int tid = threadIdx.x;
    const int n = static_cast<int>((a.shape >> 17) & 31u) * 64;  // the workgroup size
    const int H = static_cast<int>(a.shape & 0x1ffffu);
    const int ng = H / E;  // groups per row
    const int span = S * n;
    const int row_bytes = 2 * H;
    const size_t base = static_cast<size_t>(row) * static_cast<size_t>(H);  // the row's first element
    const uint16_t* x0 = static_cast<const uint16_t*>(a.x.p[0]) + base;
    const int shift = static_cast<int>((reinterpret_cast<uintptr_t>(x0) & 127u) / sizeof(G));
    const bool single = ng <= span;               // one span: rotate; longer rows: shift
    const int nidx = single ? span : ng + shift;  // lane indexes that cover the row
    const int first = tid - shift;                // group of the lane's first index
    const int first_off = static_cast<int>(sizeof(G)) * ((single && first < 0) ? first + span : first);
    // byte offset of the lane's u-th group in the span from index i0
    auto offset = [=](int i0, int u) {
        return (i0 == 0 && u == 0) ? first_off : static_cast<int>(sizeof(G)) * (i0 + u * n + first);
    };
    Rsrc rx[WL];
#pragma unroll
    for (int r = 0; r < WL; ++r) rx[r] = make_rsrc(static_cast<const uint16_t*>(a.x.p[r]) + base, row_bytes);
    const Rsrc rres = make_rsrc(static_cast<const uint16_t*>(a.residual) + base, row_bytes);
    const Rsrc rw = make_rsrc(a.weight, row_bytes);
    const Rsrc rro = make_rsrc(static_cast<uint16_t*>(a.residual_out) + base, row_bytes);
    const Rsrc rno = make_rsrc(static_cast<uint16_t*>(a.norm_out) + base, row_bytes);

    double ss = 0.0;
    G keep[S];  // residual_out of the last span
    G wk[S];    // weight of the last span, loaded with its inputs
    for (int i0 = 0; i0 < nidx; i0 += span) {
        // every load of the span first (the ranks kept, residual, weight), then the arithmetic
        G xv[WL][S];
        G rs[S];
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int off = offset(i0, u);
#pragma unroll
            for (int r = 0; r < WL; ++r) xv[r][u] = B::template ld<kBufNT>(rx[r], off);
            rs[u] = B::template ld<kBufNT>(rres, off);
            wk[u] = B::template ld<0>(rw, off);
        }
        // keep the scheduler from interleaving the arithmetic (and its waits) into the loads
        __builtin_amdgcn_sched_barrier(0);
        // binary32 rank sums, rank order 0, 1, ..., W-1 for every element
        float acc[S][E];
#pragma unroll
        for (int u = 0; u < S; ++u) {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                acc[u][k] = Group<E>::get(xv[0][u], k);
#pragma unroll
                for (int r = 1; r < WL; ++r) acc[u][k] = acc[u][k] + Group<E>::get(xv[r][u], k);
            }
        }
        if constexpr (W == 0) {
            // the generic kernel (up to 16 ranks, W known at run time) adds the ranks
            // after x_0 one at a time, which keeps its registers within budget
            for (int r = 1; r < world; ++r) {
                const Rsrc rr = make_rsrc(static_cast<const uint16_t*>(a.x.p[r]) + base, row_bytes);
                G v[S];
#pragma unroll
                for (int u = 0; u < S; ++u) v[u] = B::template ld<kBufNT>(rr, offset(i0, u));
#pragma unroll
                for (int u = 0; u < S; ++u)
#pragma unroll
                    for (int k = 0; k < E; ++k) acc[u][k] = acc[u][k] + Group<E>::get(v[u], k);
            }
        }
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const G rg = pack<E>(acc[u]);
            float o[E];
#pragma unroll
            for (int k = 0; k < E; ++k) o[k] = Group<E>::get(rg, k) + Group<E>::get(rs[u], k);
            const G og = pack<E>(o);
            keep[u] = og;
            B::template st<RC ? 0 : kBufNT>(og, rro, offset(i0, u));
#pragma unroll
            for (int k = 0; k < E; ++k) {
                // zero outside the row (its loads returned zeros)
                const double d = static_cast<double>(Group<E>::get(og, k));
                ss = __builtin_fma(d, d, ss);
            }
        }
    }
    __shared__ double wave_ss[16];
    ss = seg_sum(ss, 64);
    if ((tid & 63) == 0) wave_ss[tid >> 6] = ss;
    __syncthreads();
    double total = wave_ss[0];
    for (int i = 1; i < (n >> 6); ++i) total = total + wave_ss[i];
    const float inv = inv_rms(total, static_cast<double>(H), a.eps);

    if (single) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            float v[E];
#pragma unroll
            for (int k = 0; k < E; ++k) v[k] = (Group<E>::get(keep[u], k) * inv) * Group<E>::get(wk[u], k);
            B::template st<kBufNT>(pack<E>(v), rno, offset(0, u));
        }
        return;
    }
    for (int i0 = 0; i0 < nidx; i0 += span) {
        G rv[S], wv[S];
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int off = offset(i0, u);
            rv[u] = B::template ld<0>(rro, off);
            wv[u] = B::template ld<0>(rw, off);
        }
#pragma unroll
        for (int u = 0; u < S; ++u) {
            float v[E];
#pragma unroll
            for (int k = 0; k < E; ++k) v[k] = (Group<E>::get(rv[u], k) * inv) * Group<E>::get(wv[u], k);
            B::template st<kBufNT>(pack<E>(v), rno, offset(i0, u));
        }
    }
}

template <int W, int E, bool RC>
__global__ void __launch_bounds__(scalar_max_threads<W>()) scalar_kernel(const ScalarArgs<(W > 0 ? W : kMaxWorld)> a) {
    scalar_body<W, E, RC>(a);
}

// The same kernel for W <= 8 with the flat argument list (leading dwords preloaded).
template <int W, int E, bool RC>
__global__ void __launch_bounds__(scalar_max_threads<W>()) scalar_kernel_flat(ARRMS_FLAT_FUSED_PARAMS) {
    static_assert(W >= 1 && W <= 8, "flat argument lists carry at most 8 partials");
    scalar_body<W, E, RC>(fused_block<ScalarArgs<W>, W>(ARRMS_FLAT_FUSED_NAMES));
}

// ---------------------------------------------------------------- launchers
// Argument blocks.  Each returns false when a size does not fit its packed
// field (the planner never produces such a plan; the launch is then refused).
template <int WA>
bool row_args(const Args& a, RowArgs<WA>* r) {
    const int tpr16 = a.threads_per_row / 16;
    int rpb_log2 = 0;
    while ((1 << rpb_log2) < a.rows_per_block) ++rpb_log2;
    if (a.nvec > 0xffff || a.threads_per_row % 16 || tpr16 < 1 || tpr16 > 127 || (1 << rpb_log2) != a.rows_per_block ||
        rpb_log2 > 7 || a.world > 31)
        return false;
    *r = RowArgs<WA>{};
    r->x = pack_ptrs<WA>(a);
    r->residual = a.residual;
    r->weight = a.weight;
    r->residual_out = a.residual_out;
    r->norm_out = a.norm_out;
    r->eps = a.eps;
    r->tokens = a.tokens;
    r->xcd_chunk = a.xcd_chunk;
    r->shape = static_cast<uint32_t>(a.nvec) | static_cast<uint32_t>(tpr16) << 16 |
               static_cast<uint32_t>(rpb_log2) << 23 | static_cast<uint32_t>(a.world) << 26;
    return true;
}

// The flat argument list of the row and scalar twins, from their argument block.
template <int WA, class K>
FlatFusedArgs flat_fused(const K& r) {
    FlatFusedArgs f{};
    f.tokens = r.tokens;
    f.xcd_chunk = r.xcd_chunk;
    f.shape = r.shape;
    f.eps = r.eps;
    f.residual = r.residual;
    for (int i = 0; i < WA && i < 8; ++i) f.x[i] = r.x.p[i];
    f.weight = r.weight;
    f.residual_out = r.residual_out;
    f.norm_out = r.norm_out;
    return f;
}

// `fn` is the flat twin when a.preload is set (W <= 8), else the by-value kernel.
template <int WA>
hipError_t launch_row_with(const void* fn, const Args& a, int grid, int block, hipStream_t s) {
    RowArgs<WA> r;
    if (!row_args<WA>(a, &r)) return hipErrorInvalidValue;
    if (a.preload) {
        if (WA > 8) return hipErrorInvalidValue;
        FlatFusedArgs f = flat_fused<WA>(r);
        return launch_flat(fn, f, grid, block, s);
    }
    return launch_with(fn, r, grid, block, s);
}

bool splith_fits(const Args& a, int block) {
    return a.nvec <= 0xffff && a.chunk_vec <= 0xffff && a.chunks <= 0xffff && block <= 0xffff && a.world <= 31;
}

template <int WA>
hipError_t launch_splith_partial_with(const void* fn, const Args& a, int grid, int block, hipStream_t s) {
    SplitPartialArgs<WA> r{};
    r.x = pack_ptrs<WA>(a);
    r.residual = a.residual;
    r.residual_out = a.residual_out;
    r.ws = a.ws;
    r.blocks = a.blocks;
    r.xcd_chunk = a.xcd_chunk;
    r.vec = static_cast<uint32_t>(a.nvec) | static_cast<uint32_t>(a.chunk_vec) << 16;
    r.shape = static_cast<uint32_t>(a.chunks) | static_cast<uint32_t>(a.world) << 16;
    return launch_with(fn, r, grid, block, s);
}

template <int WA>
hipError_t launch_scalar_with(const void* fn, const Args& a, int grid, int block, hipStream_t s) {
    const int e_code = a.elems_per_load == 4 ? 2 : (a.elems_per_load == 2 ? 1 : 0);
    if (block % 64 || block < 64 || block > 1024 || a.world > 31 || a.hidden < 1 ||
        a.hidden > 0x1ffff ||
        (1 << e_code) != a.elems_per_load || a.hidden % a.elems_per_load)
        return hipErrorInvalidValue;
    ScalarArgs<WA> r{};
    r.x = pack_ptrs<WA>(a);
    r.residual = a.residual;
    r.weight = a.weight;
    r.residual_out = a.residual_out;
    r.norm_out = a.norm_out;
    r.eps = a.eps;
    r.tokens = a.tokens;
    r.xcd_chunk = a.xcd_chunk;
    r.shape = static_cast<uint32_t>(a.hidden) | static_cast<uint32_t>(block / 64) << 17 |
              static_cast<uint32_t>(a.world) << 22 | static_cast<uint32_t>(e_code) << 27;
    if (a.preload) {
        if (WA > 8) return hipErrorInvalidValue;
        FlatFusedArgs f = flat_fused<WA>(r);
        return launch_flat(fn, f, grid, block, s);
    }
    return launch_with(fn, r, grid, block, s);
}

// The by-value kernel, or its flat twin (W <= 8 only; nullptr for other W).
template <int W, int VPT, bool RC>
const void* row_sym(bool flat) {
    if constexpr (W >= 1 && W <= 8) {
        if (flat) return reinterpret_cast<const void*>(&row_kernel_flat<W, VPT, RC>);
    } else {
        if (flat) return nullptr;
    }
    return reinterpret_cast<const void*>(&row_kernel<W, VPT, RC>);
}

// Instantiated (W, VPT) pairs: those whose (W + 2) * VPT live vectors fit the
// register budget the host planner allows (40); others are never planned.
template <int VPT, bool RC>
const void* row_fn(int world, bool flat) {
    if (VPT == 8 && world > 3) return nullptr;
    switch (world) {
        case 1: return row_sym<1, VPT, RC>(flat);
        case 2: return row_sym<2, VPT, RC>(flat);
        case 3: return row_sym<3, VPT, RC>(flat);
        default: break;
    }
    if constexpr (VPT <= 4) {
        switch (world) {
            case 4: return row_sym<4, VPT, RC>(flat);
            case 5: return row_sym<5, VPT, RC>(flat);
            case 6: return row_sym<6, VPT, RC>(flat);
            case 7: return row_sym<7, VPT, RC>(flat);
            case 8: return row_sym<8, VPT, RC>(flat);
            default: break;
        }
    }
    if constexpr (VPT <= 2) {
        if (world == 16) return row_sym<16, VPT, RC>(flat);
        return row_sym<0, VPT, RC>(flat);
    }
    return nullptr;
}

template <int VPT>
const void* splith_fn(int world) {
    switch (world) {
        case 1: return reinterpret_cast<const void*>(&splith_partial_kernel<1, VPT>);
        case 2: return reinterpret_cast<const void*>(&splith_partial_kernel<2, VPT>);
        case 3: return reinterpret_cast<const void*>(&splith_partial_kernel<3, VPT>);
        case 4: return reinterpret_cast<const void*>(&splith_partial_kernel<4, VPT>);
        case 5: return reinterpret_cast<const void*>(&splith_partial_kernel<5, VPT>);
        case 6: return reinterpret_cast<const void*>(&splith_partial_kernel<6, VPT>);
        case 7: return reinterpret_cast<const void*>(&splith_partial_kernel<7, VPT>);
        case 8: return reinterpret_cast<const void*>(&splith_partial_kernel<8, VPT>);
        default: break;
    }
    if constexpr (VPT == 1) {
        if (world == 16) return reinterpret_cast<const void*>(&splith_partial_kernel<16, 1>);
        return reinterpret_cast<const void*>(&splith_partial_kernel<0, 1>);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_row(const Args& a, int vpt, int grid, int block, hipStream_t s) {
    const void* fn = nullptr;
    const bool rc = a.ro_cached != 0;
    const bool flat = a.preload != 0;
    switch (vpt) {
        case 1: fn = rc ? row_fn<1, true>(a.world, flat) : row_fn<1, false>(a.world, flat); break;
        case 2: fn = rc ? row_fn<2, true>(a.world, flat) : row_fn<2, false>(a.world, flat); break;
        case 4: fn = rc ? row_fn<4, true>(a.world, flat) : row_fn<4, false>(a.world, flat); break;
        case 8: fn = rc ? row_fn<8, true>(a.world, flat) : row_fn<8, false>(a.world, flat); break;
        default: return hipErrorInvalidValue;
    }
    if (!fn) return hipErrorInvalidValue;
    // row_kernel<W, VPT, RC> takes RowArgs<W> for W <= 8 and RowArgs<16> otherwise
    switch (a.world) {
        case 1: return launch_row_with<1>(fn, a, grid, block, s);
        case 2: return launch_row_with<2>(fn, a, grid, block, s);
        case 3: return launch_row_with<3>(fn, a, grid, block, s);
        case 4: return launch_row_with<4>(fn, a, grid, block, s);
        case 5: return launch_row_with<5>(fn, a, grid, block, s);
        case 6: return launch_row_with<6>(fn, a, grid, block, s);
        case 7: return launch_row_with<7>(fn, a, grid, block, s);
        case 8: return launch_row_with<8>(fn, a, grid, block, s);
        default: return launch_row_with<kMaxWorld>(fn, a, grid, block, s);
    }
}

hipError_t launch_splith(const Args& a, int vpt, int grid, int block, hipStream_t s) {
    if (a.preload) return hipErrorInvalidValue;  // split-H has no flat twins (decode sizes only)
    const void* fn = nullptr;
    switch (vpt) {
        case 1: fn = splith_fn<1>(a.world); break;
        case 2: fn = splith_fn<2>(a.world); break;
        default: return hipErrorInvalidValue;
    }
    if (!fn || !splith_fits(a, block) || a.chunk_vec != block * vpt) return hipErrorInvalidValue;
    hipError_t e;
    switch (a.world) {
        case 1: e = launch_splith_partial_with<1>(fn, a, grid, block, s); break;
        case 2: e = launch_splith_partial_with<2>(fn, a, grid, block, s); break;
        case 3: e = launch_splith_partial_with<3>(fn, a, grid, block, s); break;
        case 4: e = launch_splith_partial_with<4>(fn, a, grid, block, s); break;
        case 5: e = launch_splith_partial_with<5>(fn, a, grid, block, s); break;
        case 6: e = launch_splith_partial_with<6>(fn, a, grid, block, s); break;
        case 7: e = launch_splith_partial_with<7>(fn, a, grid, block, s); break;
        case 8: e = launch_splith_partial_with<8>(fn, a, grid, block, s); break;
        default: e = launch_splith_partial_with<kMaxWorld>(fn, a, grid, block, s); break;
    }
    if (e != hipSuccess) return e;
    SplitNormArgs n{};
    n.residual_out = a.residual_out;
    n.weight = a.weight;
    n.norm_out = a.norm_out;
    n.ws = a.ws;
    n.eps = a.eps;
    n.blocks = a.blocks;
    n.xcd_chunk = a.xcd_chunk;
    n.vec = static_cast<uint32_t>(a.nvec) | static_cast<uint32_t>(a.chunk_vec) << 16;
    n.shape = static_cast<uint32_t>(a.chunks) | static_cast<uint32_t>(block) << 16;
    return launch_with(reinterpret_cast<const void*>(&splith_norm_kernel), n, grid, block, s);
}

template <int W, int E, bool RC>
const void* scalar_sym(bool flat) {
    if constexpr (W >= 1 && W <= 8) {
        if (flat) return reinterpret_cast<const void*>(&scalar_kernel_flat<W, E, RC>);
    } else {
        if (flat) return nullptr;
    }
    return reinterpret_cast<const void*>(&scalar_kernel<W, E, RC>);
}

template <int E, bool RC>
const void* scalar_fn(int world, bool flat) {
    switch (world) {
        case 1: return scalar_sym<1, E, RC>(flat);
        case 2: return scalar_sym<2, E, RC>(flat);
        case 3: return scalar_sym<3, E, RC>(flat);
        case 4: return scalar_sym<4, E, RC>(flat);
        case 5: return scalar_sym<5, E, RC>(flat);
        case 6: return scalar_sym<6, E, RC>(flat);
        case 7: return scalar_sym<7, E, RC>(flat);
        case 8: return scalar_sym<8, E, RC>(flat);
        default: return scalar_sym<0, E, RC>(flat);
    }
}

hipError_t launch_scalar(const Args& a, int grid, int block, hipStream_t s) {
    const void* fn = nullptr;
    const bool rc = a.ro_cached != 0;
    // the rank loop is the generic instance (any rank count, ranks after x_0 added one at a time)
    const int w = a.rank_loop ? 0 : a.world;
    const bool flat = a.preload != 0;
    switch (a.elems_per_load) {
        case 1: fn = rc ? scalar_fn<1, true>(w, flat) : scalar_fn<1, false>(w, flat); break;
        case 2: fn = rc ? scalar_fn<2, true>(w, flat) : scalar_fn<2, false>(w, flat); break;
        case 4: fn = rc ? scalar_fn<4, true>(w, flat) : scalar_fn<4, false>(w, flat); break;
        default: return hipErrorInvalidValue;
    }
    if (!fn) return hipErrorInvalidValue;
    if (a.rank_loop) return launch_scalar_with<kMaxWorld>(fn, a, grid, block, s);
    switch (a.world) {
        case 1: return launch_scalar_with<1>(fn, a, grid, block, s);
        case 2: return launch_scalar_with<2>(fn, a, grid, block, s);
        case 3: return launch_scalar_with<3>(fn, a, grid, block, s);
        case 4: return launch_scalar_with<4>(fn, a, grid, block, s);
        case 5: return launch_scalar_with<5>(fn, a, grid, block, s);
        case 6: return launch_scalar_with<6>(fn, a, grid, block, s);
        case 7: return launch_scalar_with<7>(fn, a, grid, block, s);
        case 8: return launch_scalar_with<8>(fn, a, grid, block, s);
        default: return launch_scalar_with<kMaxWorld>(fn, a, grid, block, s);
    }
}

}  // namespace arrms
