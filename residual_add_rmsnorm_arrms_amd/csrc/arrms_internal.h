// Internal interface between the C-ABI host code (arrms_api.cpp) and the gfx950
// kernels (arrms_kernels.hip).  Not installed; the public interface is include/arrms.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "arrms.h"

namespace arrms {

constexpr int kMaxWorld = 16;

// The W rank-partial base pointers travel by value inside the kernel arguments,
// so a call needs no host-to-device copy of the pointer array.
struct Partials {
    const void* p[kMaxWorld];
};

// One call's description, filled by the host code; each launcher packs the
// fields its kernel needs into that kernel's argument block (below).
struct Args {
    Partials x;             // W device pointers, BF16 [tokens][hidden]
    const void* residual;   // BF16 [tokens][hidden]
    const void* weight;     // BF16 [hidden]
    void* residual_out;     // BF16 [tokens][hidden]; may equal residual
    void* norm_out;         // BF16 [tokens][hidden]
    void* reduced;          // rank sum only: BF16 [tokens][hidden] output
    double* ws;             // split-H: [tokens][chunks] binary64 partial sums of squares
    double hidden_d;        // H as binary64 (the divisor of the mean of squares)
    float eps;
    int world;              // W
    int tokens;             // T
    int hidden;             // H
    int nvec;               // H / 8: 16-byte vectors per row (vector variants)
    int threads_per_row;    // row: lanes that share one row
    int rows_per_block;     // row: rows per workgroup
    int chunks;             // split-H: chunks per row
    int chunk_vec;          // split-H: vectors per chunk
    int blocks;             // logical workgroups (the launched grid may add XCD padding)
    int xcd_chunk;          // K > 0: runs of K consecutive blocks per XCD (grid a multiple of 8K)
    int elems_per_load;     // scalar: BF16 elements per load (1, 2 or 4); rank sum: 1, 2, 4 or 8
    int head;               // rank sum only: elements before the aligned start of x.p[] / reduced
    int ro_cached;          // row, scalar: 1 write-back stores for residual_out, 0 streaming stores
    int rank_loop;          // rank sum, scalar: 1 add the ranks after x_0 one load round at a time
    int preload;            // row, scalar, rank sum with W <= 8: 1 launch the kernels whose leading
                            // arguments the dispatcher preloads into scalar registers
    long long count;        // rank sum only: elements from the aligned start (tokens * hidden - head)
};

// ------------------------------------------------- per-kernel argument blocks
// What each kernel receives, packed from Args by its launcher.  On MI355X with
// ROCm 7 the host cost of a launch steps from about 2.8 us to about 3.7 us when
// the explicit kernel arguments grow past 112 bytes, and reading blockDim or
// gridDim in a kernel adds the implicit-argument block (about 0.3 us more).  So
// the blocks below stay within 112 bytes for every W <= 8 (the generic and
// W = 16 kernels carry 16 pointers and are larger), and the kernels take their
// sizes from these fields, never from blockDim or gridDim.  Small sizes share
// one packed word.

// The partial pointers: W of them for kernels specialised on W, 16 otherwise.
template <int WA>
struct Ptrs {
    const void* p[WA];
};

// Row variant.  shape: bits 0-15 nvec (H / 8), 16-22 threads_per_row / 16,
// 23-25 log2(rows_per_block), 26-30 W.
template <int WA>
struct RowArgs {
    Ptrs<WA> x;
    const void* residual;
    const void* weight;
    void* residual_out;
    void* norm_out;
    float eps;
    int tokens;
    int xcd_chunk;
    uint32_t shape;
};

// Split-H phase 1.  vec: bits 0-15 nvec, 16-31 chunk_vec; shape: bits 0-15
// chunks per row, 16-20 W.  The workgroup has chunk_vec / VPT lanes.
template <int WA>
struct SplitPartialArgs {
    Ptrs<WA> x;
    const void* residual;
    void* residual_out;
    double* ws;
    int blocks;
    int xcd_chunk;
    uint32_t vec;
    uint32_t shape;
};

// Split-H phase 2.  vec as in phase 1; shape: bits 0-15 chunks per row,
// 16-31 lanes per workgroup.
struct SplitNormArgs {
    const void* residual_out;
    const void* weight;
    void* norm_out;
    const double* ws;
    float eps;
    int blocks;
    int xcd_chunk;
    uint32_t vec;
    uint32_t shape;
};

// Scalar variant (narrow loads, one row per workgroup).  shape: bits 0-16 H,
// 17-21 lanes per workgroup / 64, 22-26 W, 27-28 log2(elements per load).
template <int WA>
struct ScalarArgs {
    Ptrs<WA> x;
    const void* residual;
    const void* weight;
    void* residual_out;
    void* norm_out;
    float eps;
    int tokens;
    int xcd_chunk;
    uint32_t shape;
};

// Rank sum alone (256 lanes per workgroup).  x and reduced point at the first
// aligned element; `head` elements before it and the count % E after the last
// whole group are done element-wise by the last workgroup.
template <int WA>
struct ReduceArgs {
    Ptrs<WA> x;
    void* reduced;
    long long count;
    int blocks;
    int xcd_chunk;
    int world;
    int head;
};

// The first WA partial pointers of a call (the rest of Ptrs<16> stays null).
template <int WA>
inline Ptrs<WA> pack_ptrs(const Args& a) {
    Ptrs<WA> x = {};
    for (int r = 0; r < a.world && r < WA; ++r) x.p[r] = a.x.p[r];
    return x;
}

// Launch `fn` with one argument block passed by value.
template <typename K>
inline hipError_t launch_with(const void* fn, const K& args, int grid, int block, hipStream_t s) {
    void* p[] = {const_cast<K*>(&args)};
    return hipLaunchKernel(fn, dim3(grid), dim3(block), p, 0, s);
}

// ------------------------------------------------- preloaded argument lists
// gfx950 can preload the first 14 dwords of a kernel's arguments into scalar
// registers when it launches a wave, but only arguments passed as scalars (not an
// aggregate passed by value).  A wave of the kernels above first waits for its
// argument block to arrive from memory; the twins below take their arguments as a
// flat list whose leading 14 dwords are what a wave needs first (sizes, the
// residual and the first four partial pointers), so their waves start without
// that round trip.  Each twin receives the same values as its by-value original
// and rebuilds the same argument block, so the two compute the same bits.  The
// flat list costs the host more per launch, so the planner takes the twins only
// for calls long enough to hide that (arrms_plan_t::kernarg_preload).
//
// Host copy of the flat list of the row and scalar twins, in parameter order:
// 4 + 2 + 8 * 2 + 3 * 2 = 28 dwords, 112 bytes; partials past W are null.
struct FlatFusedArgs {
    int tokens;
    int xcd_chunk;
    uint32_t shape;
    float eps;
    const void* residual;
    const void* x[8];
    const void* weight;
    void* residual_out;
    void* norm_out;
};

// Host copy of the flat list of the rank-sum twins: 4 + 2 + 8 * 2 + 2 = 24
// dwords, 96 bytes; the output pointer last, so that the first four partials are
// among the preloaded dwords.
struct FlatReduceArgs {
    int blocks;
    int xcd_chunk;
    int world;
    int head;
    long long count;
    const void* x[8];
    void* reduced;
};

// Launch `fn` with the fields of a flat argument list, one kernel parameter each.
inline hipError_t launch_flat(const void* fn, FlatFusedArgs& f, int grid, int block, hipStream_t s) {
    void* p[] = {&f.tokens, &f.xcd_chunk, &f.shape, &f.eps, &f.residual, &f.x[0], &f.x[1], &f.x[2],
                 &f.x[3], &f.x[4], &f.x[5], &f.x[6], &f.x[7], &f.weight, &f.residual_out, &f.norm_out};
    return hipLaunchKernel(fn, dim3(grid), dim3(block), p, 0, s);
}

inline hipError_t launch_flat(const void* fn, FlatReduceArgs& f, int grid, int block, hipStream_t s) {
    void* p[] = {&f.blocks, &f.xcd_chunk, &f.world, &f.head, &f.count, &f.x[0], &f.x[1], &f.x[2],
                 &f.x[3], &f.x[4], &f.x[5], &f.x[6], &f.x[7], &f.reduced};
    return hipLaunchKernel(fn, dim3(grid), dim3(block), p, 0, s);
}

// Each launcher returns the hipError_t of the launch itself.
hipError_t launch_row(const Args& a, int vec_per_thread, int grid, int block, hipStream_t s);
// Split-H launches two kernels on `s`: the partial pass, then the norm pass.
hipError_t launch_splith(const Args& a, int vec_per_thread, int grid, int block, hipStream_t s);
hipError_t launch_scalar(const Args& a, int grid, int block, hipStream_t s);
// Rank sum only (reduced = BF16 sum of the partials), flat over a.head + a.count
// elements, with loads of a.elems_per_load elements.  16-byte loads (8 elements)
// take 1, 2 or 4 vectors per lane per partial for W <= 8, only 1 for the 16-wide
// rank arrays of larger W (register budget); narrower loads take 16 bytes per lane.
hipError_t launch_reduce(const Args& a, int vec_per_thread, int grid, int block, hipStream_t s);

// Load width of the rank sum, flat over memory: the widest E in {8, 4, 2, 1}, at
// most max_elems, such that every pointer (the W partials and the output) has the
// same offset modulo 2E bytes, and the number of elements before the first
// 2E-aligned one (at most `count`).  Pointers are 2-byte aligned, so E = 1 always
// qualifies.
inline void reduce_alignment(const void* const* partials, int world, const void* reduced, long long count,
                             int max_elems, int* elems, int* head) {
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(reduced);
    int e = max_elems >= 8 ? 8 : (max_elems >= 4 ? 4 : (max_elems >= 2 ? 2 : 1));
    for (; e > 1; e /= 2) {
        const uintptr_t m = static_cast<uintptr_t>(2 * e - 1);
        bool same = true;
        for (int r = 0; r < world; ++r)
            if (((reinterpret_cast<uintptr_t>(partials[r]) ^ p0) & m) != 0) same = false;
        if (same) break;
    }
    const uintptr_t m = static_cast<uintptr_t>(2 * e - 1);
    long long h = static_cast<long long>(((2 * e - (p0 & m)) & m) / 2);
    if (h > count) h = count;
    *elems = e;
    *head = static_cast<int>(h);
}

// Does a planned call's split-H workspace, tokens x chunks_per_row doubles, fit
// a workspace of `capacity` doubles?  Plans of the other variants use none.
inline bool splith_workspace_fits(const arrms_plan_t& p, int tokens, long long capacity) {
    return p.variant != ARRMS_VARIANT_SPLITH ||
           (p.chunks_per_row > 0 && static_cast<long long>(tokens) * p.chunks_per_row <= capacity);
}

// Launch a planned fused call (plan from arrms_plan) on `stream` of the current
// device; `ws` is the split-H workspace (at least tokens x chunks_per_row doubles
// for a split-H plan, unused otherwise).  Returns the hipError_t of the launch.
hipError_t launch_fused(const arrms_plan_t& p, const void* const* partials, int world, int tokens, int hidden,
                        const void* residual, const void* weight, float eps, void* residual_out, void* norm_out,
                        double* ws, hipStream_t stream);

}  // namespace arrms
