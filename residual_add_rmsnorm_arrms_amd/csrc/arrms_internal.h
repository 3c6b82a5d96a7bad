// Internal interface between the C-ABI host code (arrms_api.cpp) and the gfx950
// kernels (arrms_kernels.hip).  Not installed; the public interface is include/arrms.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace arrms {

constexpr int kMaxWorld = 16;

// The W rank-partial base pointers travel by value inside the kernel arguments,
// so a call needs no host-to-device copy of the pointer array.
struct Partials {
    const void* p[kMaxWorld];
};

// Kernel arguments, shared by every variant (passed by value).
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
    long long count;        // rank sum only: elements (tokens * hidden)
};

// Each launcher returns the hipError_t of the launch itself.
hipError_t launch_row(const Args& a, int vec_per_thread, int grid, int block, hipStream_t s);
// Split-H launches two kernels on `s`: the partial pass, then the norm pass.
hipError_t launch_splith(const Args& a, int vec_per_thread, int grid, int block, hipStream_t s);
hipError_t launch_scalar(const Args& a, int grid, int block, hipStream_t s);
// Rank sum only (reduced = BF16 sum of the partials), flat over a.count elements.
// reduce_kernel instances: 16-byte vectors per lane per partial of 1, 2 or 4
// for W <= 8, only 1 for the 16-wide rank arrays of larger W (register budget).
hipError_t launch_reduce(const Args& a, int vec_per_thread, int grid, int block, hipStream_t s);
hipError_t launch_reduce_scalar(const Args& a, int grid, int block, hipStream_t s);

}  // namespace arrms
