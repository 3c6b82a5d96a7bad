// gfx950 kernels of the rank sum alone: reduced = BF16(sum over the W rank
// partials), the first line of the contract of the page "[TLERaw] Add NVSHMEM
// allreduce RMSNorm tutorial" (FlagTree PR #1122, section Summary), i.e. the
// page's collective stage (section Implementation 1) on one GPU's share.  Same
// arithmetic as the fused kernels: binary32 sum in rank order from x_0, one
// rounding to BF16.  Bound by HBM bandwidth: 2 * (W + 1) bytes per element.
#include <hip/hip_runtime.h>

#include "arrms_device.h"

namespace arrms {
namespace {

using namespace dev;

// Workgroup size of both rank-sum kernels (the host plans 256 lanes).
constexpr int kReduceLanes = 256;

// ------------------------------------------------------------ rank sum only
// The contract's first line on its own (the page's collective stage, locally):
// reduced = BF16(sum of the W partials), flat over a.count = T*H elements.
// Each lane sums VPT 16-byte vectors (at stride 256) of every partial;
// the last count % 8 elements go element-wise in the last block.
template <int W, int kReduceVpt>
__global__ void __launch_bounds__(kReduceLanes) reduce_kernel(const ReduceArgs<(W > 0 ? W : kMaxWorld)> a) {
    constexpr int WA = W > 0 ? W : kMaxWorld;
    const int world = W > 0 ? W : a.world;
    const int block = logical_block(a.xcd_chunk, a.blocks);
    if (block < 0) return;
    const size_t nvec = static_cast<size_t>(a.count) / 8;
    const size_t first = static_cast<size_t>(block) * kReduceLanes * kReduceVpt + threadIdx.x;
    bool ok[kReduceVpt];
    u32x4 xv[kReduceVpt][WA];
#pragma unroll
    for (int k = 0; k < kReduceVpt; ++k) {
        const size_t v = first + static_cast<size_t>(k) * kReduceLanes;
        ok[k] = v < nvec;
        if (ok[k]) {
#pragma unroll
            for (int r = 0; r < WA; ++r)
                if (W > 0 || r < world) xv[k][r] = ld4_stream(a.x.p[r], v);
        }
    }
#pragma unroll
    for (int k = 0; k < kReduceVpt; ++k)
        if (ok[k]) st4_stream(a.reduced, first + static_cast<size_t>(k) * kReduceLanes, reduced_vec<W>(xv[k], world));
    if (block == a.blocks - 1) {  // the count % 8 elements past the last whole vector
        for (size_t e = nvec * 8 + threadIdx.x; e < static_cast<size_t>(a.count); e += kReduceLanes) {
            float acc = lo_f32(static_cast<const uint16_t*>(a.x.p[0])[e]);
            for (int r = 1; r < world; ++r) acc = acc + lo_f32(static_cast<const uint16_t*>(a.x.p[r])[e]);
            static_cast<uint16_t*>(a.reduced)[e] = cvt1(acc);
        }
    }
}

// Rank sum only, element-wise, for pointers that are not 16-byte aligned.
__global__ void __launch_bounds__(kReduceLanes) reduce_scalar_kernel(const ReduceArgs<kMaxWorld> a) {
    const size_t stride = static_cast<size_t>(a.grid) * kReduceLanes;
    for (size_t e = static_cast<size_t>(blockIdx.x) * kReduceLanes + threadIdx.x; e < static_cast<size_t>(a.count);
         e += stride) {
        float acc = lo_f32(static_cast<const uint16_t*>(a.x.p[0])[e]);
        for (int r = 1; r < a.world; ++r) acc = acc + lo_f32(static_cast<const uint16_t*>(a.x.p[r])[e]);
        static_cast<uint16_t*>(a.reduced)[e] = cvt1(acc);
    }
}

template <int VPT>
const void* reduce_fn(int world) {
    switch (world) {
        case 1: return reinterpret_cast<const void*>(&reduce_kernel<1, VPT>);
        case 2: return reinterpret_cast<const void*>(&reduce_kernel<2, VPT>);
        case 3: return reinterpret_cast<const void*>(&reduce_kernel<3, VPT>);
        case 4: return reinterpret_cast<const void*>(&reduce_kernel<4, VPT>);
        case 5: return reinterpret_cast<const void*>(&reduce_kernel<5, VPT>);
        case 6: return reinterpret_cast<const void*>(&reduce_kernel<6, VPT>);
        case 7: return reinterpret_cast<const void*>(&reduce_kernel<7, VPT>);
        case 8: return reinterpret_cast<const void*>(&reduce_kernel<8, VPT>);
        default: break;
    }
    if constexpr (VPT == 1) return reinterpret_cast<const void*>(&reduce_kernel<0, 1>);
    return nullptr;
}

template <int WA>
hipError_t launch_reduce_with(const void* fn, const Args& a, int grid, hipStream_t s) {
    ReduceArgs<WA> r{};
    r.x = pack_ptrs<WA>(a);
    r.reduced = a.reduced;
    r.count = a.count;
    r.blocks = a.blocks;
    r.xcd_chunk = a.xcd_chunk;
    r.world = a.world;
    r.grid = grid;
    return launch_with(fn, r, grid, kReduceLanes, s);
}

}  // namespace

hipError_t launch_reduce(const Args& a, int vpt, int grid, int block, hipStream_t s) {
    const void* fn = nullptr;
    switch (vpt) {
        case 1: fn = reduce_fn<1>(a.world); break;
        case 2: fn = reduce_fn<2>(a.world); break;
        case 4: fn = reduce_fn<4>(a.world); break;
        default: return hipErrorInvalidValue;
    }
    if (!fn || block != kReduceLanes) return hipErrorInvalidValue;
    // reduce_kernel<W, VPT> takes ReduceArgs<W> for W <= 8 and ReduceArgs<16> otherwise
    switch (a.world) {
        case 1: return launch_reduce_with<1>(fn, a, grid, s);
        case 2: return launch_reduce_with<2>(fn, a, grid, s);
        case 3: return launch_reduce_with<3>(fn, a, grid, s);
        case 4: return launch_reduce_with<4>(fn, a, grid, s);
        case 5: return launch_reduce_with<5>(fn, a, grid, s);
        case 6: return launch_reduce_with<6>(fn, a, grid, s);
        case 7: return launch_reduce_with<7>(fn, a, grid, s);
        case 8: return launch_reduce_with<8>(fn, a, grid, s);
        default: return launch_reduce_with<kMaxWorld>(fn, a, grid, s);
    }
}

hipError_t launch_reduce_scalar(const Args& a, int grid, int block, hipStream_t s) {
    if (block != kReduceLanes) return hipErrorInvalidValue;
    return launch_reduce_with<kMaxWorld>(reinterpret_cast<const void*>(&reduce_scalar_kernel), a, grid, s);
}

}  // namespace arrms
