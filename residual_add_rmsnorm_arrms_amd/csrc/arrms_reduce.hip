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

// Workgroup size of the rank-sum kernel (the host plans 256 lanes).
constexpr int kReduceLanes = 256;

// ------------------------------------------------------------ rank sum only
// The contract's first line on its own (the page's collective stage, locally):
// reduced = BF16(sum of the W partials), flat over the T*H elements, so only the
// pointers' alignment decides the load width.  The host picks the widest width E
// (8, 4, 2 or 1 elements: 16-, 8-, 4- or 2-byte loads) at which every pointer has
// the same offset, and passes the pointers advanced to their first E-aligned
// element.  Each lane sums L groups of E elements (at stride 256) of every
// partial, all loads issued first; the last workgroup adds the `head` elements
// before the aligned start and the count % E after the last whole group, element
// by element.
// Each workgroup reaches its groups through buffer resources that span exactly
// its own whole groups of each tensor: the hardware's range check returns zeros
// for a load past them and drops such a store, so no group index is clamped or
// branched on, and one 32-bit offset per group serves every tensor.
template <int W, int L, int E>
__device__ __forceinline__ void reduce_body(const ReduceArgs<(W > 0 ? W : kMaxWorld)>& a) {
    typedef typename Group<E>::T G;
    typedef Buf<E> B;
    constexpr int WA = W > 0 ? W : kMaxWorld;
    const int world = W > 0 ? W : a.world;
    const int block = logical_block(a.xcd_chunk, a.blocks);
    if (block < 0) return;
    const long long ng = a.count / E;  // whole groups from the aligned start
    const long long g0 = static_cast<long long>(block) * kReduceLanes * L;
    if (g0 < ng) {  // (a call of fewer elements than one group has only its head and tail)
        const long long span = ng - g0 < kReduceLanes * L ? ng - g0 : kReduceLanes * L;
        const int bytes = static_cast<int>(span) * static_cast<int>(sizeof(G));
        const size_t first = static_cast<size_t>(g0) * E;  // the workgroup's first element
        G xv[L][WA];
        // rank by rank, so that each rank's resource lives only while its loads issue
#pragma unroll
        for (int r = 0; r < WA; ++r) {
            if (W > 0 || r < world) {
                const Rsrc rx = make_rsrc(static_cast<const uint16_t*>(a.x.p[r]) + first, bytes);
#pragma unroll
                for (int k = 0; k < L; ++k)
                    xv[k][r] = B::template ld<kBufNT>(
                        rx, (k * kReduceLanes + static_cast<int>(threadIdx.x)) * static_cast<int>(sizeof(G)));
            }
        }
        const Rsrc rout = make_rsrc(static_cast<uint16_t*>(a.reduced) + first, bytes);
#pragma unroll
        for (int k = 0; k < L; ++k) {
            const int off = (k * kReduceLanes + static_cast<int>(threadIdx.x)) * static_cast<int>(sizeof(G));
            float sum[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float acc = Group<E>::get(xv[k][0], e);
#pragma unroll
                for (int r = 1; r < WA; ++r)
                    if (W > 0 || r < world) acc = acc + Group<E>::get(xv[k][r], e);
                sum[e] = acc;
            }
            B::template st<kBufNT>(pack<E>(sum), rout, off);
        }
    }
    if (block == a.blocks - 1) {  // the head and the tail, element-wise
        const long long tail0 = ng * E;
        const int extra = a.head + static_cast<int>(a.count - tail0);
        for (int j = threadIdx.x; j < extra; j += kReduceLanes) {
            const long long e = j < a.head ? static_cast<long long>(j - a.head) : tail0 + (j - a.head);
            float acc = lo_f32(static_cast<const uint16_t*>(a.x.p[0])[e]);
            for (int r = 1; r < world; ++r) acc = acc + lo_f32(static_cast<const uint16_t*>(a.x.p[r])[e]);
            static_cast<uint16_t*>(a.reduced)[e] = cvt1(acc);
        }
    }
}

template <int W, int L, int E>
__global__ void __launch_bounds__(kReduceLanes) reduce_kernel(const ReduceArgs<(W > 0 ? W : kMaxWorld)> a) {
    reduce_body<W, L, E>(a);
}

// The same kernel for W <= 8 with a flat argument list (FlatReduceArgs on the host),
// whose leading dwords are preloaded into scalar registers.
template <int W, int L, int E>
__global__ void __launch_bounds__(kReduceLanes) reduce_kernel_flat(
    int blocks, int xcd_chunk, int world, int head, long long count, const void* x0, const void* x1, const void* x2,
    const void* x3, const void* x4, const void* x5, const void* x6, const void* x7, void* reduced) {
    static_assert(W >= 1 && W <= 8, "flat argument lists carry at most 8 partials");
    const void* const x[8] = {x0, x1, x2, x3, x4, x5, x6, x7};
    ReduceArgs<W> a;
#pragma unroll
    for (int r = 0; r < W; ++r) a.x.p[r] = x[r];
    a.reduced = reduced;
    a.count = count;
    a.blocks = blocks;
    a.xcd_chunk = xcd_chunk;
    a.world = world;
    a.head = head;
    reduce_body<W, L, E>(a);
}

// The same sum for six ranks or more with the ranks added one load round at a time:
// x_0's groups, then each further rank's groups added in rank order (the arithmetic is
// unchanged).  Only L groups of one rank are in registers at a time, so a CU runs many
// workgroups, which pays once each CU has enough of them to cover the round trips.
template <int L, int E>
__global__ void __launch_bounds__(kReduceLanes) reduce_loop_kernel(const ReduceArgs<kMaxWorld> a) {
    typedef typename Group<E>::T G;
    typedef Buf<E> B;
    const int block = logical_block(a.xcd_chunk, a.blocks);
    if (block < 0) return;
    const long long ng = a.count / E;
    const long long g0 = static_cast<long long>(block) * kReduceLanes * L;
    if (g0 < ng) {
        const long long span = ng - g0 < kReduceLanes * L ? ng - g0 : kReduceLanes * L;
        const int bytes = static_cast<int>(span) * static_cast<int>(sizeof(G));
        const size_t first = static_cast<size_t>(g0) * E;
        int off[L];
#pragma unroll
        for (int k = 0; k < L; ++k) off[k] = (k * kReduceLanes + static_cast<int>(threadIdx.x)) * static_cast<int>(sizeof(G));
        float acc[L][E];
        {
            const Rsrc r0 = make_rsrc(static_cast<const uint16_t*>(a.x.p[0]) + first, bytes);
            G v[L];
#pragma unroll
            for (int k = 0; k < L; ++k) v[k] = B::template ld<kBufNT>(r0, off[k]);
#pragma unroll
            for (int k = 0; k < L; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[k][e] = Group<E>::get(v[k], e);
        }
        for (int r = 1; r < a.world; ++r) {
            const Rsrc rr = make_rsrc(static_cast<const uint16_t*>(a.x.p[r]) + first, bytes);
            G v[L];
#pragma unroll
            for (int k = 0; k < L; ++k) v[k] = B::template ld<kBufNT>(rr, off[k]);
#pragma unroll
            for (int k = 0; k < L; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[k][e] = acc[k][e] + Group<E>::get(v[k], e);
        }
        const Rsrc rout = make_rsrc(static_cast<uint16_t*>(a.reduced) + first, bytes);
#pragma unroll
        for (int k = 0; k < L; ++k) B::template st<kBufNT>(pack<E>(acc[k]), rout, off[k]);
    }
    if (block == a.blocks - 1) {  // the head and the tail, element-wise
        const long long tail0 = ng * E;
        const int extra = a.head + static_cast<int>(a.count - tail0);
        for (int j = threadIdx.x; j < extra; j += kReduceLanes) {
            const long long e = j < a.head ? static_cast<long long>(j - a.head) : tail0 + (j - a.head);
            float acc = lo_f32(static_cast<const uint16_t*>(a.x.p[0])[e]);
            for (int r = 1; r < a.world; ++r) acc = acc + lo_f32(static_cast<const uint16_t*>(a.x.p[r])[e]);
            static_cast<uint16_t*>(a.reduced)[e] = cvt1(acc);
        }
    }
}

template <int W, int L, int E>
const void* reduce_sym(bool flat) {
    return flat ? reinterpret_cast<const void*>(&reduce_kernel_flat<W, L, E>)
                : reinterpret_cast<const void*>(&reduce_kernel<W, L, E>);
}

// The by-value kernel, or its flat twin (W <= 8 only; nullptr for more ranks).
template <int L, int E>
const void* reduce_fn(int world, bool flat) {
    switch (world) {
        case 1: return reduce_sym<1, L, E>(flat);
        case 2: return reduce_sym<2, L, E>(flat);
        case 3: return reduce_sym<3, L, E>(flat);
        case 4: return reduce_sym<4, L, E>(flat);
        case 5: return reduce_sym<5, L, E>(flat);
        case 6: return reduce_sym<6, L, E>(flat);
        case 7: return reduce_sym<7, L, E>(flat);
        case 8: return reduce_sym<8, L, E>(flat);
        default: break;
    }
    // more than 8 ranks: one 16 bytes' worth of groups per lane (register budget)
    if constexpr (L * E == 8) {
        if (!flat) return reinterpret_cast<const void*>(&reduce_kernel<0, L, E>);
    }
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
    r.head = a.head;
    if (a.preload) {  // `fn` is the flat twin
        if (WA > 8) return hipErrorInvalidValue;
        FlatReduceArgs f{};
        f.blocks = r.blocks;
        f.xcd_chunk = r.xcd_chunk;
        f.world = r.world;
        f.head = r.head;
        f.count = r.count;
        for (int i = 0; i < WA && i < 8; ++i) f.x[i] = r.x.p[i];
        f.reduced = r.reduced;
        return launch_flat(fn, f, grid, kReduceLanes, s);
    }
    return launch_with(fn, r, grid, kReduceLanes, s);
}

}  // namespace

hipError_t launch_reduce(const Args& a, int vpt, int grid, int block, hipStream_t s) {
    const void* fn = nullptr;
    if (a.rank_loop) {
        if (a.preload) return hipErrorInvalidValue;  // the loop kernel serves any rank count: no flat twin
        switch (a.elems_per_load) {
            case 8: fn = reinterpret_cast<const void*>(&reduce_loop_kernel<1, 8>); break;
            case 4: fn = reinterpret_cast<const void*>(&reduce_loop_kernel<2, 4>); break;
            case 2: fn = reinterpret_cast<const void*>(&reduce_loop_kernel<4, 2>); break;
            case 1: fn = reinterpret_cast<const void*>(&reduce_loop_kernel<8, 1>); break;
            default: return hipErrorInvalidValue;
        }
        if (vpt > 1 || block != kReduceLanes || a.head < 0 || a.head >= a.elems_per_load) return hipErrorInvalidValue;
        return launch_reduce_with<kMaxWorld>(fn, a, grid, s);
    }
    const bool flat = a.preload != 0;
    switch (a.elems_per_load) {
        case 8:
            switch (vpt) {
                case 1: fn = reduce_fn<1, 8>(a.world, flat); break;
                case 2: fn = reduce_fn<2, 8>(a.world, flat); break;
                case 4: fn = reduce_fn<4, 8>(a.world, flat); break;
                default: return hipErrorInvalidValue;
            }
            break;
        case 4: fn = reduce_fn<2, 4>(a.world, flat); break;
        case 2: fn = reduce_fn<4, 2>(a.world, flat); break;
        case 1: fn = reduce_fn<8, 1>(a.world, flat); break;
        default: return hipErrorInvalidValue;
    }
    if (!fn || block != kReduceLanes || a.head < 0 || a.head >= a.elems_per_load) return hipErrorInvalidValue;
    // reduce_kernel<W, L, E> takes ReduceArgs<W> for W <= 8 and ReduceArgs<16> otherwise
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

}  // namespace arrms
