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

#include "arrms_internal.h"

namespace arrms {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- BF16 helpers
// A dword holds two BF16 values: element 2i in the low half, 2i+1 in the high
// half.  Widening is exact: the BF16 bits are the top half of a binary32.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 -> nearest BF16 value (ties to even), returned as a binary32 bit
// pattern whose low 16 bits are zero.  Adding 0x7fff plus the lowest kept bit
// carries into the kept half exactly when the dropped half exceeds one half,
// or equals one half with an odd kept half.  A NaN keeps its top half with
// the quiet bit set.
__device__ __forceinline__ uint32_t round_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
    const uint32_t quiet_nan = (u | 0x00400000u) & 0xffff0000u;
    return __builtin_isnan(f) ? quiet_nan : rounded;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo_rounded, uint32_t hi_rounded) {
    return (lo_rounded >> 16) | hi_rounded;
}

// 16-byte loads and stores.  The partials and the residual are read exactly
// once, so they are loaded with the non-temporal (streaming) hint; the weight,
// read by every row, is loaded normally so that it stays cached.  The outputs
// are written once and not read again by this kernel: streaming stores.
__device__ __forceinline__ u32x4 ld4(const void* base, size_t i) {
    return static_cast<const u32x4*>(base)[i];
}
__device__ __forceinline__ u32x4 ld4_stream(const void* base, size_t i) {
    return __builtin_nontemporal_load(static_cast<const u32x4*>(base) + i);
}
__device__ __forceinline__ void st4(void* base, size_t i, u32x4 v) { static_cast<u32x4*>(base)[i] = v; }
__device__ __forceinline__ void st4_stream(void* base, size_t i, u32x4 v) {
    __builtin_nontemporal_store(v, static_cast<u32x4*>(base) + i);
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  With xcd_chunk = K > 0 the launched grid is a multiple of 8K and
// the i-th workgroup an XCD receives takes logical block (8 * (i / K) + x) * K
// + i % K (x = its XCD): runs of K consecutive blocks (rows) stay on one XCD,
// and at any moment the 8 XCDs work on neighbouring runs.  K = 0 keeps the
// hardware's round-robin order.  Returns -1 for padding blocks past a.blocks.
__device__ __forceinline__ int logical_block(const Args& a) {
    const int b = blockIdx.x;
    const int k = a.xcd_chunk;
    if (k == 0) return b;
    const int x = b & 7;
    const int i = b >> 3;
    const int j = i / k;
    const int l = (j * 8 + x) * k + (i - j * k);
    return l < a.blocks ? l : -1;
}

// ---------------------------------------------------------------- reductions
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                          static_cast<uint32_t>(lo));
}

// Lane i reads lane i ^ 16 within each half-wave: ds_swizzle bit-mask mode,
// and-mask 0x1f, or-mask 0, xor-mask 0x10.
__device__ __forceinline__ double swizzle_xor16_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_ds_swizzle(static_cast<int>(b), 0x401F);
    const int hi = __builtin_amdgcn_ds_swizzle(static_cast<int>(b >> 32), 0x401F);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                          static_cast<uint32_t>(lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), lane);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                          static_cast<uint32_t>(lo));
}

// Sum of v over aligned groups of `width` lanes (16, 32 or 64); every lane of a
// group receives the group's sum.  Butterfly order: lane ^ 1, ^ 2 (DPP quad
// permutes), the other quad of each 8 (row_half_mirror), the other 8 of each 16
// (row_mirror), the other 16 of each 32 (ds_swizzle), then the two half-waves
// (readlane).  After each step a group's lanes hold equal values, so the mirror
// permutes act as xor partners, and binary64 addition being commutative gives
// every lane bit-identical sums.  The order is fixed, so results are
// deterministic; they can differ from a sequential sum in the last binary64
// bit, which changes the binary32 1/RMS only when the exact value lies within
// about 2^-29 relative of a binary32 rounding boundary.  Needs all 64 lanes
// active.
__device__ __forceinline__ double seg_sum(double v, int width) {
    v = v + dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v = v + dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v = v + dpp_f64<0x141>(v);  // row_half_mirror
    v = v + dpp_f64<0x140>(v);  // row_mirror
    if (width >= 32) v = v + swizzle_xor16_f64(v);
    if (width >= 64) v = readlane_f64(v, 0) + readlane_f64(v, 32);
    return v;
}

// 1 / RMS of a row from its binary64 sum of squares.
__device__ __forceinline__ float inv_rms(double sum_sq, double hidden, float eps) {
    return static_cast<float>(1.0 / sqrt(sum_sq / hidden + static_cast<double>(eps)));
}

// ------------------------------------------------------- per-vector arithmetic
// Rank sum, reduced rounding and residual add for one 16-byte vector (8
// elements) of a row; accumulates the squares into ss and returns residual_out.
// binary32 rank sum, in rank order from x_0, of the two elements in dword j.
template <int W>
__device__ __forceinline__ void rank_sum(const u32x4 (&xv)[W > 0 ? W : kMaxWorld], int world, int j, float& a_lo,
                                         float& a_hi) {
    constexpr int WA = W > 0 ? W : kMaxWorld;
    a_lo = lo_f32(xv[0][j]);
    a_hi = hi_f32(xv[0][j]);
#pragma unroll
    for (int r = 1; r < WA; ++r) {
        if (W > 0 || r < world) {
            a_lo = a_lo + lo_f32(xv[r][j]);
            a_hi = a_hi + hi_f32(xv[r][j]);
        }
    }
}

// `reduced` for one vector: the rank sum rounded to BF16.
template <int W>
__device__ __forceinline__ u32x4 reduced_vec(const u32x4 (&xv)[W > 0 ? W : kMaxWorld], int world) {
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float a_lo, a_hi;
        rank_sum<W>(xv, world, j, a_lo, a_hi);
        out[j] = pack2(round_bf16(a_lo), round_bf16(a_hi));
    }
    return out;
}

template <int W>
__device__ __forceinline__ u32x4 residual_vec(const u32x4 (&xv)[W > 0 ? W : kMaxWorld], int world,
                                              u32x4 rv, double& ss) {
    u32x4 ro;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float a_lo, a_hi;
        rank_sum<W>(xv, world, j, a_lo, a_hi);
        const uint32_t o_lo = round_bf16(__uint_as_float(round_bf16(a_lo)) + lo_f32(rv[j]));
        const uint32_t o_hi = round_bf16(__uint_as_float(round_bf16(a_hi)) + hi_f32(rv[j]));
        const double d_lo = static_cast<double>(__uint_as_float(o_lo));
        const double d_hi = static_cast<double>(__uint_as_float(o_hi));
        ss = ss + d_lo * d_lo;  // exact square of a BF16 value in binary64
        ss = ss + d_hi * d_hi;
        ro[j] = pack2(o_lo, o_hi);
    }
    return ro;
}

// norm_out for one vector from residual_out, 1/RMS and the weight.
__device__ __forceinline__ u32x4 norm_vec(u32x4 ro, float inv, u32x4 wv) {
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float n_lo = (lo_f32(ro[j]) * inv) * lo_f32(wv[j]);
        const float n_hi = (hi_f32(ro[j]) * inv) * hi_f32(wv[j]);
        out[j] = pack2(round_bf16(n_lo), round_bf16(n_hi));
    }
    return out;
}

// ---------------------------------------------------------------- row variant
// threads_per_row lanes own one token row (16 or 32 lanes: several rows per
// wave; a multiple of 64: one or more whole waves per row), rows_per_block rows
// per workgroup.  Lane l handles vectors l, l + tpr, ..., l + (VPT-1)*tpr of the
// row, so at each step a wave reads 1 KiB of contiguous memory per input.  All
// (W + 2) * VPT loads of a lane are issued before any arithmetic; residual_out
// stays in registers for the second pass.
// Largest workgroup of a row kernel; the host planner uses the same table.
template <int W, int VPT>
constexpr int row_max_threads() {
    return (W == 0 || W > 8) ? (VPT == 1 ? 512 : 256) : (VPT == 1 ? 1024 : (VPT <= 4 ? 512 : 256));
}

template <int W, int VPT>
__global__ void __launch_bounds__((row_max_threads<W, VPT>())) row_kernel(const Args a) {
    constexpr int WA = W > 0 ? W : kMaxWorld;
    const int world = W > 0 ? W : a.world;
    const int tpr = a.threads_per_row;
    const int block = logical_block(a);
    if (block < 0) return;  // padding workgroup of the XCD mapping (whole workgroup)
    const int tid = threadIdx.x;
    const int row_in_block = tid / tpr;
    const int lane = tid - row_in_block * tpr;
    const int row = block * a.rows_per_block + row_in_block;
    const bool row_ok = row < a.tokens;
    const size_t base = static_cast<size_t>(row_ok ? row : 0) * static_cast<size_t>(a.nvec);

    bool ok[VPT];
    u32x4 xv[VPT][WA];
    u32x4 rv[VPT];
    u32x4 wv[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lane + k * tpr;
        ok[k] = row_ok && v < a.nvec;
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
            st4_stream(a.residual_out, base + lane + k * tpr, ro[k]);
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
    const float inv = inv_rms(ss, a.hidden_d, a.eps);

#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (ok[k]) st4_stream(a.norm_out, base + lane + k * tpr, norm_vec(ro[k], inv, wv[k]));
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
__global__ void __launch_bounds__(splith_max_threads<W>()) splith_partial_kernel(const Args a) {
    constexpr int WA = W > 0 ? W : kMaxWorld;
    const int world = W > 0 ? W : a.world;
    const int block = logical_block(a);
    if (block < 0) return;
    const int row = block / a.chunks;
    const int chunk = block - row * a.chunks;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int v0 = chunk * a.chunk_vec;
    const int v1 = min(a.nvec, v0 + a.chunk_vec);
    const size_t base = static_cast<size_t>(row) * static_cast<size_t>(a.nvec);

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
        a.ws[static_cast<size_t>(row) * a.chunks + chunk] = t;
    }
}

__global__ void __launch_bounds__(1024) splith_norm_kernel(const Args a) {
    const int block = logical_block(a);
    if (block < 0) return;
    const int row = block / a.chunks;
    const int chunk = block - row * a.chunks;
    const int tid = threadIdx.x;
    const int v0 = chunk * a.chunk_vec;
    const int v1 = min(a.nvec, v0 + a.chunk_vec);
    const size_t base = static_cast<size_t>(row) * static_cast<size_t>(a.nvec);
    const double* part = a.ws + static_cast<size_t>(row) * a.chunks;
    double total = part[0];
    for (int c = 1; c < a.chunks; ++c) total = total + part[c];
    const float inv = inv_rms(total, a.hidden_d, a.eps);
    for (int v = v0 + tid; v < v1; v += blockDim.x)
        st4_stream(a.norm_out, base + v, norm_vec(ld4(a.residual_out, base + v), inv, ld4(a.weight, v)));
}

// -------------------------------------------------------------- scalar variant
// Any H and any 2-byte alignment: one row per workgroup, one BF16 element per
// lane per step.  residual_out is written in the first pass and re-read in the
// second by the same lane (same addresses, program order), so H is unbounded.
__global__ void __launch_bounds__(256) scalar_kernel(const Args a) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int H = a.hidden;
    const size_t base = static_cast<size_t>(row) * static_cast<size_t>(H);
    const uint16_t* res = static_cast<const uint16_t*>(a.residual);
    const uint16_t* w = static_cast<const uint16_t*>(a.weight);
    uint16_t* ro_out = static_cast<uint16_t*>(a.residual_out);
    uint16_t* n_out = static_cast<uint16_t*>(a.norm_out);

    double ss = 0.0;
    for (int h = tid; h < H; h += nthreads) {
        float acc = lo_f32(static_cast<const uint16_t*>(a.x.p[0])[base + h]);
        for (int r = 1; r < a.world; ++r) acc = acc + lo_f32(static_cast<const uint16_t*>(a.x.p[r])[base + h]);
        const uint32_t o = round_bf16(__uint_as_float(round_bf16(acc)) + lo_f32(res[base + h]));
        ro_out[base + h] = static_cast<uint16_t>(o >> 16);
        const double d = static_cast<double>(__uint_as_float(o));
        ss = ss + d * d;
    }
    __shared__ double wave_ss[4];
    ss = seg_sum(ss, 64);
    if ((tid & 63) == 0) wave_ss[tid >> 6] = ss;
    __syncthreads();
    double total = wave_ss[0];
    for (int i = 1; i < (nthreads >> 6); ++i) total = total + wave_ss[i];
    const float inv = inv_rms(total, a.hidden_d, a.eps);
    for (int h = tid; h < H; h += nthreads) {
        const float n = (lo_f32(ro_out[base + h]) * inv) * lo_f32(w[h]);
        n_out[base + h] = static_cast<uint16_t>(round_bf16(n) >> 16);
    }
}

// ------------------------------------------------------------ rank sum only
// The contract's first line on its own (the page's collective stage, locally):
// reduced = BF16(sum of the W partials), flat over a.count = T*H elements.
// Each lane sums VPT 16-byte vectors (at stride blockDim) of every partial;
// the last count % 8 elements go element-wise in the last block.
template <int W, int kReduceVpt>
__global__ void __launch_bounds__(256) reduce_kernel(const Args a) {
    constexpr int WA = W > 0 ? W : kMaxWorld;
    const int world = W > 0 ? W : a.world;
    const int block = logical_block(a);
    if (block < 0) return;
    const size_t nvec = static_cast<size_t>(a.count) / 8;
    const size_t first = static_cast<size_t>(block) * blockDim.x * kReduceVpt + threadIdx.x;
    bool ok[kReduceVpt];
    u32x4 xv[kReduceVpt][WA];
#pragma unroll
    for (int k = 0; k < kReduceVpt; ++k) {
        const size_t v = first + static_cast<size_t>(k) * blockDim.x;
        ok[k] = v < nvec;
        if (ok[k]) {
#pragma unroll
            for (int r = 0; r < WA; ++r)
                if (W > 0 || r < world) xv[k][r] = ld4_stream(a.x.p[r], v);
        }
    }
#pragma unroll
    for (int k = 0; k < kReduceVpt; ++k)
        if (ok[k]) st4_stream(a.reduced, first + static_cast<size_t>(k) * blockDim.x, reduced_vec<W>(xv[k], world));
    if (block == a.blocks - 1) {  // the count % 8 elements past the last whole vector
        for (size_t e = nvec * 8 + threadIdx.x; e < static_cast<size_t>(a.count); e += blockDim.x) {
            float acc = lo_f32(static_cast<const uint16_t*>(a.x.p[0])[e]);
            for (int r = 1; r < world; ++r) acc = acc + lo_f32(static_cast<const uint16_t*>(a.x.p[r])[e]);
            static_cast<uint16_t*>(a.reduced)[e] = static_cast<uint16_t>(round_bf16(acc) >> 16);
        }
    }
}

// Rank sum only, element-wise, for pointers that are not 16-byte aligned.
__global__ void __launch_bounds__(256) reduce_scalar_kernel(const Args a) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < static_cast<size_t>(a.count);
         e += stride) {
        float acc = lo_f32(static_cast<const uint16_t*>(a.x.p[0])[e]);
        for (int r = 1; r < a.world; ++r) acc = acc + lo_f32(static_cast<const uint16_t*>(a.x.p[r])[e]);
        static_cast<uint16_t*>(a.reduced)[e] = static_cast<uint16_t>(round_bf16(acc) >> 16);
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch(const void* fn, const Args& a, int grid, int block, hipStream_t s) {
    void* args[] = {const_cast<Args*>(&a)};
    return hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0, s);
}

// Instantiated (W, VPT) pairs: those whose (W + 2) * VPT live vectors fit the
// register budget the host planner allows (40); others are never planned.
template <int VPT>
const void* row_fn(int world) {
    if (VPT == 8 && world > 3) return nullptr;
    switch (world) {
        case 1: return reinterpret_cast<const void*>(&row_kernel<1, VPT>);
        case 2: return reinterpret_cast<const void*>(&row_kernel<2, VPT>);
        case 3: return reinterpret_cast<const void*>(&row_kernel<3, VPT>);
        default: break;
    }
    if constexpr (VPT <= 4) {
        switch (world) {
            case 4: return reinterpret_cast<const void*>(&row_kernel<4, VPT>);
            case 5: return reinterpret_cast<const void*>(&row_kernel<5, VPT>);
            case 6: return reinterpret_cast<const void*>(&row_kernel<6, VPT>);
            case 7: return reinterpret_cast<const void*>(&row_kernel<7, VPT>);
            case 8: return reinterpret_cast<const void*>(&row_kernel<8, VPT>);
            default: break;
        }
    }
    if constexpr (VPT <= 2) {
        if (world == 16) return reinterpret_cast<const void*>(&row_kernel<16, VPT>);
        return reinterpret_cast<const void*>(&row_kernel<0, VPT>);
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

}  // namespace

hipError_t launch_reduce(const Args& a, int vpt, int grid, int block, hipStream_t s) {
    const void* fn = nullptr;
    switch (vpt) {
        case 1: fn = reduce_fn<1>(a.world); break;
        case 2: fn = reduce_fn<2>(a.world); break;
        case 4: fn = reduce_fn<4>(a.world); break;
        default: return hipErrorInvalidValue;
    }
    if (!fn) return hipErrorInvalidValue;
    return launch(fn, a, grid, block, s);
}

hipError_t launch_reduce_scalar(const Args& a, int grid, int block, hipStream_t s) {
    return launch(reinterpret_cast<const void*>(&reduce_scalar_kernel), a, grid, block, s);
}

hipError_t launch_row(const Args& a, int vpt, int grid, int block, hipStream_t s) {
    const void* fn = nullptr;
    switch (vpt) {
        case 1: fn = row_fn<1>(a.world); break;
        case 2: fn = row_fn<2>(a.world); break;
        case 4: fn = row_fn<4>(a.world); break;
        case 8: fn = row_fn<8>(a.world); break;
        default: return hipErrorInvalidValue;
    }
    if (!fn) return hipErrorInvalidValue;
    return launch(fn, a, grid, block, s);
}

hipError_t launch_splith(const Args& a, int vpt, int grid, int block, hipStream_t s) {
    const void* fn = nullptr;
    switch (vpt) {
        case 1: fn = splith_fn<1>(a.world); break;
        case 2: fn = splith_fn<2>(a.world); break;
        default: return hipErrorInvalidValue;
    }
    if (!fn) return hipErrorInvalidValue;
    const hipError_t e = launch(fn, a, grid, block, s);
    if (e != hipSuccess) return e;
    return launch(reinterpret_cast<const void*>(&splith_norm_kernel), a, grid, block, s);
}

hipError_t launch_scalar(const Args& a, int grid, int block, hipStream_t s) {
    return launch(reinterpret_cast<const void*>(&scalar_kernel), a, grid, block, s);
}

}  // namespace arrms
