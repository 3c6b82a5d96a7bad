// Device helpers shared by the gfx950 kernels of the fused rank-partial sum +
// residual add + RMSNorm (arrms_kernels.hip) and of the rank sum alone
// (arrms_reduce.hip): BF16 conversion and rounding, streaming 16-byte memory
// access, the XCD block mapping, cross-lane binary64 reductions and the
// per-vector arithmetic of every step.  See arrms_kernels.hip for the
// operation and its rounding points.
#pragma once

#include <hip/hip_runtime.h>

#include "arrms_internal.h"

namespace arrms {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- BF16 helpers
// A dword holds two BF16 values: element 2i in the low half, 2i+1 in the high
// half.  Widening is exact: the BF16 bits are the top half of a binary32.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 -> BF16, round to nearest, ties to even: gfx950's packed
// conversion (v_cvt_pk_bf16_f32) under the default rounding mode, with binary32
// denormals preserved (the kernels are built without flush-to-zero).  A carry
// out of the largest finite values gives infinity; a NaN stays a NaN (its
// payload is the hardware's).  cvt2 packs two results into one dword, the
// first in the low half; cvt1 returns one BF16 bit pattern.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t cvt1(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

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

// ------------------------------------------------- groups of E BF16 elements
// The unit one load moves: E consecutive BF16 elements (E = 1, 2, 4 or 8: a 2-,
// 4-, 8- or 16-byte load), with access to element k (k = 0 lowest) and packing of
// E binary32 values rounded to BF16.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int E> struct Group;
template <> struct Group<1> {
    typedef uint16_t T;
    static __device__ __forceinline__ float get(T g, int) { return lo_f32(g); }
};
template <> struct Group<2> {
    typedef uint32_t T;
    static __device__ __forceinline__ float get(T g, int k) { return k ? hi_f32(g) : lo_f32(g); }
};
template <> struct Group<4> {
    typedef u32x2 T;
    static __device__ __forceinline__ float get(T g, int k) { return (k & 1) ? hi_f32(g[k >> 1]) : lo_f32(g[k >> 1]); }
};
template <> struct Group<8> {
    typedef u32x4 T;
    static __device__ __forceinline__ float get(T g, int k) { return (k & 1) ? hi_f32(g[k >> 1]) : lo_f32(g[k >> 1]); }
};

template <int E>
__device__ __forceinline__ typename Group<E>::T pack(const float (&v)[E]) {
    if constexpr (E == 1) {
        return cvt1(v[0]);
    } else if constexpr (E == 2) {
        return cvt2(v[0], v[1]);
    } else if constexpr (E == 4) {
        return u32x2{cvt2(v[0], v[1]), cvt2(v[2], v[3])};
    } else {
        return u32x4{cvt2(v[0], v[1]), cvt2(v[2], v[3]), cvt2(v[4], v[5]), cvt2(v[6], v[7])};
    }
}

// ----------------------------------------------------- buffer-resource access
// A buffer resource describes `bytes` bytes from `base`; an access through it at a
// 32-bit byte offset is checked by the hardware against that range: a load outside
// it returns zero and a store outside it is dropped (the raw-buffer range check of
// the GCN/CDNA buffer instructions; the offset is a VGPR, no SGPR offset is used).
// The fourth descriptor word, 0x00020000, is the 32-bit data format that untyped
// buffer accesses need on this GPU family.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}

// Cache-policy operand of the buffer instructions: the non-temporal (streaming) bit.
constexpr int kBufNT = 2;

// Loads and stores of one E-element group at a byte offset; AUX = kBufNT or 0.
template <int E> struct Buf;
template <> struct Buf<1> {
    template <int AUX> static __device__ __forceinline__ uint16_t ld(Rsrc r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX);
    }
    template <int AUX> static __device__ __forceinline__ void st(uint16_t v, Rsrc r, int off) {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, AUX);
    }
};
template <> struct Buf<2> {
    template <int AUX> static __device__ __forceinline__ uint32_t ld(Rsrc r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
    }
    template <int AUX> static __device__ __forceinline__ void st(uint32_t v, Rsrc r, int off) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, AUX);
    }
};
template <> struct Buf<4> {
    typedef decltype(__builtin_amdgcn_raw_buffer_load_b64(Rsrc(), 0, 0, 0)) Raw;
    template <int AUX> static __device__ __forceinline__ u32x2 ld(Rsrc r, int off) {
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
    }
    template <int AUX> static __device__ __forceinline__ void st(u32x2 v, Rsrc r, int off) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(Raw, v), r, off, 0, AUX);
    }
};

template <> struct Buf<8> {
    typedef decltype(__builtin_amdgcn_raw_buffer_load_b128(Rsrc(), 0, 0, 0)) Raw;
    template <int AUX> static __device__ __forceinline__ u32x4 ld(Rsrc r, int off) {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    }
    template <int AUX> static __device__ __forceinline__ void st(u32x4 v, Rsrc r, int off) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(Raw, v), r, off, 0, AUX);
    }
};

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  With xcd_chunk = K > 0 the launched grid is a multiple of 8K and
// the i-th workgroup an XCD receives takes logical block (8 * (i / K) + x) * K
// + i % K (x = its XCD): runs of K consecutive blocks (rows) stay on one XCD,
// and at any moment the 8 XCDs work on neighbouring runs.  K = 0 keeps the
// hardware's round-robin order.  Returns -1 for padding blocks past `blocks`.  K is
// uniform, so the power-of-two test is one scalar branch; the division it saves is
// about 40 scalar instructions at the start of every workgroup (measured on MI355X:
// 0.2 % faster at W=4 H=2048 T=4096, 0.7 % at T=1024, 1 % at W=1).
__device__ __forceinline__ int logical_block(int xcd_chunk, int blocks) {
    const int b = blockIdx.x;
    const int k = xcd_chunk;
    if (k == 0) return b;
    const int x = b & 7;
    const int i = b >> 3;
    int j, r;  // i = j * k + r
    if ((k & (k - 1)) == 0) {  // every automatic K: a shift and a mask instead of a division
        const int sh = __builtin_ctz(static_cast<unsigned>(k));
        j = i >> sh;
        r = i & (k - 1);
    } else {
        j = i / k;
        r = i - j * k;
    }
    const int l = (j * 8 + x) * k + r;
    return l < blocks ? l : -1;
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
        out[j] = cvt2(a_lo, a_hi);
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
        const uint32_t red = cvt2(a_lo, a_hi);
        const uint32_t o = cvt2(lo_f32(red) + lo_f32(rv[j]), hi_f32(red) + hi_f32(rv[j]));
        const double d_lo = static_cast<double>(lo_f32(o));
        const double d_hi = static_cast<double>(hi_f32(o));
        // The square of a BF16 value is exact in binary64, so the fused
        // multiply-add rounds once, exactly as square-then-add does.
        ss = __builtin_fma(d_lo, d_lo, ss);
        ss = __builtin_fma(d_hi, d_hi, ss);
        ro[j] = o;
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
        out[j] = cvt2(n_lo, n_hi);
    }
    return out;
}

}  // namespace dev
}  // namespace arrms
