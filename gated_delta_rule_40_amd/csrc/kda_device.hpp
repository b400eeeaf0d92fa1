// kda_device.hpp -- gfx950 device helpers shared by the libkda kernels:
// vector types, bf16 conversion and MFMA fragment handling.
//
// MFMA conventions used throughout (one 64-lane wave, lane l, group j = l/16,
// row/col m = l%16):
//   * 16x16 accumulator tile D: lane l holds D[4j+i][m], i = 0..3.
//   * An operand "K-block" is a slab of the contraction index consumed by
//     one bf16 16x16x32 MFMA (KB = 32) or by four fp32 16x16x4 MFMAs (KB = 16).
//     In a K-block, lane group j carries contraction indices
//        bf16: {4j..4j+3} U {16+4j..16+4j+3}   (8 values, element e)
//        fp32: {4j..4j+3}                        (element i feeds instruction i)
//     A operands are read as A[m][those k]; B operands as B[those k][m].
//     Because A and B use the same assignment, any fixed assignment gives the
//     same product, and this one makes an accumulator tile pair (rows = k)
//     usable directly as the B operand of the next contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace kda {

// Host side: raise a kernel's dynamic-LDS limit to `bytes` once per device
// (the attribute belongs to the device that is current when it is set).
// `done` holds one bit per device id below 64, set after a successful call;
// devices beyond that are set on every launch.  Thread-safe.
inline hipError_t ensure_lds_limit(const void *kern, int bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f(bf16_t x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f(f16_t x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return static_cast<bf16_t>(x); }
template <> __device__ __forceinline__ f16_t from_f<f16_t>(float x) { return static_cast<f16_t>(x); }

// ---------------------------------------------------------------- fragments
template <typename T> struct Mma;

// 2-byte operand types (bf16, fp16) share one layout: 16x16x32 MFMA per
// K-block, 16x16x16 MFMA for 16-wide contractions.
template <typename H, typename V8, typename V4> struct Mma2 {
    static constexpr int KB = 32;     // contraction indices per K-block
    typedef V8 frag;                   // per-lane operand of one K-block
    typedef V4 frag16;                 // per-lane operand of a 16-wide contraction

    // A[m][k0 + K-block indices of group j], from a row-major LDS row.
    __device__ static __forceinline__ frag load(const H *row, int k0, int j) {
        const V4 lo = *reinterpret_cast<const V4 *>(row + k0 + 4 * j);
        const V4 hi = *reinterpret_cast<const V4 *>(row + k0 + 16 + 4 * j);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // The same K-block from a row stored in the permuted order of kperm: the
    // eight values of group j sit contiguously at 8j (one 16-byte read).
    __device__ static __forceinline__ frag load_p(const H *row, int k0, int j) {
        return *reinterpret_cast<const V8 *>(row + k0 + 8 * j);
    }
    // Same as load, each value multiplied by s[k] (fp32 per-channel scale) before rounding.
    __device__ static __forceinline__ frag load_scaled(const H *row, const float *s, int k0, int j) {
        const V4 lo = *reinterpret_cast<const V4 *>(row + k0 + 4 * j);
        const V4 hi = *reinterpret_cast<const V4 *>(row + k0 + 16 + 4 * j);
        const f32x4 slo = *reinterpret_cast<const f32x4 *>(s + k0 + 4 * j);
        const f32x4 shi = *reinterpret_cast<const f32x4 *>(s + k0 + 16 + 4 * j);
        frag r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = from_f<H>(to_f(lo[e]) * slo[e]);
            r[e + 4] = from_f<H>(to_f(hi[e]) * shi[e]);
        }
        return r;
    }
    // B operand from the accumulator tiles covering rows k0..k0+31 (t[0], t[1]),
    // each value multiplied by `scale` (an exact power of two) before rounding.
    __device__ static __forceinline__ frag from_acc(const f32x4 *t, float scale = 1.f) {
        frag r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = from_f<H>(t[0][e] * scale);
            r[e + 4] = from_f<H>(t[1][e] * scale);
        }
        return r;
    }
    // 16-wide contraction: group j carries k = 4j..4j+3.
    __device__ static __forceinline__ frag16 load16(const H *row, int k0, int j) {
        return *reinterpret_cast<const V4 *>(row + k0 + 4 * j);
    }
    __device__ static __forceinline__ frag16 from_acc16(const f32x4 &t, float scale = 1.f) {
        frag16 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = from_f<H>(t[e] * scale);
        return r;
    }
};

template <> struct Mma<bf16_t> : Mma2<bf16_t, bf16x8, bf16x4> {
    __device__ static __forceinline__ f32x4 mma(const frag &a, const frag &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mma16(const frag16 &a, const frag16 &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<f16_t> : Mma2<f16_t, f16x8, f16x4> {
    __device__ static __forceinline__ f32x4 mma(const frag &a, const frag &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mma16(const frag16 &a, const frag16 &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KB = 16;
    typedef f32x4 frag;
    typedef f32x4 frag16;

    __device__ static __forceinline__ frag load(const float *row, int k0, int j) {
        return *reinterpret_cast<const f32x4 *>(row + k0 + 4 * j);
    }
    __device__ static __forceinline__ frag load_p(const float *row, int k0, int j) { return load(row, k0, j); }
    __device__ static __forceinline__ frag load_scaled(const float *row, const float *s, int k0, int j) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(row + k0 + 4 * j);
        const f32x4 y = *reinterpret_cast<const f32x4 *>(s + k0 + 4 * j);
        return x * y;
    }
    __device__ static __forceinline__ frag from_acc(const f32x4 *t, float scale = 1.f) { return t[0] * scale; }
    __device__ static __forceinline__ f32x4 mma(const frag &a, const frag &b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    __device__ static __forceinline__ frag16 load16(const float *row, int k0, int j) { return load(row, k0, j); }
    __device__ static __forceinline__ frag16 from_acc16(const f32x4 &t, float scale = 1.f) { return t * scale; }
    __device__ static __forceinline__ f32x4 mma16(const frag16 &a, const frag16 &b, f32x4 c) { return mma(a, b, c); }
};

// Storage position of contraction index k in a row read with load_p: for
// 2-byte operands, inside each 32-block the indices of lane group j
// ({4j..4j+3} and {16+4j..16+4j+3}) are stored contiguously at 8j..8j+7, so
// 4-aligned runs of k stay contiguous; fp32 rows are stored in order.
template <typename T>
__device__ __forceinline__ int kperm(int k) {
    if (sizeof(T) == 4) return k;
    return (k & ~31) | (((k & 15) >> 2) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// ------------------------------------------------------------- small loads
template <typename T> struct Pair;       // two adjacent elements of a row
template <> struct Pair<bf16_t> { typedef bf16x2 type; };
template <> struct Pair<f16_t> { typedef f16x2 type; };
template <> struct Pair<float> { typedef f32x2 type; };

template <typename T> struct Quad;       // four adjacent elements of a row
template <> struct Quad<bf16_t> { typedef bf16x4 type; };
template <> struct Quad<f16_t> { typedef f16x4 type; };
template <> struct Quad<float> { typedef f32x4 type; };

template <typename T>
__device__ __forceinline__ f32x2 load_pair(const T *p) {
    const typename Pair<T>::type x = *reinterpret_cast<const typename Pair<T>::type *>(p);
    f32x2 r;
    r[0] = to_f(x[0]);
    r[1] = to_f(x[1]);
    return r;
}
template <typename T>
__device__ __forceinline__ void store_pair(T *p, float a, float b) {
    typename Pair<T>::type x;
    x[0] = from_f<T>(a);
    x[1] = from_f<T>(b);
    *reinterpret_cast<typename Pair<T>::type *>(p) = x;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Flags of a segment-plan entry {sequence, t0, t1, flags}: the sequence's
// first and last segment.
enum { SEG_FIRST = 1, SEG_LAST = 2 };

// Exact power-of-two scale that maps a magnitude m into [2^13, 2^14):
// returns 2^(13 - floor(log2 m)) for finite normal m > 0, else 1.  Used to
// keep fp16 MFMA operands in range without changing their relative rounding.
// Branch-free: the exponent arithmetic runs on every lane and a select
// picks 1 for the special cases.
__device__ __forceinline__ float pow2_scale(float m) {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);
    const int se = min(max(13 - (e - 127) + 127, 1), 254);
    return __uint_as_float((uint32_t)((e == 0 || e == 0xff) ? 127 : se) << 23);
}
// 1/s for a scale s returned by pow2_scale (exact).
__device__ __forceinline__ float pow2_inv(float s) {
    const uint32_t e = (__float_as_uint(s) >> 23) & 0xffu;
    return __uint_as_float((254u - e) << 23);
}
// Maximum over the four lane groups (j = lane/16) that share a column, with
// the gfx950 lane swaps (VALU, no LDS round trip): permlane16_swap(x, x)
// returns rows {0,0,2,2} and {1,1,3,3} of x (a row = 16 lanes), and
// permlane32_swap(x, x) the lower and the upper half-wave, each in both halves.
// For m >= 0 (magnitudes): non-negative floats order as their bit patterns, so
// the maxima are integer maxima, which need no NaN canonicalisation.
__device__ __forceinline__ float colmax(float m) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const uint32_t u = max(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(max(b[0], b[1]));
}
// Lane movement inside each 16-lane row by DPP (VALU, no LDS round trip):
// quad_perm(1,0,3,2) = 0xB1 and quad_perm(2,3,0,1) = 0x4E swap neighbours at
// distance 1 and 2, row_ror:4 = 0x124 and row_ror:8 = 0x128 rotate the row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Maximum over the 16 lanes of each row, for m >= 0 (integer maxima as in colmax).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_movu(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float rowmax16(float m) {
    uint32_t u = __float_as_uint(m);
    u = max(u, dpp_movu<0xB1>(u));
    u = max(u, dpp_movu<0x4E>(u));
    u = max(u, dpp_movu<0x124>(u));
    return __uint_as_float(max(u, dpp_movu<0x128>(u)));
}
// Maximum over the whole wave, for m >= 0.
__device__ __forceinline__ float wavemax(float m) { return colmax(rowmax16(m)); }
// Sum over each aligned group of 8 lanes, in every lane of the group
// (row_half_mirror = 0x141 pairs lane l with 7 - l).
__device__ __forceinline__ float sum8(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    return x + dpp_mov<0x141>(x);
}
// Sum over the whole wave, in every lane.
__device__ __forceinline__ float wavesum(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    x += dpp_mov<0x124>(x);
    x += dpp_mov<0x128>(x);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// m folded with |x| elementwise, as two three-input maxima (v_max3 with |.|).
__device__ __forceinline__ float absmax_acc(float m, const f32x4 &x) {
    m = fmaxf(fmaxf(m, fabsf(x[0])), fabsf(x[1]));
    return fmaxf(fmaxf(m, fabsf(x[2])), fabsf(x[3]));
}
__device__ __forceinline__ float absmax4(const f32x4 &x) {
    return fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
}

}  // namespace kda
