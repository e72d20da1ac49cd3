// dn_device.h -- device helpers shared by the gfx950 kernels of the delta-rule library:
// element types, vector types, and the MFMA fragment conventions used to chain
// matrix-core products without a round trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// Element access. E is the storage type of q, k, v, beta, g and o (float or bf16).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Four consecutive elements as a vector (8 bytes for bf16, 16 for fp32).
template <typename E> struct Vec4;
template <> struct Vec4<float> { typedef f32x4 type; };
template <> struct Vec4<bf16> { typedef bf16x4 type; };

// ---------------------------------------------------------------------------
// MFMA fragments.
//
// A matrix-core product D(16x16, fp32) += A(16 x 32) * B(32 x 16) is issued as
// one v_mfma_f32_16x16x32_bf16 for bf16 operands and as eight
// v_mfma_f32_16x16x4_f32 for fp32 operands. In both cases lane l = 16*g + r
// (g = l / 16, r = l % 16) supplies eight operand values per 32-wide block of
// the contraction index, and the result tile is held as
//      D-tile: lane (g, n) holds D[4g + i][n], i = 0..3.
// The eight contraction indices a lane supplies are
//      pi(g, j) = 4g + j            for j = 0..3
//               = 16 + 4g + (j - 4) for j = 4..7
// for row r of A (A-fragment) and for column r of B (B-fragment). Because the
// product sums over all 32 indices, any bijection works as long as A and B
// agree; this one is chosen because it is exactly what a lane holds in the
// two D-tiles covering rows 0..15 and 16..31 of a 32-row block. So the result
// of one product, split into 32-row blocks, is directly the B-fragment of a
// following product that contracts over those rows, and a product computed
// transposed (rows = the next product's contraction index) is directly an
// A-fragment. This is what lets the chunk kernels chain their products in
// registers.
// ---------------------------------------------------------------------------
template <typename E> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
}

// Fragment from two D-tiles (rows 0..15 -> values 0..3, rows 16..31 -> values 4..7),
// rounded to the operand type, optionally scaling each value.
template <typename E>
__device__ __forceinline__ typename Frag<E>::type frag_from_tiles(const f32x4& lo, const f32x4& hi) {
    typename Frag<E>::type f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = from_f32<E>(lo[i]);
        f[4 + i] = from_f32<E>(hi[i]);
    }
    return f;
}

// Fragment of a row-major matrix M (leading dimension ld, in elements) for the
// 32-wide contraction block starting at column k0: lane (g, r) reads
// M[row0 + r][k0 + 4g .. +3] and M[row0 + r][k0 + 16 + 4g .. +3].
// Works on LDS or global memory; both halves are 4-element vector reads.
template <typename E>
__device__ __forceinline__ typename Frag<E>::type frag_rows(const E* M, int ld, int row0, int k0,
                                                            int lane) {
    const int g = lane >> 4, r = lane & 15;
    const E* p = M + (row0 + r) * ld + k0 + 4 * g;
    typedef typename Vec4<E>::type V4;
    V4 a = *reinterpret_cast<const V4*>(p);
    V4 b = *reinterpret_cast<const V4*>(p + 16);
    typename Frag<E>::type f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = a[i];
        f[4 + i] = b[i];
    }
    return f;
}

// Same as frag_rows, but every value is multiplied (in fp32) by a per-row
// factor rs (rows) or per-column factor cs (contraction index) before rounding.
template <typename E>
__device__ __forceinline__ typename Frag<E>::type frag_rows_scaled(const E* M, int ld, int row0,
                                                                   int k0, int lane, float rs,
                                                                   const float* cs) {
    const int g = lane >> 4, r = lane & 15;
    const E* p = M + (row0 + r) * ld + k0 + 4 * g;
    typedef typename Vec4<E>::type V4;
    V4 a = *reinterpret_cast<const V4*>(p);
    V4 b = *reinterpret_cast<const V4*>(p + 16);
    typename Frag<E>::type f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float ca = cs ? cs[k0 + 4 * g + i] : 1.0f;
        float cb = cs ? cs[k0 + 16 + 4 * g + i] : 1.0f;
        f[i] = from_f32<E>(to_f32(a[i]) * rs * ca);
        f[4 + i] = from_f32<E>(to_f32(b[i]) * rs * cb);
    }
    return f;
}

// Workgroup barrier that waits only for this wave's LDS (and scalar) memory
// operations, leaving its global loads in flight. HIP's __syncthreads() also
// drains outstanding global loads, which would stall a software pipeline that
// prefetches the next iteration's operands across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Wave-wide inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        float y = __shfl_up(x, off, WAVE);
        if (lane >= off) x += y;
    }
    return x;
}

__device__ __forceinline__ float readlane_f(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

}  // namespace dn
