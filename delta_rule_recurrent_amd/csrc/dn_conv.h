// dn_conv.h -- per-lane helpers of the gated layer's prologue and epilogue
// (gfx950): eight consecutive channels of a token row in registers, the
// width-4 causal convolution as packed bf16 dot products, SiLU and the L2 norm
// with the hardware transcendentals, and lane sums inside a row of 16 lanes.
// Shared by the layer kernels and the prefill prep that runs the prologue in
// its load stage, so that both compute the same bits.
#pragma once

#include "dn_device.h"

namespace dn {

// Eight consecutive elements <-> fp32.
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)a[i];
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = x[i]; b[i] = x[4 + i]; }
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (bf16)x[i];
    *reinterpret_cast<bf16x8*>(p) = a;
}

// Eight consecutive elements kept in their storage type (fewer registers while in flight).
template <typename E> struct Raw8;
template <> struct Raw8<bf16> { bf16x8 v; };
template <> struct Raw8<float> { f32x4 a, b; };
__device__ __forceinline__ void load_raw(const bf16* p, Raw8<bf16>& r) {
    r.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load_raw(const float* p, Raw8<float>& r) {
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ float elem(const Raw8<bf16>& r, int i) { return (float)r.v[i]; }
__device__ __forceinline__ float elem(const Raw8<float>& r, int i) { return i < 4 ? r.a[i] : r.b[i - 4]; }
__device__ __forceinline__ void set_elem(Raw8<bf16>& r, int i, bf16 x) { r.v[i] = x; }
__device__ __forceinline__ void set_elem(Raw8<float>& r, int i, float x) {
    if (i < 4) r.a[i] = x;
    else r.b[i - 4] = x;
}

// bf16 pairs: channel i of two rows as one 32-bit word (the earlier row in the
// low half), picked with a byte permute; and the fp32 dot product of two pairs
// plus an accumulator (products of bf16 values are exact in fp32).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ unsigned pair_of(const Raw8<bf16>& early, const Raw8<bf16>& late, int i) {
    const unsigned a = __builtin_bit_cast(u32x4, early.v)[i / 2];
    const unsigned b = __builtin_bit_cast(u32x4, late.v)[i / 2];
    return __builtin_amdgcn_perm(b, a, (i & 1) ? 0x07060302u : 0x05040100u);
}
__device__ __forceinline__ float dot2(unsigned x, unsigned w, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, w),
                                           acc, false);
}

// SiLU with the hardware exp2 and reciprocal (each within 1 ulp): x / (1 + e^-x).
// Large negative x gives e^-x = inf and a zero reciprocal, so the result is -0.
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// 1 / max(sqrt(s), 1e-12) for a sum of squares s >= 0, with the hardware rsqrt.
__device__ __forceinline__ float inv_norm(float s) { return __builtin_amdgcn_rsqf(fmaxf(s, 1e-24f)); }

// Sum over the `WIDTH` consecutive lanes that hold one row (8 or 16, aligned), with
// data-parallel-primitive moves inside a row of 16 lanes: swap neighbours, swap
// pairs (each quad then holds its sum), mirror within eight lanes, mirror within
// sixteen. The additions pair up as in a butterfly, so every lane of the row ends
// with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float s) {
    return s + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), CTRL,
                                                                  0xF, 0xF, false));
}
template <int WIDTH>
__device__ __forceinline__ float row_sum(float s) {
    static_assert(WIDTH == 8 || WIDTH == 16, "rows of 8 or 16 lanes");
    s = dpp_add<0xB1>(s);    // quad_perm [1,0,3,2]
    s = dpp_add<0x4E>(s);    // quad_perm [2,3,0,1]
    s = dpp_add<0x141>(s);   // row_half_mirror
    if (WIDTH == 16) s = dpp_add<0x140>(s);   // row_mirror
    return s;
}

// The prologue of eight consecutive tokens t0 .. t0+7 (t0 >= 0) of one
// D-channel segment for one lane of a lane group (D/8 lanes, eight channels
// each), as the layer's prologue kernel computes them: the width-4 causal
// convolution with the three inputs before t0 (earlier rows, else the carried
// history, else zeros), SiLU, and for key segments the L2 norm times qs.
//   xs    qkv row of the sequence's token 0 at this lane's first channel
//         (rows C elements apart); T the sequence's length
//   cw    conv_w at this lane's first channel ([C][4])
//   cst   this lane's 24 history entries ([C][3] at its first channel), or null
//   dst   output row of token t0 for this lane (rows ldd apart), bf16; rows at
//         or past T are written as zeros
//   gdst  null, or a second destination (rows D apart) for the rows before T
// Every lane of the group must take part (the norm is a lane sum).
template <int D>
__device__ __forceinline__ void prologue_run8(const bf16* __restrict__ xs, long C, long T, long t0,
                                              const bf16* __restrict__ cw, const bf16* cst, bool is_key,
                                              float qs, bf16* dst, int ldd, bf16* gdst) {
    constexpr int LPR = D / 8;
    constexpr int R8 = 8;
    Raw8<bf16> hr[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const long tt = t0 - 3 + j;
        if (tt >= 0) {
            // (a run wholly past T reads in-bounds rows; its outputs are zeros)
            load_raw(xs + min(tt, T - 1) * C, hr[j]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) set_elem(hr[j], i, cst ? cst[i * 3 + 3 + tt] : from_f32<bf16>(0.0f));
        }
    }
    const int last = (int)min((long)R8 - 1, T - 1 - t0);   // the run's last row before T
    Raw8<bf16> x[R8];
#pragma unroll
    for (int r = 0; r < R8; ++r) load_raw(xs + (t0 + min(r, last)) * C, x[r]);
    Raw8<bf16> wr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) load_raw(cw + 8 * j, wr[j]);
    unsigned w01[8], w23[8], p2[8], p1[8];   // pairs (t-3, t-2) and (t-2, t-1)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4 wd = __builtin_bit_cast(u32x4, wr[i / 2].v);
        w01[i] = wd[2 * (i % 2)];
        w23[i] = wd[2 * (i % 2) + 1];
        p2[i] = pair_of(hr[0], hr[1], i);
        p1[i] = pair_of(hr[1], hr[2], i);
    }
#pragma unroll
    for (int r = 0; r < R8; ++r) {
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const unsigned p0 = pair_of(r == 0 ? hr[2] : x[r - 1], x[r], i);   // (t-1, t)
            y[i] = dot2(p0, w23[i], dot2(p2[i], w01[i], 0.0f));
            p2[i] = p1[i];
            p1[i] = p0;
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            y[i] = silu(y[i]);
            ss += y[i] * y[i];
        }
        if (is_key) {
            const float sc = qs * inv_norm(row_sum<LPR>(ss));
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] *= sc;
        }
        if (r > last) {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = 0.0f;
        }
        store8(dst + r * ldd, y);
        if (gdst && r <= last) store8(gdst + r * D, y);
    }
}

}  // namespace dn
