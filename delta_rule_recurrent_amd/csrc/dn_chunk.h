// dn_chunk.h -- device helpers of the chunkwise kernels (gfx950): token tiles
// staged through registers, operand fragments read from row-major tiles and
// from global memory, small fp32 products on the matrix cores, and
// range-checked buffer loads.
#pragma once

#include "dn_device.h"
#include "dn_launch.h"

namespace dn {

// ---------------------------------------------------------------------------
// Workspace layout of one (head, chunk) block, for a chunk of CH tokens (64
// unless stated; NT = CH / 16 token tiles, CB = CH / 32 token blocks).
// Fragment arrays are [tile][k-block][lane][8] elements of E (see the fragment
// convention in dn_device.h); D-tile arrays are [tile][tile][lane][4].
//   W   [NT token tiles][DK/32][64][8]     W = T (beta e^G K)          A-fragments
//   Qt  [NT token tiles][DK/32][64][8]     Q~ = e^G * Q (KDA only)     A-fragments
//   Kt  [DK/16 chan tiles][CB][64][8]      K~^T = (e^{G_C - G} K)^T    A-fragments
//   At  [NT token tiles][CB][64][8]        attn = tril(Q K^T D)         A-fragments
//   Uu  [DV/16 col tiles][NT token tiles][64][4]  u = T (beta V)        D-tiles
//                                          (a 16-column slice is contiguous)
//   gam [DK] float                         e^{G_C} per key channel (Gated: all equal)
//   eg  [CH] float                         e^{G_t} per token (Gated / DeltaNet: the
//                                          scan reads Q itself and scales Q S by it)
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, int CH = CHUNK>
struct WsLayout {
    static constexpr long NT = CH / 16, CB = CH / 32;
    static constexpr long W_OFF = 0;
    static constexpr long Q_OFF = W_OFF + NT * (DK / 32) * 64 * 8;
    static constexpr long K_OFF = Q_OFF + NT * (DK / 32) * 64 * 8;
    static constexpr long A_OFF = K_OFF + (DK / 16) * CB * 64 * 8;
    static constexpr long U_OFF = A_OFF + NT * CB * 64 * 8;
    static constexpr long E_END = U_OFF + NT * (DV / 16) * 64 * 4;
    static constexpr long GAM_BYTE_OFF = (E_END * (long)sizeof(E) + 255) / 256 * 256;
    static constexpr long EG_BYTE_OFF = GAM_BYTE_OFF + DK * 4L;
    static constexpr long BYTES = (EG_BYTE_OFF + CH * 4L + 255) / 256 * 256;
};

template <typename E> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; };
template <> struct Vec16<float> { typedef f32x4 type; };

// A [64 x D] token-major tile held in registers while it is in flight: each
// thread carries four tokens of ITER 16-byte column vectors.
template <typename E, int D>
struct TileRegs {
    typedef typename Vec16<E>::type V16;
    static constexpr int VEC = 16 / sizeof(E);
    static constexpr int NV = D / VEC;
    static constexpr int ITER = (16 * NV + 255) / 256;
    V16 x[ITER][4];
};

// Load a tile (rows >= L read as zero). The row index is clamped instead of
// the load being skipped, so every load is unconditional and the compiler can
// wait for exactly these loads later, with other memory operations in flight.
template <typename E, int D>
__device__ __forceinline__ void tile_load(TileRegs<E, D>& r, const E* __restrict__ src, int L,
                                          int tid, int Lmask = -1) {
    // rows are read at min(t, L - 1) (L >= 1) and kept where t < Lmask
    // (Lmask defaults to L; an empty chunk passes L = 1, Lmask = 0)
    if (Lmask < 0) Lmask = L;
    typedef TileRegs<E, D> R;
    typedef typename R::V16 V16;
#pragma unroll
    for (int it = 0; it < R::ITER; ++it) {
        const int idx = min(tid + 256 * it, 16 * R::NV - 1);
        const int tq = idx / R::NV, cv = idx % R::NV;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = 4 * tq + u;
            const V16 val = *reinterpret_cast<const V16*>(src + (long)min(t, L - 1) * D + cv * R::VEC);
            r.x[it][u] = (t < Lmask) ? val : V16{};
        }
    }
}

// Write a loaded tile into LDS as row-major rows[64][ldr] and/or transposed
// trans[D][ldt] (token index contiguous, written as 4-token vectors).
template <typename E, int D, bool ROWS, bool TRANS>
__device__ __forceinline__ void tile_store(const TileRegs<E, D>& r, E* rows, int ldr, E* trans,
                                           int ldt, int tid) {
    typedef TileRegs<E, D> R;
    typedef typename R::V16 V16;
    typedef typename Vec4<E>::type V4;
#pragma unroll
    for (int it = 0; it < R::ITER; ++it) {
        const int idx = tid + 256 * it;
        if (idx >= 16 * R::NV) break;
        const int tq = idx / R::NV, cv = idx % R::NV;
        if (ROWS) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *reinterpret_cast<V16*>(rows + (4 * tq + u) * ldr + cv * R::VEC) = r.x[it][u];
        }
        if (TRANS) {
#pragma unroll
            for (int e = 0; e < R::VEC; ++e) {
                V4 c4;
#pragma unroll
                for (int u = 0; u < 4; ++u) c4[u] = r.x[it][u][e];
                *reinterpret_cast<V4*>(trans + (cv * R::VEC + e) * ldt + 4 * tq) = c4;
            }
        }
    }
}

// The level of the binary split of a chunk's tokens that holds the pair of
// token indices a > b: one plus the highest bit in which they differ (1..4 for
// a pair inside one 16-token tile).
__device__ __forceinline__ int pair_level(int a, int b) { return 32 - __clz(a ^ b); }

// fp32 16x16x16 product on the matrix cores, acc += X * Y, with X a 16x16
// block of a row-major fp32 LDS matrix and Y a 16x16 D-tile held in
// registers. Step s of the four 16x16x4 products contracts index 4g + s from
// lane group g, which is exactly the value D-tile lane (g, n) holds in its
// element s, so Y never goes through LDS.
__device__ __forceinline__ f32x4 mma16_lds_reg(const float* X, int ldx, int lane, const f32x4& Y,
                                               f32x4 acc) {
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[r * ldx + 4 * g + s], Y[s], acc, 0, 0, 0);
    return acc;
}


// Fragments in a second contraction order, for products whose operands are
// both loaded this way (K K^T, Q K^T, and K I / V I below): lane (g, r) holds
// the 8 consecutive channels 8g .. 8g+7 of row r of a 32-wide block, one
// 16-byte load. Any order works for a contraction as long as both operands
// use it; this one reads each row in 64-byte pieces instead of 32-byte ones.
// Rows >= L (past the end of the sequence, only in its last chunk) repeat row
// L - 1: the row index is clamped so that every load is unconditional and in
// bounds. Such rows never reach a stored result: their beta and log-decay are
// zero, so they add nothing to A, T, W, u or the state, and the outputs of
// those rows are not written.
template <typename E>
__device__ __forceinline__ typename Frag<E>::type frag_rows8_g(const E* __restrict__ M, int ld,
                                                               int row0, int k0, int lane, int L) {
    typedef typename Frag<E>::type F;
    const int g = lane >> 4, r = lane & 15;
    const E* p = M + (long)min(row0 + r, L - 1) * ld + k0 + 8 * g;
    if constexpr (sizeof(F) == 16) {
        return *reinterpret_cast<const F*>(p);
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
        F f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = a[i];
            f[4 + i] = b[i];
        }
        return f;
    }
}

// B-fragment of the identity in that order, for the 16 columns 16h .. 16h+15
// of a 32-wide block: lane (g, n) supplies I[8g + j][16h + n].
template <typename E>
__device__ __forceinline__ typename Frag<E>::type ident8_frag(int h, int lane) {
    const int g = lane >> 4, n = lane & 15;
    typename Frag<E>::type f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = from_f32<E>(8 * g + j == 16 * h + n ? 1.f : 0.f);
    return f;
}

// Fragment from two D-tiles (rows r0 + 4gq + e and r0 + 16 + 4gq + e) with
// each row scaled by s[row] (an LDS table) before rounding.
template <typename E>
__device__ __forceinline__ typename Frag<E>::type frag_from_tiles_rs(const f32x4& lo, const f32x4& hi,
                                                                     const float* s, int r0, int lane) {
    const int gq = lane >> 4;
    const f32x4 slo = *reinterpret_cast<const f32x4*>(s + r0 + 4 * gq);
    const f32x4 shi = *reinterpret_cast<const f32x4*>(s + r0 + 16 + 4 * gq);
    typename Frag<E>::type f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = from_f32<E>(lo[e] * slo[e]);
        f[4 + e] = from_f32<E>(hi[e] * shi[e]);
    }
    return f;
}

// Orders this wavefront's LDS accesses around a switch of who reads what
// (LDS operations of one wavefront complete in order; this also waits for
// them, and keeps the compiler from moving LDS accesses across).
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Raw buffer loads through a resource descriptor held in scalar registers:
// the base address is uniform, each lane adds a fixed 32-bit offset, and no
// per-load 64-bit address arithmetic is needed. Bytes at or past `bytes` read
// as zero (the load is range-checked). 0x00020000 is the gfx9 descriptor word
// for untyped 32-bit-element buffers.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename T>
__device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, int voff) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8 || sizeof(T) == 16 || sizeof(T) == 32,
                  "4, 8, 16 or 32 bytes");
    T out;
    if constexpr (sizeof(T) == 4) {
        const int x = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
        __builtin_memcpy(&out, &x, 4);
    } else if constexpr (sizeof(T) == 8) {
        const i32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
        __builtin_memcpy(&out, &x, 8);
    } else if constexpr (sizeof(T) == 16) {
        const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
        __builtin_memcpy(&out, &x, 16);
    } else {
        const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
        const i32x4 y = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, 0);
        __builtin_memcpy(&out, &x, 16);
        __builtin_memcpy(reinterpret_cast<char*>(&out) + 16, &y, 16);
    }
    return out;
}
// Raw 16-byte buffer store: dropped (no write, no fault) when the offset is
// at or past the resource's byte count.
template <typename T>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, int voff, const T& v) {
    static_assert(sizeof(T) == 16, "16 bytes");
    i32x4 x;
    __builtin_memcpy(&x, &v, 16);
    __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, 0, 0);
}


}  // namespace dn
