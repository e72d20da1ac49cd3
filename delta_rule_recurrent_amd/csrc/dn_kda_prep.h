// dn_kda_prep.h -- KDA's chunk-parallel step for one (head, 64-token chunk) on
// four wavefronts (gfx950): the UT/WY quantities of the chunk written to its
// workspace block, as the scan in chunk.hip reads them (page "A walk through
// of the DeltaNet family of linear attention variants", KDA section; the
// chunked form of page "28. Linear attention and Gated DeltaNet", section
// "The chunked form: recurrence as matrix multiplication"). Used by the
// two-phase prep (chunk_kda.hip) and by the one-launch prefill (chunk.hip).
#pragma once

#include "dn_device.h"
#include "dn_launch.h"
#include "dn_chunk.h"

namespace dn {

// ---------------------------------------------------------------------------
// KDA prep: four wavefronts per (head, chunk).
// ---------------------------------------------------------------------------
// Workspace contents as the scan reads them for KDA: W, Q~ = e^G * Q, K~^T,
// attn, u and the per-channel chunk decay e^{G_C}, in about 67 KiB of LDS at
// d = 128 (two workgroups per compute unit), for bf16 and fp32 at d = 64 and 128.
//
// The decay of a pair i > j, exp(G_i - G_j) per key channel, stays inside the
// contraction over channels. It is split at a token r with i > r >= j, so
// that both factors are decays (exponent <= 0) and nothing can overflow: r is
// the last token of the lower half of the smallest aligned group of 2^lv
// tokens holding both, lv = 1..6 the highest bit in which i and j differ
//     exp(G_i - G_j) = exp(G_i - G_r) exp(G_r - G_j).
// At one level every token t has a single factor f(t): exp(G_t - G_r) in the
// upper half of its group and exp(G_r - G_t) in the lower half. With
// Z = K * f and Zq = Q * f (per token and channel), Z Z^T and Z Zq^T hold the
// exact decayed products for every pair of that level (the others are
// discarded). Levels 1..4 pair tokens inside a 16-token tile, levels 5 and 6
// pair whole tiles: (1,0), (3,2) at level 5 and (2,0), (2,1), (3,0), (3,1) at 6.
//
// The work is split so that each wavefront takes two exponentials per token
// and channel:
//   wavefront 0: levels 1..4 of token tiles 0 and 1, with attn's diagonal
//                q_i . k_i; after the second barrier the blocked inverse T and
//                T diag(beta) into LDS;
//   wavefront 1: the same for token tiles 2 and 3; after the second barrier
//                attn's fragments from LDS;
//   wavefront 2: levels 5 and 6 (the tiles below the diagonal); after the
//                second barrier V with tokens as the contraction index into LDS;
//   wavefront 3: K~^T = (e^{G_C - G} K)^T, Q~ and X = e^G K through identity
//                products on the matrix cores;
// and after the third barrier wavefronts 0..2 form u = T diag(beta) V (a share
// of the value tiles each) while wavefront 3 forms W = T diag(beta) X.
// G is kept as the running sum of log2-decays (the log-decay times log2 e), so
// that every factor is one exp2 of a difference.
template <typename E> struct Vec2;
template <> struct Vec2<float> { typedef float __attribute__((ext_vector_type(2))) type; };
template <> struct Vec2<bf16> { typedef __bf16 __attribute__((ext_vector_type(2))) type; };
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <typename E, int DK, int DV>
struct KdaPrepLds {
    static constexpr int LDG = DK + 4;                 // G rows (fp32)
    static constexpr int LDF = 68;                     // A and attn (fp32 64 x 64)
    static constexpr int LDT = 64 + 16 / sizeof(E);    // T diag(beta) in the operand type
    static constexpr long G_BYTES = 64L * LDG * 4;
    static constexpr long V_BYTES = (DV / 16) * 2L * 64 * 8 * sizeof(E);
    static constexpr long F_BYTES = 64L * LDF * 4;
    static_assert(V_BYTES <= G_BYTES, "V's fragments take G's place");
    static_assert(64L * LDT * (long)sizeof(E) <= F_BYTES, "T diag(beta) takes A's place");
    // G, then (after the second barrier) V as B-fragments
    __align__(16) float G[G_BYTES / 4];
    // A, then T's diagonal blocks in place, then T diag(beta)
    __align__(16) float A[F_BYTES / 4];
    // attn, entries i >= j
    __align__(16) float At[F_BYTES / 4];
    __align__(16) float bs[64];
};

__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight G values of row `row` at channels c .. c+7 (two 16-byte LDS reads).
__device__ __forceinline__ void g_row8(const float* G, int ldg, int row, int c, float (&o)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(G + row * ldg + c);
    const f32x4 b = *reinterpret_cast<const f32x4*>(G + row * ldg + c + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[j] = a[j];
        o[4 + j] = b[j];
    }
}

// Level fragments of one row: the decay between the row's token and the
// reference token, exp2(-|G_row - G_ref|), applied to the row's key (zk) and,
// with Q, query (zq) values. G never increases along the chunk (every
// log-decay is <= 0), so this is exp2(G_row - G_ref) in the upper half of the
// row's group and exp2(G_ref - G_row) in the lower half; the sign costs no
// instruction (the exponential's source modifiers).
template <typename E, bool Q>
__device__ __forceinline__ void level_frags(const typename Frag<E>::type& kx,
                                            const typename Frag<E>::type& qx, const float (&gi)[8],
                                            const float (&gr)[8],
                                            typename Frag<E>::type& zk, typename Frag<E>::type& zq) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float f = exp2_raw(-fabsf(gi[j] - gr[j]));
        zk[j] = from_f32<E>(to_f32(kx[j]) * f);
        if (Q) zq[j] = from_f32<E>(to_f32(qx[j]) * f);
    }
}

// Four K and four Q fragments (rows = tokens, the 8 consecutive channels
// 8g .. 8g+7 of a 32-channel block per lane). Wavefronts 2 and 3 hold the four
// token tiles of one channel block in each and stream the blocks one ahead of
// their use; wavefronts 0 and 1 hold one token tile's (up to) four channel
// blocks in each. Both uses share the same registers.
template <typename E>
struct KQSlice {
    typename Frag<E>::type k[4], q[4];
};
template <typename E, int DK>
__device__ __forceinline__ void load_tile(KQSlice<E>& s, const E* __restrict__ q, const E* __restrict__ k,
                                          long tokk, int L, int tt, int lane) {
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
        s.k[kb] = frag_rows8_g<E>(k + tokk * DK, DK, 16 * tt, 32 * kb, lane, L);
        s.q[kb] = frag_rows8_g<E>(q + tokk * DK, DK, 16 * tt, 32 * kb, lane, L);
    }
}
template <typename E, int DK>
__device__ __forceinline__ void load_slice(KQSlice<E>& s, const E* __restrict__ q, const E* __restrict__ k,
                                           long tokk, int L, int kb, int lane) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        s.k[tt] = frag_rows8_g<E>(k + tokk * DK, DK, 16 * tt, 32 * kb, lane, L);
        s.q[tt] = frag_rows8_g<E>(q + tokk * DK, DK, 16 * tt, 32 * kb, lane, L);
    }
}

// Levels 1..4 of token tiles t0 and t0+1: the strictly lower entries of A's
// diagonal tiles (times beta_i) and attn's lower entries with its diagonal.
template <typename E, int DK>
__device__ __forceinline__ void kda_intra(const KQSlice<E> (&sl)[2], int t0, const float* G, const float* bs,
                                          float* As, float* At, int lane) {
    typedef typename Frag<E>::type F;
    constexpr int KB = DK / 32, LDG = DK + 4, LDF = 68;
    const int gq = lane >> 4, n = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int tt = t0 + h;
        f32x4 sA[4], sT[4], dg = zero4();
#pragma unroll
        for (int lv = 0; lv < 4; ++lv) sA[lv] = sT[lv] = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int c = 32 * kb + 8 * gq;
            float gi[8];
            g_row8(G, LDG, 16 * tt + n, c, gi);
#pragma unroll
            for (int lv = 1; lv <= 4; ++lv) {
                const int sz = 1 << lv, half = sz >> 1;
                const int ref = 16 * tt + (n & ~(sz - 1)) + half - 1;
                float gr[8];
                g_row8(G, LDG, ref, c, gr);
                F zk, zq;
                level_frags<E, true>(sl[h].k[kb], sl[h].q[kb], gi, gr, zk, zq);
                sA[lv - 1] = mma(zk, zk, sA[lv - 1]);   // (Z Z^T)[i][j]
                sT[lv - 1] = mma(zk, zq, sT[lv - 1]);   // (Z Zq^T)[j][i] = attn^T
            }
            dg = mma(sl[h].k[kb], sl[h].q[kb], dg);     // (K Q^T): its diagonal q_i . k_i
        }
        auto pick = [&](const f32x4* S, int lv, int e) {
            return lv == 1 ? S[0][e] : lv == 2 ? S[1][e] : lv == 3 ? S[2][e] : S[3][e];
        };
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int a = 4 * gq + e;   // D-tile row (local token)
            // A: row i = a, column j = n (strictly below the diagonal)
            if (a > n) As[(16 * tt + a) * LDF + 16 * tt + n] = bs[16 * tt + a] * pick(sA, pair_level(a, n), e);
            // attn^T: row j = a, column i = n (on and below attn's diagonal)
            if (n > a) At[(16 * tt + n) * LDF + 16 * tt + a] = pick(sT, pair_level(n, a), e);
            if (n == a) At[(16 * tt + n) * LDF + 16 * tt + a] = dg[e];
        }
    }
}

// Levels 5 and 6: the tiles below the diagonal of A (times beta_i) and attn.
template <typename E, int DK>
__device__ __forceinline__ void kda_cross(KQSlice<E> (&sl)[2], const E* __restrict__ q, const E* __restrict__ k,
                                          long tokk, int L, const float* G, const float* bs, float* As, float* At,
                                          int lane) {
    typedef typename Frag<E>::type F;
    constexpr int KB = DK / 32, LDG = DK + 4, LDF = 68;
    const int gq = lane >> 4, n = lane & 15;
    f32x4 a10 = zero4(), a32 = zero4(), a20 = zero4(), a21 = zero4(), a30 = zero4(), a31 = zero4();
    f32x4 t10 = zero4(), t32 = zero4(), t20 = zero4(), t21 = zero4(), t30 = zero4(), t31 = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const KQSlice<E>& x = sl[kb & 1];
        const int c = 32 * kb + 8 * gq;
        float g6[8];
        g_row8(G, LDG, 31, c, g6);   // level 6's reference token
        F z6lo[2];                   // level 6, tiles 0 and 1 (lower half)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            float g5[8];
            g_row8(G, LDG, 32 * pp + 15, c, g5);   // level 5's reference token of the pair
            F z5k[2], z5q[2], z6k[2], z6q[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tt = 2 * pp + h;
                float gi[8];
                g_row8(G, LDG, 16 * tt + n, c, gi);
                level_frags<E, true>(x.k[tt], x.q[tt], gi, g5, z5k[h], z5q[h]);
                level_frags<E, true>(x.k[tt], x.q[tt], gi, g6, z6k[h], z6q[h]);
            }
            if (pp == 0) {
                // level 5: tiles (1, 0)
                a10 = mma(z5k[1], z5k[0], a10);
                t10 = mma(z5k[0], z5q[1], t10);
                z6lo[0] = z6k[0];
                z6lo[1] = z6k[1];
            } else {
                // level 5: tiles (3, 2); level 6: (2,0), (2,1), (3,0), (3,1)
                a32 = mma(z5k[1], z5k[0], a32);
                t32 = mma(z5k[0], z5q[1], t32);
                a20 = mma(z6k[0], z6lo[0], a20);
                t20 = mma(z6lo[0], z6q[0], t20);
                a21 = mma(z6k[0], z6lo[1], a21);
                t21 = mma(z6lo[1], z6q[0], t21);
                a30 = mma(z6k[1], z6lo[0], a30);
                t30 = mma(z6lo[0], z6q[1], t30);
                a31 = mma(z6k[1], z6lo[1], a31);
                t31 = mma(z6lo[1], z6q[1], t31);
            }
        }
        if (kb + 2 < KB) load_slice<E, DK>(sl[kb & 1], q, k, tokk, L, kb + 2, lane);
    }
    // A (rows i = 16 it + 4gq + e, columns j = 16 jt + n) and attn (from attn^T
    // tiles: rows j = 16 jt + 4gq + e, columns i = 16 it + n)
    auto put = [&](int it, int jt, const f32x4& a, const f32x4& t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * it + 4 * gq + e;
            As[i * LDF + 16 * jt + n] = bs[i] * a[e];
        }
        *reinterpret_cast<f32x4*>(At + (16 * it + n) * LDF + 16 * jt + 4 * gq) = t;
    };
    put(1, 0, a10, t10);
    put(3, 2, a32, t32);
    put(2, 0, a20, t20);
    put(2, 1, a21, t21);
    put(3, 0, a30, t30);
    put(3, 1, a31, t31);
}

// K~^T = (e^{G_C - G} K)^T (A-fragments, rows = key channels) and Q~ = e^G * Q
// (A-fragments, rows = tokens) into the workspace; X = e^G K with tokens as the
// contraction index (B-fragments, for W) into xf.
template <typename E, int DK>
__device__ __forceinline__ void kda_factors(KQSlice<E> (&sl)[2], const E* __restrict__ q, const E* __restrict__ k,
                                            long tokk, int L, const float* G, typename Frag<E>::type* Kf,
                                            typename Frag<E>::type* Qf, typename Frag<E>::type (&xf)[DK / 16][2],
                                            int lane) {
    typedef typename Frag<E>::type F;
    constexpr int KB = DK / 32, LDG = DK + 4;
    const int gq = lane >> 4, n = lane & 15;
    const F id0 = ident8_frag<E>(0, lane), id1 = ident8_frag<E>(1, lane);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const KQSlice<E>& x = sl[kb & 1];
        const int c = 32 * kb + 8 * gq;
        float gl[8];
        g_row8(G, LDG, 63, c, gl);   // the chunk's last token
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            F kt_[2], xs[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tt = 2 * pp + h;
                float gi[8];
                g_row8(G, LDG, 16 * tt + n, c, gi);
                F qs;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float fk = exp2_raw(gl[j] - gi[j]);   // e^{G_C - G_t}
                    const float fg = exp2_raw(gi[j]);           // e^{G_t}
                    kt_[h][j] = from_f32<E>(to_f32(x.k[tt][j]) * fk);
                    xs[h][j] = from_f32<E>(to_f32(x.k[tt][j]) * fg);
                    qs[j] = from_f32<E>(to_f32(x.q[tt][j]) * fg);
                }
                // I Q~ is Q~^T: two of its tiles stacked over channels are an
                // A-fragment of Q~ (rows = tokens)
                Qf[(tt * KB + kb) * 64 + lane] = frag_from_tiles<E>(mma(id0, qs, zero4()), mma(id1, qs, zero4()));
            }
            // K~ I and X I are D-tiles with rows = tokens; the pair's two
            // stacked over tokens are A-fragments of K~^T (rows = channels) and
            // B-fragments of X
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const F& id = hh ? id1 : id0;
                const int ct = 2 * kb + hh;
                Kf[(ct * 2 + pp) * 64 + lane] = frag_from_tiles<E>(mma(kt_[0], id, zero4()), mma(kt_[1], id, zero4()));
                xf[ct][pp] = frag_from_tiles<E>(mma(xs[0], id, zero4()), mma(xs[1], id, zero4()));
            }
        }
        if (kb + 2 < KB) load_slice<E, DK>(sl[kb & 1], q, k, tokk, L, kb + 2, lane);
    }
}

template <typename E, int DK, int DV>
__device__ __forceinline__ void kda_prep4_item(const E* __restrict__ q, const E* __restrict__ k,
                                               const E* __restrict__ v, const E* __restrict__ beta,
                                               const E* __restrict__ g, char* __restrict__ blk,
                                               KdaPrepLds<E, DK, DV>& lds, long tok0, long tokk, int L,
                                               int w, int lane) {
    typedef WsLayout<E, DK, DV> Lw;
    typedef KdaPrepLds<E, DK, DV> Sm;
    typedef typename Frag<E>::type F;
    typedef typename Vec4<E>::type V4;
    typedef typename Vec2<E>::type V2;
    constexpr int KB = DK / 32, VB = DV / 32, VT = DV / 16;
    constexpr int LDG = Sm::LDG, LDF = Sm::LDF, LDT = Sm::LDT;
    const int gq = lane >> 4, n = lane & 15;

    F* Wf = reinterpret_cast<F*>(reinterpret_cast<E*>(blk) + Lw::W_OFF);
    F* Qf = reinterpret_cast<F*>(reinterpret_cast<E*>(blk) + Lw::Q_OFF);
    F* Kf = reinterpret_cast<F*>(reinterpret_cast<E*>(blk) + Lw::K_OFF);
    F* Af = reinterpret_cast<F*>(reinterpret_cast<E*>(blk) + Lw::A_OFF);
    V4* Uf = reinterpret_cast<V4*>(reinterpret_cast<E*>(blk) + Lw::U_OFF);
    float* gam = reinterpret_cast<float*>(blk + Lw::GAM_BYTE_OFF);
    float* G = lds.G;
    float* As = lds.A;
    float* At = lds.At;
    E* Tu = reinterpret_cast<E*>(lds.A);
    F* Vl = reinterpret_cast<F*>(lds.G);

    // ---- 1. loads, all issued up front: the log-decay runs (below), beta of
    //         token `lane`, and the K and Q fragments each wavefront works on
    //         (wavefronts 0 and 1: two token tiles each; 2 and 3: the first two
    //         32-channel blocks of all four, the rest streamed one block ahead)
    // Log-decay: wavefront w sums the channels [w DK/4, (w+1) DK/4), one pair of
    // channels and a run of RL consecutive tokens per lane (R runs per pair).
    constexpr int P = DK / 8, R = 64 / P, RL = 64 / R;
    const int pr = lane % P, run = lane / P;
    const int c0 = w * (DK / 4) + 2 * pr;
    V2 graw[RL];
#pragma unroll
    for (int t = 0; t < RL; ++t)
        graw[t] = *reinterpret_cast<const V2*>(g + (tok0 + min(run * RL + t, L - 1)) * DK + c0);
    const E braw = beta[tok0 + min(lane, L - 1)];
    KQSlice<E> sl[2];
    if (w < 2) {
        load_tile<E, DK>(sl[0], q, k, tokk, L, 2 * w, lane);
        load_tile<E, DK>(sl[1], q, k, tokk, L, 2 * w + 1, lane);
    } else {
        load_slice<E, DK>(sl[0], q, k, tokk, L, 0, lane);
        load_slice<E, DK>(sl[1], q, k, tokk, L, 1, lane);
    }

    // running sums (rows past the end of the sequence add zero), the runs'
    // totals passed on across lanes, G (in log2 units) into LDS
    {
        float s0 = 0.f, s1 = 0.f, r0[RL], r1[RL];
#pragma unroll
        for (int t = 0; t < RL; ++t) {
            const bool in = run * RL + t < L;
            s0 += in ? to_f32(graw[t][0]) : 0.f;
            s1 += in ? to_f32(graw[t][1]) : 0.f;
            r0[t] = s0;
            r1[t] = s1;
        }
        float i0 = s0, i1 = s1;   // inclusive prefix of the run totals over runs
#pragma unroll
        for (int off = 1; off < R; off <<= 1) {
            const float y0 = __shfl_up(i0, off * P, 64), y1 = __shfl_up(i1, off * P, 64);
            if (run >= off) {
                i0 += y0;
                i1 += y1;
            }
        }
        const float cy0 = i0 - s0, cy1 = i1 - s1;
        constexpr float LOG2E = 1.4426950408889634f;
#pragma unroll
        for (int t = 0; t < RL; ++t)
            *reinterpret_cast<f32x2*>(G + (run * RL + t) * LDG + c0) = f32x2{(r0[t] + cy0) * LOG2E, (r1[t] + cy1) * LOG2E};
        if (run == R - 1) {
            // e^{G_C}: the state's decay over the chunk, per key channel
            *reinterpret_cast<f32x2*>(gam + c0) = f32x2{exp2_raw((r0[RL - 1] + cy0) * LOG2E),
                                                        exp2_raw((r1[RL - 1] + cy1) * LOG2E)};
        }
    }
    if (w == 0) lds.bs[lane] = lane < L ? to_f32(braw) : 0.f;
    lds_barrier();   // G and beta are in LDS
    const float* bs = lds.bs;

    // ---- 2. the decayed products and factors
    F xf[DK / 16][2];   // (wavefront 3) X = e^G K, B-fragments over tokens
    F vf[4][VB];        // (wavefront 2) V, rows = tokens
    if (w < 2) {
        kda_intra<E, DK>(sl, 2 * w, G, bs, As, At, lane);
    } else if (w == 2) {
        kda_cross<E, DK>(sl, q, k, tokk, L, G, bs, As, At, lane);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int kb = 0; kb < VB; ++kb) vf[tt][kb] = frag_rows8_g<E>(v + tok0 * DV, DV, 16 * tt, 32 * kb, lane, L);
    } else {
        kda_factors<E, DK>(sl, q, k, tokk, L, G, Kf, Qf, xf, lane);
    }
    lds_barrier();   // A and attn are complete; G is no longer read

    // ---- 3. the blocked inverse (0), attn's fragments (1), V's transposes (2)
    if (w == 0) {
        // 3a: diagonal blocks by forward substitution, lane (block gq, column n):
        //     T_jj = 1, T_ij = -sum_{j <= m < i} A_im T_mj; written over the block of A
        {
            const int b0 = 16 * gq, j = n;
            float tc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) tc[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc += As[(b0 + i) * LDF + b0 + m] * tc[m];
                tc[i] = (i > j) ? -acc : tc[i];
            }
            lds_fence();
#pragma unroll
            for (int i = 0; i < 16; ++i) As[(b0 + i) * LDF + b0 + j] = tc[i];
        }
        lds_fence();
        // 3b: T_IJ = -T_II sum_{J <= K < I} A_IK T_KJ on the matrix cores (fp32)
        f32x4 tm[4][4];
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) tm[J][J][e] = As[(16 * J + 4 * gq + e) * LDF + 16 * J + n];
#pragma unroll
        for (int I = 1; I < 4; ++I) {
#pragma unroll
            for (int J = 0; J < I; ++J) {
                f32x4 Rr = zero4();
#pragma unroll
                for (int K = J; K < I; ++K) Rr = mma16_lds_reg(As + 16 * I * LDF + 16 * K, LDF, lane, tm[K][J], Rr);
                tm[I][J] = -mma16_lds_reg(As + 16 * I * LDF + 16 * I, LDF, lane, Rr, zero4());
            }
        }
        lds_fence();   // every read of A and of the diagonal blocks has returned
        // T diag(beta) (lower triangular) in the operand type, over the fp32
        // region; lane (gq, n) holds column 16J + n of tile (I, J)
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            const float cb = bs[16 * J + n];
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Tu[(16 * I + 4 * gq + e) * LDT + 16 * J + n] = from_f32<E>(I >= J ? tm[I][J][e] * cb : 0.f);
        }
    } else if (w == 1) {
        // attn = tril(...) as A-fragments (rows i, contraction over j)
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int i = 16 * it + n;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(At + i * LDF + 32 * kb + 4 * gq);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(At + i * LDF + 32 * kb + 16 + 4 * gq);
                F f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[e] = from_f32<E>(32 * kb + 4 * gq + e <= i ? lo[e] : 0.f);
                    f[4 + e] = from_f32<E>(32 * kb + 16 + 4 * gq + e <= i ? hi[e] : 0.f);
                }
                Af[(it * 2 + kb) * 64 + lane] = f;
            }
    } else if (w == 2) {
        // V with tokens as the contraction index (D = V I), into LDS over G
        const F id0 = ident8_frag<E>(0, lane), id1 = ident8_frag<E>(1, lane);
#pragma unroll
        for (int nt = 0; nt < VT; ++nt) {
            f32x4 d[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) d[tt] = mma(vf[tt][nt >> 1], (nt & 1) ? id1 : id0, zero4());
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) Vl[(nt * 2 + kt) * 64 + lane] = frag_from_tiles<E>(d[2 * kt], d[2 * kt + 1]);
        }
    }
    lds_barrier();   // T diag(beta) and V are in LDS

    if (w < 3) {
        // ---- 4. u = T diag(beta) V as D-tiles (rows = tokens), value tiles w, w+3, ...
        F tu[4][2];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) tu[tt][kt] = frag_rows<E>(Tu, LDT, 16 * tt, 32 * kt, lane);
        for (int nt = w; nt < VT; nt += 3) {
            F vb[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) vb[kt] = Vl[(nt * 2 + kt) * 64 + lane];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) acc = mma(tu[tt][kt], vb[kt], acc);
                V4 u4;
#pragma unroll
                for (int e = 0; e < 4; ++e) u4[e] = from_f32<E>(acc[e]);
                Uf[(nt * 4 + tt) * 64 + lane] = u4;
            }
        }
    } else {
        // ---- 4'. W = T diag(beta) X: W^T tiles (rows = key channels) for each
        //          token tile, stacked over channel tiles = A-fragments of W
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            F tf[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) tf[kt] = frag_rows<E>(Tu, LDT, 16 * tt, 32 * kt, lane);
            f32x4 wt[DK / 16];
#pragma unroll
            for (int mt = 0; mt < DK / 16; ++mt) {
                wt[mt] = zero4();
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) wt[mt] = mma(xf[mt][kt], tf[kt], wt[mt]);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) Wf[(tt * KB + kb) * 64 + lane] = frag_from_tiles<E>(wt[2 * kb], wt[2 * kb + 1]);
        }
    }
}

}  // namespace dn
