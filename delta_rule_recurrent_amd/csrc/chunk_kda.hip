// chunk_kda.hip -- KDA's chunk-parallel phase (per-key-channel decay) on gfx950:
// the UT/WY quantities of every (head, 64-token chunk) written to the chunk
// workspace that the scan in chunk.hip reads (page "A walk through of the
// DeltaNet family of linear attention variants", KDA section; the chunked form
// of page "28. Linear attention and Gated DeltaNet", section "The chunked
// form: recurrence as matrix multiplication").
#include "dn_device.h"
#include "dn_launch.h"
#include "dn_chunk.h"

namespace dn {

// ---------------------------------------------------------------------------
// KDA prep on two wavefronts per (head, chunk).
// ---------------------------------------------------------------------------
// Same workspace contents as chunk_prep_kernel's KDA form (W, Q~, K~^T, attn,
// u, the per-channel chunk decay), in about 69 KiB of LDS at d = 128 (two
// units per compute unit) and for fp32 at d = 128 as well.
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
//   wavefront 0: levels 1..4 (the diagonal tiles of A and attn, and attn's
//                diagonal q_i . k_i); after the second barrier the blocked
//                inverse T and T diag(beta); after the third u = T diag(beta) V.
//   wavefront 1: levels 5 and 6 (the tiles below the diagonal), K~^T, Q~ and
//                X = e^G K through identity products; after the second barrier
//                attn's fragments and V with tokens as the contraction index;
//                after the third W = T diag(beta) X.
// Each wavefront takes four exponentials per token and channel. G is kept as
// the running sum of log2-decays (the log-decay times log2 e) so that every
// factor is one exp2 of a difference.
template <typename E> struct Vec2;
template <> struct Vec2<float> { typedef float __attribute__((ext_vector_type(2))) type; };
template <> struct Vec2<bf16> { typedef __bf16 __attribute__((ext_vector_type(2))) type; };

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

// Level fragments of one row: the factor exp2(sg (G_row - G_ref)) applied to
// the row's key (zk) and, with Q, query (zq) values; sg = +1 in the upper half
// of the row's group, -1 in the lower half (the exponent is then <= 0).
template <typename E, bool Q>
__device__ __forceinline__ void level_frags(const typename Frag<E>::type& kx,
                                            const typename Frag<E>::type& qx, const float (&gi)[8],
                                            const float (&gr)[8], float sg,
                                            typename Frag<E>::type& zk, typename Frag<E>::type& zq) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float f = exp2_raw(sg * (gi[j] - gr[j]));
        zk[j] = from_f32<E>(to_f32(kx[j]) * f);
        if (Q) zq[j] = from_f32<E>(to_f32(qx[j]) * f);
    }
}

template <typename E, int DK, int DV>
__device__ __forceinline__ void kda_prep2_item(const E* __restrict__ q, const E* __restrict__ k,
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
    //         token `lane`, K and Q fragments (rows = tokens, 8 consecutive
    //         channels per lane); wavefront 1 loads V after its level products
    // Log-decay: wavefront w sums the channels [w DK/2, (w+1) DK/2), one pair of
    // channels and a run of RL consecutive tokens per lane (R runs per pair).
    constexpr int P = DK / 4, R = 64 / P, RL = 64 / R;
    const int pr = lane % P, run = lane / P;
    const int c0 = w * (DK / 2) + 2 * pr;
    V2 graw[RL];
#pragma unroll
    for (int t = 0; t < RL; ++t)
        graw[t] = *reinterpret_cast<const V2*>(g + (tok0 + min(run * RL + t, L - 1)) * DK + c0);
    const E braw = beta[tok0 + min(lane, L - 1)];
    F kf[4][KB], qf[4][KB];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kf[tt][kb] = frag_rows8_g<E>(k + tokk * DK, DK, 16 * tt, 32 * kb, lane, L);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qf[tt][kb] = frag_rows8_g<E>(q + tokk * DK, DK, 16 * tt, 32 * kb, lane, L);

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
        for (int t = 0; t < RL; ++t) {
            typedef float __attribute__((ext_vector_type(2))) f2;
            *reinterpret_cast<f2*>(G + (run * RL + t) * LDG + c0) = f2{(r0[t] + cy0) * LOG2E, (r1[t] + cy1) * LOG2E};
        }
        if (run == R - 1) {
            // e^{G_C}: the state's decay over the chunk, per key channel
            typedef float __attribute__((ext_vector_type(2))) f2;
            *reinterpret_cast<f2*>(gam + c0) = f2{exp2_raw((r0[RL - 1] + cy0) * LOG2E),
                                                  exp2_raw((r1[RL - 1] + cy1) * LOG2E)};
        }
    }
    if (w == 0) lds.bs[lane] = lane < L ? to_f32(braw) : 0.f;
    lds_barrier();   // G and beta are in LDS
    const float* bs = lds.bs;

    if (w == 0) {
        // ---- 2. levels 1..4: the diagonal tiles of A and attn
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 sA[4], sT[4], dg = zero4();
#pragma unroll
            for (int lv = 0; lv < 4; ++lv) sA[lv] = sT[lv] = zero4();
            const int row = 16 * tt + n;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int c = 32 * kb + 8 * gq;
                float gi[8];
                g_row8(G, LDG, row, c, gi);
#pragma unroll
                for (int lv = 1; lv <= 4; ++lv) {
                    const int sz = 1 << lv, half = sz >> 1;
                    const int ref = 16 * tt + (n & ~(sz - 1)) + half - 1;
                    float gr[8];
                    g_row8(G, LDG, ref, c, gr);
                    F zk, zq;
                    level_frags<E, true>(kf[tt][kb], qf[tt][kb], gi, gr, (n & (sz - 1)) >= half ? 1.f : -1.f, zk, zq);
                    sA[lv - 1] = mma(zk, zk, sA[lv - 1]);   // (Z Z^T)[i][j]
                    sT[lv - 1] = mma(zk, zq, sT[lv - 1]);   // (Z Zq^T)[j][i] = attn^T
                }
                dg = mma(kf[tt][kb], qf[tt][kb], dg);       // (K Q^T): its diagonal q_i . k_i
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
        lds_barrier();   // A and attn are complete; G is no longer read

        // ---- 3. UT transform T = (I + A)^-1, blocked over 16x16 tiles
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
        lds_barrier();   // T diag(beta) and V are in LDS

        // ---- 5. u = T diag(beta) V as D-tiles (rows = tokens), value tile by value tile
        F tu[4][2];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) tu[tt][kt] = frag_rows<E>(Tu, LDT, 16 * tt, 32 * kt, lane);
#pragma unroll
        for (int nt = 0; nt < VT; ++nt) {
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
        return;
    }

    // ---- 2'. (wavefront 1) levels 5 and 6: the tiles below the diagonal; per
    //          channel block also K~^T, Q~ and X = e^G K (identity products).
    //          Token tiles are taken in pairs (0, 1) and (2, 3): level 5 pairs
    //          the two tiles of a pair, level 6 the first pair with the second.
    f32x4 a10 = zero4(), a32 = zero4(), a20 = zero4(), a21 = zero4(), a30 = zero4(), a31 = zero4();
    f32x4 t10 = zero4(), t32 = zero4(), t20 = zero4(), t21 = zero4(), t30 = zero4(), t31 = zero4();
    F xf[DK / 16][2];
    const F id0 = ident8_frag<E>(0, lane), id1 = ident8_frag<E>(1, lane);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int c = 32 * kb + 8 * gq;
        float gl[8], g6[8];
        g_row8(G, LDG, 63, c, gl);   // the chunk's last token
        g_row8(G, LDG, 31, c, g6);   // level 6's reference token
        F z6lo[2];                   // level 6, tiles 0 and 1 (lower half)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            float g5[8];
            g_row8(G, LDG, 32 * pp + 15, c, g5);   // level 5's reference token of the pair
            F z5k[2], z5q[2], z6k[2], z6q[2], kt_[2], xs[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tt = 2 * pp + h;
                float gi[8];
                g_row8(G, LDG, 16 * tt + n, c, gi);
                level_frags<E, true>(kf[tt][kb], qf[tt][kb], gi, g5, h ? 1.f : -1.f, z5k[h], z5q[h]);
                level_frags<E, true>(kf[tt][kb], qf[tt][kb], gi, g6, pp ? 1.f : -1.f, z6k[h], z6q[h]);
                F qs;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float fk = exp2_raw(gl[j] - gi[j]);   // e^{G_C - G_t}
                    const float fg = exp2_raw(gi[j]);           // e^{G_t}
                    kt_[h][j] = from_f32<E>(to_f32(kf[tt][kb][j]) * fk);
                    xs[h][j] = from_f32<E>(to_f32(kf[tt][kb][j]) * fg);
                    qs[j] = from_f32<E>(to_f32(qf[tt][kb][j]) * fg);
                }
                // I Q~ is Q~^T: two of its tiles stacked over channels are an
                // A-fragment of Q~ (rows = tokens)
                Qf[(tt * KB + kb) * 64 + lane] =
                    frag_from_tiles<E>(mma(id0, qs, zero4()), mma(id1, qs, zero4()));
            }
            // level 5: tile pair (1, 0) or (3, 2)
            if (pp == 0) {
                a10 = mma(z5k[1], z5k[0], a10);
                t10 = mma(z5k[0], z5q[1], t10);
                z6lo[0] = z6k[0];
                z6lo[1] = z6k[1];
            } else {
                a32 = mma(z5k[1], z5k[0], a32);
                t32 = mma(z5k[0], z5q[1], t32);
                // level 6: (2,0), (2,1), (3,0), (3,1)
                a20 = mma(z6k[0], z6lo[0], a20);
                t20 = mma(z6lo[0], z6q[0], t20);
                a21 = mma(z6k[0], z6lo[1], a21);
                t21 = mma(z6lo[1], z6q[0], t21);
                a30 = mma(z6k[1], z6lo[0], a30);
                t30 = mma(z6lo[0], z6q[1], t30);
                a31 = mma(z6k[1], z6lo[1], a31);
                t31 = mma(z6lo[1], z6q[1], t31);
            }
            // K~ I and X I are D-tiles with rows = tokens; the pair's two
            // stacked over tokens are A-fragments of K~^T (rows = channels) and
            // B-fragments of X
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const F& id = hh ? id1 : id0;
                const int ct = 2 * kb + hh;
                Kf[(ct * 2 + pp) * 64 + lane] =
                    frag_from_tiles<E>(mma(kt_[0], id, zero4()), mma(kt_[1], id, zero4()));
                xf[ct][pp] = frag_from_tiles<E>(mma(xs[0], id, zero4()), mma(xs[1], id, zero4()));
            }
        }
    }
    // V (rows = tokens), for its transposes after the barrier
    F vf[4][VB];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int kb = 0; kb < VB; ++kb) vf[tt][kb] = frag_rows8_g<E>(v + tok0 * DV, DV, 16 * tt, 32 * kb, lane, L);
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
    lds_barrier();   // A and attn are complete; G is no longer read

    // ---- 3'. attn = tril(...) as A-fragments (rows i, contraction over j), and
    //          V with tokens as the contraction index into LDS (over G)
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
#pragma unroll
    for (int nt = 0; nt < VT; ++nt) {
        f32x4 d[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) d[tt] = mma(vf[tt][nt >> 1], (nt & 1) ? id1 : id0, zero4());
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) Vl[(nt * 2 + kt) * 64 + lane] = frag_from_tiles<E>(d[2 * kt], d[2 * kt + 1]);
    }
    lds_barrier();   // T diag(beta) and V are in LDS

    // ---- 4. W = T diag(beta) X: W^T tiles (rows = key channels) for each token
    //         tile, stacked over channel tiles = A-fragments of W
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

template <typename E, int DK, int DV, bool VARLEN>
__global__ __launch_bounds__(128) void chunk_prep_kda2_kernel(const E* __restrict__ q,
                                                              const E* __restrict__ k,
                                                              const E* __restrict__ v,
                                                              const E* __restrict__ beta,
                                                              const E* __restrict__ g,
                                                              char* __restrict__ ws, int T,
                                                              int nchunks, HeadMap hm,
                                                              const int2* __restrict__ ctab) {
    __shared__ KdaPrepLds<E, DK, DV> lds;
    const long item = blockIdx.x;
    const long bh = item / nchunks;
    long tok0, tokk;
    int L;
    if constexpr (VARLEN) {
        // packed sequences: item = head * nchunks + global chunk, the chunk's
        // first token and length from the chunk table (length 0: unused slot)
        const int2 e = ctab[item % nchunks];
        if (e.y == 0) return;
        tok0 = tokk = bh * T + e.x;
        L = e.y;
    } else {
        const int t0 = (int)(item % nchunks) * CHUNK;
        tok0 = bh * T + t0;
        tokk = hm.key(bh) * T + t0;
        L = min(CHUNK, T - t0);
    }
    kda_prep2_item<E, DK, DV>(q, k, v, beta, g, ws + item * WsLayout<E, DK, DV>::BYTES, lds, tok0, tokk, L,
                              (int)(threadIdx.x >> 6), (int)(threadIdx.x & 63));
}


template <typename E, int D>
hipError_t launch_kda_prep(const void* q, const void* k, const void* v, const void* beta, const void* g,
                           void* ws, long nitems, int T, int nchunks, HeadMap hm, const void* ctab,
                           hipStream_t st) {
    if (ctab)
        hipLaunchKernelGGL((chunk_prep_kda2_kernel<E, D, D, true>), dim3((unsigned)nitems), dim3(128), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g, (char*)ws, T,
                           nchunks, hm, (const int2*)ctab);
    else
        hipLaunchKernelGGL((chunk_prep_kda2_kernel<E, D, D, false>), dim3((unsigned)nitems), dim3(128), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g, (char*)ws, T,
                           nchunks, hm, (const int2*)nullptr);
    return hipGetLastError();
}

template hipError_t launch_kda_prep<bf16, 64>(const void*, const void*, const void*, const void*, const void*,
                                              void*, long, int, int, HeadMap, const void*, hipStream_t);
template hipError_t launch_kda_prep<bf16, 128>(const void*, const void*, const void*, const void*, const void*,
                                               void*, long, int, int, HeadMap, const void*, hipStream_t);
template hipError_t launch_kda_prep<float, 64>(const void*, const void*, const void*, const void*, const void*,
                                               void*, long, int, int, HeadMap, const void*, hipStream_t);
template hipError_t launch_kda_prep<float, 128>(const void*, const void*, const void*, const void*, const void*,
                                                void*, long, int, int, HeadMap, const void*, hipStream_t);

}  // namespace dn
