// gdr_chunk.hip -- chunked form of the generalized delta rule (fp32), for gfx950.
//
// The transition S_t = (diag(w_t) - (a_t * kr_t) kr_t^T) S_{t-1} + kw_t v_t^T
// (page "DeltaNet: Memory That Edits", section "The generalized delta rule";
// the pages give no chunked form, so it is derived here). Within a chunk of
// C tokens (16, 32 or 64), with G_t the running sum of g = log w (G_{-1} = 0) and
// l = a * kr, the removal read-outs z_s = kr_s^T S_{s-1} obey the unit
// lower-triangular system
//     (I + M) Z = R^ S_0 + N V,
//     M_sj = sum_c kr_sc l_jc e^{G_{s-1,c} - G_{j,c}},  N_sj = (same with kw_j),  j < s,
//     R^_s = kr_s e^{G_{s-1}},
// so Z = Wz S_0 + uz with Wz = T R^, uz = T N V, T = (I + M)^-1. The chunk is
// then the affine map
//     S_C = P S_0 + Sh,   P = diag(e^{G_C}) - L~^T Wz,   Sh = Kw~^T V - L~^T uz,
//     O   = Qp S_0 + Oh,  Qp = Q^ - A_l Wz,            Oh = A_kw V - A_l uz,
// with L~_s = l_s e^{G_C - G_s}, Kw~_s = kw_s e^{G_C - G_s}, Q^_t = q_t e^{G_t} and
// A_x[t][s] = sum_c q_tc x_sc e^{G_{t,c} - G_{s,c}} (s <= t). Every exponent is
// <= 0. A short last chunk is padded with zero inputs and g = 0, which leaves
// every formula exact (padded tokens contribute nothing and decay nothing).
//
// The per-chunk maps are computed by a few kernels over a per-chunk fp32
// workspace (an elementwise pass, the four decay-weighted contractions, the
// triangular inverse, then tiled products on the fp32 matrix cores), and a
// scan applies the maps chunk after chunk, also on the matrix cores.
#include "dn_device.h"
#include "dn_launch.h"

namespace dn {
namespace {

// Chunk lengths this path is built for (template parameter C below).
constexpr bool gdr_chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }

// Per-chunk workspace, in floats, for head size D and chunk length C.
template <int D, int C>
struct GdrWs {
    static constexpr long G = 0;                 // running log-decay [C][D]
    static constexpr long R = G + C * D;         // R^ = kr e^{G_{s-1}}; then Qp (A-fragment order)
    static constexpr long L = R + C * D;         // L~ = a kr e^{G_C - G}
    static constexpr long K = L + C * D;         // Kw~ = kw e^{G_C - G}
    static constexpr long V = K + C * D;         // v (zero-padded)
    static constexpr long W = V + C * D;         // Wz = T R^
    static constexpr long U = W + C * D;         // uz = T N V
    static constexpr long M = U + C * D;         // M [C][C]
    static constexpr long N = M + C * C;         // N
    static constexpr long AK = N + C * C;        // A_kw
    static constexpr long AL = AK + C * C;       // A_l
    static constexpr long T = AL + C * C;        // (I + M)^-1
    static constexpr long P = T + C * C;         // P [D][D] (A-fragment order, see the products)
    static constexpr long SH = P + (long)D * D;  // Sh [D][D] (fragment order, see the products)
    static constexpr long QP = SH + (long)D * D; // Q^ = q e^{G} [C][D]
    static constexpr long OH = QP + C * D;       // Oh [C][D] (fragment order)
    static constexpr long FLOATS = OH + C * D;   // a multiple of 64 floats (256 bytes)
    static_assert(FLOATS % 64 == 0, "256-byte blocks");
};

// ---- 1. elementwise: G, R^, L~, Kw~, V, Q^ (into the Qp slot). A thread
//         owns NG groups of four consecutive channels of one token and issues
//         every input load of its groups before the first is used. g is staged
//         in LDS and summed there over tokens (one thread per channel, the sum
//         in a register); the outputs are then written as 16-byte vectors,
//         reading the running sums from LDS.
template <typename E, int D, int C>
__global__ __launch_bounds__(256) void gdr_elem_kernel(const E* __restrict__ q,
                                                       const E* __restrict__ kw,
                                                       const E* __restrict__ v,
                                                       const E* __restrict__ kr,
                                                       const E* __restrict__ a,
                                                       const E* __restrict__ g,
                                                       float* __restrict__ ws, int T, int nchunks) {
    typedef GdrWs<D, C> Ws;
    typedef typename Vec4<E>::type V4;
    constexpr int G4 = D / 4;              // four-channel groups per token
    constexpr int NG = C * G4 / 256;       // groups per thread
    static_assert(C * G4 % 256 == 0, "whole groups per thread");
    __shared__ __align__(16) float sG[C][D + 4];
    const long item = blockIdx.x;
    const long bh = item / nchunks;
    const int c = (int)(item % nchunks);
    const int L = min(C, T - c * C);
    float* w = ws + item * Ws::FLOATS;
    const long row0 = bh * T + (long)c * C;
    const int tid = threadIdx.x;

    V4 xg[NG], xq[NG], xkw[NG], xkr[NG], xa[NG], xv[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int gi = tid + 256 * k, t = gi / G4, ch = (gi % G4) * 4;
        xg[k] = xq[k] = xkw[k] = xkr[k] = xa[k] = xv[k] = V4{};
        if (t < L) {
            const long i = (row0 + t) * D + ch;
            xg[k] = *reinterpret_cast<const V4*>(g + i);
            xq[k] = *reinterpret_cast<const V4*>(q + i);
            xkw[k] = *reinterpret_cast<const V4*>(kw + i);
            xkr[k] = *reinterpret_cast<const V4*>(kr + i);
            xa[k] = *reinterpret_cast<const V4*>(a + i);
            xv[k] = *reinterpret_cast<const V4*>(v + i);   // d_v == d_k
        }
    }
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int gi = tid + 256 * k, t = gi / G4, ch = (gi % G4) * 4;
        f32x4 x;
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = to_f32(xg[k][u]);
        *reinterpret_cast<f32x4*>(&sG[t][ch]) = x;
    }
    __syncthreads();
    if (tid < D) {
        float Gr = 0.f;
#pragma unroll 8
        for (int t = 0; t < C; ++t) {
            Gr += sG[t][tid];
            sG[t][tid] = Gr;
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int gi = tid + 256 * k, t = gi / G4, ch = (gi % G4) * 4;
        const long e = (long)t * D + ch;
        const f32x4 Gt = *reinterpret_cast<const f32x4*>(&sG[t][ch]);
        const f32x4 Gm = t > 0 ? *reinterpret_cast<const f32x4*>(&sG[t - 1][ch]) : zero4();
        const f32x4 GC = *reinterpret_cast<const f32x4*>(&sG[C - 1][ch]);
        f32x4 oR, oV, oL, oK, oQ;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float dec = __expf(GC[u] - Gt[u]);
            const float krv = to_f32(xkr[k][u]);
            oR[u] = krv * __expf(Gm[u]);
            oV[u] = to_f32(xv[k][u]);
            oL[u] = to_f32(xa[k][u]) * krv * dec;
            oK[u] = to_f32(xkw[k][u]) * dec;
            oQ[u] = to_f32(xq[k][u]) * __expf(Gt[u]);
        }
        *reinterpret_cast<f32x4*>(w + Ws::G + e) = Gt;
        *reinterpret_cast<f32x4*>(w + Ws::R + e) = oR;
        *reinterpret_cast<f32x4*>(w + Ws::V + e) = oV;
        *reinterpret_cast<f32x4*>(w + Ws::L + e) = oL;
        *reinterpret_cast<f32x4*>(w + Ws::K + e) = oK;
        *reinterpret_cast<f32x4*>(w + Ws::QP + e) = oQ;
    }
}

// ---- 2. the decay-weighted contractions M, N (j < s) and A_kw, A_l (j <= s).
//         Tokens fall into sub-blocks of 16. For s in sub-block I and j in an
//         earlier sub-block J, with b = 16 I - 1 (the token before sub-block I)
//         and e = 16 J + 15 (the last token of sub-block J), the decay factors
//         split per channel into three with exponents <= 0:
//             e^{G_{s-1} - G_j} = e^{G_{s-1} - G_b} e^{G_b - G_e} e^{G_e - G_j}
//         (and the same with G_s for the read-out forms). The first depends on
//         the row only, the last on the column only and the middle on (I, J), so
//         these 16 x 16 blocks are products of scaled rows over the channels, run
//         on the fp32 matrix cores: wave w computes one of the four outputs for
//         every pair of sub-blocks. Pairs inside one sub-block keep one
//         exponential per pair and channel on the VALU (a factor through a fixed
//         token could overflow there): thread (sl, jl) of the 16 x 16 grid takes
//         the pair (sl, jl) of the first half of the diagonal blocks when jl < sl
//         and the mirrored pair (15 - sl, 15 - jl) of the second half when jl > sl.
//         The entries j == s (no decay) are dot products per token, summed by the
//         threads that stage the token. The channels are staged in LDS in blocks
//         of 16, the next block's inputs loaded while this one is used.
template <typename E, int D, int C>
__global__ __launch_bounds__(256) void gdr_pairs_kernel(const E* __restrict__ q,
                                                        const E* __restrict__ kw,
                                                        const E* __restrict__ kr,
                                                        const E* __restrict__ a,
                                                        float* __restrict__ ws, int T, int nchunks) {
    typedef GdrWs<D, C> Ws;
    typedef typename Vec4<E>::type V4;
    constexpr int SB = 16, NSB = C / SB, NPAIR = NSB * (NSB - 1) / 2;
    constexpr int CB = 16, LD = CB + 4;          // channels per block; row stride (16-byte aligned)
    constexpr int NDIR = (NSB + 1) / 2;          // diagonal blocks taken by the direct pairs
    constexpr int NLD = C * CB / 4;              // four-channel groups per block
    static_assert(NLD <= 256, "one group per thread");
    __shared__ __align__(16) float sG[C][LD], sKr[C][LD], sL[C][LD], sKw[C][LD];
    __shared__ __align__(16) float sQg[C][LD], sRm[C][LD], sQm[C][LD], sLc[C][LD], sKc[C][LD];
    __shared__ __align__(16) float sDk[NPAIR > 0 ? NPAIR : 1][CB];

    const long item = blockIdx.x;
    const long bh = item / nchunks;
    const int c = (int)(item % nchunks);
    const int L = min(C, T - c * C);
    float* w = ws + item * Ws::FLOATS;
    const long row0 = bh * T + (long)c * C;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;

    // staging role: token lt, channels lc .. lc + 3 of the block
    const int lt = tid / (CB / 4), lc = 4 * (tid % (CB / 4));
    const bool lin = tid < NLD && lt < L;
    const long gi = (row0 + lt) * D + lc;
    V4 rq, rkw, rkr, ra;
    f32x4 rg;
    auto fetch = [&](int c0) {
        if (tid < NLD) {
            rg = *reinterpret_cast<const f32x4*>(w + Ws::G + lt * D + c0 + lc);
            if (lin) {
                rq = *reinterpret_cast<const V4*>(q + gi + c0);
                rkw = *reinterpret_cast<const V4*>(kw + gi + c0);
                rkr = *reinterpret_cast<const V4*>(kr + gi + c0);
                ra = *reinterpret_cast<const V4*>(a + gi + c0);
            }
        }
    };

    // VALU role
    const int sl = tid / SB, jl = tid % SB;
    const bool dgl = sl == jl, mir = jl > sl;
    int prow[NDIR], pcol[NDIR], prm[NDIR];
    bool pok[NDIR];
#pragma unroll
    for (int v = 0; v < NDIR; ++v) {
        int I = mir ? NDIR + v : v;
        pok[v] = !dgl && I < NSB;
        I = min(I, NSB - 1);
        prow[v] = SB * I + (mir ? SB - 1 - sl : sl);
        pcol[v] = SB * I + (mir ? SB - 1 - jl : jl);
        prm[v] = max(prow[v] - 1, 0);
    }
    float m[NDIR], n[NDIR], ak[NDIR], al[NDIR];
#pragma unroll
    for (int v = 0; v < NDIR; ++v) m[v] = n[v] = ak[v] = al[v] = 0.f;
    float dak = 0.f, dal = 0.f;   // A_kw[lt][lt], A_l[lt][lt] (staging role)

    // matrix-core role: wave wv computes M (0), N (1), A_kw (2) or A_l (3)
    const int fr = lane & 15, fg = lane >> 4;
    const float(*Aop)[LD] = wv < 2 ? sRm : sQm;
    const float(*Bop)[LD] = (wv == 0 || wv == 3) ? sLc : sKc;
    f32x4 acc[NPAIR > 0 ? NPAIR : 1];
#pragma unroll
    for (int p = 0; p < NPAIR; ++p) acc[p] = zero4();

    fetch(0);
    for (int c0 = 0; c0 < D; c0 += CB) {
        __syncthreads();   // the previous block's readers are done
        f32x4 xq = zero4(), xkw = zero4(), xkr = zero4(), xl = zero4();
        if (tid < NLD) {
            if (lin) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xq[i] = to_f32(rq[i]);
                    xkw[i] = to_f32(rkw[i]);
                    xkr[i] = to_f32(rkr[i]);
                    xl[i] = to_f32(ra[i]) * xkr[i];
                }
            }
            *reinterpret_cast<f32x4*>(&sG[lt][lc]) = rg;
            *reinterpret_cast<f32x4*>(&sKw[lt][lc]) = xkw;
            *reinterpret_cast<f32x4*>(&sKr[lt][lc]) = xkr;
            *reinterpret_cast<f32x4*>(&sL[lt][lc]) = xl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dak += xq[i] * xkw[i];
                dal += xq[i] * xl[i];
            }
        }
        if (c0 + CB < D) fetch(c0 + CB);
        __syncthreads();
        // scaled rows (exponents <= 0): q e^{g}, and the factors through the sub-block ends
        if (tid < NLD) {
            const int I = lt / SB;
            const f32x4 Gt = *reinterpret_cast<const f32x4*>(&sG[lt][lc]);
            const f32x4 Gm = lt > 0 ? *reinterpret_cast<const f32x4*>(&sG[lt - 1][lc]) : zero4();
            const f32x4 Gb = I > 0 ? *reinterpret_cast<const f32x4*>(&sG[SB * I - 1][lc]) : zero4();
            const f32x4 Ge = *reinterpret_cast<const f32x4*>(&sG[SB * I + SB - 1][lc]);
            f32x4 qg, rm, qm, lcv, kcv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qg[i] = xq[i] * __expf(Gt[i] - Gm[i]);
                rm[i] = xkr[i] * __expf(Gm[i] - Gb[i]);
                qm[i] = xq[i] * __expf(Gt[i] - Gb[i]);
                const float dec = __expf(Ge[i] - Gt[i]);
                lcv[i] = xl[i] * dec;
                kcv[i] = xkw[i] * dec;
            }
            *reinterpret_cast<f32x4*>(&sQg[lt][lc]) = qg;
            *reinterpret_cast<f32x4*>(&sRm[lt][lc]) = rm;
            *reinterpret_cast<f32x4*>(&sQm[lt][lc]) = qm;
            *reinterpret_cast<f32x4*>(&sLc[lt][lc]) = lcv;
            *reinterpret_cast<f32x4*>(&sKc[lt][lc]) = kcv;
        }
        if (NPAIR > 0 && tid < NPAIR * CB) {
            // e^{G_b - G_e} of the pair of sub-blocks (I, J), J < I
            const int p = tid / CB, ch = tid % CB;
            int I = 1, J = p;
            while (J >= I) {
                J -= I;
                ++I;
            }
            sDk[p][ch] = __expf(sG[SB * I - 1][ch] - sG[SB * J + SB - 1][ch]);
        }
        __syncthreads();

        // pairs inside a sub-block
#pragma unroll 1
        for (int c4 = 0; c4 < CB; c4 += 4) {
#pragma unroll
            for (int v = 0; v < NDIR; ++v) {
                const f32x4 gm = *reinterpret_cast<const f32x4*>(&sG[prm[v]][c4]);
                const f32x4 gj = *reinterpret_cast<const f32x4*>(&sG[pcol[v]][c4]);
                const f32x4 xr = *reinterpret_cast<const f32x4*>(&sKr[prow[v]][c4]);
                const f32x4 xg = *reinterpret_cast<const f32x4*>(&sQg[prow[v]][c4]);
                const f32x4 xl = *reinterpret_cast<const f32x4*>(&sL[pcol[v]][c4]);
                const f32x4 xk = *reinterpret_cast<const f32x4*>(&sKw[pcol[v]][c4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = __expf(gm[i] - gj[i]);
                    const float e1 = e * xr[i], e2 = e * xg[i];
                    m[v] += e1 * xl[i];
                    n[v] += e1 * xk[i];
                    ak[v] += e2 * xk[i];
                    al[v] += e2 * xl[i];
                }
            }
        }
        // pairs across sub-blocks: lane (fg, fr) supplies channel 4 fg + i of
        // row fr to the i-th 16 x 16 x 4 product
#pragma unroll
        for (int p = 0, I = 1, J = 0; p < NPAIR; ++p) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(&Aop[SB * I + fr][4 * fg]);
            const f32x4 bv = *reinterpret_cast<const f32x4*>(&Bop[SB * J + fr][4 * fg]) *
                             *reinterpret_cast<const f32x4*>(&sDk[p][4 * fg]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[p] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[i], acc[p], 0, 0, 0);
            if (++J == I) {
                J = 0;
                ++I;
            }
        }
    }

    float* const out[4] = {w + Ws::M, w + Ws::N, w + Ws::AK, w + Ws::AL};
    // diagonal blocks (every entry written: values below the diagonal, zeros above)
#pragma unroll
    for (int v = 0; v < NDIR; ++v) {
        if (pok[v]) {
            const int at = prow[v] * C + pcol[v];
            out[0][at] = m[v];
            out[1][at] = n[v];
            out[2][at] = ak[v];
            out[3][at] = al[v];
        }
    }
    if (mir) {
#pragma unroll
        for (int I = 0; I < NSB; ++I) {
            const int at = (SB * I + sl) * C + SB * I + jl;
            out[0][at] = out[1][at] = out[2][at] = out[3][at] = 0.f;
        }
    }
    // the entries j == s: the four staging threads of token lt hold a quarter
    // of its channels each (adjacent lanes)
#pragma unroll
    for (int off = 1; off < CB / 4; off <<= 1) {
        dak += __shfl_xor(dak, off, WAVE);
        dal += __shfl_xor(dal, off, WAVE);
    }
    if (tid < NLD && lc == 0) {
        const int at = lt * (C + 1);
        out[0][at] = out[1][at] = 0.f;
        out[2][at] = dak;
        out[3][at] = dal;
    }
    // blocks across sub-blocks: the product below the diagonal, zeros above
    float* const o = w + (wv == 0 ? Ws::M : wv == 1 ? Ws::N : wv == 2 ? Ws::AK : Ws::AL);
#pragma unroll
    for (int p = 0, I = 1, J = 0; p < NPAIR; ++p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[(SB * I + 4 * fg + i) * C + SB * J + fr] = acc[p][i];
            o[(SB * J + 4 * fg + i) * C + SB * I + fr] = 0.f;
        }
        if (++J == I) {
            J = 0;
            ++I;
        }
    }
}

// ---- 3. T = (I + M)^-1 by forward substitution; lane j computes column j:
//         T_ij = [i == j] - sum_{m < i} M_im T_mj (M strictly lower, so T_ij = 0 for i < j).
//         The column stays in registers (both loops unrolled); row i of M is read
//         from LDS as 16-byte vectors, the same address in every lane, and the
//         sum is split over four accumulators.
template <int D, int C>
__global__ __launch_bounds__(WAVE) void gdr_tinv_kernel(float* __restrict__ ws) {
    typedef GdrWs<D, C> Ws;
    __shared__ __align__(16) float sM[C][C + 4];
    float* w = ws + (long)blockIdx.x * Ws::FLOATS;
    const int j = threadIdx.x;
    if (j < C) {
        for (int i = 0; i < C; ++i) sM[i][j] = w[Ws::M + i * C + j];
    }
    __syncthreads();
    if (j >= C) return;
    float t[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m4 = 0; m4 < (i & ~3); m4 += 4) {
            const f32x4 mv = *reinterpret_cast<const f32x4*>(&sM[i][m4]);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] += mv[u] * t[m4 + u];
        }
#pragma unroll
        for (int m = i & ~3; m < i; ++m) acc[m & 3] += sM[i][m] * t[m];
        t[i] = (i == j ? 1.f : 0.f) - ((acc[0] + acc[1]) + (acc[2] + acc[3]));
    }
#pragma unroll
    for (int i = 0; i < C; ++i) w[Ws::T + i * C + j] = t[i];
}

// ---- 4. batched fp32 product inside every chunk's workspace:
//         C = sum over one or two terms of alpha op(A) B  (+ beta C)  (+ diag(e^x)),
//         op(A) = A or A^T; op(A) (M x KK), B (KK x N), C (M x N), row-major
//         with the given leading dimensions; x (optional) is a length-M vector
//         whose exponentials are added on the diagonal. With `chain`, the
//         second term's B is the first term's result (M == KK <= 64: the
//         workgroup holds all its rows), kept in LDS. With `tiled` = 1, C is
//         written in the scan's accumulator order: 16 x 16 tiles of 256 floats,
//         tiles row-major, and in a tile lane (g, n) holds rows 4g .. 4g + 3 of
//         column n (ldc = N; beta 0, no diagonal). With `tiled` = 2, C is written
//         in the scan's A-fragment order: blocks of 16 rows x 32 columns (512
//         floats, blocks row-major), in a block first the columns 4g .. 4g + 3 of
//         row r at (16 g + r) * 4, then the columns 16 + 4g .. at 256 + the same
//         (ldc = N). The beta term reads C row-major at offBeta when that is
//         given (a different slot), else C itself. Every product here
//         contracts over the KK tokens of a chunk. A workgroup stages each
//         term's op(A) rows (times alpha) and B columns in LDS (the contraction
//         zero-padded to a multiple of 32) and accumulates a 64 x 64 tile on the
//         fp32 matrix cores: wave w the rows 16w .. 16w + 15 (when they exist:
//         M is a multiple of 16), four 16-column tiles. N is a multiple of 64.
struct GemmTerm {
    long offA;
    int lda, transA;
    long offB;
    int ldb;
    float alpha;
};

template <int KK>
__global__ __launch_bounds__(256) void gdr_gemm_kernel(float* __restrict__ ws, long stride, int M,
                                                       int tm, int tn, GemmTerm t0, GemmTerm t1,
                                                       int nterms, int chain, long offC, int ldc,
                                                       int tiled, float beta, long offDiag,
                                                       long offBeta) {
    constexpr int KP = (KK + 31) / 32 * 32;
    __shared__ __align__(16) float As[64][KP + 4];   // op(A) rows: As[m][k]
    __shared__ float Bs[KP][64 + 1];                 // Bs[k][n]
    // block = (chunk item, output tile row, output tile column)
    const long tiles = (long)tm * tn;
    const long item = blockIdx.x / tiles;
    const int tile = (int)(blockIdx.x % tiles);
    float* w = ws + item * stride;
    float* Cm = w + offC;
    const int m0 = (tile / tn) * 64, n0 = (tile % tn) * 64;
    const int rows = min(64, M - m0);
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int gq = lane >> 4, r = lane & 15;
    const bool active = 16 * wv < rows;
    f32x4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = zero4();

    for (int term = 0; term < nterms; ++term) {
        const GemmTerm t = term == 0 ? t0 : t1;
        const float* A = w + t.offA;
        const float* B = w + t.offB;
        const bool fromAcc = chain && term == 1;
        if (term > 0) __syncthreads();   // the previous term's readers are done
        if (fromAcc) {
            // B = the first term's result: rows 16 wv + 4 gq + i (< M = KK), the
            // other rows keep the zeros staged with the first term
            if (active) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Bs[16 * wv + 4 * gq + i][16 * ct + r] = acc[ct][i];
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) acc[ct] = zero4();
        }
        // 16 bytes per load (every offset and leading dimension is a multiple of
        // 4 floats); rows and contraction indices past the operands read as zero
        for (int e = tid; e < KP * 16; e += 256) {
            const int k = e / 16, c4 = (e % 16) * 4;
            if (!fromAcc) {
                f32x4 bv = zero4();
                if (k < KK) bv = *reinterpret_cast<const f32x4*>(B + (long)k * t.ldb + n0 + c4);
#pragma unroll
                for (int u = 0; u < 4; ++u) Bs[k][c4 + u] = bv[u];
            }
            if (t.transA) {
                // A^T: A is KK x M; columns m0 + c4 .. of A are rows of op(A)
                f32x4 av = zero4();
                if (k < KK && c4 < rows)
                    av = *reinterpret_cast<const f32x4*>(A + (long)k * t.lda + m0 + c4);
#pragma unroll
                for (int u = 0; u < 4; ++u) As[c4 + u][k] = t.alpha * av[u];
            }
        }
        if (!t.transA) {
            for (int e = tid; e < 64 * (KP / 4); e += 256) {
                const int mr = e / (KP / 4), k4 = (e % (KP / 4)) * 4;
                f32x4 av = zero4();
                if (mr < rows && k4 < KK)
                    av = *reinterpret_cast<const f32x4*>(A + (long)(m0 + mr) * t.lda + k4);
                *reinterpret_cast<f32x4*>(&As[mr][k4]) = t.alpha * av;
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int kb = 0; kb < KP / 32; ++kb) {
                f32x8 af;   // row 16 wv + r at contraction indices 4gq .. 4gq + 3, 16 + 4gq .. 16 + 4gq + 3
                const f32x4 lo4 = *reinterpret_cast<const f32x4*>(&As[16 * wv + r][32 * kb + 4 * gq]);
                const f32x4 hi4 = *reinterpret_cast<const f32x4*>(&As[16 * wv + r][32 * kb + 16 + 4 * gq]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    af[j] = lo4[j];
                    af[4 + j] = hi4[j];
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    f32x8 bf;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        bf[j] = Bs[32 * kb + (j < 4 ? 4 * gq + j : 16 + 4 * gq + j - 4)][16 * ct + r];
                    acc[ct] = mma(af, bf, acc[ct]);
                }
            }
        }
    }
    if (!active) return;
    if (tiled == 2) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + 16 * wv + 4 * gq + i, col = n0 + 16 * ct + r;
                float val = acc[ct][i];
                if (beta != 0.f) val += beta * w[offBeta + (long)row * ldc + col];
                if (offDiag >= 0 && row == col) val += __expf(w[offDiag + row]);
                const int c = col & 31;
                const long off = ((long)(row >> 4) * (ldc >> 5) + (col >> 5)) * 512 + (c >> 4) * 256 +
                                 (((c & 15) >> 2) * 16 + (row & 15)) * 4 + (c & 3);
                Cm[off] = val;
            }
        return;
    }
    if (tiled) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const long tile = (long)((m0 >> 4) + wv) * (ldc >> 4) + (n0 >> 4) + ct;
            *reinterpret_cast<f32x4*>(Cm + tile * 256 + (gq * 16 + r) * 4) = acc[ct];
        }
        return;
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + 16 * wv + 4 * gq + i, col = n0 + 16 * ct + r;
            float* dst = Cm + (long)row * ldc + col;
            float val = acc[ct][i];
            if (beta != 0.f) val += beta * (offBeta >= 0 ? w[offBeta + (long)row * ldc + col] : *dst);
            if (offDiag >= 0 && row == col) val += __expf(w[offDiag + row]);
            *dst = val;
        }
}

// ---- 5. the scan: one workgroup (four wavefronts) per (head, 16 value
//         columns) applies the maps chunk after chunk on the fp32 matrix cores
//         (the fragment convention of dn_device.h). Wave w owns S rows
//         32w .. 32w + 31 (d = 128; 16w .. 16w + 15 at d = 64) and read-out rows
//         16w .. 16w + 15 (those below C) as 16 x 16 accumulator tiles. Per chunk: the A-fragments
//         of P and Qp are loaded straight from the workspace (they do not depend
//         on S), two chunks ahead; S goes through LDS once to become B-fragments,
//         and S <- P S + Sh, O = Qp S + Oh accumulate from the Sh and Oh tiles.
//         When the number of heads is a multiple of 8, the column tiles of a head
//         run on one XCD (workgroup b is dealt to XCD b mod 8) and share its L2.
template <int D, int C>
struct GdrScanOps {
    static constexpr int RTW = D / 64;   // 16-row tiles of S per wavefront
    static constexpr int KB = D / 32;    // 32-wide blocks of the contraction over key channels
    f32x8 pa[RTW][KB], qa[KB];           // A-fragments of P and Qp
    f32x4 sh[RTW], oh;                   // this wavefront's tiles of Sh and Oh
};

template <int D, int C>
__device__ __forceinline__ void gdr_scan_load(GdrScanOps<D, C>& x, const float* __restrict__ wc,
                                              int vt, int w, int gq, int r, bool orw) {
    typedef GdrWs<D, C> Ws;
    typedef GdrScanOps<D, C> O;
    // lane (gq, r) holds row r of the tile at contraction indices 4gq .. 4gq + 3
    // and 16 + 4gq .. 16 + 4gq + 3 of each 32-block
#pragma unroll
    for (int kb = 0; kb < O::KB; ++kb) {
#pragma unroll
        for (int rt = 0; rt < O::RTW; ++rt) {
            // P is stored in A-fragment order: 1 KiB of lo values, then 1 KiB of hi
            const float* src = wc + Ws::P + ((long)(O::RTW * w + rt) * (D / 32) + kb) * 512 + (gq * 16 + r) * 4;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 256);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x.pa[rt][kb][j] = lo[j];
                x.pa[rt][kb][4 + j] = hi[j];
            }
        }
        // Qp in A-fragment order in the slot of R^ (read-out rows exist for the
        // first C / 16 wavefronts; the others read rows 0 .. 15, whose products
        // they never store)
        const float* src = wc + Ws::R + ((long)(orw ? w : 0) * (D / 32) + kb) * 512 + (gq * 16 + r) * 4;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 256);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x.qa[kb][j] = lo[j];
            x.qa[kb][4 + j] = hi[j];
        }
    }
    // Sh and Oh are stored in fragment order: one 16-byte load per tile
    const int fo = (gq * 16 + r) * 4;
#pragma unroll
    for (int rt = 0; rt < O::RTW; ++rt)
        x.sh[rt] = *reinterpret_cast<const f32x4*>(wc + Ws::SH + ((long)(O::RTW * w + rt) * (D / 16) + vt) * 256 + fo);
    x.oh = *reinterpret_cast<const f32x4*>(wc + Ws::OH + ((long)(orw ? w : 0) * (D / 16) + vt) * 256 + fo);
}

// One element stored through a buffer resource (0x00020000: the gfx9 word for
// untyped 32-bit-element buffers). The hardware drops a store whose byte
// offset is at or past the resource's size, so a store that must not happen
// needs no branch; with every store unconditional the compiler knows how many
// are in flight and can wait for the loads issued before them alone.
template <typename E>
__device__ __forceinline__ void store_ranged(E* base, unsigned bytes, unsigned voff, float x) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
    if constexpr (sizeof(E) == 2) {
        const E h = from_f32<E>(x);
        unsigned short u;
        __builtin_memcpy(&u, &h, 2);
        __builtin_amdgcn_raw_buffer_store_b16(u, rs, (int)voff, 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, (int)voff, 0, 0);
    }
}

template <typename E, int D, int C>
__global__ __launch_bounds__(256) void gdr_chunk_scan_kernel(const float* __restrict__ ws,
                                                             const float* S0, E* __restrict__ o,
                                                             float* S_final, int T, int nchunks) {
    typedef GdrWs<D, C> Ws;
    typedef GdrScanOps<D, C> O;
    constexpr int NT = D / 16;      // 16-column tiles per head
    constexpr int RTW = O::RTW, KB = O::KB;
    __shared__ float sS[D][16 + 1];
    const long b = blockIdx.x, heads = gridDim.x / NT;
    long bh;
    int vt;
    if (heads % 8 == 0) {
        bh = b % 8 + 8 * ((b / 8) / NT);
        vt = (int)((b / 8) % NT);
    } else {
        bh = b / NT;
        vt = (int)(b % NT);
    }
    const int n0 = 16 * vt;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int gq = lane >> 4, r = lane & 15;
    const bool ORW = 16 * w < C;   // this wavefront holds read-out rows

    f32x4 S[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const long row = 16 * (RTW * w + rt) + 4 * gq + i;
            S[rt][i] = S0 ? S0[(bh * D + row) * D + n0 + r] : 0.f;
        }

    const float* wh = ws + bh * nchunks * Ws::FLOATS;
    // Three register sets rotate: the maps of chunk c + 2 load while chunk c is
    // applied. The steps are unrolled by three with no exit between them; the
    // steps past the last chunk load that chunk again, store nothing and keep S.
    auto step = [&](int c, const O& cur) {
        const bool valid = c < nchunks;
        const int L = valid ? min(C, T - c * C) : 0;
        __syncthreads();   // every B-fragment read of the previous S is done
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sS[16 * (RTW * w + rt) + 4 * gq + i][r] = S[rt][i];
        __syncthreads();
        f32x4 sn[RTW], oa = cur.oh;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) sn[rt] = cur.sh[rt];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x8 sb;   // B-fragment: column r of the tile at the same contraction indices
#pragma unroll
            for (int j = 0; j < 8; ++j) sb[j] = sS[32 * kb + (j < 4 ? 4 * gq + j : 16 + 4 * gq + j - 4)][r];
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) sn[rt] = mma(cur.pa[rt][kb], sb, sn[rt]);
            oa = mma(cur.qa[kb], sb, oa);
        }
        // rows t >= L of the last chunk, the rows of wavefronts without read-out
        // rows and every row of a step past the end fall outside the resource
        E* const oc = o + (bh * T + (long)c * C) * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * w + 4 * gq + i;
            const unsigned off = ORW ? (unsigned)((t * D + n0 + r) * (int)sizeof(E)) : 0x40000000u;
            store_ranged<E>(oc, (unsigned)(L * D * (int)sizeof(E)), off, oa[i]);
        }
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) S[rt] = valid ? sn[rt] : S[rt];
    };
    const int last = nchunks - 1;
    auto load = [&](O& x, int c) {
        gdr_scan_load<D, C>(x, wh + (long)min(c, last) * Ws::FLOATS, vt, w, gq, r, ORW);
    };
    O s0, s1, s2;
    load(s0, 0);
    load(s1, 1);
    for (int c = 0; c < nchunks; c += 3) {
        load(s2, c + 2);
        step(c, s0);
        load(s0, c + 3);
        step(c + 1, s1);
        load(s1, c + 4);
        step(c + 2, s2);
    }
    if (S_final) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long row = 16 * (RTW * w + rt) + 4 * gq + i;
                S_final[(bh * D + row) * D + n0 + r] = S[rt][i];
            }
    }
}

template <int D, int C>
hipError_t gemm(float* ws, long items, int M, int N, GemmTerm t0, const GemmTerm* t1, long offC,
                int ldc, float beta, long offDiag, hipStream_t st, bool chain = false,
                int tiled = 0, long offBeta = -1) {
    if (M % 16 || N % 64) return hipErrorInvalidValue;
    if (chain && (!t1 || M != C || M > 64)) return hipErrorInvalidValue;
    if (tiled && (ldc != N || (tiled == 1 && (beta != 0.f || offDiag >= 0)))) return hipErrorInvalidValue;
    if (tiled == 2 && beta != 0.f && offBeta < 0) return hipErrorInvalidValue;   // in place would race
    const int tm = (M + 63) / 64, tn = N / 64;
    gdr_gemm_kernel<C><<<(unsigned)(items * tm * tn), 256, 0, st>>>(
        ws, GdrWs<D, C>::FLOATS, M, tm, tn, t0, t1 ? *t1 : t0, t1 ? 2 : 1, chain ? 1 : 0, offC, ldc,
        tiled, beta, offDiag, offBeta);
    return hipGetLastError();
}

template <typename E, int D, int C>
hipError_t gdr_chunk_t(const void* q, const void* kw, const void* v, const void* kr,
                       const void* a, const void* g, const float* S0, void* o, float* S_final,
                       void* wsv, int BH, int T, hipStream_t st) {
    typedef GdrWs<D, C> Ws;
    if (T <= 0 || BH <= 0) return hipErrorInvalidValue;   // the scan assumes at least one chunk
    const int nchunks = (T + C - 1) / C;
    const long items = (long)BH * nchunks;
    float* ws = static_cast<float*>(wsv);
    hipError_t e;
    gdr_elem_kernel<E, D, C><<<(unsigned)items, 256, 0, st>>>(
        (const E*)q, (const E*)kw, (const E*)v, (const E*)kr, (const E*)a, (const E*)g, ws, T, nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gdr_pairs_kernel<E, D, C><<<(unsigned)items, 256, 0, st>>>((const E*)q, (const E*)kw, (const E*)kr,
                                                               (const E*)a, ws, T, nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gdr_tinv_kernel<D, C><<<(unsigned)items, C, 0, st>>>(ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // Wz = T R^, uz = T (N V)                             (C x D each)
    const GemmTerm tWz{Ws::T, C, 0, Ws::R, D, 1.f}, tNV{Ws::N, C, 0, Ws::V, D, 1.f};
    const GemmTerm tuz{Ws::T, C, 0, 0, 0, 1.f};   // B: the result of tNV
    if ((e = gemm<D, C>(ws, items, C, D, tWz, nullptr, Ws::W, D, 0.f, -1, st))) return e;
    if ((e = gemm<D, C>(ws, items, C, D, tNV, &tuz, Ws::U, D, 0.f, -1, st, true))) return e;
    // P = diag(e^{G_C}) - L~^T Wz;  Sh = Kw~^T V - L~^T uz  (D x D)
    const GemmTerm tP{Ws::L, D, 1, Ws::W, D, -1.f};
    const GemmTerm tSh0{Ws::K, D, 1, Ws::V, D, 1.f}, tSh1{Ws::L, D, 1, Ws::U, D, -1.f};
    if ((e = gemm<D, C>(ws, items, D, D, tP, nullptr, Ws::P, D, 0.f, Ws::G + (long)(C - 1) * D, st,
                        false, 2)))
        return e;
    if ((e = gemm<D, C>(ws, items, D, D, tSh0, &tSh1, Ws::SH, D, 0.f, -1, st, false, 1))) return e;
    // Qp = Q^ - A_l Wz, in the scan's fragment order into the slot of R^ (no
    // longer needed once Wz is formed);  Oh = A_kw V - A_l uz   (C x D)
    const GemmTerm tQp{Ws::AL, C, 0, Ws::W, D, -1.f};
    const GemmTerm tOh0{Ws::AK, C, 0, Ws::V, D, 1.f}, tOh1{Ws::AL, C, 0, Ws::U, D, -1.f};
    if ((e = gemm<D, C>(ws, items, C, D, tQp, nullptr, Ws::R, D, 1.f, -1, st, false, 2, Ws::QP))) return e;
    if ((e = gemm<D, C>(ws, items, C, D, tOh0, &tOh1, Ws::OH, D, 0.f, -1, st, false, 1))) return e;
    gdr_chunk_scan_kernel<E, D, C><<<(unsigned)((long)BH * (D / 16)), 256, 0, st>>>(
        ws, S0, (E*)o, S_final, T, nchunks);
    return hipGetLastError();
}

template <typename E, int D>
hipError_t gdr_chunk_c(int chunk, const void* q, const void* kw, const void* v, const void* kr,
                       const void* a, const void* g, const float* S0, void* o, float* S_final,
                       void* ws, int BH, int T, hipStream_t st) {
    if (chunk == 16) return gdr_chunk_t<E, D, 16>(q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st);
    if (chunk == 32) return gdr_chunk_t<E, D, 32>(q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st);
    return gdr_chunk_t<E, D, 64>(q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st);
}

template <int D>
long ws_floats(int chunk) {
    return chunk == 16 ? GdrWs<D, 16>::FLOATS : chunk == 32 ? GdrWs<D, 32>::FLOATS : GdrWs<D, 64>::FLOATS;
}

}  // namespace

size_t gdr_chunk_workspace_bytes(long long BH, long long T, int d, int chunk) {
    if (!gdr_chunk_ok(chunk)) return 0;
    const long long nchunks = (T + chunk - 1) / chunk;
    const long long per = d == 128 ? ws_floats<128>(chunk) : ws_floats<64>(chunk);
    return (size_t)(BH * nchunks * per * 4);
}

hipError_t launch_gdr_chunk(int dtype, const void* q, const void* kw, const void* v,
                            const void* kr, const void* a, const void* g, const float* S0,
                            void* o, float* S_final, void* ws, int BH, int T, int d, int chunk,
                            hipStream_t st) {
    if (!gdr_chunk_ok(chunk)) return hipErrorNotSupported;
    if (dtype == DT_BF16)
        return d == 128 ? gdr_chunk_c<bf16, 128>(chunk, q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st)
                        : gdr_chunk_c<bf16, 64>(chunk, q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st);
    return d == 128 ? gdr_chunk_c<float, 128>(chunk, q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st)
                    : gdr_chunk_c<float, 64>(chunk, q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st);
}

}  // namespace dn
