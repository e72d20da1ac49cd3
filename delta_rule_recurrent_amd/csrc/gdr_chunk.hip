// gdr_chunk.hip -- chunked form of the generalized delta rule (fp32), for gfx950.
//
// The transition S_t = (diag(w_t) - (a_t * kr_t) kr_t^T) S_{t-1} + kw_t v_t^T
// (page "DeltaNet: Memory That Edits", section "The generalized delta rule";
// the pages give no chunked form, so it is derived here). Within a chunk of
// C = 64 tokens, with G_t the running sum of g = log w (G_{-1} = 0) and
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
// This path is built for plain correctness and a bounded cost, not speed: the
// per-chunk maps are computed by a few simple kernels over a per-chunk fp32
// workspace (an elementwise pass, the four decay-weighted contractions, the
// triangular inverse, then tiled fp32 products), and a scan applies the maps
// chunk after chunk.
#include "dn_device.h"
#include "dn_launch.h"

namespace dn {
namespace {

constexpr int GC = 64;   // chunk length

// Per-chunk workspace, in floats, for head size D.
template <int D>
struct GdrWs {
    static constexpr long G = 0;                 // running log-decay [C][D]
    static constexpr long R = G + GC * D;        // R^ = kr e^{G_{s-1}}
    static constexpr long L = R + GC * D;        // L~ = a kr e^{G_C - G}
    static constexpr long K = L + GC * D;        // Kw~ = kw e^{G_C - G}
    static constexpr long V = K + GC * D;        // v (zero-padded)
    static constexpr long W = V + GC * D;        // Wz = T R^
    static constexpr long NV = W + GC * D;       // N V
    static constexpr long U = NV + GC * D;       // uz = T N V
    static constexpr long M = U + GC * D;        // M [C][C]
    static constexpr long N = M + GC * GC;       // N
    static constexpr long AK = N + GC * GC;      // A_kw
    static constexpr long AL = AK + GC * GC;     // A_l
    static constexpr long T = AL + GC * GC;      // (I + M)^-1
    static constexpr long P = T + GC * GC;       // P [D][D]
    static constexpr long SH = P + (long)D * D;  // Sh [D][D]
    static constexpr long QP = SH + (long)D * D; // Qp [C][D] (Q^ until the product)
    static constexpr long OH = QP + GC * D;      // Oh [C][D]
    static constexpr long FLOATS = OH + GC * D;  // a multiple of 64 floats (256 bytes)
};

// ---- 1. elementwise: G, R^, L~, Kw~, V, Q^ (into the Qp slot), P = diag(e^{G_C}).
//         g is staged in LDS and summed there over tokens (one thread per
//         channel); every other output is then written by all threads, rows
//         of consecutive channels, reading the running sums from LDS.
template <typename E, int D>
__global__ __launch_bounds__(256) void gdr_elem_kernel(const E* __restrict__ q,
                                                       const E* __restrict__ kw,
                                                       const E* __restrict__ v,
                                                       const E* __restrict__ kr,
                                                       const E* __restrict__ a,
                                                       const E* __restrict__ g,
                                                       float* __restrict__ ws, int T, int nchunks) {
    typedef GdrWs<D> Ws;
    __shared__ float sG[GC][D + 1];
    const long item = blockIdx.x;
    const long bh = item / nchunks;
    const int c = (int)(item % nchunks);
    const int L = min(GC, T - c * GC);
    float* w = ws + item * Ws::FLOATS;
    const long row0 = bh * T + (long)c * GC;
    const int tid = threadIdx.x;
    for (int e = tid; e < GC * D; e += 256) {
        const int t = e / D, ch = e % D;
        sG[t][ch] = t < L ? to_f32(g[(row0 + t) * D + ch]) : 0.f;
    }
    __syncthreads();
    if (tid < D) {
        float Gr = 0.f;
        for (int t = 0; t < GC; ++t) {
            Gr += sG[t][tid];
            sG[t][tid] = Gr;
        }
    }
    __syncthreads();
    for (int e = tid; e < GC * D; e += 256) {
        const int t = e / D, ch = e % D;
        const bool in = t < L;
        const long i = (row0 + t) * D + ch;
        const float Gt = sG[t][ch], Gm = t > 0 ? sG[t - 1][ch] : 0.f, GCh = sG[GC - 1][ch];
        const float dec = __expf(GCh - Gt);
        const float krv = in ? to_f32(kr[i]) : 0.f;
        w[Ws::G + e] = Gt;
        w[Ws::R + e] = krv * __expf(Gm);
        w[Ws::V + e] = in ? to_f32(v[i]) : 0.f;   // d_v == d_k
        w[Ws::L + e] = in ? to_f32(a[i]) * krv * dec : 0.f;
        w[Ws::K + e] = in ? to_f32(kw[i]) * dec : 0.f;
        w[Ws::QP + e] = in ? to_f32(q[i]) * __expf(Gt) : 0.f;
    }
    for (int e = tid; e < D * D; e += 256) {
        const int r = e / D, cc = e % D;
        w[Ws::P + e] = r == cc ? __expf(sG[GC - 1][r]) : 0.f;
    }
}

// ---- 2. the decay-weighted contractions M, N (j < s) and A_kw, A_l (j <= s),
//         over the key channels in blocks of 32 staged in LDS. Thread: row s =
//         tid / 4, columns j = tid % 4 + 4 jj.
template <typename E, int D>
__global__ __launch_bounds__(256) void gdr_pairs_kernel(const E* __restrict__ q,
                                                        const E* __restrict__ kw,
                                                        const E* __restrict__ kr,
                                                        const E* __restrict__ a,
                                                        float* __restrict__ ws, int T, int nchunks) {
    typedef GdrWs<D> Ws;
    constexpr int CB = 32, LD = CB + 1;
    __shared__ float sG[GC][LD], sKr[GC][LD], sL[GC][LD], sKw[GC][LD], sQ[GC][LD];
    const long item = blockIdx.x;
    const long bh = item / nchunks;
    const int c = (int)(item % nchunks);
    const int L = min(GC, T - c * GC);
    float* w = ws + item * Ws::FLOATS;
    const long row0 = bh * T + (long)c * GC;
    const int tid = threadIdx.x;
    const int s = tid >> 2, jg = tid & 3;
    float m[16], n[16], ak[16], al[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) m[jj] = n[jj] = ak[jj] = al[jj] = 0.f;

    for (int c0 = 0; c0 < D; c0 += CB) {
        __syncthreads();   // the previous block's reads are done
        for (int e = tid; e < GC * CB; e += 256) {
            const int t = e / CB, ch = e % CB;
            const bool in = t < L;
            const long i = (row0 + t) * D + c0 + ch;
            sG[t][ch] = w[Ws::G + t * D + c0 + ch];
            const float krv = in ? to_f32(kr[i]) : 0.f;
            sKr[t][ch] = krv;
            sL[t][ch] = in ? to_f32(a[i]) * krv : 0.f;
            sKw[t][ch] = in ? to_f32(kw[i]) : 0.f;
            sQ[t][ch] = in ? to_f32(q[i]) : 0.f;
        }
        __syncthreads();
        for (int ch = 0; ch < CB; ++ch) {
            const float Gs = sG[s][ch], Gm = s > 0 ? sG[s - 1][ch] : 0.f;
            const float krs = sKr[s][ch], qs = sQ[s][ch];
            // e^{G_s - G_j} = e^{G_{s-1} - G_j} e^{g_s}: one exponential per pair
            const float egq = __expf(Gs - Gm) * qs;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int j = jg + 4 * jj;
                const float lj = sL[j][ch], kj = sKw[j][ch];
                if (j < s) {
                    const float e = __expf(Gm - sG[j][ch]);
                    const float e1 = e * krs, e2 = e * egq;
                    m[jj] += e1 * lj;
                    n[jj] += e1 * kj;
                    ak[jj] += e2 * kj;
                    al[jj] += e2 * lj;
                } else if (j == s) {
                    ak[jj] += qs * kj;
                    al[jj] += qs * lj;
                }
            }
        }
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        const int j = jg + 4 * jj;
        w[Ws::M + s * GC + j] = m[jj];
        w[Ws::N + s * GC + j] = n[jj];
        w[Ws::AK + s * GC + j] = ak[jj];
        w[Ws::AL + s * GC + j] = al[jj];
    }
}

// ---- 3. T = (I + M)^-1 by forward substitution; lane j computes column j:
//         T_ij = [i == j] - sum_{m < i} M_im T_mj (M strictly lower, so T_ij = 0 for i < j).
template <int D>
__global__ __launch_bounds__(WAVE) void gdr_tinv_kernel(float* __restrict__ ws) {
    typedef GdrWs<D> Ws;
    __shared__ float sM[GC][GC + 1];
    __shared__ float sT[GC][GC + 1];
    float* w = ws + (long)blockIdx.x * Ws::FLOATS;
    const int j = threadIdx.x;
    for (int i = 0; i < GC; ++i) sM[i][j] = w[Ws::M + i * GC + j];
    __syncthreads();
    for (int i = 0; i < GC; ++i) {
        float acc = 0.f;
        for (int m = 0; m < i; ++m) acc += sM[i][m] * sT[m][j];
        sT[i][j] = (i == j ? 1.f : 0.f) - acc;
    }
    for (int i = 0; i < GC; ++i) w[Ws::T + i * GC + j] = sT[i][j];
}

// ---- 4. batched fp32 product inside every chunk's workspace:
//         C = alpha op(A) B + beta C, op(A) = A or A^T; op(A) (M x 64), B
//         (64 x N), C (M x N), row-major with the given leading dimensions.
//         Every product here contracts over the 64 tokens of a chunk. A
//         workgroup stages its op(A) rows and B columns (64 x 64 each) in LDS
//         and computes a 64 x 64 tile on the fp32 matrix cores: wave w the rows
//         16w .. 16w + 15, four 16-column tiles. M and N are multiples of 64.
__global__ __launch_bounds__(256) void gdr_gemm_kernel(float* __restrict__ ws, long stride, int tm,
                                                       int tn, long offA, int lda, int transA,
                                                       long offB, int ldb, long offC, int ldc,
                                                       float alpha, float beta) {
    constexpr int KK = GC;
    __shared__ __align__(16) float As[64][KK + 4];   // op(A) rows: As[m][k]
    __shared__ float Bs[KK][64 + 1];                 // Bs[k][n]
    // block = (chunk item, output tile row, output tile column)
    const long tiles = (long)tm * tn;
    const long item = blockIdx.x / tiles;
    const int tile = (int)(blockIdx.x % tiles);
    float* w = ws + item * stride;
    const float* A = w + offA;
    const float* B = w + offB;
    float* Cm = w + offC;
    const int m0 = (tile / tn) * 64, n0 = (tile % tn) * 64;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int gq = lane >> 4, r = lane & 15;
    // 16 bytes per load (every offset and leading dimension is a multiple of 4 floats)
    for (int e = tid; e < KK * 16; e += 256) {
        const int hi = e / 16, lo = (e % 16) * 4;
        const f32x4 bv = *reinterpret_cast<const f32x4*>(B + (long)hi * ldb + n0 + lo);
#pragma unroll
        for (int u = 0; u < 4; ++u) Bs[hi][lo + u] = bv[u];
        if (transA) {
            // A^T: columns m0 + lo .. of A are rows of op(A)
            const f32x4 av = *reinterpret_cast<const f32x4*>(A + (long)hi * lda + m0 + lo);
#pragma unroll
            for (int u = 0; u < 4; ++u) As[lo + u][hi] = av[u];
        } else {
            *reinterpret_cast<f32x4*>(&As[hi][lo]) =
                *reinterpret_cast<const f32x4*>(A + (long)(m0 + hi) * lda + lo);
        }
    }
    __syncthreads();
    f32x4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = zero4();
#pragma unroll
    for (int kb = 0; kb < KK / 32; ++kb) {
        f32x8 af;   // row 16 wv + r at contraction indices 4gq .. 4gq + 3, 16 + 4gq .. 16 + 4gq + 3
        const f32x4 lo4 = *reinterpret_cast<const f32x4*>(&As[16 * wv + r][32 * kb + 4 * gq]);
        const f32x4 hi4 = *reinterpret_cast<const f32x4*>(&As[16 * wv + r][32 * kb + 16 + 4 * gq]);
#pragma unroll
        for (int j = 0; j < 4; ++j) { af[j] = lo4[j]; af[4 + j] = hi4[j]; }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            f32x8 bf;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                bf[j] = Bs[32 * kb + (j < 4 ? 4 * gq + j : 16 + 4 * gq + j - 4)][16 * ct + r];
            acc[ct] = mma(af, bf, acc[ct]);
        }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float* dst = Cm + (long)(m0 + 16 * wv + 4 * gq + i) * ldc + n0 + 16 * ct + r;
            *dst = alpha * acc[ct][i] + (beta != 0.f ? beta * *dst : 0.f);
        }
}

// ---- 5. the scan: one workgroup (four wavefronts) per (head, 32 value
//         columns) applies the maps chunk after chunk on the fp32 matrix cores
//         (the fragment convention of dn_device.h). Wave w owns S rows
//         32w .. 32w + 31 (d = 128; 16w .. 16w + 15 at d = 64) and read-out rows
//         16w .. 16w + 15 as 16 x 16 accumulator tiles. Per chunk: the A-fragments
//         of P and Qp are loaded straight from the workspace (they do not depend
//         on S), S goes through LDS once to become B-fragments, and
//         S <- P S + Sh, O = Qp S + Oh accumulate from the Sh and Oh tiles.
template <typename E, int D>
__global__ __launch_bounds__(256) void gdr_chunk_scan_kernel(const float* __restrict__ ws,
                                                             const float* S0, E* __restrict__ o,
                                                             float* S_final, int T, int nchunks) {
    typedef GdrWs<D> Ws;
    constexpr int NB = 32;          // value columns per workgroup (two 16-column tiles)
    constexpr int RTW = D / 64;     // 16-row tiles of S per wavefront
    constexpr int KB = D / 32;      // 32-wide blocks of the contraction over key channels
    __shared__ float sS[D][NB + 1];
    const long bh = blockIdx.x / (D / NB);
    const int n0 = (int)(blockIdx.x % (D / NB)) * NB;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int gq = lane >> 4, r = lane & 15;

    f32x4 S[RTW][2];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long row = 16 * (RTW * w + rt) + 4 * gq + i;
                S[rt][ct][i] = S0 ? S0[(bh * D + row) * D + n0 + 16 * ct + r] : 0.f;
            }

    for (int c = 0; c < nchunks; ++c) {
        const float* wc = ws + (bh * nchunks + c) * Ws::FLOATS;
        const int L = min(GC, T - c * GC);
        // A-fragments: lane (gq, r) holds row r of the tile at contraction
        // indices 4gq .. 4gq + 3 and 16 + 4gq .. 16 + 4gq + 3 of each 32-block
        f32x8 pa[RTW][KB], qa[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
                const float* src = wc + Ws::P + (long)(16 * (RTW * w + rt) + r) * D + 32 * kb + 4 * gq;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
#pragma unroll
                for (int j = 0; j < 4; ++j) { pa[rt][kb][j] = lo[j]; pa[rt][kb][4 + j] = hi[j]; }
            }
            const float* src = wc + Ws::QP + (long)(16 * w + r) * D + 32 * kb + 4 * gq;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) { qa[kb][j] = lo[j]; qa[kb][4 + j] = hi[j]; }
        }
        f32x4 sn[RTW][2], oa[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt)
                    sn[rt][ct][i] = wc[Ws::SH + (long)(16 * (RTW * w + rt) + 4 * gq + i) * D + n0 + 16 * ct + r];
                oa[ct][i] = wc[Ws::OH + (long)(16 * w + 4 * gq + i) * D + n0 + 16 * ct + r];
            }
        }
        __syncthreads();   // every B-fragment read of the previous S is done
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) sS[16 * (RTW * w + rt) + 4 * gq + i][16 * ct + r] = S[rt][ct][i];
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                f32x8 sb;   // B-fragment: column r of the tile at the same contraction indices
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    sb[j] = sS[32 * kb + (j < 4 ? 4 * gq + j : 16 + 4 * gq + j - 4)][16 * ct + r];
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt) sn[rt][ct] = mma(pa[rt][kb], sb, sn[rt][ct]);
                oa[ct] = mma(qa[kb], sb, oa[ct]);
            }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * gq + i;
                if (t < L) o[(bh * T + (long)c * GC + t) * D + n0 + 16 * ct + r] = from_f32<E>(oa[ct][i]);
            }
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) S[rt][ct] = sn[rt][ct];
    }
    if (S_final) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const long row = 16 * (RTW * w + rt) + 4 * gq + i;
                    S_final[(bh * D + row) * D + n0 + 16 * ct + r] = S[rt][ct][i];
                }
    }
}

// (every product contracts over the chunk's 64 tokens: K == GC)
template <int D>
hipError_t gemm(float* ws, long items, int M, int N, int K, long offA, int lda, int transA,
                long offB, int ldb, long offC, int ldc, float alpha, float beta, hipStream_t st) {
    if (K != GC || M % 64 || N % 64) return hipErrorInvalidValue;
    const int tm = M / 64, tn = N / 64;
    gdr_gemm_kernel<<<(unsigned)(items * tm * tn), 256, 0, st>>>(ws, GdrWs<D>::FLOATS, tm, tn,
                                                                 offA, lda, transA, offB, ldb,
                                                                 offC, ldc, alpha, beta);
    return hipGetLastError();
}

template <typename E, int D>
hipError_t gdr_chunk_t(const void* q, const void* kw, const void* v, const void* kr,
                       const void* a, const void* g, const float* S0, void* o, float* S_final,
                       void* wsv, int BH, int T, hipStream_t st) {
    typedef GdrWs<D> Ws;
    const int nchunks = (T + GC - 1) / GC;
    const long items = (long)BH * nchunks;
    float* ws = static_cast<float*>(wsv);
    hipError_t e;
    gdr_elem_kernel<E, D><<<(unsigned)items, 256, 0, st>>>(
        (const E*)q, (const E*)kw, (const E*)v, (const E*)kr, (const E*)a, (const E*)g, ws, T, nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gdr_pairs_kernel<E, D><<<(unsigned)items, 256, 0, st>>>((const E*)q, (const E*)kw, (const E*)kr,
                                                            (const E*)a, ws, T, nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gdr_tinv_kernel<D><<<(unsigned)items, WAVE, 0, st>>>(ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // Wz = T R^, NV = N V, uz = T NV                       (C x D each)
    if ((e = gemm<D>(ws, items, GC, D, GC, Ws::T, GC, 0, Ws::R, D, Ws::W, D, 1.f, 0.f, st))) return e;
    if ((e = gemm<D>(ws, items, GC, D, GC, Ws::N, GC, 0, Ws::V, D, Ws::NV, D, 1.f, 0.f, st))) return e;
    if ((e = gemm<D>(ws, items, GC, D, GC, Ws::T, GC, 0, Ws::NV, D, Ws::U, D, 1.f, 0.f, st))) return e;
    // P = diag(e^{G_C}) - L~^T Wz;  Sh = Kw~^T V - L~^T uz  (D x D)
    if ((e = gemm<D>(ws, items, D, D, GC, Ws::L, D, 1, Ws::W, D, Ws::P, D, -1.f, 1.f, st))) return e;
    if ((e = gemm<D>(ws, items, D, D, GC, Ws::K, D, 1, Ws::V, D, Ws::SH, D, 1.f, 0.f, st))) return e;
    if ((e = gemm<D>(ws, items, D, D, GC, Ws::L, D, 1, Ws::U, D, Ws::SH, D, -1.f, 1.f, st))) return e;
    // Qp = Q^ - A_l Wz;  Oh = A_kw V - A_l uz               (C x D)
    if ((e = gemm<D>(ws, items, GC, D, GC, Ws::AL, GC, 0, Ws::W, D, Ws::QP, D, -1.f, 1.f, st))) return e;
    if ((e = gemm<D>(ws, items, GC, D, GC, Ws::AK, GC, 0, Ws::V, D, Ws::OH, D, 1.f, 0.f, st))) return e;
    if ((e = gemm<D>(ws, items, GC, D, GC, Ws::AL, GC, 0, Ws::U, D, Ws::OH, D, -1.f, 1.f, st))) return e;
    gdr_chunk_scan_kernel<E, D><<<(unsigned)((long)BH * (D / 32)), 256, 0, st>>>(
        ws, S0, (E*)o, S_final, T, nchunks);
    return hipGetLastError();
}

}  // namespace

size_t gdr_chunk_workspace_bytes(long long BH, long long T, int d) {
    const long long nchunks = (T + GC - 1) / GC;
    const long long per = d == 128 ? GdrWs<128>::FLOATS : GdrWs<64>::FLOATS;
    return (size_t)(BH * nchunks * per * 4);
}

hipError_t launch_gdr_chunk(int dtype, const void* q, const void* kw, const void* v,
                            const void* kr, const void* a, const void* g, const float* S0,
                            void* o, float* S_final, void* ws, int BH, int T, int d,
                            hipStream_t st) {
    if (dtype == DT_BF16)
        return d == 128 ? gdr_chunk_t<bf16, 128>(q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st)
                        : gdr_chunk_t<bf16, 64>(q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st);
    return d == 128 ? gdr_chunk_t<float, 128>(q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st)
                    : gdr_chunk_t<float, 64>(q, kw, v, kr, a, g, S0, o, S_final, ws, BH, T, st);
}

}  // namespace dn
