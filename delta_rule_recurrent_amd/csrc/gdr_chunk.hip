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
//         C = alpha op(A) B + beta C, op(A) = A or A^T; A (M x K after op), B
//         (K x N), C (M x N), all row-major with the given leading dimensions.
//         64 x 64 output tile per workgroup, 4 x 4 outputs per thread, the
//         contraction in steps of 16 through LDS. M, N multiples of 64 and K
//         of 16 (checked by the caller).
__global__ __launch_bounds__(256) void gdr_gemm_kernel(float* __restrict__ ws, long stride, int tm,
                                                       int tn, int K, long offA, int lda,
                                                       int transA, long offB, int ldb, long offC,
                                                       int ldc, float alpha, float beta) {
    __shared__ float As[16][64 + 4], Bs[16][64 + 4];
    // block = (chunk item, output tile row, output tile column)
    const long tiles = (long)tm * tn;
    const long item = blockIdx.x / tiles;
    const int tile = (int)(blockIdx.x % tiles);
    float* w = ws + item * stride;
    const float* A = w + offA;
    const float* B = w + offB;
    float* Cm = w + offC;
    const int m0 = (tile / tn) * 64, n0 = (tile % tn) * 64;
    const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        __syncthreads();
        for (int e = tid; e < 16 * 64; e += 256) {
            const int kk = e / 64, mm = e % 64;
            As[kk][mm] = transA ? A[(long)(k0 + kk) * lda + m0 + mm] : A[(long)(m0 + mm) * lda + k0 + kk];
            Bs[kk][mm] = B[(long)(k0 + kk) * ldb + n0 + mm];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = As[kk][tr * 4 + i];
                bv[i] = Bs[kk][tc * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jn = 0; jn < 4; ++jn) acc[i][jn] += av[i] * bv[jn];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
            float* dst = Cm + (long)(m0 + tr * 4 + i) * ldc + n0 + tc * 4 + jn;
            *dst = alpha * acc[i][jn] + (beta != 0.f ? beta * *dst : 0.f);
        }
}

// ---- 5. the scan: one workgroup per (head, 32 value columns) applies the maps
//         chunk after chunk, S (D x 32, fp32) in LDS; each thread reads its rows
//         of P and Qp from memory (cached), which measured faster than staging
//         whole chunks in LDS (the LDS reads of S then bound the step).
template <typename E, int D>
__global__ __launch_bounds__(256) void gdr_chunk_scan_kernel(const float* __restrict__ ws,
                                                             const float* S0, E* __restrict__ o,
                                                             float* S_final, int T, int nchunks) {
    typedef GdrWs<D> Ws;
    constexpr int NB = 32;                 // value columns per workgroup
    constexpr int SPT = D * NB / 256;      // state outputs per thread
    constexpr int OPT = GC * NB / 256;     // read-out outputs per thread
    __shared__ float sS[D][NB + 1];
    const long bh = blockIdx.x / (D / NB);
    const int n0 = (int)(blockIdx.x % (D / NB)) * NB;
    const int tid = threadIdx.x;
    for (int e = tid; e < D * NB; e += 256) {
        const int r = e / NB, cc = e % NB;
        sS[r][cc] = S0 ? S0[(bh * D + r) * D + n0 + cc] : 0.f;
    }
    // thread -> state row ks, columns kn .. kn + SPT - 1; read-out row to, columns on .. on + OPT - 1
    const int ks = tid / (NB / SPT), kn = (tid % (NB / SPT)) * SPT;
    const int to = tid / (NB / OPT), on = (tid % (NB / OPT)) * OPT;
    for (int c = 0; c < nchunks; ++c) {
        const float* w = ws + (bh * nchunks + c) * Ws::FLOATS;
        const int L = min(GC, T - c * GC);
        __syncthreads();   // S of the previous chunk is in LDS
        float so[SPT], oo[OPT];
#pragma unroll
        for (int i = 0; i < SPT; ++i) so[i] = w[Ws::SH + (long)ks * D + n0 + kn + i];
#pragma unroll
        for (int i = 0; i < OPT; ++i) oo[i] = w[Ws::OH + to * D + n0 + on + i];
        for (int m = 0; m < D; ++m) {
            const float p = w[Ws::P + (long)ks * D + m];
            const float qp = w[Ws::QP + to * D + m];
#pragma unroll
            for (int i = 0; i < SPT; ++i) so[i] += p * sS[m][kn + i];
#pragma unroll
            for (int i = 0; i < OPT; ++i) oo[i] += qp * sS[m][on + i];
        }
        if (to < L) {
#pragma unroll
            for (int i = 0; i < OPT; ++i)
                o[(bh * T + (long)c * GC + to) * D + n0 + on + i] = from_f32<E>(oo[i]);
        }
        __syncthreads();   // every read of the old S is done
#pragma unroll
        for (int i = 0; i < SPT; ++i) sS[ks][kn + i] = so[i];
    }
    __syncthreads();
    if (S_final) {
        for (int e = tid; e < D * NB; e += 256) {
            const int r = e / NB, cc = e % NB;
            S_final[(bh * D + r) * D + n0 + cc] = sS[r][cc];
        }
    }
}

// (every product contracts over the chunk's 64 tokens: K == GC)
template <int D>
hipError_t gemm(float* ws, long items, int M, int N, int K, long offA, int lda, int transA,
                long offB, int ldb, long offC, int ldc, float alpha, float beta, hipStream_t st) {
    const int tm = M / 64, tn = N / 64;
    gdr_gemm_kernel<<<(unsigned)(items * tm * tn), 256, 0, st>>>(ws, GdrWs<D>::FLOATS, tm, tn, K,
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
