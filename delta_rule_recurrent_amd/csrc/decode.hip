// decode.hip -- fused single-token decode step and token-by-token recurrence (gfx950).
//
// Per (sequence, head) state S is d_k x d_v fp32, row-major (row = key channel).
// One token: S~ = Diag(alpha) S; p = S~^T k; u = beta (v - p); S = S~ + k u^T;
// o = S^T q (page "28. Linear attention and Gated DeltaNet", section "The
// recurrent form"; page "A walk through of the DeltaNet family of linear
// attention variants", fused recurrent KDA). The selective state-space kind
// drops the correction: u = v, S = alpha S + k v^T (page 28, section "Forget:
// decay").
#include "dn_device.h"
#include "dn_launch.h"

namespace dn {

// ---------------------------------------------------------------------------
// Decode step. HBM-bound: each fp32 state element is read once and written
// once. NSPLIT 256-thread workgroups per (sequence, head), each over DV/NSPLIT
// value columns; thread t owns a column quad (4 consecutive value columns, one
// 16-byte vector per row) on the rows rg, rg + RG, rg + 2RG, ... The column
// sums p = S~^T k and r = S~^T q are reduced across row groups with lane
// shuffles and one LDS exchange, and the read-out uses
// o = S_new^T q = r + u (k . q), so the state is streamed through registers
// exactly once.
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, int KIND, int NSPLIT>
__global__ __launch_bounds__(256) void decode_step_kernel(const E* __restrict__ q,
                                                          const E* __restrict__ k,
                                                          const E* __restrict__ v,
                                                          const E* __restrict__ beta,
                                                          const E* __restrict__ g,
                                                          float* __restrict__ S,
                                                          E* __restrict__ o, HeadMap hm) {
    constexpr int CW = DV / NSPLIT;   // value columns of this workgroup
    constexpr int CQ = CW / 4;        // column quads per row
    constexpr int RG = 256 / CQ;      // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    static_assert(DK % RG == 0 && CQ <= WAVE, "unsupported head size");
    typedef typename Vec4<E>::type V4;

    const long bh = blockIdx.x / NSPLIT;
    const long bk = hm.key(bh);   // q, k row (uniform: computed once, before any load)
    const int col0 = (int)(blockIdx.x % NSPLIT) * CW;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const int cq = t % CQ, rg = t / CQ;

    float* Sp = S + bh * DK * DV + col0 + 4 * cq;
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = *reinterpret_cast<const f32x4*>(Sp + (rg + RG * i) * DV);

    __shared__ float sk[DK], sq[DK], sa[DK];
    __shared__ f32x4 red_p[4][CQ], red_r[4][CQ];
    __shared__ float red_kq[4];
    if (t < DK) {
        sk[t] = to_f32(k[bk * DK + t]);
        sq[t] = to_f32(q[bk * DK + t]);
        if (KIND == KIND_KDA) sa[t] = __expf(to_f32(g[bh * DK + t]));
    }
    const V4 vraw = *reinterpret_cast<const V4*>(v + bh * DV + col0 + 4 * cq);
    const float b = KIND == KIND_SSM ? 1.0f : to_f32(beta[bh]);
    const float a = (KIND == KIND_GATED || KIND == KIND_SSM) ? __expf(to_f32(g[bh])) : 1.0f;
    __syncthreads();

    f32x4 p = zero4(), r = zero4();
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        if (KIND == KIND_KDA) s[i] *= sa[row];
        else if (KIND == KIND_GATED || KIND == KIND_SSM) s[i] *= a;
        p += sk[row] * s[i];
        r += sq[row] * s[i];
        kq += sk[row] * sq[row];
    }
    // Row groups inside one wavefront differ in lane bits >= log2(CQ).
#pragma unroll
    for (int off = CQ; off < WAVE; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] += __shfl_xor(p[e], off, WAVE);
            r[e] += __shfl_xor(r[e], off, WAVE);
        }
        kq += __shfl_xor(kq, off, WAVE);
    }
    if (lane < CQ) {
        red_p[w][lane] = p;
        red_r[w][lane] = r;
    }
    if (lane == 0) red_kq[w] = kq;
    __syncthreads();
    p = red_p[0][cq] + red_p[1][cq] + red_p[2][cq] + red_p[3][cq];
    r = red_r[0][cq] + red_r[1][cq] + red_r[2][cq] + red_r[3][cq];
    kq = red_kq[0] + red_kq[1] + red_kq[2] + red_kq[3];

    f32x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = to_f32(vraw[e]);
    const f32x4 u = KIND == KIND_SSM ? vv : b * (vv - p);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        s[i] += sk[row] * u;
        *reinterpret_cast<f32x4*>(Sp + row * DV) = s[i];
    }
    if (rg == 0) {
        const f32x4 ov = r + u * kq;
        V4 ow;
#pragma unroll
        for (int e = 0; e < 4; ++e) ow[e] = from_f32<E>(ov[e]);
        *reinterpret_cast<V4*>(o + bh * DV + col0 + 4 * cq) = ow;
    }
}

// ---------------------------------------------------------------------------
// Token-by-token recurrence. One wavefront per (sequence, head, 64-column
// slice); lane j carries column j of the state (d_k fp32 values) in registers
// through all T tokens, so p = S~^T k and o = S^T q are lane-local dot
// products and the key/query entries are broadcast with readlane. The inputs
// of the next four tokens are kept in flight (a four-deep register ring).
// ---------------------------------------------------------------------------
template <typename E, int DK, int KIND>
struct TokenIn {
    float k[DK / WAVE], q[DK / WAVE], a[DK / WAVE];
    float v, b, ga;
};

template <typename E, int DK, int DV, int KIND>
__device__ __forceinline__ void token_load(TokenIn<E, DK, KIND>& x, const E* __restrict__ q,
                                           const E* __restrict__ k, const E* __restrict__ v,
                                           const E* __restrict__ beta, const E* __restrict__ g,
                                           long bh, int t, int T, int col, int lane) {
    constexpr int KPL = DK / WAVE;
    if (t < T) {
        const long tok = bh * T + t;
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            x.k[m] = to_f32(k[tok * DK + lane + WAVE * m]);
            x.q[m] = to_f32(q[tok * DK + lane + WAVE * m]);
            x.a[m] = (KIND == KIND_KDA) ? to_f32(g[tok * DK + lane + WAVE * m]) : 0.f;
        }
        x.v = to_f32(v[tok * DV + col]);
        x.b = KIND == KIND_SSM ? 1.f : to_f32(beta[tok]);
        x.ga = (KIND == KIND_GATED || KIND == KIND_SSM) ? to_f32(g[tok]) : 0.f;
    }
}

template <typename E, int DK, int DV, int KIND, bool SNAP = false>
__global__ __launch_bounds__(64) void recurrent_kernel(const E* __restrict__ q,
                                                       const E* __restrict__ k,
                                                       const E* __restrict__ v,
                                                       const E* __restrict__ beta,
                                                       const E* __restrict__ g,
                                                       const float* __restrict__ S0,
                                                       E* __restrict__ o,
                                                       float* __restrict__ S_final, int T,
                                                       float* __restrict__ S_snap) {
    constexpr int NS = DV / WAVE;
    constexpr int KPL = DK / WAVE;
    constexpr int RING = 4;
    const long bh = blockIdx.x / NS;
    const int slice = blockIdx.x % NS;
    const int lane = threadIdx.x;
    const int col = slice * WAVE + lane;

    float s[DK];
#pragma unroll
    for (int r = 0; r < DK; ++r) s[r] = S0 ? S0[(bh * DK + r) * DV + col] : 0.f;

    TokenIn<E, DK, KIND> ring[RING];
#pragma unroll
    for (int u = 0; u < RING; ++u) token_load<E, DK, DV, KIND>(ring[u], q, k, v, beta, g, bh, u, T, col, lane);

    for (int t0 = 0; t0 < T; t0 += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            const int t = t0 + u;
            if (t < T) {
                TokenIn<E, DK, KIND>& x = ring[u];
                if (KIND == KIND_GATED || KIND == KIND_SSM) {
                    const float a = __expf(x.ga);
#pragma unroll
                    for (int r = 0; r < DK; ++r) s[r] *= a;
                } else if (KIND == KIND_KDA) {
                    float ea[KPL];
#pragma unroll
                    for (int m = 0; m < KPL; ++m) ea[m] = __expf(x.a[m]);
#pragma unroll
                    for (int r = 0; r < DK; ++r) s[r] *= readlane_f(ea[r / WAVE], r % WAVE);
                }
                float p = 0.f;
#pragma unroll
                for (int r = 0; r < DK; ++r) p += readlane_f(x.k[r / WAVE], r % WAVE) * s[r];
                const float uu = KIND == KIND_SSM ? x.v : x.b * (x.v - p);
#pragma unroll
                for (int r = 0; r < DK; ++r) s[r] += readlane_f(x.k[r / WAVE], r % WAVE) * uu;
                float out = 0.f;
#pragma unroll
                for (int r = 0; r < DK; ++r) out += readlane_f(x.q[r / WAVE], r % WAVE) * s[r];
                o[(bh * T + t) * DV + col] = from_f32<E>(out);
                if constexpr (SNAP) {
                    // the state after token t, [bh][t][DK][DV]
#pragma unroll
                    for (int r = 0; r < DK; ++r) S_snap[((bh * T + t) * DK + r) * DV + col] = s[r];
                }
            }
            token_load<E, DK, DV, KIND>(ring[u], q, k, v, beta, g, bh, t + RING, T, col, lane);
        }
    }
    if (S_final) {
#pragma unroll
        for (int r = 0; r < DK; ++r) S_final[(bh * DK + r) * DV + col] = s[r];
    }
}

__global__ void state_copy_kernel(const float* __restrict__ S0, float* __restrict__ S_final,
                                  long long n) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) S_final[i] = S0 ? S0[i] : 0.f;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename E, int D>
static hipError_t decode_t(int kind, const void* q, const void* k, const void* v, const void* beta,
                           const void* g, float* S, void* o, int BH, hipStream_t st, HeadMap hm) {
    const E *q_ = (const E*)q, *k_ = (const E*)k, *v_ = (const E*)v, *b_ = (const E*)beta,
            *g_ = (const E*)g;
    E* o_ = (E*)o;
    // four workgroups per state, one quarter of the value columns each (the
    // column sums are independent per column): finer work units keep more of
    // the state stream in flight per CU (measured 80.9 -> 78.6 us per step at
    // 256 x 16 heads, d = 128)
    constexpr int NS = 4;
    dim3 grid((unsigned)((long)BH * NS)), block(256);
    if (kind == KIND_DELTANET)
        hipLaunchKernelGGL((decode_step_kernel<E, D, D, KIND_DELTANET, NS>), grid, block, 0, st, q_, k_, v_, b_, g_, S, o_, hm);
    else if (kind == KIND_GATED)
        hipLaunchKernelGGL((decode_step_kernel<E, D, D, KIND_GATED, NS>), grid, block, 0, st, q_, k_, v_, b_, g_, S, o_, hm);
    else if (kind == KIND_SSM)
        hipLaunchKernelGGL((decode_step_kernel<E, D, D, KIND_SSM, NS>), grid, block, 0, st, q_, k_, v_, b_, g_, S, o_, hm);
    else
        hipLaunchKernelGGL((decode_step_kernel<E, D, D, KIND_KDA, NS>), grid, block, 0, st, q_, k_, v_, b_, g_, S, o_, hm);
    return hipGetLastError();
}

hipError_t launch_decode(int kind, int dtype, const void* q, const void* k, const void* v,
                         const void* beta, const void* g, float* S, void* o, int BH, int dk,
                         int dv, hipStream_t st, HeadMap hm) {
    (void)dv;
    if (dtype == DT_BF16)
        return dk == 128 ? decode_t<bf16, 128>(kind, q, k, v, beta, g, S, o, BH, st, hm)
                         : decode_t<bf16, 64>(kind, q, k, v, beta, g, S, o, BH, st, hm);
    return dk == 128 ? decode_t<float, 128>(kind, q, k, v, beta, g, S, o, BH, st, hm)
                     : decode_t<float, 64>(kind, q, k, v, beta, g, S, o, BH, st, hm);
}

template <typename E, int D, bool SNAP>
static hipError_t recurrent_launch(int kind, const E* q_, const E* k_, const E* v_, const E* b_,
                                   const E* g_, const float* S0, E* o_, float* S_final, int BH,
                                   int T, float* S_snap, hipStream_t st) {
    dim3 grid((unsigned)BH * (D / WAVE)), block(WAVE);
    if (kind == KIND_DELTANET)
        hipLaunchKernelGGL((recurrent_kernel<E, D, D, KIND_DELTANET, SNAP>), grid, block, 0, st, q_, k_, v_, b_, g_, S0, o_, S_final, T, S_snap);
    else if (kind == KIND_GATED)
        hipLaunchKernelGGL((recurrent_kernel<E, D, D, KIND_GATED, SNAP>), grid, block, 0, st, q_, k_, v_, b_, g_, S0, o_, S_final, T, S_snap);
    else if (kind == KIND_SSM)
        hipLaunchKernelGGL((recurrent_kernel<E, D, D, KIND_SSM, SNAP>), grid, block, 0, st, q_, k_, v_, b_, g_, S0, o_, S_final, T, S_snap);
    else
        hipLaunchKernelGGL((recurrent_kernel<E, D, D, KIND_KDA, SNAP>), grid, block, 0, st, q_, k_, v_, b_, g_, S0, o_, S_final, T, S_snap);
    return hipGetLastError();
}

template <typename E, int D>
static hipError_t recurrent_t(int kind, const void* q, const void* k, const void* v,
                              const void* beta, const void* g, const float* S0, void* o,
                              float* S_final, int BH, int T, hipStream_t st, float* S_snap) {
    const E *q_ = (const E*)q, *k_ = (const E*)k, *v_ = (const E*)v, *b_ = (const E*)beta,
            *g_ = (const E*)g;
    if (S_snap) return recurrent_launch<E, D, true>(kind, q_, k_, v_, b_, g_, S0, (E*)o, S_final, BH, T, S_snap, st);
    return recurrent_launch<E, D, false>(kind, q_, k_, v_, b_, g_, S0, (E*)o, S_final, BH, T, nullptr, st);
}

hipError_t launch_recurrent(int kind, int dtype, const void* q, const void* k, const void* v,
                            const void* beta, const void* g, const float* S0, void* o,
                            float* S_final, int BH, int T, int dk, int dv, hipStream_t st,
                            float* S_snap) {
    (void)dv;
    if (dtype == DT_BF16)
        return dk == 128 ? recurrent_t<bf16, 128>(kind, q, k, v, beta, g, S0, o, S_final, BH, T, st, S_snap)
                         : recurrent_t<bf16, 64>(kind, q, k, v, beta, g, S0, o, S_final, BH, T, st, S_snap);
    return dk == 128 ? recurrent_t<float, 128>(kind, q, k, v, beta, g, S0, o, S_final, BH, T, st, S_snap)
                     : recurrent_t<float, 64>(kind, q, k, v, beta, g, S0, o, S_final, BH, T, st, S_snap);
}

hipError_t launch_state_copy(const float* S0, float* S_final, long long n, hipStream_t st) {
    const int block = 256;
    const long long grid = (n + block - 1) / block;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)grid), dim3(block), 0, st, S0, S_final, n);
    return hipGetLastError();
}

}  // namespace dn
