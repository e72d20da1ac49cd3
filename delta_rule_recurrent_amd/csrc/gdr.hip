// gdr.hip -- the generalized delta rule, token by token, for gfx950.
//
// Page "DeltaNet: Memory That Edits", section "The generalized delta rule": the
// transition separates the roles the delta rule ties together,
//     S_t = (diag(w_t) - (a_t * kr_t) kr_t^T) S_{t-1} + kw_t v_t^T,   o_t = S_t^T q_t,
// with a per-key-channel decay w_t = exp(g_t), a removal key kr_t, a write key
// kw_t and a per-channel removal rate a_t (a diagonal-plus-low-rank key-space
// transition). The state is d_k x d_v fp32, rows = key channels.
//
// One wavefront per (sequence, head, 64 value columns): lane j carries column j
// of the state (d_k values) in registers through all tokens. Every term of the
// update is local to the column: p_j = kr . S[:, j] (before the decay), then
// S[:, j] = w * S[:, j] - (a * kr) p_j + kw v_j and o_j = q . S[:, j]. The
// per-channel vectors of a token are spread over the lanes and broadcast with
// readlane; the next four tokens' inputs are kept in flight. A single token
// takes gdr_step_kernel below, which streams the state once.
#include "dn_device.h"
#include "dn_launch.h"

namespace dn {
namespace {

template <int DK>
struct GdrIn {
    // lane holds entries lane + 64 m of the key-channel vectors, as loaded
    float q[DK / WAVE], kw[DK / WAVE], kr[DK / WAVE], a[DK / WAVE], g[DK / WAVE];
    float v;
};

template <typename E, int DK, int DV>
__device__ __forceinline__ void gdr_load(GdrIn<DK>& x, const E* __restrict__ q,
                                         const E* __restrict__ kw, const E* __restrict__ v,
                                         const E* __restrict__ kr, const E* __restrict__ a,
                                         const E* __restrict__ g, long bh, int t, int T, int col,
                                         int lane) {
    if (t < T) {
        const long tok = bh * T + t;
#pragma unroll
        for (int m = 0; m < DK / WAVE; ++m) {
            const long i = tok * DK + lane + WAVE * m;
            x.q[m] = to_f32(q[i]);
            x.kw[m] = to_f32(kw[i]);
            x.kr[m] = to_f32(kr[i]);
            x.a[m] = to_f32(a[i]);
            x.g[m] = to_f32(g[i]);
        }
        x.v = to_f32(v[tok * DV + col]);
    }
}

// S0 and S_final may be the same buffer: each lane reads its column before the
// first token and writes it after the last.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(WAVE) void gdr_recurrent_kernel(
    const E* __restrict__ q, const E* __restrict__ kw, const E* __restrict__ v,
    const E* __restrict__ kr, const E* __restrict__ a, const E* __restrict__ g, const float* S0,
    E* __restrict__ o, float* S_final, int T) {
    constexpr int NS = DV / WAVE;
    constexpr int KPL = DK / WAVE;
    constexpr int RING = 4;
    const long bh = blockIdx.x / NS;
    const int lane = threadIdx.x;
    const int col = (int)(blockIdx.x % NS) * WAVE + lane;

    float s[DK];
#pragma unroll
    for (int r = 0; r < DK; ++r) s[r] = S0 ? S0[(bh * DK + r) * DV + col] : 0.f;

    GdrIn<DK> ring[RING];
#pragma unroll
    for (int u = 0; u < RING; ++u) gdr_load<E, DK, DV>(ring[u], q, kw, v, kr, a, g, bh, u, T, col, lane);

    for (int t0 = 0; t0 < T; t0 += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            const int t = t0 + u;
            if (t < T) {
                const GdrIn<DK>& x = ring[u];
                float ak[KPL], w[KPL];
#pragma unroll
                for (int m = 0; m < KPL; ++m) {
                    ak[m] = x.a[m] * x.kr[m];
                    w[m] = __expf(x.g[m]);
                }
                float p = 0.f;   // kr^T S_{t-1}, this column
#pragma unroll
                for (int r = 0; r < DK; ++r) p += readlane_f(x.kr[r / WAVE], r % WAVE) * s[r];
#pragma unroll
                for (int r = 0; r < DK; ++r)
                    s[r] = readlane_f(w[r / WAVE], r % WAVE) * s[r] -
                           readlane_f(ak[r / WAVE], r % WAVE) * p +
                           readlane_f(x.kw[r / WAVE], r % WAVE) * x.v;
                float out = 0.f;
#pragma unroll
                for (int r = 0; r < DK; ++r) out += readlane_f(x.q[r / WAVE], r % WAVE) * s[r];
                o[(bh * T + t) * DV + col] = from_f32<E>(out);
            }
            gdr_load<E, DK, DV>(ring[u], q, kw, v, kr, a, g, bh, t + RING, T, col, lane);
        }
    }
    if (S_final) {
#pragma unroll
        for (int r = 0; r < DK; ++r) S_final[(bh * DK + r) * DV + col] = s[r];
    }
}

// ---------------------------------------------------------------------------
// One token (decode). HBM-bound, so every state element is read once and
// written once: NSPLIT 256-thread workgroups per (sequence, head), each over
// DV/NSPLIT value columns; thread t owns a column quad on rows rg, rg + RG, ...
// The read-out is formed from the old state,
//     o = (q * w)^T S - (q . (a * kr)) p + (q . kw) v,   p = kr^T S,
// so the column sums p and (q * w)^T S and the two scalars are reduced across
// row groups (lane shuffles, then one LDS exchange) before the update is
// written. S0 NULL reads zeros; S_final NULL writes nothing; S_final == S0 is
// safe (each thread reads its elements before writing them).
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, int NSPLIT>
__global__ __launch_bounds__(256) void gdr_step_kernel(
    const E* __restrict__ q, const E* __restrict__ kw, const E* __restrict__ v,
    const E* __restrict__ kr, const E* __restrict__ a, const E* __restrict__ g, const float* S0,
    E* __restrict__ o, float* S_final) {
    constexpr int CW = DV / NSPLIT;   // value columns of this workgroup
    constexpr int CQ = CW / 4;        // column quads per row
    constexpr int RG = 256 / CQ;      // row groups
    constexpr int RPT = DK / RG;      // rows per thread
    static_assert(DK % RG == 0 && CQ <= WAVE, "unsupported head size");
    typedef typename Vec4<E>::type V4;

    const long bh = blockIdx.x / NSPLIT;
    const int col0 = (int)(blockIdx.x % NSPLIT) * CW;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const int cq = t % CQ, rg = t / CQ;
    const long base = bh * DK * DV + col0 + 4 * cq;

    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = S0 ? *reinterpret_cast<const f32x4*>(S0 + base + (rg + RG * i) * DV) : zero4();

    __shared__ float skr[DK], sak[DK], sw[DK], skw[DK], sq[DK], sqw[DK];
    __shared__ f32x4 red_p[4][CQ], red_r[4][CQ];
    __shared__ float red_s[4][2];
    if (t < DK) {
        const long i = bh * DK + t;
        const float r_ = to_f32(kr[i]), w_ = __expf(to_f32(g[i])), q_ = to_f32(q[i]);
        skr[t] = r_;
        sak[t] = to_f32(a[i]) * r_;
        sw[t] = w_;
        skw[t] = to_f32(kw[i]);
        sq[t] = q_;
        sqw[t] = q_ * w_;
    }
    const V4 vraw = *reinterpret_cast<const V4*>(v + bh * DV + col0 + 4 * cq);
    __syncthreads();

    f32x4 p = zero4(), r = zero4();
    float qak = 0.f, qkw = 0.f;   // q . (a * kr) and q . kw over this thread's rows
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        p += skr[row] * s[i];
        r += sqw[row] * s[i];
        qak += sq[row] * sak[row];
        qkw += sq[row] * skw[row];
    }
    // Row groups inside one wavefront differ in lane bits >= log2(CQ).
#pragma unroll
    for (int off = CQ; off < WAVE; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] += __shfl_xor(p[e], off, WAVE);
            r[e] += __shfl_xor(r[e], off, WAVE);
        }
        qak += __shfl_xor(qak, off, WAVE);
        qkw += __shfl_xor(qkw, off, WAVE);
    }
    if (lane < CQ) {
        red_p[w][lane] = p;
        red_r[w][lane] = r;
    }
    if (lane == 0) {
        red_s[w][0] = qak;
        red_s[w][1] = qkw;
    }
    __syncthreads();
    p = red_p[0][cq] + red_p[1][cq] + red_p[2][cq] + red_p[3][cq];
    r = red_r[0][cq] + red_r[1][cq] + red_r[2][cq] + red_r[3][cq];
    qak = red_s[0][0] + red_s[1][0] + red_s[2][0] + red_s[3][0];
    qkw = red_s[0][1] + red_s[1][1] + red_s[2][1] + red_s[3][1];

    f32x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = to_f32(vraw[e]);
    if (S_final) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + RG * i;
            *reinterpret_cast<f32x4*>(S_final + base + row * DV) =
                sw[row] * s[i] - sak[row] * p + skw[row] * vv;
        }
    }
    if (rg == 0) {
        const f32x4 ov = r - qak * p + qkw * vv;
        V4 ow;
#pragma unroll
        for (int e = 0; e < 4; ++e) ow[e] = from_f32<E>(ov[e]);
        *reinterpret_cast<V4*>(o + bh * DV + col0 + 4 * cq) = ow;
    }
}

template <typename E, int D>
hipError_t gdr_t(const void* q, const void* kw, const void* v, const void* kr, const void* a,
                 const void* g, const float* S0, void* o, float* S_final, int BH, int T,
                 hipStream_t st) {
    if (T == 1) {
        // four workgroups per state, a quarter of the value columns each
        constexpr int NS = 4;
        gdr_step_kernel<E, D, D, NS><<<(unsigned)((long)BH * NS), 256, 0, st>>>(
            (const E*)q, (const E*)kw, (const E*)v, (const E*)kr, (const E*)a, (const E*)g, S0,
            (E*)o, S_final);
        return hipGetLastError();
    }
    const long blocks = (long)BH * (D / WAVE);
    gdr_recurrent_kernel<E, D, D><<<(unsigned)blocks, WAVE, 0, st>>>(
        (const E*)q, (const E*)kw, (const E*)v, (const E*)kr, (const E*)a, (const E*)g, S0, (E*)o,
        S_final, T);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdr_recurrent(int dtype, const void* q, const void* kw, const void* v,
                                const void* kr, const void* a, const void* g, const float* S0,
                                void* o, float* S_final, int BH, int T, int d, hipStream_t st) {
    if (dtype == DT_BF16)
        return d == 128 ? gdr_t<bf16, 128>(q, kw, v, kr, a, g, S0, o, S_final, BH, T, st)
                        : gdr_t<bf16, 64>(q, kw, v, kr, a, g, S0, o, S_final, BH, T, st);
    return d == 128 ? gdr_t<float, 128>(q, kw, v, kr, a, g, S0, o, S_final, BH, T, st)
                    : gdr_t<float, 64>(q, kw, v, kr, a, g, S0, o, S_final, BH, T, st);
}

}  // namespace dn
