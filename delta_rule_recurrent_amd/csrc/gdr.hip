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
// readlane; the next four tokens' inputs are kept in flight.
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

template <typename E, int D>
hipError_t gdr_t(const void* q, const void* kw, const void* v, const void* kr, const void* a,
                 const void* g, const float* S0, void* o, float* S_final, int BH, int T,
                 hipStream_t st) {
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
