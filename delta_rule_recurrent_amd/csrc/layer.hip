// layer.hip -- the gated layer's work around the rule, as single-pass HBM kernels for gfx950.
//
// Page "28. Linear attention and Gated DeltaNet", section "The full layer": after
// the input projections, the q, k and v channels (token-major, one row of
// C = 2*Hk*dk + Hv*dv channels per token, q then k then v) go through a depthwise
// causal convolution of width 4 over time and SiLU; the channels are split into
// key heads (q, k) and value heads (v); q and k are L2-normalised and q is scaled
// by dk^-1/2; beta = sigmoid(b) and g = -exp(A_log) * softplus(a + dt_bias). After
// the rule, each value head's read-out is RMS-normalised, multiplied by a weight
// vector and by SiLU(z).
//
// All three kernels move every byte once: the prologue reads the projected rows
// and writes the head-major q, k, v that the chunk and decode kernels take; the
// epilogue reads the head-major read-out and z and writes token-major rows for the
// output projection. Arithmetic is fp32 with one rounding to the storage type at
// each output.
#include "dn_device.h"
#include "dn_launch.h"

namespace dn {
namespace {

constexpr int LAYER_WG = 256;   // threads per workgroup of the layer kernels
constexpr int RUN = 8;          // consecutive tokens one lane group convolves in registers
constexpr int CONV_K = 4;       // convolution width (its state: the last 3 inputs)
constexpr int EPI_ROWS = 64;    // rows of the read-out per epilogue workgroup

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

// SiLU with the hardware exp2 and reciprocal (each within 1 ulp): x / (1 + e^-x).
// Large negative x gives e^-x = inf and a zero reciprocal, so the result is -0.
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// 1 / max(sqrt(s), 1e-12) for a sum of squares s >= 0, with the hardware rsqrt.
__device__ __forceinline__ float inv_norm(float s) { return __builtin_amdgcn_rsqf(fmaxf(s, 1e-24f)); }

// Sum over the `width` consecutive lanes that hold one row (width a power of two).
template <int WIDTH>
__device__ __forceinline__ float row_sum(float s) {
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m /= 2) s += __shfl_xor(s, m, WAVE);
    return s;
}

// ---------------------------------------------------------------------------
// Prologue. Grid (ceil(T / (GROUPS*RUN)), 2*Hk + Hv, B), 256 threads. Block y
// picks one head-sized channel segment (q head, k head or v head); D/8 lanes
// (a lane group) hold one token row of it, eight channels per lane, and each
// group convolves RUN consecutive tokens, keeping the last three inputs in
// registers, so every input element is read once (plus a 3-row halo per run).
// The v-segment blocks also compute the gates of their value head.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(LAYER_WG) void layer_prologue_kernel(
    const E* __restrict__ qkv, const E* __restrict__ conv_w, const E* cstate, E* cout,
    const E* __restrict__ bin, const E* __restrict__ ain, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, E* __restrict__ q, E* __restrict__ k, E* __restrict__ v,
    E* __restrict__ beta, E* __restrict__ g, float bscale, int T, int Hk, int Hv) {
    constexpr int LPR = D / 8;
    constexpr int GROUPS = LAYER_WG / LPR;
    constexpr float QSCALE = D == 64 ? 0.125f : 0.08838834764831845f;   // D^-1/2
    const int s = blockIdx.y, b = blockIdx.z;
    const int grp = threadIdx.x / LPR, l = threadIdx.x % LPR;
    const long t0 = (long)blockIdx.x * (GROUPS * RUN) + (long)grp * RUN;
    if (t0 >= T) return;   // whole lane groups leave together; no block barrier follows
    const long C = (long)(2 * Hk + Hv) * D;
    const long c = (long)s * D + l * 8;   // first of this lane's eight channels

    // Filter taps of the eight channels: conv_w [C][4], 32 consecutive elements.
    float w[8][CONV_K];
    {
        float a[8], bb[8], cc[8], dd[8];
        load8(conv_w + c * CONV_K, a);
        load8(conv_w + c * CONV_K + 8, bb);
        load8(conv_w + c * CONV_K + 16, cc);
        load8(conv_w + c * CONV_K + 24, dd);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float* src = i < 2 ? a : i < 4 ? bb : i < 6 ? cc : dd;
            const int o = (i % 2) * 4;
#pragma unroll
            for (int j = 0; j < CONV_K; ++j) w[i][j] = src[o + j];
        }
    }

    // The three inputs before t0: earlier rows of qkv, else the carried state
    // [B][C][3] (oldest first: input t < 0 is state entry 3 + t), else zeros.
    float h[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const long tt = t0 - 3 + j;
        if (tt >= 0) {
            load8(qkv + ((long)b * T + tt) * C + c, h[j]);
        } else if (cstate) {
#pragma unroll
            for (int i = 0; i < 8; ++i) h[j][i] = to_f32(cstate[((long)b * C + c + i) * 3 + 3 + tt]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) h[j][i] = 0.0f;
        }
    }

    // All RUN rows are loaded up front (rows past the end re-read the last one);
    // only the stores are predicated.
    Raw8<E> x[RUN];
#pragma unroll
    for (int r = 0; r < RUN; ++r) {
        const long tt = t0 + r < T ? t0 + r : (long)T - 1;
        load_raw(qkv + ((long)b * T + tt) * C + c, x[r]);
    }

    E* out;
    long head;
    int hs;
    if (s < Hk) { out = q; head = s; hs = Hk; }
    else if (s < 2 * Hk) { out = k; head = s - Hk; hs = Hk; }
    else { out = v; head = s - 2 * Hk; hs = Hv; }
    E* orow = out + (((long)b * hs + head) * T + t0) * D + l * 8;
    const bool is_key = s < 2 * Hk;
    const float qs = s < Hk ? QSCALE : 1.0f;

#pragma unroll
    for (int r = 0; r < RUN; ++r) {
        float y[8];
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float xi = elem(x[r], i);
            const float acc = w[i][0] * h[0][i] + w[i][1] * h[1][i] + w[i][2] * h[2][i] + w[i][3] * xi;
            y[i] = silu(acc);
            ss += y[i] * y[i];
            h[0][i] = h[1][i];
            h[1][i] = h[2][i];
            h[2][i] = xi;
        }
        if (is_key) {
            const float sc = qs * inv_norm(row_sum<LPR>(ss));
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] *= sc;
        }
        if (t0 + r < T) store8(orow + (long)r * D, y);
    }

    // The new convolution state (the last three inputs of each channel) is
    // written by the group of the first run, the only one that reads the old
    // state, after its reads: an in-place update cannot race with them. For
    // T < 3 the oldest entries come from the old state (input t < 0 is entry
    // 3 + t), re-read here by the same lanes.
    if (cout && t0 == 0) {
        float nh[24];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const long tt = (long)T - 3 + j;
            float rv[8];
            if (tt >= 0) {
                load8(qkv + ((long)b * T + tt) * C + c, rv);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    rv[i] = cstate ? to_f32(cstate[((long)b * C + c + i) * 3 + 3 + tt]) : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) nh[3 * i + j] = rv[i];
        }
        const long so = ((long)b * C + c) * 3;
        store8(cout + so, *reinterpret_cast<const float(*)[8]>(nh));
        store8(cout + so + 8, *reinterpret_cast<const float(*)[8]>(nh + 8));
        store8(cout + so + 16, *reinterpret_cast<const float(*)[8]>(nh + 16));
    }

    if (s >= 2 * Hk) {
        const int hv = s - 2 * Hk;
        const float nA = g ? -__expf(A_log[hv]) : 0.0f;
        const float bias = g ? dt_bias[hv] : 0.0f;
        for (int r = l; r < RUN; r += LPR) {
            const long t = t0 + r;
            if (t >= T) break;
            const long src = ((long)b * T + t) * Hv + hv;
            const long dst = ((long)b * Hv + hv) * T + t;
            beta[dst] = from_f32<E>(bscale / (1.0f + __expf(-to_f32(bin[src]))));
            if (g) {
                const float z = to_f32(ain[src]) + bias;
                const float sp = fmaxf(z, 0.0f) + log1pf(__expf(-fabsf(z)));   // softplus
                g[dst] = from_f32<E>(nA * sp);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Prologue of a single token (decode). One lane group per (sequence, segment):
// the group reads its channels' three-entry history and the new input,
// convolves, and writes the shifted history back (to conv_state_out, which may
// be conv_state itself: every lane reads its own 24 entries before writing
// them, and no other lane touches them). Grid ceil(B*(2*Hk + Hv) / GROUPS).
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(LAYER_WG) void layer_prologue_step_kernel(
    const E* __restrict__ qkv, const E* __restrict__ conv_w, const E* cstate, E* cout,
    const E* __restrict__ bin, const E* __restrict__ ain, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, E* __restrict__ q, E* __restrict__ k, E* __restrict__ v,
    E* __restrict__ beta, E* __restrict__ g, float bscale, int B, int Hk, int Hv) {
    constexpr int LPR = D / 8;
    constexpr int GROUPS = LAYER_WG / LPR;
    constexpr float QSCALE = D == 64 ? 0.125f : 0.08838834764831845f;
    const int NS = 2 * Hk + Hv;
    const long gi = (long)blockIdx.x * GROUPS + threadIdx.x / LPR;
    if (gi >= (long)B * NS) return;   // whole lane groups leave together
    const int l = threadIdx.x % LPR;
    const long b = gi / NS;
    const int s = (int)(gi % NS);
    const long C = (long)NS * D;
    const long c = (long)s * D + l * 8;

    Raw8<E> xr, w0, w1, w2, w3, h0, h1, h2;
    load_raw(qkv + b * C + c, xr);
    load_raw(conv_w + c * CONV_K, w0);
    load_raw(conv_w + c * CONV_K + 8, w1);
    load_raw(conv_w + c * CONV_K + 16, w2);
    load_raw(conv_w + c * CONV_K + 24, w3);
    const long so = (b * C + c) * 3;   // this lane's 24 history entries, channel-major
    if (cstate) {
        load_raw(cstate + so, h0);
        load_raw(cstate + so + 8, h1);
        load_raw(cstate + so + 16, h2);
    }
    float y[8], ss = 0.0f;
    float hist[24];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hist[i] = cstate ? elem(h0, i) : 0.0f;
        hist[8 + i] = cstate ? elem(h1, i) : 0.0f;
        hist[16 + i] = cstate ? elem(h2, i) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // channel i: taps conv_w[c+i][0..3] are elements 4i..4i+3 of the 32 loaded
        const Raw8<E>& wr = i < 2 ? w0 : i < 4 ? w1 : i < 6 ? w2 : w3;
        const int o = (i % 2) * 4;
        const float xi = elem(xr, i);
        const float acc = elem(wr, o) * hist[3 * i] + elem(wr, o + 1) * hist[3 * i + 1] +
                          elem(wr, o + 2) * hist[3 * i + 2] + elem(wr, o + 3) * xi;
        y[i] = silu(acc);
        ss += y[i] * y[i];
    }
    if (cout) {
        float nh[24];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            nh[3 * i] = hist[3 * i + 1];
            nh[3 * i + 1] = hist[3 * i + 2];
            nh[3 * i + 2] = elem(xr, i);
        }
        // shifted history of stored values: exact in the storage type
        store8(cout + so, *reinterpret_cast<const float(*)[8]>(nh));
        store8(cout + so + 8, *reinterpret_cast<const float(*)[8]>(nh + 8));
        store8(cout + so + 16, *reinterpret_cast<const float(*)[8]>(nh + 16));
    }
    E* out;
    long row;
    if (s < Hk) { out = q; row = b * Hk + s; }
    else if (s < 2 * Hk) { out = k; row = b * Hk + s - Hk; }
    else { out = v; row = b * Hv + s - 2 * Hk; }
    if (s < 2 * Hk) {
        const float sc = (s < Hk ? QSCALE : 1.0f) * inv_norm(row_sum<LPR>(ss));
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] *= sc;
    }
    store8(out + row * D + l * 8, y);
    if (s >= 2 * Hk && l == 0) {
        const int hv = s - 2 * Hk;
        const long i = b * Hv + hv;   // [B,1,Hv] in, [B,Hv,1] out: the same index
        beta[i] = from_f32<E>(bscale / (1.0f + __expf(-to_f32(bin[i]))));
        if (g) {
            const float z = to_f32(ain[i]) + dt_bias[hv];
            g[i] = from_f32<E>(-__expf(A_log[hv]) * (fmaxf(z, 0.0f) + log1pf(__expf(-fabsf(z)))));
        }
    }
}

// New convolution state for an empty input (T == 0: the old state, or zeros),
// [B][C][3]; written the same way for any T. One thread per (sequence,
// channel); it reads everything it needs before writing, so the new state may
// overwrite the old one.
template <typename E>
__global__ __launch_bounds__(LAYER_WG) void conv_state_kernel(const E* __restrict__ qkv,
                                                              const E* cstate, E* cout, int T,
                                                              long C, long n) {
    const long i = (long)blockIdx.x * LAYER_WG + threadIdx.x;
    if (i >= n) return;
    const long b = i / C, c = i % C;
    E val[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const long tt = (long)T - 3 + j;
        if (tt >= 0) val[j] = qkv[((long)b * T + tt) * C + c];
        else val[j] = cstate ? cstate[i * 3 + 3 + tt] : from_f32<E>(0.0f);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) cout[i * 3 + j] = val[j];
}

// ---------------------------------------------------------------------------
// Epilogue. EPI_ROWS rows of the head-major read-out o [B][Hv][T][D] per workgroup
// (consecutive rows, so a wave reads a contiguous span); D/8 lanes per row.
//   out[b][t][hv*D + c] = w[c] * round(o * rsqrt(mean(o^2) + eps)) * SiLU(z[b][t][hv*D + c])
// with the normalised value rounded to the storage type before the products.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(LAYER_WG) void layer_epilogue_kernel(
    const E* __restrict__ o, const E* __restrict__ z, const E* __restrict__ nw,
    E* __restrict__ out, long rows, int T, int Hv, float eps) {
    constexpr int LPR = D / 8;
    constexpr int GROUPS = LAYER_WG / LPR;
    constexpr int PER = EPI_ROWS / GROUPS;
    const int grp = threadIdx.x / LPR, l = threadIdx.x % LPR;
    const long base = (long)blockIdx.x * EPI_ROWS;
    float wv[8];
    load8(nw + l * 8, wv);

    Raw8<E> ov[PER], zv[PER];
    long zoff[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        long row = base + p * GROUPS + grp;
        if (row >= rows) row = rows - 1;
        const long bh = row / T, t = row % T;
        const long bb = bh / Hv, hv = bh % Hv;
        zoff[p] = ((bb * T + t) * Hv + hv) * D + l * 8;
        load_raw(o + row * D + l * 8, ov[p]);
        load_raw(z + zoff[p], zv[p]);
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += elem(ov[p], i) * elem(ov[p], i);
        ss = row_sum<LPR>(ss);
        const float r = rsqrtf(ss * (1.0f / D) + eps);
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float nrm = to_f32(from_f32<E>(elem(ov[p], i) * r));
            y[i] = wv[i] * nrm * silu(elem(zv[p], i));
        }
        if (base + p * GROUPS + grp < rows) store8(out + zoff[p], y);
    }
}

template <typename E, int D>
hipError_t prologue_launch(const void* qkv, const void* conv_w, const void* cstate,
                           void* cstate_out, const void* b, const void* a, const float* A_log,
                           const float* dt_bias, void* q, void* k, void* v, void* beta, void* g,
                           float bs, int B, int T, int Hk, int Hv, hipStream_t st) {
    const E* x = static_cast<const E*>(qkv);
    const long C = (long)(2 * Hk + Hv) * D;
    if (T == 1) {
        constexpr int GROUPS = LAYER_WG / (D / 8);
        const long groups = (long)B * (2 * Hk + Hv);
        layer_prologue_step_kernel<E, D><<<(unsigned)((groups + GROUPS - 1) / GROUPS), LAYER_WG, 0,
                                           st>>>(
            x, static_cast<const E*>(conv_w), static_cast<const E*>(cstate),
            static_cast<E*>(cstate_out), static_cast<const E*>(b), static_cast<const E*>(a), A_log,
            dt_bias, static_cast<E*>(q), static_cast<E*>(k), static_cast<E*>(v),
            static_cast<E*>(beta), static_cast<E*>(g), bs, B, Hk, Hv);
        return hipGetLastError();
    }
    if (T > 0) {
        constexpr int TILE = (LAYER_WG / (D / 8)) * RUN;
        const dim3 grid((unsigned)((T + TILE - 1) / TILE), (unsigned)(2 * Hk + Hv), (unsigned)B);
        layer_prologue_kernel<E, D><<<grid, LAYER_WG, 0, st>>>(
            x, static_cast<const E*>(conv_w), static_cast<const E*>(cstate),
            static_cast<E*>(cstate_out), static_cast<const E*>(b), static_cast<const E*>(a), A_log, dt_bias,
            static_cast<E*>(q), static_cast<E*>(k), static_cast<E*>(v), static_cast<E*>(beta),
            static_cast<E*>(g), bs, T, Hk, Hv);
        return hipGetLastError();
    }
    if (cstate_out) {   // T == 0: the state passes through (or becomes zeros)
        const long n = (long)B * C;
        conv_state_kernel<E><<<(unsigned)((n + LAYER_WG - 1) / LAYER_WG), LAYER_WG, 0, st>>>(
            x, static_cast<const E*>(cstate), static_cast<E*>(cstate_out), T, C, n);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename E, int D>
hipError_t epilogue_launch(const void* o, const void* z, const void* w, void* out, int B, int Hv,
                           int T, float eps, hipStream_t st) {
    const long rows = (long)B * Hv * T;
    if (rows == 0) return hipSuccess;
    layer_epilogue_kernel<E, D><<<(unsigned)((rows + EPI_ROWS - 1) / EPI_ROWS), LAYER_WG, 0, st>>>(
        static_cast<const E*>(o), static_cast<const E*>(z), static_cast<const E*>(w),
        static_cast<E*>(out), rows, T, Hv, eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layer_prologue(int dtype, const void* qkv, const void* conv_w,
                                 const void* conv_state, void* conv_state_out, const void* b,
                                 const void* a, const float* A_log, const float* dt_bias, void* q,
                                 void* k, void* v, void* beta, void* g, float bs, int B, int T,
                                 int Hk, int Hv, int d, hipStream_t st) {
    if (dtype == DT_BF16) {
        return d == 64 ? prologue_launch<bf16, 64>(qkv, conv_w, conv_state, conv_state_out, b, a,
                                                   A_log, dt_bias, q, k, v, beta, g, bs, B, T, Hk, Hv, st)
                       : prologue_launch<bf16, 128>(qkv, conv_w, conv_state, conv_state_out, b, a,
                                                    A_log, dt_bias, q, k, v, beta, g, bs, B, T, Hk, Hv, st);
    }
    return d == 64 ? prologue_launch<float, 64>(qkv, conv_w, conv_state, conv_state_out, b, a,
                                                A_log, dt_bias, q, k, v, beta, g, bs, B, T, Hk, Hv, st)
                   : prologue_launch<float, 128>(qkv, conv_w, conv_state, conv_state_out, b, a,
                                                 A_log, dt_bias, q, k, v, beta, g, bs, B, T, Hk, Hv, st);
}

hipError_t launch_layer_epilogue(int dtype, const void* o, const void* z, const void* norm_w,
                                 void* out, int B, int Hv, int T, int d, float eps,
                                 hipStream_t st) {
    if (dtype == DT_BF16) {
        return d == 64 ? epilogue_launch<bf16, 64>(o, z, norm_w, out, B, Hv, T, eps, st)
                       : epilogue_launch<bf16, 128>(o, z, norm_w, out, B, Hv, T, eps, st);
    }
    return d == 64 ? epilogue_launch<float, 64>(o, z, norm_w, out, B, Hv, T, eps, st)
                   : epilogue_launch<float, 128>(o, z, norm_w, out, B, Hv, T, eps, st);
}

}  // namespace dn
