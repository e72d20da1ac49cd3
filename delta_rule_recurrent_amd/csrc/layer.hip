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
// The prologue and epilogue kernels move every byte once: the prologue reads the
// projected rows and writes the head-major q, k, v that the chunk and decode
// kernels take; the epilogue reads the head-major read-out and z and writes
// token-major rows for the output projection. For one decode token the whole
// layer step is one kernel (the prologue in the decode step's load stage, the
// norm in its store stage). Arithmetic is fp32 with one rounding to the storage
// type at each output.
#include <type_traits>

#include "dn_device.h"
#include "dn_launch.h"
#include "dn_conv.h"

namespace dn {
namespace {

constexpr int LAYER_WG = 256;   // threads per workgroup of the layer kernels
constexpr int RUN = 8;          // consecutive tokens one lane group convolves in registers
constexpr int CONV_K = 4;       // convolution width (its state: the last 3 inputs)
constexpr int EPI_ROWS = 32;    // rows of the output per epilogue workgroup

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

    // The three inputs before t0: earlier rows of qkv, else the carried state
    // [B][C][3] (oldest first: input t < 0 is state entry 3 + t), else zeros.
    Raw8<E> hr[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const long tt = t0 - 3 + j;
        if (tt >= 0) {
            load_raw(qkv + ((long)b * T + tt) * C + c, hr[j]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                set_elem(hr[j], i, cstate ? cstate[((long)b * C + c + i) * 3 + 3 + tt] : from_f32<E>(0.0f));
        }
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

    // All RUN rows are loaded up front, each a fixed stride after the first. A
    // run that reaches past the end (only the last one of a sequence) re-reads
    // its last row for the missing ones and predicates its stores; every other
    // run takes the same code without the checks.
    const E* xrow = qkv + ((long)b * T + t0) * C + c;
    auto run = [&](auto whole) {
        constexpr bool WHOLE = decltype(whole)::value;
        const int last = WHOLE ? RUN - 1 : (int)(T - 1 - t0);
        Raw8<E> x[RUN];
#pragma unroll
        for (int r = 0; r < RUN; ++r) load_raw(xrow + (long)(WHOLE ? r : min(r, last)) * C, x[r]);
        // SiLU, the key heads' norm and scale, the store of one output row.
        auto finish = [&](int r, float (&y)[8]) {
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                y[i] = silu(y[i]);
                ss += y[i] * y[i];
            }
            if (is_key) {
                const float sc = qs * inv_norm(row_sum<LPR>(ss));
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] *= sc;
            }
            if (WHOLE || r <= last) store8(orow + r * D, y);
        };
        if constexpr (sizeof(E) == 2) {
            // conv_w [C][4]: the taps of channel i are 32-bit words 2i (taps 0, 1)
            // and 2i + 1 (taps 2, 3) of the lane's 64 bytes; the inputs go in as
            // pairs of consecutive tokens, so each output is two pair products.
            Raw8<E> wr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) load_raw(conv_w + c * CONV_K + 8 * j, wr[j]);
            unsigned w01[8], w23[8], p2[8], p1[8];   // pairs (t-3, t-2) and (t-2, t-1)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 wd = __builtin_bit_cast(u32x4, wr[i / 2].v);
                w01[i] = wd[2 * (i % 2)];
                w23[i] = wd[2 * (i % 2) + 1];
                p2[i] = pair_of(hr[0], hr[1], i);
                p1[i] = pair_of(hr[1], hr[2], i);
            }
#pragma unroll
            for (int r = 0; r < RUN; ++r) {
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const unsigned p0 = pair_of(r == 0 ? hr[2] : x[r - 1], x[r], i);   // (t-1, t)
                    y[i] = dot2(p0, w23[i], dot2(p2[i], w01[i], 0.0f));
                    p2[i] = p1[i];
                    p1[i] = p0;
                }
                finish(r, y);
            }
        } else {
            float w[8][CONV_K], h[3][8];
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
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) h[j][i] = elem(hr[j], i);
#pragma unroll
            for (int r = 0; r < RUN; ++r) {
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float xi = elem(x[r], i);
                    y[i] = w[i][0] * h[0][i] + w[i][1] * h[1][i] + w[i][2] * h[2][i] + w[i][3] * xi;
                    h[0][i] = h[1][i];
                    h[1][i] = h[2][i];
                    h[2][i] = xi;
                }
                finish(r, y);
            }
        }
    };
    if (t0 + RUN <= T) run(std::true_type{});
    else run(std::false_type{});

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

// ---------------------------------------------------------------------------
// The whole layer for one token (decode) in one kernel: the prologue in the
// rule's load stage, the gated RMSNorm in its store stage (page "28. Linear
// attention and Gated DeltaNet", section "The full layer", steps 2-7, with the
// recurrent step of section "The recurrent form"). One 256-thread workgroup
// per (sequence b, value head h) holds the whole D x D state of its head, so
// the RMS over the head's D read-out columns needs no exchange between
// workgroups (splitting a state over four workgroups, as the decode step
// does, needs such an exchange: through agent-coherent stores, loads and an
// arrival count it made the step slower, not faster).
//  * Load stage. Wavefront 0 requests the token's inputs first, then every
//    thread its share of the state (thread t: column quad t % (D/4), rows
//    t / (D/4) + RG i); loads complete in order, so wavefront 0 forms q, k
//    (key head h / (Hv/Hk)) and v while the state is in flight, exactly as
//    the single-token prologue does: D/8 lanes per segment, eight channels
//    each, the convolution with the carried history, SiLU, the L2 norms as
//    lane sums (q also scaled by D^-1/2), each rounded to the storage type;
//    one lane forms beta and g. They go to LDS for the whole workgroup.
//  * The rule: S~ = alpha S, p = S~^T k, u = beta (v - p), S = S~ + k u^T,
//    o = S^T q = S~^T q + u (k . q), as in the decode step (the state is read
//    and written once).
//  * Store stage. The threads of row group 0 hold o for their column quads;
//    o is rounded to the storage type (as the rule's output would be), its
//    RMS over the D columns is a lane sum over those threads, and
//    out = w * round(o * rsqrt(mean(o^2) + eps)) * SiLU(z).
// The new convolution history of this token goes to cout: v channels by every
// workgroup, the q and k channels of a key head by the first value head of
// its group only (one writer per channel). Every lane reads its own entries
// before writing them, so cout may be cstate itself when each key head serves
// one value head (with shared key heads other workgroups still read them).
// ---------------------------------------------------------------------------
template <typename E, int D, bool GATED>
__global__ __launch_bounds__(LAYER_WG) void layer_decode_kernel(
    const E* __restrict__ qkv, const E* __restrict__ conv_w, const E* cstate, E* cout,
    const E* __restrict__ bin, const E* __restrict__ ain, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const E* __restrict__ z, const E* __restrict__ nw,
    float* __restrict__ S, E* __restrict__ out, float bscale, float eps, int Hk, int Hv) {
    constexpr int LPR = D / 8;            // lanes per channel segment
    constexpr int CQ = D / 4;             // column quads per state row
    constexpr int RG = LAYER_WG / CQ;     // row groups
    constexpr int RPT = D / RG;           // rows per thread
    constexpr float QSCALE = D == 64 ? 0.125f : 0.08838834764831845f;   // D^-1/2
    static_assert(D % RG == 0 && CQ <= WAVE && 3 * LPR < WAVE, "unsupported head size");
    typedef typename Vec4<E>::type V4;

    const long bh = blockIdx.x;
    const long b = bh / Hv;
    const int h = (int)(bh % Hv);
    const int grp = Hv / Hk, hk = h / grp;
    const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
    const int cq = t % CQ, rg = t / CQ;
    const long C = (long)(2 * Hk + Hv) * D;

    const int seg = lane / LPR, l = lane % LPR;   // wavefront 0: 0 q, 1 k, 2 v
    const bool pro = w == 0 && seg < 3;
    const long c = (seg < 2 ? (long)(seg * Hk + hk) * D : (long)(2 * Hk + h) * D) + l * 8;
    const long so = (b * C + c) * 3;   // this lane's 24 history entries, channel-major
    Raw8<E> xr, w0, w1, w2, w3, h0, h1, h2;
    if (pro) {
        load_raw(qkv + b * C + c, xr);
        load_raw(conv_w + c * CONV_K, w0);
        load_raw(conv_w + c * CONV_K + 8, w1);
        load_raw(conv_w + c * CONV_K + 16, w2);
        load_raw(conv_w + c * CONV_K + 24, w3);
        if (cstate) {
            load_raw(cstate + so, h0);
            load_raw(cstate + so + 8, h1);
            load_raw(cstate + so + 16, h2);
        }
    }
    const bool gl = w == 0 && lane == WAVE - 1;   // the lane that forms the gates
    float bin_v = 0.f, ain_v = 0.f, alog_v = 0.f;
    if (gl) {
        bin_v = to_f32(bin[b * Hv + h]);
        if (GATED) {
            ain_v = to_f32(ain[b * Hv + h]) + dt_bias[h];
            alog_v = A_log[h];
        }
    }
    // the store stage's z and norm weights (row group 0: lanes 0 .. CQ-1 of
    // wavefront 0)
    const long oc = (b * Hv + h) * D + 4 * cq;   // [B][Hv*D]: the same as [B][1][Hv*D]
    V4 zv, wv;
    if (rg == 0) {
        zv = *reinterpret_cast<const V4*>(z + oc);
        wv = *reinterpret_cast<const V4*>(nw + 4 * cq);
    }

    float* Sp = S + bh * D * D + 4 * cq;
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = *reinterpret_cast<const f32x4*>(Sp + (rg + RG * i) * D);

    __shared__ float sq[D], sk[D], sv[D], sgate[2];
    __shared__ f32x4 red_p[4][CQ], red_r[4][CQ];
    __shared__ float red_kq[4];

    if (pro) {
        float y[8], ss = 0.0f, hist[24];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            hist[i] = cstate ? elem(h0, i) : 0.0f;
            hist[8 + i] = cstate ? elem(h1, i) : 0.0f;
            hist[16 + i] = cstate ? elem(h2, i) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const Raw8<E>& wr = i < 2 ? w0 : i < 4 ? w1 : i < 6 ? w2 : w3;
            const int o = (i % 2) * 4;
            const float xi = elem(xr, i);
            const float acc = elem(wr, o) * hist[3 * i] + elem(wr, o + 1) * hist[3 * i + 1] +
                              elem(wr, o + 2) * hist[3 * i + 2] + elem(wr, o + 3) * xi;
            y[i] = silu(acc);
            ss += y[i] * y[i];
        }
        if (cout && (seg == 2 || h % grp == 0)) {
            float nh[24];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                nh[3 * i] = hist[3 * i + 1];
                nh[3 * i + 1] = hist[3 * i + 2];
                nh[3 * i + 2] = elem(xr, i);
            }
            store8(cout + so, *reinterpret_cast<const float(*)[8]>(nh));
            store8(cout + so + 8, *reinterpret_cast<const float(*)[8]>(nh + 8));
            store8(cout + so + 16, *reinterpret_cast<const float(*)[8]>(nh + 16));
        }
        // the lane sum runs in every lane of the segment (rows of LPR lanes)
        const float tot = row_sum<LPR>(ss);
        const float sc = seg == 0 ? QSCALE * inv_norm(tot) : seg == 1 ? inv_norm(tot) : 1.0f;
        float* dst = seg == 0 ? sq : seg == 1 ? sk : sv;
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[l * 8 + i] = to_f32(from_f32<E>(y[i] * sc));
    } else if (gl) {
        sgate[0] = to_f32(from_f32<E>(bscale / (1.0f + __expf(-bin_v))));
        if (GATED)
            sgate[1] = to_f32(from_f32<E>(-__expf(alog_v) * (fmaxf(ain_v, 0.0f) + log1pf(__expf(-fabsf(ain_v))))));
    }
    __syncthreads();

    const float beta = sgate[0];
    const float alpha = GATED ? __expf(sgate[1]) : 1.0f;
    f32x4 p = zero4(), r = zero4();
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        if (GATED) s[i] *= alpha;
        p += sk[row] * s[i];
        r += sq[row] * s[i];
        kq += sk[row] * sq[row];
    }
    // row groups inside one wavefront differ in lane bits >= log2(CQ)
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

    f32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = beta * (sv[4 * cq + e] - p[e]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        s[i] += sk[row] * u;
        *reinterpret_cast<f32x4*>(Sp + row * D) = s[i];
    }
    if (rg == 0) {
        // row group 0 is lanes 0 .. CQ-1 of wavefront 0: the read-out of the
        // head's D columns, four per lane
        const f32x4 ov = r + u * kq;
        float on[4], ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            on[e] = to_f32(from_f32<E>(ov[e]));
            ss += on[e] * on[e];
        }
#pragma unroll
        for (int off = 1; off < CQ; off <<= 1) ss += __shfl_xor(ss, off, CQ);
        const float rr = rsqrtf(ss * (1.0f / D) + eps);
        V4 res;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float nrm = to_f32(from_f32<E>(on[e] * rr));
            res[e] = from_f32<E>(to_f32(wv[e]) * nrm * silu(to_f32(zv[e])));
        }
        *reinterpret_cast<V4*>(out + oc) = res;
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
// Epilogue. EPI_ROWS consecutive rows of the token-major output out [B][T][Hv][D]
// per workgroup, D/8 lanes per row: a wave reads z and writes out as contiguous
// spans, and reads the head-major read-out o [B][Hv][T][D] one head row at a time
// (the layout that measured fastest: two of the three streams are contiguous).
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
        const long bt = row / Hv, hv = row % Hv;
        const long bb = bt / T, t = bt % T;
        zoff[p] = row * D + l * 8;
        load_raw(o + ((bb * Hv + hv) * T + t) * D + l * 8, ov[p]);
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

template <typename E, int D>
hipError_t decode_layer_launch(const void* qkv, const void* conv_w, const void* cstate, void* cout,
                               const void* b, const void* a, const float* A_log, const float* dt_bias,
                               const void* z, const void* nw, float* S, void* out, float bs, float eps,
                               int B, int Hk, int Hv, hipStream_t st) {
    const unsigned grid = (unsigned)((long)B * Hv);
    if (a) {
        layer_decode_kernel<E, D, true><<<grid, LAYER_WG, 0, st>>>(
            static_cast<const E*>(qkv), static_cast<const E*>(conv_w), static_cast<const E*>(cstate),
            static_cast<E*>(cout), static_cast<const E*>(b), static_cast<const E*>(a), A_log, dt_bias,
            static_cast<const E*>(z), static_cast<const E*>(nw), S, static_cast<E*>(out), bs, eps, Hk, Hv);
    } else {
        layer_decode_kernel<E, D, false><<<grid, LAYER_WG, 0, st>>>(
            static_cast<const E*>(qkv), static_cast<const E*>(conv_w), static_cast<const E*>(cstate),
            static_cast<E*>(cout), static_cast<const E*>(b), nullptr, nullptr, nullptr,
            static_cast<const E*>(z), static_cast<const E*>(nw), S, static_cast<E*>(out), bs, eps, Hk, Hv);
    }
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

hipError_t launch_layer_decode(int dtype, const void* qkv, const void* conv_w, const void* conv_state,
                               void* conv_state_out, const void* b, const void* a, const float* A_log,
                               const float* dt_bias, const void* z, const void* norm_w, float eps, float* S,
                               void* out, float bs, int B, int Hk, int Hv, int d, hipStream_t st) {
    if (dtype == DT_BF16) {
        return d == 64 ? decode_layer_launch<bf16, 64>(qkv, conv_w, conv_state, conv_state_out, b, a, A_log,
                                                       dt_bias, z, norm_w, S, out, bs, eps, B, Hk, Hv, st)
                       : decode_layer_launch<bf16, 128>(qkv, conv_w, conv_state, conv_state_out, b, a, A_log,
                                                        dt_bias, z, norm_w, S, out, bs, eps, B, Hk, Hv, st);
    }
    return d == 64 ? decode_layer_launch<float, 64>(qkv, conv_w, conv_state, conv_state_out, b, a, A_log,
                                                    dt_bias, z, norm_w, S, out, bs, eps, B, Hk, Hv, st)
                   : decode_layer_launch<float, 128>(qkv, conv_w, conv_state, conv_state_out, b, a, A_log,
                                                     dt_bias, z, norm_w, S, out, bs, eps, B, Hk, Hv, st);
}

}  // namespace dn
