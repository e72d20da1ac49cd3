// chunk.hip -- chunkwise-parallel prefill (chunk C = 64) on gfx950 matrix cores.
//
// For one chunk of one (sequence, head), with G_i the running sum of the
// log-decay inside the chunk (per key channel for KDA), the UT/WY form is
//     A   = strict_tril(beta_i k_i . k_j exp(G_i - G_j))
//     T   = (I + A)^-1                      (unit lower triangular)
//     W   = T (beta exp(G) K),  u = T (beta V)
//     U   = u - W S0                         (values actually written)
//     O   = (Q exp(G)) S0 + tril(Q K^T exp(G_i - G_j)) U
//     S1  = exp(G_C) S0 + (K exp(G_C - G))^T U
// (page "28. Linear attention and Gated DeltaNet", section "The chunked form:
// recurrence as matrix multiplication"; page "DeltaNet: Memory That Edits",
// section "Training it: the WY trick"; with per-channel decay for KDA,
// page "A walk through of the DeltaNet family of linear attention variants").
//
// Kernels:
//   chunk_prep_kernel  one workgroup per (head, chunk), all chunks in parallel:
//                      G, A (MFMA), T (forward substitution in LDS), W, u
//                      (MFMA), the masked decayed Q K^T and the decay-scaled
//                      K^T (fp32 at d = 128); everything the sequential part needs is
//                      written to the workspace in the exact per-lane MFMA
//                      fragment order the scan loads (one coalesced 16-byte
//                      load per lane per fragment).
//   chunk_scan_kernel  one workgroup per (head, 32- or 16-column value tile):
//                      the fp32 state tile lives in MFMA accumulators across
//                      all chunks; per chunk U = u - W S, O = Q~ S + attn U,
//                      S = gamma S + K~^T U, chained through two small LDS
//                      exchanges of bf16 fragments.
//   chunk_prep2_kernel the prep on two wavefronts per (head, chunk) (Gated
//                      DeltaNet / DeltaNet; same workspace contents).
//   chunk_fused_kernel both in one launch: prep workgroups hand chunk blocks
//                      to the scan workgroups of the same XCD as they finish
//                      (long sequences, bf16).
// KDA's prep (per-channel decay) is in chunk_kda.hip; it writes the same
// workspace blocks, which the scan here reads.
#include <atomic>
#include <cstdlib>
#include <random>

#include "dn_device.h"
#include "dn_launch.h"
#include "dn_chunk.h"
#include "dn_kda_prep.h"
#include "dn_conv.h"

namespace dn {

// LDS carve-up of the prep kernel (bytes). Regions X and Y are reused as the
// work moves on (each switch is separated by a workgroup barrier):
//   X : K rows     -> fp32 T (diagonal 16x16 inverses)          -> T' = T diag(beta e^G)
//   Y : Q rows     -> fp32 system matrix A                      -> T'' = T diag(beta)
//   KT: K^T (token index contiguous)
//   VT: V^T
template <typename E, int DK, int DV, int KIND>
struct PrepSmem {
    static_assert(KIND != KIND_KDA, "KDA has its own prep kernel");
    static constexpr int KP = 16 / sizeof(E);  // row padding: one 16-byte vector
    static constexpr int LDK = DK + KP;        // [64][DK] tiles
    static constexpr int LDT = 64 + KP;        // [D][64] tiles
    static constexpr int LDF = 68;             // fp32 64x64 matrices
    static constexpr long cmax(long a, long b) { return a > b ? a : b; }
    static constexpr long SZ_X = cmax(cmax(64L * LDK * sizeof(E), 64L * LDF * 4), 64L * LDT * sizeof(E));
    static constexpr long SZ_Y = SZ_X;
    static constexpr long OFF_X = 0;
    static constexpr long OFF_Y = OFF_X + SZ_X;
    static constexpr long OFF_KT = OFF_Y + SZ_Y;
    static constexpr long OFF_VT = OFF_KT + (long)DK * LDT * sizeof(E);
    static constexpr long TOTAL = OFF_VT + (long)DV * LDT * sizeof(E);
};

// ---------------------------------------------------------------------------
// Prep kernel: one workgroup (4 wavefronts) per (head, chunk); DeltaNet, Gated
// DeltaNet and the state-space kind in fp32 at d = 128, where the two-wavefront
// prep's fragments do not fit its registers.
// ---------------------------------------------------------------------------
// Two workgroups share a compute unit where the LDS allows it; the register
// budget is capped accordingly.
template <typename E, int DK, int DV, int KIND, bool VARLEN = false>
__global__ __launch_bounds__(256, (PrepSmem<E, DK, DV, KIND>::TOTAL + 1024) * 2 <= 163840 ? 2 : 1)
void chunk_prep_kernel(const E* __restrict__ q,
                                                         const E* __restrict__ k,
                                                         const E* __restrict__ v,
                                                         const E* __restrict__ beta,
                                                         const E* __restrict__ g,
                                                         char* __restrict__ ws, int T,
                                                         int nchunks, int nitems, HeadMap hm,
                                                         const int2* __restrict__ ctab = nullptr) {
    typedef WsLayout<E, DK, DV> Lw;
    typedef PrepSmem<E, DK, DV, KIND> Sm;
    typedef typename Frag<E>::type F;
    typedef typename Vec4<E>::type V4;
    constexpr int LDK = Sm::LDK, LDT = Sm::LDT, LDF = Sm::LDF;

    __shared__ __align__(16) char smem[Sm::TOTAL];
    __shared__ float Gs[64], eG[64], eGC[64], bs[64];
    E* Ks = reinterpret_cast<E*>(smem + Sm::OFF_X);
    E* Qs = reinterpret_cast<E*>(smem + Sm::OFF_Y);
    float* Tf = reinterpret_cast<float*>(smem + Sm::OFF_X);
    float* As = reinterpret_cast<float*>(smem + Sm::OFF_Y);
    E* Tp = reinterpret_cast<E*>(smem + Sm::OFF_X);
    E* Tpp = reinterpret_cast<E*>(smem + Sm::OFF_Y);
    E* KsT = reinterpret_cast<E*>(smem + Sm::OFF_KT);
    E* VsT = reinterpret_cast<E*>(smem + Sm::OFF_VT);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int gq = lane >> 4, n = lane & 15;

    // Persistent loop over (head, chunk) items: the inputs of the next item are
    // loaded into registers while the current one is computed, and written to
    // LDS when it is done. Prefetches are unconditional (the item index is
    // clamped to the last item).
    TileRegs<E, DK> rk, rq;
    TileRegs<E, DV> rv;
    // beta and log-decay of token `lane` (wave 0), kept as loaded: converting
    // (or masking) them right after the load would make the wave wait for
    // every prefetch load issued before them
    E pbr{}, pgr{};
    bool pin = false;   // token `lane` is inside the chunk
    auto fetch = [&](int it) {
        const int fc = it % nchunks;
        long ftok, fkey;
        int fL, fA;   // tokens of the chunk; fA >= 1 bounds the row addresses
        if constexpr (VARLEN) {
            // packed sequences: item = head * nchunks + global chunk, the chunk's
            // first token and length from the chunk table (length 0: unused slot)
            const int2 e = ctab[fc];
            ftok = fkey = (long)(it / nchunks) * T + e.x;
            fL = e.y;
            fA = max(e.y, 1);
        } else {
            ftok = (long)(it / nchunks) * T + (long)fc * CHUNK;
            fkey = hm.key(it / nchunks) * T + (long)fc * CHUNK;   // q, k row
            fL = fA = min(CHUNK, T - fc * CHUNK);
        }
        tile_load<E, DK>(rk, k + fkey * DK, fA, tid, fL);
        tile_load<E, DK>(rq, q + fkey * DK, fA, tid, fL);
        tile_load<E, DV>(rv, v + ftok * DV, fA, tid, fL);
        if (w == 0) {
            const long tk = ftok + min(lane, fA - 1);
            if (KIND != KIND_SSM) pbr = beta[tk];
            if (KIND == KIND_GATED || KIND == KIND_SSM) pgr = g[tk];
            pin = lane < fL;
        }
    };
    int item = blockIdx.x;
    fetch(item);
    for (;;) {
    const int c = item % nchunks;
    const long bh = item / nchunks;
    const int t0 = c * CHUNK;
    const int L = min(CHUNK, T - t0);

    char* blk = ws + ((long)bh * nchunks + c) * Lw::BYTES;
    E* Wf = reinterpret_cast<E*>(blk) + Lw::W_OFF;
    E* Kf = reinterpret_cast<E*>(blk) + Lw::K_OFF;
    E* Af = reinterpret_cast<E*>(blk) + Lw::A_OFF;
    E* Uf = reinterpret_cast<E*>(blk) + Lw::U_OFF;
    float* gam = reinterpret_cast<float*>(blk + Lw::GAM_BYTE_OFF);
    float* eg = reinterpret_cast<float*>(blk + Lw::EG_BYTE_OFF);

    const long tok0 = (long)bh * T + t0;

    // ---- 1. beta, log-decay and its running sum inside the chunk; stage tiles
    // the state-space kind has no write strength and no correction: beta = 1
    // (u = V) and A = 0 (T = I); the W it gets is never read by its scan
    const float pb = pin ? (KIND == KIND_SSM ? 1.f : to_f32(pbr)) : 0.f;
    const float pg = (KIND == KIND_GATED || KIND == KIND_SSM) && pin ? to_f32(pgr) : 0.f;
    if (w == 0) bs[lane] = pb;
    if (w == 0) {
        const float G = wave_inclusive_sum(pg, lane);
        const float GC = readlane_f(G, 63);
        Gs[lane] = G;
        eG[lane] = __expf(G);
        eGC[lane] = __expf(GC - G);
        // the chunk decay, replicated per key channel so that the scan reads
        // it like KDA's (vector loads; no scalar load on its critical path)
        for (int ch = lane; ch < DK; ch += 64) gam[ch] = __expf(GC);
    }
    tile_store<E, DK, true, true>(rk, Ks, LDK, KsT, LDT, tid);
    tile_store<E, DK, true, false>(rq, Qs, LDK, nullptr, 0, tid);
    tile_store<E, DV, false, true>(rv, nullptr, 0, VsT, LDT, tid);
    lds_barrier();
    fetch((int)min((long)item + gridDim.x, (long)nitems - 1));
    // ---- 2. attn -> A-fragments; raw K K^T kept in registers
    // Wave w owns token tile w: rows i in [16w, 16w+16) of A and of attn.
    f32x4 sa[4];
    {
        F ka[DK / 32], qa[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            ka[kb] = frag_rows<E>(Ks, LDK, 16 * w, 32 * kb, lane);
            qa[kb] = frag_rows<E>(Qs, LDK, 16 * w, 32 * kb, lane);
        }
        f32x4 at[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            sa[jt] = zero4();
            at[jt] = zero4();
            if (jt <= w) {
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const F kj = frag_rows<E>(Ks, LDK, 16 * jt, 32 * kb, lane);
                    if (KIND != KIND_SSM) sa[jt] = mma(ka[kb], kj, sa[jt]);  // (K K^T)[i][j]
                    at[jt] = mma(kj, qa[kb], at[jt]);  // (K Q^T)[j][i] = attn^T
                }
            }
            // attn^T tile: rows j = 16jt + 4gq + e, column i = 16w + n (causal, incl. diagonal)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * jt + 4 * gq + e, i = 16 * w + n;
                at[jt][e] = i >= j ? __expf(Gs[i] - Gs[j]) * at[jt][e] : 0.f;
            }
        }
        // attn^T computed with rows = j lands directly as A-fragments of attn (rows i)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            reinterpret_cast<F*>(Af)[(w * 2 + kb) * 64 + lane] = frag_from_tiles<E>(at[2 * kb], at[2 * kb + 1]);
        // the scan reads Q itself and applies the per-token factor e^G to Q S
        if (w == 0) eg[lane] = eG[lane];
    }
    // K~^T = (e^{G_C - G} K)^T, A-fragments with rows = key channels
    for (int p = w; p < (DK / 16) * 2; p += 4) {
        const int mt = p >> 1, kb = p & 1;
        reinterpret_cast<F*>(Kf)[p * 64 + lane] = frag_rows_scaled<E>(KsT, LDT, 16 * mt, 32 * kb, lane, 1.f, eGC);
    }
    lds_barrier();  // K and Q rows are dead from here on

    // ---- 2b. system matrix A = strict_tril(beta_i K K^T D) into region Y -----
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * w + 4 * gq + e, j = 16 * jt + n;
            float val = 0.f;
            if (i > j) val = bs[i] * __expf(Gs[i] - Gs[j]) * sa[jt][e];
            As[i * LDF + j] = val;
        }
    lds_barrier();

    // ---- 3. UT transform T = (I + A)^-1, blocked over 16x16 tiles ------------
    // 3a: wave w inverts its diagonal tile by forward substitution, lane = column:
    //     T_jj = 1, T_ij = -sum_{j <= m < i} A_im T_mj  (rows and columns inside the tile)
    {
        const int j = n;
        const int b0 = 16 * w;
        float tc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tc[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc += As[(b0 + i) * LDF + b0 + m] * tc[m];
            if (i > j) tc[i] = -acc;
        }
        if (gq == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) Tf[(b0 + i) * LDF + b0 + j] = tc[i];
        }
    }
    lds_barrier();
    // 3b: wave w computes column tile w of T downwards on the matrix cores:
    //     T_Iw = -T_II * sum_{w <= K < I} A_IK T_Kw   (16x16 tiles, fp32)
    f32x4 tcol[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) tcol[I] = zero4();
    {
        f32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = Tf[(16 * w + 4 * gq + e) * LDF + 16 * w + n];
#pragma unroll
        for (int I = 0; I < 4; ++I)
            if (I == w) tcol[I] = d;
    }
#pragma unroll
    for (int I = 1; I < 4; ++I) {
        if (I > w) {
            f32x4 R = zero4();
#pragma unroll
            for (int K = 0; K < I; ++K)
                if (K >= w) R = mma16_lds_reg(As + 16 * I * LDF + 16 * K, LDF, lane, tcol[K], R);
            const f32x4 t = mma16_lds_reg(Tf + 16 * I * LDF + 16 * I, LDF, lane, R, zero4());
            tcol[I] = -t;
        }
    }
    lds_barrier();  // A and the diagonal inverses are dead from here on
    // T' = T diag(beta e^G) into region X, T'' = T diag(beta) into region Y
    {
        const int j = 16 * w + n;
        const float sb = bs[j];
        const float sbg = bs[j] * eG[j];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * gq + e;
                Tp[i * LDT + j] = from_f32<E>(tcol[I][e] * sbg);
                Tpp[i * LDT + j] = from_f32<E>(tcol[I][e] * sb);
            }
    }
    lds_barrier();

    // ---- 4. W^T = X^T T'^T, computed transposed so it lands as A-fragments of W
    //         (X = K, T' = T diag(beta e^G))
    {
        const E* XT = KsT;
        const E* TT = Tp;
        f32x4 wt[DK / 16];
#pragma unroll
        for (int mt = 0; mt < DK / 16; ++mt) {
            wt[mt] = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                wt[mt] = mma(frag_rows<E>(XT, LDT, 16 * mt, 32 * kb, lane),
                             frag_rows<E>(TT, LDT, 16 * w, 32 * kb, lane), wt[mt]);
        }
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
            reinterpret_cast<F*>(Wf)[(w * (DK / 32) + kb) * 64 + lane] =
                frag_from_tiles<E>(wt[2 * kb], wt[2 * kb + 1]);
    }
    // ---- 5. u = T diag(beta) V for token tile w (D-tiles) -------------------
#pragma unroll
    for (int nt = 0; nt < DV / 16; ++nt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            acc = mma(frag_rows<E>(Tpp, LDT, 16 * w, 32 * kb, lane),
                      frag_rows<E>(VsT, LDT, 16 * nt, 32 * kb, lane), acc);
        V4 u4;
#pragma unroll
        for (int e = 0; e < 4; ++e) u4[e] = from_f32<E>(acc[e]);
        reinterpret_cast<V4*>(Uf)[(nt * 4 + w) * 64 + lane] = u4;
    }

    if ((long)item + gridDim.x >= nitems) break;
    item += gridDim.x;
    lds_barrier();   // every wave is done with this item's LDS data
    }
}

// ---------------------------------------------------------------------------
// Prep kernel, two wavefronts per (head, chunk): Gated DeltaNet and DeltaNet.
// ---------------------------------------------------------------------------
// Same results and workspace layout as chunk_prep_kernel, split over two
// wavefronts that meet at a single LDS barrier (about 37 KB of LDS per chunk,
// two wavefronts per SIMD):
//   wavefront 0: A = strict_tril(beta K K^T D), the blocked inverse T, the
//                scaled copies T diag(beta e^G) and T diag(beta) into LDS;
//                after the barrier u = T diag(beta) V.
//   wavefront 1: attn = tril(Q K^T D), K~^T, K and V with tokens as the
//                contraction index (V into LDS); after the barrier
//                W = T diag(beta e^G) K.
//  * K, Q and V fragments with rows = tokens come straight from global memory,
//    in the 8-consecutive-channel contraction order (16-byte loads).
//  * With the token index as the contraction index (B-fragments of K and V,
//    A-fragments of K~^T = (e^{G_C - G} K)^T), K and V come from a product
//    with an identity fragment on the matrix cores: D = K I holds K as D-tiles
//    (exactly), and two D-tiles stacked over tokens are such a fragment.
//  * Each scaled T is rounded once to the operand type.


// The gated layer's inputs for the prep that runs the layer's prologue in its
// load stage (bf16, d = 128): the projected channel rows qkv [B][T][C] with
// C = (2 Hk + Hv) 128 (q of the key heads, then k, then v of the value heads),
// the filter taps [C][4], the carried history [B][C][3] (or null: zeros) and
// its successor (written by the items of each sequence's last chunk; must not
// overlap the old one), the gate inputs b, a [B][T][Hv] (a null: no decay),
// and where the normalised, scaled q rows go for the scan ([B][Hk][T][128]).
struct LayerIn {
    const bf16* qkv;
    const bf16* conv_w;
    const bf16* cstate;
    bf16* cout;
    const bf16* bin;
    const bf16* ain;
    const float* A_log;
    const float* dt_bias;
    bf16* qhat;
    float bscale;
    int T, Hk, Hv;
};

template <typename E, int DK, int DV, int CH = CHUNK>
struct Prep2Smem {
    static constexpr int LDF = CH + 4;                 // fp32 CH x CH: A, then T's diagonal blocks
    static constexpr int LDT = CH + 16 / sizeof(E);    // T diag(.) in the operand type (two)
    static constexpr long AT_BYTES = (long)CH * LDF * 4 > 2L * CH * LDT * (long)sizeof(E)
                                         ? (long)CH * LDF * 4
                                         : 2L * CH * LDT * (long)sizeof(E);
    // V as B-fragments (contraction over tokens), [DV/16 value tiles][CH/32][64 lanes]
    static constexpr long V_BYTES = (DV / 16) * (CH / 32) * 64L * 8 * sizeof(E);
    static constexpr long BYTES = AT_BYTES + V_BYTES;
};

// Per-token tables of one chunk of CH tokens in LDS: running log-decay G,
// beta e^G, e^{G_C - G} and beta; lane l holds tokens l, l + 64, ... (bv, gv
// zero past the chunk's end). Returns e^{G_C}.
template <int CH>
__device__ __forceinline__ float token_tables(const float (&bv)[(CH + 63) / 64], const float (&gv)[(CH + 63) / 64],
                                              int lane, float* Gs, float* sX, float* sK, float* bs, float* eG) {
    constexpr int TH = (CH + 63) / 64;
    float G[TH];
#pragma unroll
    for (int h = 0; h < TH; ++h) {
        G[h] = wave_inclusive_sum(gv[h], lane);
        if (h > 0) G[h] += readlane_f(G[h - 1], 63);
    }
    const float GC = readlane_f(G[TH - 1], CH >= 64 ? 63 : CH - 1);
#pragma unroll
    for (int h = 0; h < TH; ++h) {
        const int t = 64 * h + lane;
        if (CH >= 64 || t < CH) {
            const float e = __expf(G[h]);
            Gs[t] = G[h];
            sX[t] = bv[h] * e;
            sK[t] = __expf(GC - G[h]);
            bs[t] = bv[h];
            if (eG) eG[t] = e;
        }
    }
    return __expf(GC);
}

// LDS of one two-wavefront prep unit.
template <typename E, int DK, int DV, int CH = CHUNK>
struct Prep2Lds {
    __align__(16) char smem[Prep2Smem<E, DK, DV, CH>::BYTES];
    // per wavefront: running log-decay, beta e^G, e^{G_C - G}, beta of each token
    __align__(16) float tab[2][4][CH];
};

// One (head bh, chunk c) item of CH tokens (32, 64 or 128) on two wavefronts
// (w = 0, 1 of the unit), its results written to the workspace block `blk`.
// Each of the two wavefronts passes exactly one workgroup barrier.
// LAYER: q, k, v, beta and g are not read; the item forms them from the
// layer's inputs `li` for sequence lb, value head lh, tokens lt0 .. lt0+L-1
// (section 1 below), exactly as the layer's prologue kernel would.
template <typename E, int DK, int DV, int KIND, int CH = CHUNK, bool LAYER = false>
__device__ __forceinline__ void prep2_item(const E* __restrict__ q, const E* __restrict__ k,
                                           const E* __restrict__ v, const E* __restrict__ beta,
                                           const E* __restrict__ g, char* __restrict__ blk,
                                           Prep2Lds<E, DK, DV, CH>& lds, long tok0, long tokk, int L,
                                           int w, int lane, const LayerIn& li = LayerIn{}, long lb = 0,
                                           int lh = 0, long lt0 = 0) {
    typedef WsLayout<E, DK, DV, CH> Lw;
    typedef Prep2Smem<E, DK, DV, CH> Sm;
    typedef typename Frag<E>::type F;
    typedef typename Vec4<E>::type V4;
    constexpr int KB = DK / 32, CT = DK / 16, VB = DV / 32, VT = DV / 16;
    constexpr int NT = CH / 16, CB = CH / 32, TH = (CH + 63) / 64;
    constexpr int LDF = Sm::LDF, LDT = Sm::LDT;
    // past 64 tokens, V's fragments are loaded after attn (register room)
    constexpr bool LATE_V = CH > 64;

    char* smem = lds.smem;
    float(*tab)[4][CH] = lds.tab;
    float* As = reinterpret_cast<float*>(smem);   // A, then T's diagonal blocks in place
    E* Tw = reinterpret_cast<E*>(smem);           // T diag(beta e^G), once the inverse is done
    E* Tu = Tw + CH * LDT;                        // T diag(beta)
    F* Vl = reinterpret_cast<F*>(smem + Sm::AT_BYTES);

    const int gq = lane >> 4, n = lane & 15;
    // tok0: the chunk's first token (value-head row), tokk: the same token in
    // the q, k rows; L: tokens of the chunk (1..CH)

    F* Wf = reinterpret_cast<F*>(reinterpret_cast<E*>(blk) + Lw::W_OFF);
    F* Kf = reinterpret_cast<F*>(reinterpret_cast<E*>(blk) + Lw::K_OFF);
    F* Af = reinterpret_cast<F*>(reinterpret_cast<E*>(blk) + Lw::A_OFF);
    V4* Uf = reinterpret_cast<V4*>(reinterpret_cast<E*>(blk) + Lw::U_OFF);
    float* gam = reinterpret_cast<float*>(blk + Lw::GAM_BYTE_OFF);
    float* eg = reinterpret_cast<float*>(blk + Lw::EG_BYTE_OFF);

    // ---- 1. every load of this wavefront is issued up front, so that a single
    //         memory latency covers them: beta and the log-decay of tokens
    //         `lane` (+ 64), then the K fragments (rows = tokens, contraction =
    //         key channels, in the 8-consecutive-channel order; both
    //         wavefronts), then (wavefront 1) Q and V in the same order
    E braw[TH], graw[TH];
    F kf[NT][KB];
    F qa[NT][KB], vf[NT][VB];
    if constexpr (LAYER) {
        // ---- 1'. the layer's prologue in the load stage. Wavefront 0 forms the
        //          64 k rows (its key head), wavefront 1 the v rows (its value
        //          head), four lane groups x two runs of eight tokens each, into
        //          the two LDS regions that A and V's fragments use later; after
        //          a barrier both read their fragments (same order as the global
        //          loads below), and after a second one wavefront 1 forms the q
        //          rows over V's region (and stores them for the scan) while
        //          wavefront 0 starts on A. The gates are formed per token.
        static_assert(sizeof(E) == 2 && DK == 128 && DV == 128 && CH == 64,
                      "the layer prep is built for bf16, d = 128, chunks of 64");
        constexpr int LDK = DK + 8;   // padded k rows in the A region
        constexpr float QSCALE = 0.08838834764831845f;   // 128^-1/2
        const long C = (long)(2 * li.Hk + li.Hv) * DK;
        const int grpv = li.Hv / li.Hk, hk = lh / grpv;
        const long T = li.T;
        const bf16* xs0 = li.qkv + lb * T * C;   // the sequence's token 0
        const int lg = lane >> 4, l16 = lane & 15;
        {
            const long gi = (lb * T + lt0 + min(lane, L - 1)) * li.Hv + lh;
            braw[0] = from_f32<E>(li.bscale / (1.0f + __expf(-to_f32(li.bin[gi]))));
            graw[0] = E{};
            if (KIND == KIND_GATED) {
                const float zz = to_f32(li.ain[gi]) + li.dt_bias[lh];
                graw[0] = from_f32<E>(-__expf(li.A_log[lh]) * (fmaxf(zz, 0.0f) + log1pf(__expf(-fabsf(zz)))));
            }
        }
        E* ktile = reinterpret_cast<E*>(smem);                 // k rows over A's region
        E* vtile = reinterpret_cast<E*>(smem + Sm::AT_BYTES);  // v, then q rows over V's region
        const bf16* cst0 = li.cstate ? li.cstate + lb * C * 3 : nullptr;
        {
            const long cs = (w == 0 ? (long)(li.Hk + hk) * DK : (long)(2 * li.Hk + lh) * DK) + 8 * l16;
            E* tile = w == 0 ? ktile : vtile;
            const int ldt = w == 0 ? LDK : DV;
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const int r0 = 16 * lg + 8 * run;
                prologue_run8<DK>(xs0 + cs, C, T, lt0 + r0, li.conv_w + cs * 4, cst0 ? cst0 + cs * 3 : nullptr,
                                  w == 0, 1.0f, tile + r0 * ldt + 8 * l16, ldt, nullptr);
            }
        }
        // the sequence's last chunk: the new history (the last three inputs of
        // each channel) of this head's v channels, and of its key head's q and k
        // channels from the first value head of the key head's group
        if (li.cout && lt0 + CH >= T) {
            const int seg = w == 0 ? (lg == 1 ? 0 : lg == 2 ? 1 : -1) : (lg == 1 ? 2 : -1);
            if (seg >= 0 && (seg == 2 || lh % grpv == 0)) {
                const long cs = (seg < 2 ? (long)(seg * li.Hk + hk) * DK : (long)(2 * li.Hk + lh) * DK) + 8 * l16;
                float nh[24];
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const long tt = T - 3 + j;
                    float rv[8];
                    if (tt >= 0) {
                        load8(xs0 + tt * C + cs, rv);
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) rv[i] = cst0 ? to_f32(cst0[(cs + i) * 3 + 3 + tt]) : 0.0f;
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) nh[3 * i + j] = rv[i];
                }
                bf16* co = li.cout + (lb * C + cs) * 3;
                store8(co, *reinterpret_cast<const float(*)[8]>(nh));
                store8(co + 8, *reinterpret_cast<const float(*)[8]>(nh + 8));
                store8(co + 16, *reinterpret_cast<const float(*)[8]>(nh + 16));
            }
        }
        lds_barrier();   // the k and v rows are in LDS
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                kf[tt][kb] = *reinterpret_cast<const F*>(ktile + (16 * tt + n) * LDK + 32 * kb + 8 * gq);
        if (w == 1) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int kb = 0; kb < VB; ++kb)
                    vf[tt][kb] = *reinterpret_cast<const F*>(vtile + (16 * tt + n) * DV + 32 * kb + 8 * gq);
        }
        lds_barrier();   // both wavefronts have their fragments: the regions are free
        if (w == 1) {
            const long cs = (long)hk * DK + 8 * l16;
            bf16* qdst = lh % grpv == 0 ? li.qhat + ((lb * li.Hk + hk) * T + lt0) * DK + 8 * l16 : nullptr;
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const int r0 = 16 * lg + 8 * run;
                prologue_run8<DK>(xs0 + cs, C, T, lt0 + r0, li.conv_w + cs * 4, cst0 ? cst0 + cs * 3 : nullptr,
                                  true, QSCALE, vtile + r0 * DV + 8 * l16, DV, qdst ? qdst + r0 * DK : nullptr);
            }
            lds_fence();
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    qa[tt][kb] = *reinterpret_cast<const F*>(vtile + (16 * tt + n) * DV + 32 * kb + 8 * gq);
            lds_fence();   // read before V's fragments go over them
        }
    } else {
#pragma unroll
        for (int h = 0; h < TH; ++h) {
            const long tk = tok0 + min(64 * h + lane, L - 1);
            braw[h] = KIND == KIND_SSM ? E{} : beta[tk];
            graw[h] = (KIND == KIND_GATED || KIND == KIND_SSM) ? g[tk] : E{};
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kf[tt][kb] = frag_rows8_g<E>(k + tokk * DK, DK, 16 * tt, 32 * kb, lane, L);
        if (w == 1) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) qa[tt][kb] = frag_rows8_g<E>(q + tokk * DK, DK, 16 * tt, 32 * kb, lane, L);
            if (!LATE_V) {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int kb = 0; kb < VB; ++kb) vf[tt][kb] = frag_rows8_g<E>(v + tok0 * DV, DV, 16 * tt, 32 * kb, lane, L);
            }
        }
    }

    // per-token tables (each wavefront its own copy; wave 0 stores the per-token
    // e^G and the chunk decay e^{G_C}, replicated per key channel)
    float* Gs = tab[w][0];
    float* sX = tab[w][1];
    float* sK = tab[w][2];
    float* bs = tab[w][3];
    {
        // the state-space kind has no write strength and no correction: beta = 1
        // (so u = V) and a zero beta e^G table (so W = 0)
        float bv[TH], gv[TH];
#pragma unroll
        for (int h = 0; h < TH; ++h) {
            bv[h] = KIND == KIND_SSM ? 1.f : to_f32(braw[h]);
            gv[h] = to_f32(graw[h]);
            if (64 * h + lane >= L) bv[h] = gv[h] = 0.f;
        }
        const float eGC = token_tables<CH>(bv, gv, lane, Gs, sX, sK, bs, w == 0 ? eg : nullptr);
        if (KIND == KIND_SSM) {
#pragma unroll
            for (int h = 0; h < TH; ++h)
                if (CH >= 64 || 64 * h + lane < CH) sX[64 * h + lane] = 0.f;
        }
        if (w == 0)
            for (int ch = lane; ch < DK; ch += 64) gam[ch] = eGC;
    }

    if (w == 0) {
        lds_fence();   // tables written
        // ---- 2. A = strict_tril(beta_i K K^T exp(G_i - G_j)) into LDS (fp32)
#pragma unroll
        for (int it = 0; it < NT; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
                f32x4 s = zero4();   // (state-space kind: A = 0, so T = I)
                if constexpr (KIND != KIND_SSM) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) s = mma(kf[it][kb], kf[jt][kb], s);
                }
                const int j = 16 * jt + n;
                const float Gj = Gs[j];
                const f32x4 Gi = *reinterpret_cast<const f32x4*>(Gs + 16 * it + 4 * gq);
                const f32x4 bi = *reinterpret_cast<const f32x4*>(bs + 16 * it + 4 * gq);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * it + 4 * gq + e;
                    const float val = bi[e] * __expf(Gi[e] - Gj) * s[e];   // inf above the diagonal is dropped
                    As[i * LDF + j] = (i > j) ? val : 0.f;
                }
            }
        lds_fence();   // A is written

        // ---- 3. UT transform T = (I + A)^-1, blocked over 16x16 tiles
        // 3a: diagonal blocks by forward substitution, lane (block 4p + gq,
        //     column n): T_jj = 1, T_ij = -sum_{j <= m < i} A_im T_mj; written
        //     over the block of A
#pragma unroll
        for (int pass = 0; pass < (NT + 3) / 4; ++pass) {
            const int blkd = 4 * pass + gq;
            if (NT % 4 == 0 || blkd < NT) {
                const int b0 = 16 * blkd, j = n;
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
        }
        lds_fence();
        // 3b: T_IJ = -T_II sum_{J <= K < I} A_IK T_KJ on the matrix cores (fp32),
        //     the column tiles J interleaved
        f32x4 tm[NT][NT];
#pragma unroll
        for (int J = 0; J < NT; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) tm[J][J][e] = As[(16 * J + 4 * gq + e) * LDF + 16 * J + n];
#pragma unroll
        for (int I = 1; I < NT; ++I) {
#pragma unroll
            for (int J = 0; J < I; ++J) {
                f32x4 R = zero4();
#pragma unroll
                for (int K = J; K < I; ++K) R = mma16_lds_reg(As + 16 * I * LDF + 16 * K, LDF, lane, tm[K][J], R);
                tm[I][J] = -mma16_lds_reg(As + 16 * I * LDF + 16 * I, LDF, lane, R, zero4());
            }
        }
        lds_fence();   // every read of A and of the diagonal blocks has returned
        // T diag(beta e^G) and T diag(beta) (lower triangular) in the operand
        // type, over the fp32 region; lane (gq, n) holds column 16J + n of tile (I, J)
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            const float cx = sX[16 * J + n], cb = bs[16 * J + n];
#pragma unroll
            for (int I = 0; I < NT; ++I)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int o = (16 * I + 4 * gq + e) * LDT + 16 * J + n;
                    Tw[o] = from_f32<E>(I >= J ? tm[I][J][e] * cx : 0.f);
                    Tu[o] = from_f32<E>(I >= J ? tm[I][J][e] * cb : 0.f);
                }
        }
    } else {
        // ---- 2'. attn = tril(Q K^T exp(G_i - G_j)) as A-fragments: attn^T tiles
        //          (rows j) stacked over two j tiles
        lds_fence();   // tables written
#pragma unroll
        for (int it = 0; it < NT; ++it) {
            f32x4 at[NT];
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) {
                at[jt] = zero4();
                if (jt <= it) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) at[jt] = mma(kf[jt][kb], qa[it][kb], at[jt]);
                    const int i = 16 * it + n;
                    const float Gi = Gs[i];
                    const f32x4 Gj = *reinterpret_cast<const f32x4*>(Gs + 16 * jt + 4 * gq);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 16 * jt + 4 * gq + e;
                        const float val = __expf(Gi - Gj[e]) * at[jt][e];   // inf above the diagonal is dropped
                        at[jt][e] = (i >= j) ? val : 0.f;
                    }
                }
            }
#pragma unroll
            for (int kb = 0; kb < CB; ++kb) Af[(it * CB + kb) * 64 + lane] = frag_from_tiles<E>(at[2 * kb], at[2 * kb + 1]);
        }
        if (LATE_V) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int kb = 0; kb < VB; ++kb) vf[tt][kb] = frag_rows8_g<E>(v + tok0 * DV, DV, 16 * tt, 32 * kb, lane, L);
        }
        // K and V with tokens as the contraction index (D = K I): K as
        // B-fragments (kept for W = T diag(beta e^G) K), K~^T = (e^{G_C - G} K)^T
        // as A-fragments (stored), V as B-fragments (to wavefront 0 through LDS)
        const F id0 = ident8_frag<E>(0, lane), id1 = ident8_frag<E>(1, lane);
#pragma unroll
        for (int nt = 0; nt < VT; ++nt) {
            f32x4 d[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) d[tt] = mma(vf[tt][nt >> 1], (nt & 1) ? id1 : id0, zero4());
#pragma unroll
            for (int kt = 0; kt < CB; ++kt) Vl[(nt * CB + kt) * 64 + lane] = frag_from_tiles<E>(d[2 * kt], d[2 * kt + 1]);
        }
        F xf[CT][CB];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x4 d[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) d[tt] = mma(kf[tt][ct >> 1], (ct & 1) ? id1 : id0, zero4());
#pragma unroll
            for (int kt = 0; kt < CB; ++kt) {
                xf[ct][kt] = frag_from_tiles<E>(d[2 * kt], d[2 * kt + 1]);
                Kf[(ct * CB + kt) * 64 + lane] = frag_from_tiles_rs<E>(d[2 * kt], d[2 * kt + 1], sK, 32 * kt, lane);
            }
        }
        lds_barrier();   // T diag(.) and V are in LDS

        // ---- 4. W = T diag(beta e^G) K: W^T tiles (rows = key channels) for each
        //         token tile, stacked over channel tiles = A-fragments of W
        //         (the state-space kind has W = 0, which its scan does not read:
        //         not written)
        if constexpr (KIND != KIND_SSM) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                F tf[CB];
#pragma unroll
                for (int kt = 0; kt < CB; ++kt) tf[kt] = frag_rows<E>(Tw, LDT, 16 * tt, 32 * kt, lane);
                f32x4 wt[CT];
#pragma unroll
                for (int mt = 0; mt < CT; ++mt) {
                    wt[mt] = zero4();
#pragma unroll
                    for (int kt = 0; kt < CB; ++kt) wt[mt] = mma(xf[mt][kt], tf[kt], wt[mt]);
                }
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) Wf[(tt * KB + kb) * 64 + lane] = frag_from_tiles<E>(wt[2 * kb], wt[2 * kb + 1]);
            }
        }
        return;
    }
    lds_barrier();   // (wavefront 0) T diag(.) and V are in LDS

    // ---- 5. u = T diag(beta) V as D-tiles (rows = tokens), value tile by value tile
    F tu[NT][CB];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int kt = 0; kt < CB; ++kt) tu[tt][kt] = frag_rows<E>(Tu, LDT, 16 * tt, 32 * kt, lane);
#pragma unroll
    for (int nt = 0; nt < VT; ++nt) {
        F vb[CB];
#pragma unroll
        for (int kt = 0; kt < CB; ++kt) vb[kt] = Vl[(nt * CB + kt) * 64 + lane];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kt = 0; kt < CB; ++kt) acc = mma(tu[tt][kt], vb[kt], acc);
            V4 u4;
#pragma unroll
            for (int e = 0; e < 4; ++e) u4[e] = from_f32<E>(acc[e]);
            Uf[(nt * NT + tt) * 64 + lane] = u4;
        }
    }
}

// Chunks of CH tokens (64 unless stated); past 64 the fragments need the whole
// register file, one unit per SIMD pair.
template <typename E, int DK, int DV, int KIND, int CH = CHUNK>
__global__ __launch_bounds__(128, CH > 64 ? 1 : 2) void chunk_prep2_kernel(const E* __restrict__ q,
                                                                           const E* __restrict__ k,
                                                                           const E* __restrict__ v,
                                                                           const E* __restrict__ beta,
                                                                           const E* __restrict__ g,
                                                                           char* __restrict__ ws, int T,
                                                                           int nchunks, HeadMap hm) {
    __shared__ Prep2Lds<E, DK, DV, CH> lds;
    const long item = blockIdx.x;
    const long bh = item / nchunks;
    const int t0 = (int)(item % nchunks) * CH;
    prep2_item<E, DK, DV, KIND, CH>(q, k, v, beta, g, ws + item * WsLayout<E, DK, DV, CH>::BYTES, lds,
                                    bh * T + t0, hm.key(bh) * T + t0, min(CH, T - t0),
                                    (int)(threadIdx.x >> 6), (int)(threadIdx.x & 63));
}

// The prep of the gated layer's prefill: one item per (head row, chunk) as
// chunk_prep2_kernel, the layer's prologue formed in the item's load stage
// (prep2_item with LAYER) instead of read from q, k, v, beta, g.
template <int KIND>
__global__ __launch_bounds__(128, 2) void chunk_prep2_layer_kernel(LayerIn li, char* __restrict__ ws,
                                                                  int nchunks) {
    __shared__ Prep2Lds<bf16, 128, 128> lds;
    const long item = blockIdx.x;
    const long bh = item / nchunks;
    const int c = (int)(item % nchunks);
    const long t0 = (long)c * CHUNK;
    prep2_item<bf16, 128, 128, KIND, CHUNK, true>(nullptr, nullptr, nullptr, nullptr, nullptr,
                                                  ws + item * WsLayout<bf16, 128, 128>::BYTES, lds, 0, 0,
                                                  (int)min((long)CHUNK, li.T - t0), (int)(threadIdx.x >> 6),
                                                  (int)(threadIdx.x & 63), li, bh / li.Hv, (int)(bh % li.Hv), t0);
}

// The same prep as the recomputation after a one-launch call: it runs only if
// that launch's hand-off failed (its error word holds gval). Launched with few
// workgroups that take the items in turn, so that the usual case (nothing to
// do) costs one round of workgroups.
template <typename E, int DK, int DV, int KIND>
__global__ __launch_bounds__(128, 2) void chunk_prep2_redo_kernel(const E* __restrict__ q,
                                                                  const E* __restrict__ k,
                                                                  const E* __restrict__ v,
                                                                  const E* __restrict__ beta,
                                                                  const E* __restrict__ g,
                                                                  char* __restrict__ ws, int T,
                                                                  int nchunks, long nitems, HeadMap hm,
                                                                  const unsigned long long* guard,
                                                                  unsigned long long gval) {
    if (__hip_atomic_load(guard, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gval) return;
    __shared__ Prep2Lds<E, DK, DV> lds;
    for (long item = blockIdx.x; item < nitems; item += gridDim.x) {
        const long bh = item / nchunks;
        const int t0 = (int)(item % nchunks) * CHUNK;
        // a lane index the compiler cannot see to be the same in every
        // iteration (see chunk_fused_kernel): without it the item's
        // lane-dependent offsets were held across iterations and spilled
        int ln;
        asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"((int)(threadIdx.x & 63)));
        prep2_item<E, DK, DV, KIND>(q, k, v, beta, g, ws + item * WsLayout<E, DK, DV>::BYTES, lds,
                                    bh * T + t0, hm.key(bh) * T + t0, min(CHUNK, T - t0),
                                    (int)(threadIdx.x >> 6), ln);
        if (item + gridDim.x < nitems) lds_barrier();   // both wavefronts are done with the LDS
    }
}

// Packed sequences of different lengths: item = head * nchunks + global chunk;
// the chunk's first token and length come from the chunk table (slots past the
// last chunk have length 0 and are skipped).
template <typename E, int DK, int DV, int KIND>
__global__ __launch_bounds__(128, 2) void chunk_prep2_varlen_kernel(const E* __restrict__ q,
                                                                    const E* __restrict__ k,
                                                                    const E* __restrict__ v,
                                                                    const E* __restrict__ beta,
                                                                    const E* __restrict__ g,
                                                                    char* __restrict__ ws, int T,
                                                                    int nchunks,
                                                                    const int2* __restrict__ ctab) {
    __shared__ Prep2Lds<E, DK, DV> lds;
    const long item = blockIdx.x;
    const int2 e = ctab[item % nchunks];
    if (e.y == 0) return;
    const long tok0 = (item / nchunks) * T + e.x;
    prep2_item<E, DK, DV, KIND>(q, k, v, beta, g, ws + item * WsLayout<E, DK, DV>::BYTES, lds,
                                tok0, tok0, e.y, (int)(threadIdx.x >> 6), (int)(threadIdx.x & 63));
}

// ---------------------------------------------------------------------------
// Scan kernel
// ---------------------------------------------------------------------------
// One wavefront per 16-token tile of a CH-token chunk (NW = CH / 16); each owns
// DK / NW key rows of the state (MTW tiles of 16).
template <typename E, int DK, int DV, int BV, int KIND, int CH = CHUNK>
struct ScanOps {
    typedef typename Frag<E>::type F;
    typedef typename Vec4<E>::type V4;
    static constexpr int NW = CH / 16;          // wavefronts = token tiles
    static constexpr int CB = CH / 32;          // contraction blocks over tokens
    static constexpr int KB = DK / 32;          // contraction blocks over key channels
    static constexpr int MTW = DK / (16 * NW);  // key-channel tiles per wave
    static_assert(MTW >= 1 && MTW * 16 * NW == DK, "key rows split evenly over the wavefronts");
    static constexpr int NT = BV / 16;          // value tiles (16 columns) per workgroup
    typedef typename Vec16<E>::type V16;
    // Gated / DeltaNet: the wave's 16 rows of Q as loaded (row-major, 16 bytes
    // per lane per load); KDA: Q~ as A-fragments from the workspace
    static constexpr int QR = 16 * DK * (int)sizeof(E) / (64 * 16);
    F w[KB], q[KB], a[CB], k[MTW][CB];
    V16 qr[QR];
    V4 u[NT];
    // chunk decay: KDA per key channel of the wave's rows (D-tile order),
    // otherwise one value for the whole state (in gam[0][0])
    f32x4 gam[KIND == KIND_KDA ? MTW : 1], eg;
};

// Where the operands of one chunk are: its workspace block and its rows of Q,
// of which the first L are in the sequence.
template <typename E>
struct ChunkSrc {
    const char* blk;
    const E* q;
    int L;
};

// Operands of one chunk for wave w of value tile vt, in four parts (one
// coalesced load per lane per fragment). The parts are issued at different
// points of the previous-but-one chunk's step, so the wave never stalls on a
// burst of loads waiting for the memory pipeline to accept them.
template <int PART, int KIND, typename E, int DK, int DV, int BV, int CH>
__device__ __forceinline__ void scan_load_part(ScanOps<E, DK, DV, BV, KIND, CH>& x, const ChunkSrc<E>& src,
                                               int vt, int w, int lane) {
    typedef WsLayout<E, DK, DV, CH> Lw;
    typedef ScanOps<E, DK, DV, BV, KIND, CH> O;
    typedef typename O::F F;
    typedef typename O::V4 V4;
    constexpr int FB = (int)sizeof(F);    // bytes of one fragment per lane
    constexpr int ES = (int)sizeof(E);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(src.blk, (unsigned)Lw::BYTES);
    if (PART == 0) {
        // (the state-space kind has no W: its prep does not write it)
        if (KIND != KIND_SSM) {
#pragma unroll
            for (int kb = 0; kb < O::KB; ++kb)
                x.w[kb] = buf_load<F>(rb, (int)(Lw::W_OFF * ES) + ((w * O::KB + kb) * 64 + lane) * FB);
        }
    } else if (PART == 1) {
        if (KIND == KIND_KDA) {
#pragma unroll
            for (int kb = 0; kb < O::KB; ++kb)
                x.q[kb] = buf_load<F>(rb, (int)(Lw::Q_OFF * ES) + ((w * O::KB + kb) * 64 + lane) * FB);
        } else {
            // contiguous 16-byte loads of the wave's rows; rows past the end of
            // the sequence are outside the descriptor's range and read as zero
            // (their outputs are not written)
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(src.q, (unsigned)(src.L * DK * ES));
#pragma unroll
            for (int i = 0; i < O::QR; ++i)
                x.qr[i] = buf_load<typename O::V16>(rq, (16 * w * DK + (i * 64 + lane) * (16 / ES)) * ES);
        }
    } else if (PART == 2) {
#pragma unroll
        for (int kb = 0; kb < O::CB; ++kb)
            x.a[kb] = buf_load<F>(rb, (int)(Lw::A_OFF * ES) + ((w * O::CB + kb) * 64 + lane) * FB);
#pragma unroll
        for (int m = 0; m < O::MTW; ++m)
#pragma unroll
            for (int kb = 0; kb < O::CB; ++kb)
                x.k[m][kb] = buf_load<F>(rb, (int)(Lw::K_OFF * ES) + (((w * O::MTW + m) * O::CB + kb) * 64 + lane) * FB);
    } else {
        const int gq = lane >> 4;
#pragma unroll
        for (int nt = 0; nt < O::NT; ++nt)
            x.u[nt] = buf_load<V4>(rb, (int)(Lw::U_OFF * ES) + (((vt * O::NT + nt) * O::NW + w) * 64 + lane) * (int)sizeof(V4));
        if (KIND == KIND_KDA) {
#pragma unroll
            for (int m = 0; m < O::MTW; ++m)
                x.gam[m] = buf_load<f32x4>(rb, (int)Lw::GAM_BYTE_OFF + (16 * (w * O::MTW + m) + 4 * gq) * 4);
        } else {
            x.gam[0][0] = buf_load<float>(rb, (int)Lw::GAM_BYTE_OFF);
        }
        if (KIND != KIND_KDA) x.eg = buf_load<f32x4>(rb, (int)Lw::EG_BYTE_OFF + (16 * w + 4 * gq) * 4);
    }
}

template <int KIND, typename E, int DK, int DV, int BV, int CH>
__device__ __forceinline__ void scan_load(ScanOps<E, DK, DV, BV, KIND, CH>& x, const ChunkSrc<E>& src, int vt,
                                          int w, int lane) {
    scan_load_part<0, KIND>(x, src, vt, w, lane);
    scan_load_part<1, KIND>(x, src, vt, w, lane);
    scan_load_part<2, KIND>(x, src, vt, w, lane);
    scan_load_part<3, KIND>(x, src, vt, w, lane);
}

// Keeps the compiler from moving memory operations across this point (the
// load parts stay where they are placed in the step).
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// One head row's sequence as the scan sees it: where its chunk blocks, q rows,
// o rows and states are, and how long it is. For a batch of equal lengths
// row bh holds tokens bh*T ..; for packed sequences of different lengths the
// rows start at the sequence offsets.
struct SeqView {
    const char* wsh;   // the row's first chunk block (its chunks are consecutive)
    long qrow;         // q row of the sequence's first token (key-head row for shared heads)
    long orow;         // o row of the sequence's first token
    long srow;         // index of the row's states in S0 / S_final / boundary states
    int len;           // tokens (>= 1)
    int nchunks;       // ceil(len / 64)
};

// One chunk of the scan for one workgroup: U = u - W S, O = Q~ S + attn U,
// S = gamma S + K~^T U. S (fp32, MFMA accumulator layout) is updated in
// place; the operands of chunk c+2 (`nxt`, from block `nblk`) are loaded in
// parts along the way; the output tile leaves through LDS as 16-byte rows.
template <typename E, int DK, int DV, int KIND, int BV, bool PF, int CH = CHUNK>
__device__ __forceinline__ void scan_step(const ScanOps<E, DK, DV, BV, KIND, CH>& cur,
                                          ScanOps<E, DK, DV, BV, KIND, CH>& nxt, const ChunkSrc<E>& nblk,
                                          f32x4 (&S)[ScanOps<E, DK, DV, BV, KIND, CH>::MTW][BV / 16],
                                          typename Frag<E>::type (*Sx)[BV / 16][64],
                                          typename Frag<E>::type (*Ux)[BV / 16][64], E* ob, E* qs,
                                          E* __restrict__ o, long orow, int len, int t0, int vt,
                                          int w, int lane, const char* pfblk, float& pf) {
    typedef ScanOps<E, DK, DV, BV, KIND, CH> Ops;
    typedef typename Ops::F F;
    typedef typename Ops::V4 V4;
    typedef typename Vec16<E>::type V16;
    constexpr int NT = Ops::NT, KB = Ops::KB, MTW = Ops::MTW, CB = Ops::CB;
    constexpr int LDO = BV + 16 / sizeof(E);   // output staging row (padded)
    const int gq = lane >> 4, n = lane & 15;

    // Gated / DeltaNet: the wave's Q rows go through its own LDS slice
    // (row-major, padded) to become A-fragments
    constexpr int LDQ = DK + 16 / sizeof(E);
    if (KIND != KIND_KDA) {
        constexpr int VEC = 16 / sizeof(E);
#pragma unroll
        for (int i = 0; i < Ops::QR; ++i) {
            const int off = (i * 64 + lane) * VEC;
            *reinterpret_cast<V16*>(qs + (off / DK) * LDQ + off % DK) = cur.qr[i];
        }
    }

    // state -> B-fragments of the contraction over key channels; key-channel
    // block kb covers the key tiles 2kb, 2kb+1: two tiles of one wave (MTW even)
    // or one tile each of the waves 2kb, 2kb+1 (MTW = 1, half a fragment each)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (MTW >= 2) {
#pragma unroll
            for (int m = 0; m < MTW; m += 2)
                Sx[(w * MTW + m) >> 1][nt][lane] = frag_from_tiles<E>(S[m][nt], S[m + 1][nt]);
        } else {
            V4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = from_f32<E>(S[0][nt][e]);
            reinterpret_cast<V4*>(&Sx[w >> 1][nt][lane])[w & 1] = h;
        }
    }
    sched_fence();
    scan_load_part<0, KIND>(nxt, nblk, vt, w, lane);
    lds_barrier();

    F qf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qf[kb] = KIND == KIND_KDA ? cur.q[kb] : frag_rows<E>(qs, LDQ, 0, 32 * kb, lane);
    f32x4 U[NT], O[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        U[nt] = zero4();
        O[nt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const F sb = Sx[kb][nt][lane];
            // state-space kind: W = 0, so U = u without the product (bitwise the same)
            if constexpr (KIND != KIND_SSM) U[nt] = mma(cur.w[kb], sb, U[nt]);
            O[nt] = mma(qf[kb], sb, O[nt]);
        }
        // Gated / DeltaNet: (e^G Q) S = e^G (Q S), per token row
        if (KIND != KIND_KDA) O[nt] *= cur.eg;
    }
    sched_fence();
    scan_load_part<1, KIND>(nxt, nblk, vt, w, lane);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        // (an opaque copy: keeps the compiler from converting this operand
        // steps early, which would make it wait for the newest loads)
        V4 uc = cur.u[nt];
        asm volatile("" : "+v"(uc));
        V4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            U[nt][e] = to_f32(uc[e]) - U[nt][e];
            h[e] = from_f32<E>(U[nt][e]);
        }
        reinterpret_cast<V4*>(&Ux[w >> 1][nt][lane])[w & 1] = h;
    }
    // decay the state (its pre-decay value is already captured in Sx)
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) S[m][nt] *= KIND == KIND_KDA ? cur.gam[m] : cur.gam[0][0];
    sched_fence();
    scan_load_part<2, KIND>(nxt, nblk, vt, w, lane);
    lds_barrier();

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int kb = 0; kb < CB; ++kb) {
            const F ub = Ux[kb][nt][lane];
            O[nt] = mma(cur.a[kb], ub, O[nt]);
#pragma unroll
            for (int m = 0; m < MTW; ++m) S[m][nt] = mma(cur.k[m][kb], ub, S[m][nt]);
        }
        // stage this wave's 16 output rows (token tile w) for row stores
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[(4 * gq + e) * LDO + 16 * nt + n] = from_f32<E>(O[nt][e]);
    }
    sched_fence();
    scan_load_part<3, KIND>(nxt, nblk, vt, w, lane);
    // 16 rows x BV columns: BV*sizeof(E) bytes per row, 16 bytes per lane.
    // Stored through a resource that ends at the sequence's last row, so rows
    // past it (and lanes past the tile, sent out of range) are dropped by the
    // hardware: the stores are unconditional, which lets the compiler count
    // them when it waits for the next step's operands (a store inside a
    // branch made it wait for every memory operation in flight instead).
    constexpr int PER_ROW = BV * sizeof(E) / 16;
    constexpr int VEC = 16 / sizeof(E);
    constexpr int NST = (16 * PER_ROW + 63) / 64;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + (orow + t0) * DV, (unsigned)(min(len - t0, CH) * DV * (int)sizeof(E)));
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int p = lane + 64 * i;
        const bool in = (16 * PER_ROW) % 64 == 0 || p < 16 * PER_ROW;
        const int pp = in ? p : 0;
        const int row = pp / PER_ROW, col = (pp % PER_ROW) * VEC;
        const V16 val = *reinterpret_cast<const V16*>(&ob[row * LDO + col]);
        buf_store16(ro, in ? ((16 * w + row) * DV + vt * BV + col) * (int)sizeof(E) : 0x40000000, val);
    }
    if constexpr (PF) {
        // Pull a later chunk's block from HBM into L2: one 4-byte load per
        // 128-byte line, the lines dealt out over the 4 NV wavefronts of the
        // head's workgroups (lanes past the block's end load nothing). The
        // value is never used; it is waited for only when the register comes
        // round again, RING steps later, so the load never holds up a step.
        asm volatile("" ::"v"(pf));
        constexpr int NV = DV / BV;
        pf = buf_load<float>(make_rsrc(pfblk, (unsigned)WsLayout<E, DK, DV, CH>::BYTES),
                             ((vt * Ops::NW + w) + lane * Ops::NW * NV) * 128);
    }
}

// LDS of one scan workgroup.
template <typename E, int DK, int DV, int KIND, int BV, int CH = CHUNK>
struct ScanLds {
    typedef typename Frag<E>::type F;
    static constexpr int KB = DK / 32, NT = BV / 16, NW = CH / 16, CB = CH / 32;
    static constexpr int LDO = BV + 16 / sizeof(E);   // output staging row (padded)
    static constexpr int LDQ = DK + 16 / sizeof(E);   // Q row (padded)
    F Sx[KB][NT][64];   // state as B-fragments (contraction over key channels)
    F Ux[CB][NT][64];   // U as B-fragments (contraction over tokens)
    __align__(16) E Ob[NW][16 * LDO];                              // per-wave output staging
    __align__(16) E Qs[KIND == KIND_KDA ? 1 : NW][16 * LDQ];      // per-wave Q rows
};

// ---------------------------------------------------------------------------
// Hand-off of workspace blocks from prep wavefronts to scan wavefronts inside
// one launch. A block is published by each of its two producing wavefronts
// with a 64-bit tag once that wavefront's stores to it have completed; the
// tag is the launch's epoch combined with the producer's XCD number, and a
// consumer accepts a block only if both tags equal the epoch combined with
// its own XCD number. Producer and consumer therefore always share an XCD
// and its L2, where completed stores are visible, so no cache write-back or
// invalidation is needed: the consumer has not read the block's lines before
// (the vector L1 starts every launch empty), so it cannot hold stale copies.
// A tag left over from an earlier launch never matches (the epoch is new for
// every launch). Waits are bounded: after `spin` polls (about a second at the
// default) a wavefront marks the launch as failed (it writes the epoch into
// an error word after the tags) and stops waiting; the others stop waiting
// once they see that. A failed launch's results are then recomputed by the
// two phases (kernels enqueued after it that do nothing unless the error word
// holds that launch's epoch), so the call's results are correct either way;
// dn_chunk_fwd_handoff_status reports that it happened.
// ---------------------------------------------------------------------------
typedef unsigned long long u64;
constexpr int SPIN_LIMIT = 1 << 20;

__device__ __forceinline__ unsigned xcc_id() {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return x & 15u;
}
__device__ __forceinline__ u64 xcc_tag(u64 epoch) { return epoch ^ ((u64)xcc_id() << 56); }
__device__ __forceinline__ u64 flag_load(const u64* f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Producer: after this wavefront's stores to the block have completed.
__device__ __forceinline__ void publish(u64* f, u64 tag, int lane) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_store(f, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Consumer: (a, b) are the block's two tags as loaded earlier; poll until both
// equal `tag` (or give up, see above).
__device__ __forceinline__ void wait_block(const u64* f, u64 a, u64 b, u64 tag, u64* err, u64 epoch,
                                        int spin, int lane) {
    if (a == tag && b == tag) return;
    for (int i = 0; i < spin; ++i) {
        __builtin_amdgcn_s_sleep(8);
        a = flag_load(f);
        b = flag_load(f + 1);
        if (a == tag && b == tag) return;
        if ((i & 1023) == 1023 && flag_load(err) == epoch) return;
    }
    if (lane == 0) __hip_atomic_store(err, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Where the hand-off tags live: after the BH * nchunks workspace blocks, two
// 64-bit tags per block, then the error word and the epoch of the last
// one-launch call (see ws_bytes_t for the rest of the tail).
template <typename E, int DK, int DV>
__device__ __forceinline__ u64* block_tags(char* ws, long BH, int nchunks) {
    return reinterpret_cast<u64*>(ws + BH * nchunks * WsLayout<E, DK, DV>::BYTES);
}

// The sequential scan of one (head bh, value tile vt) on four wavefronts.
// SYNC: the chunk blocks are produced concurrently in the same launch and
// each is waited for (tags at `tags`, expected value `tag`) before its
// operands are loaded. RING: 3 (two chunks prefetched) or 2 (one chunk; fewer
// registers held; the Gated DeltaNet one-launch form, where three measured no
// faster).
template <typename E, int DK, int DV, int KIND, int BV, bool SYNC, int RING, bool EMIT = false, int CH = CHUNK>
__device__ __forceinline__ void scan_body(const SeqView sv, const E* __restrict__ q,
                                          const float* __restrict__ S0, E* __restrict__ o,
                                          float* __restrict__ S_final, int vt, int w, int lane,
                                          ScanLds<E, DK, DV, KIND, BV, CH>& lds, const u64* tags,
                                          u64 tag, u64* err, u64 epoch, int spin,
                                          float* __restrict__ S_bound = nullptr) {
    typedef WsLayout<E, DK, DV, CH> Lw;
    typedef ScanOps<E, DK, DV, BV, KIND, CH> Ops;
    constexpr int NT = Ops::NT, MTW = Ops::MTW;
    const int gq = lane >> 4, n = lane & 15;

    // fp32 state tile: rows 16*(w*MTW + m) + 4gq + e, columns vt*BV + 16nt + n
    f32x4 S[MTW][NT];
    if (S0) {
#pragma unroll
        for (int m = 0; m < MTW; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * (w * MTW + m) + 4 * gq + e, col = vt * BV + 16 * nt + n;
                    S[m][nt][e] = S0[(sv.srow * DK + row) * DV + col];
                }
    } else {
#pragma unroll
        for (int m = 0; m < MTW; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) S[m][nt] = zero4();
    }

    // EMIT: the state after chunk cc, S_bound[bh][cc] (fp32 [DK][DV]); written
    // at the end of the step, after its loads, like the output rows
    auto emit = [&](int cc) {
        if constexpr (EMIT) {
            float* Sb = S_bound + (sv.srow * sv.nchunks + cc) * DK * DV;
#pragma unroll
            for (int m = 0; m < MTW; ++m)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * (w * MTW + m) + 4 * gq + e, col = vt * BV + 16 * nt + n;
                        Sb[row * DV + col] = S[m][nt][e];
                    }
        }
    };

    // The operands of the next RING - 1 chunks are in flight while chunk c is
    // processed (RING register sets in rotation). Prefetches are
    // unconditional (the chunk index is clamped to the last chunk):
    // straight-line code lets the compiler wait for exactly the set in use
    // instead of draining every load in flight.
    const char* wsh = sv.wsh;
    const int nchunks = sv.nchunks;
    const int last = nchunks - 1;
    auto blk = [&](int cc) {
        const int c2 = min(cc, last);
        return ChunkSrc<E>{wsh + (long)c2 * Lw::BYTES, q + (sv.qrow + (long)c2 * CH) * DK,
                           min(CH, sv.len - c2 * CH)};
    };
    // SYNC: the tags of the next block to be waited for are loaded one chunk
    // step ahead, so a block that is already published costs no wait
    u64 ta = 0, tb = 0;
    auto tags_of = [&](int cc) { return tags + 2 * min(cc, last); };
    auto ready = [&](int cc) {
        if (SYNC) {
            wait_block(tags_of(cc), ta, tb, tag, err, epoch, spin, lane);
            sched_fence();
            ta = flag_load(tags_of(cc + 1));
            tb = flag_load(tags_of(cc + 1) + 1);
        }
    };
    if (SYNC) {
        ta = flag_load(tags_of(0));
        tb = flag_load(tags_of(0) + 1);
    }
    E* ob = lds.Ob[w];
    E* qs = lds.Qs[KIND == KIND_KDA ? 0 : w];
    // KDA: L2 prefetch of the block RING + 1 chunks ahead (its operands are
    // then loaded into registers two steps later). Measured at d = 128: 5 %
    // off the KDA scan, nothing for the other kinds. Only where every block
    // was written before the launch: a prefetched line that is written later
    // could stay stale in this CU's L1.
    constexpr bool PF = !SYNC && KIND == KIND_KDA;
    auto pfb = [&](int cc) { return wsh + (long)min(cc, last) * Lw::BYTES; };
    float pf0 = 0.f, pf1 = 0.f, pf2 = 0.f;
    (void)pf2;
    // The loops run whole rounds of RING steps with no exit inside (an exit
    // between steps let the compiler sink the next operands' loads past it,
    // to just before their use); the last nchunks mod RING steps follow the
    // loop, with the operands the loop's last round loaded.
    if constexpr (RING == 2) {
        // operands of chunk c + 1 in flight while chunk c is processed
        Ops o0, o1;
        ready(0);
        scan_load<KIND>(o0, blk(0), vt, w, lane);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), see below
        const int cend = nchunks & ~1;
        int c = 0;
        for (; c < cend; c += 2) {
            ready(c + 1);
            scan_step<E, DK, DV, KIND, BV, PF, CH>(o0, o1, blk(c + 1), S, lds.Sx, lds.Ux, ob, qs, o, sv.orow, sv.len, c * CH, vt, w, lane, pfb(c + 3), pf0);
            emit(c);
            ready(c + 2);
            scan_step<E, DK, DV, KIND, BV, PF, CH>(o1, o0, blk(c + 2), S, lds.Sx, lds.Ux, ob, qs, o, sv.orow, sv.len, (c + 1) * CH, vt, w, lane, pfb(c + 4), pf1);
            emit(c + 1);
        }
        if (c < nchunks) {
            ready(c + 1);
            scan_step<E, DK, DV, KIND, BV, PF, CH>(o0, o1, blk(c + 1), S, lds.Sx, lds.Ux, ob, qs, o, sv.orow, sv.len, c * CH, vt, w, lane, pfb(c + 3), pf0);
            emit(c);
        }
    } else {
        // operands of chunks c + 1 and c + 2 in flight while chunk c is processed
        Ops o0, o1, o2;
        ready(0);
        scan_load<KIND>(o0, blk(0), vt, w, lane);
        ready(1);
        scan_load<KIND>(o1, blk(1), vt, w, lane);
        // Wait here for the sets loaded above: the loop then starts from the
        // same outstanding loads on entry as on every later iteration, and the
        // compiler waits in it for the set each step uses rather than (on the
        // strength of the entry path) for nearly everything in flight.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        const int cend = nchunks - nchunks % 3;
        int c = 0;
        for (; c < cend; c += 3) {
            ready(c + 2);
            scan_step<E, DK, DV, KIND, BV, PF, CH>(o0, o2, blk(c + 2), S, lds.Sx, lds.Ux, ob, qs, o, sv.orow, sv.len, c * CH, vt, w, lane, pfb(c + 4), pf0);
            emit(c);
            ready(c + 3);
            scan_step<E, DK, DV, KIND, BV, PF, CH>(o1, o0, blk(c + 3), S, lds.Sx, lds.Ux, ob, qs, o, sv.orow, sv.len, (c + 1) * CH, vt, w, lane, pfb(c + 5), pf1);
            emit(c + 1);
            ready(c + 4);
            scan_step<E, DK, DV, KIND, BV, PF, CH>(o2, o1, blk(c + 4), S, lds.Sx, lds.Ux, ob, qs, o, sv.orow, sv.len, (c + 2) * CH, vt, w, lane, pfb(c + 6), pf2);
            emit(c + 2);
        }
        if (c < nchunks) {
            ready(c + 2);
            scan_step<E, DK, DV, KIND, BV, PF, CH>(o0, o2, blk(c + 2), S, lds.Sx, lds.Ux, ob, qs, o, sv.orow, sv.len, c * CH, vt, w, lane, pfb(c + 4), pf0);
            emit(c);
            if (c + 1 < nchunks) {
                ready(c + 3);
                scan_step<E, DK, DV, KIND, BV, PF, CH>(o1, o0, blk(c + 3), S, lds.Sx, lds.Ux, ob, qs, o, sv.orow, sv.len, (c + 1) * CH, vt, w, lane, pfb(c + 5), pf1);
                emit(c + 1);
            }
        }
    }

    if (S_final) {
#pragma unroll
        for (int m = 0; m < MTW; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * (w * MTW + m) + 4 * gq + e, col = vt * BV + 16 * nt + n;
                    S_final[(sv.srow * DK + row) * DV + col] = S[m][nt][e];
                }
    }
}

template <typename E, int DK, int DV, int KIND, int BV, bool EMIT, int CH = CHUNK>
__global__ __launch_bounds__(4 * CH) void chunk_scan_kernel(const char* __restrict__ ws,
                                                         const E* __restrict__ q,
                                                         const float* __restrict__ S0,
                                                         E* __restrict__ o,
                                                         float* __restrict__ S_final, int T,
                                                         int nchunks, int BH,
                                                         float* __restrict__ S_bound, HeadMap hm,
                                                         const unsigned long long* guard,
                                                         unsigned long long gval) {
    // guard != NULL: recomputation after a one-launch call, done only if that
    // launch's hand-off failed (its error word holds gval)
    if (guard && __hip_atomic_load(guard, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gval) return;
    constexpr int NV = DV / BV;
    // XCD-aware mapping: consecutive workgroups go to different XCDs
    // (round-robin over 8); the NV value tiles of one head share an XCD so
    // that their common operands (W, Q~, K~^T, attn) hit the same L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vt = slot % NV;
    const long bh = (long)(slot / NV) * 8 + xcd;
    if (bh >= BH) return;
    __shared__ ScanLds<E, DK, DV, KIND, BV, CH> lds;
    const SeqView sv{ws + bh * nchunks * WsLayout<E, DK, DV, CH>::BYTES, hm.key(bh) * T, bh * T, bh, T,
                     nchunks};
    scan_body<E, DK, DV, KIND, BV, false, 3, EMIT, CH>(sv, q, S0, o, S_final, vt, (int)(threadIdx.x >> 6),
                                                    (int)(threadIdx.x & 63), lds, nullptr, 0, nullptr, 0, 0,
                                                    S_bound);
}

// The scan over packed sequences: one workgroup per (sequence n, head h, value
// tile), state row n * H + h; the sequence's chunks are the global chunks
// cs[n] .. cs[n+1] - 1 of head h. Sequence bounds are clamped to [0, T].
template <typename E, int DK, int DV, int KIND, int BV>
__global__ __launch_bounds__(256) void chunk_scan_varlen_kernel(const char* __restrict__ ws,
                                                                const E* __restrict__ q,
                                                                const float* __restrict__ S0,
                                                                E* __restrict__ o,
                                                                float* __restrict__ S_final, int T,
                                                                int nchunks, int N, int H,
                                                                const int* __restrict__ cu,
                                                                const int* __restrict__ cs) {
    constexpr int NV = DV / BV;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vt = slot % NV;
    const long bh = (long)(slot / NV) * 8 + xcd;
    if (bh >= (long)N * H) return;
    const int n = (int)(bh / H), h = (int)(bh % H);
    const int start = min(max(cu[n], 0), T);
    const int len = min(max(cu[n + 1], start), T) - start;
    if (len == 0) {
        // empty sequence: the state passes through
        if (S_final)
            for (int i = threadIdx.x; i < DK * BV; i += 256) {
                const long at = (bh * DK + i / BV) * DV + vt * BV + i % BV;
                S_final[at] = S0 ? S0[at] : 0.f;
            }
        return;
    }
    __shared__ ScanLds<E, DK, DV, KIND, BV> lds;
    const long row = (long)h * T + start;
    const SeqView sv{ws + ((long)h * nchunks + cs[n]) * WsLayout<E, DK, DV>::BYTES, row, row, bh,
                     len, (len + CHUNK - 1) / CHUNK};
    scan_body<E, DK, DV, KIND, BV, false, 3>(sv, q, S0, o, S_final, vt, (int)(threadIdx.x >> 6),
                                          (int)(threadIdx.x & 63), lds, nullptr, 0, nullptr, 0, 0);
}

// Chunk offsets of packed sequences (one workgroup): cs[n] = sum over m < n of
// ceil(len_m / 64), n = 0..N, with len_m = cu[m+1] - cu[m] clamped to [0, T].
__global__ __launch_bounds__(1024) void varlen_chunks_kernel(const int* __restrict__ cu, int N, int T,
                                                             int* __restrict__ cs) {
    __shared__ int part[1024];
    const int t = threadIdx.x;
    const int per = (N + 1023) / 1024;
    const int m0 = min(t * per, N), m1 = min(m0 + per, N);
    auto chunks = [&](int m) {
        const int a = min(max(cu[m], 0), T);
        const int b = min(max(cu[m + 1], a), T);
        return (b - a + CHUNK - 1) / CHUNK;
    };
    int sum = 0;
    for (int m = m0; m < m1; ++m) sum += chunks(m);
    part[t] = sum;
    __syncthreads();
    // inclusive scan of the per-thread sums (Hillis-Steele over 1024 entries)
    for (int off = 1; off < 1024; off <<= 1) {
        const int x = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    int run = part[t] - sum;   // exclusive prefix of this thread's range
    for (int m = m0; m < m1; ++m) {
        cs[m] = run;
        run += chunks(m);
    }
    if (t == 1023) cs[N] = part[1023];
}

// Chunk table of packed sequences: entry gc (global chunk) = (first token of
// the chunk in its head row, tokens in it); (0, 0) past the last chunk.
__global__ __launch_bounds__(256) void varlen_table_kernel(const int* __restrict__ cu,
                                                           const int* __restrict__ cs, int N, int T,
                                                           int nchunks, int2* __restrict__ ctab) {
    const int gc = blockIdx.x * 256 + threadIdx.x;
    if (gc >= nchunks) return;
    if (gc >= cs[N]) {
        ctab[gc] = make_int2(0, 0);
        return;
    }
    // the sequence n with cs[n] <= gc < cs[n + 1] (cs is nondecreasing)
    int lo = 0, hi = N;   // invariant: cs[lo] <= gc < cs[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cs[mid] <= gc) lo = mid;
        else hi = mid;
    }
    const int a = min(max(cu[lo], 0), T);
    const int b = min(max(cu[lo + 1], a), T);
    const int base = a + (gc - cs[lo]) * CHUNK;
    ctab[gc] = make_int2(base, min(CHUNK, b - base));
}

// ---------------------------------------------------------------------------
// Fused prefill: prep and scan in one launch (Gated DeltaNet / DeltaNet).
// ---------------------------------------------------------------------------
// Workgroup b runs on XCD b % 8 (the hardware deals workgroups out to the
// eight XCDs round-robin, starting over with every launch) and serves the
// heads h = x, x + 8, ... of its XCD x. On each XCD the first NP workgroups
// are prep workgroups: two units of two wavefronts, each unit taking the
// XCD's (chunk, head) items in chunk-major order, so that every head's early
// chunks come first. The workgroups after them are the scan workgroups of
// the XCD's heads, one per (head, value tile), exactly as in the scan kernel,
// except that each chunk block is waited for before it is loaded.
// Workgroups start in index order, so every prep workgroup of an XCD has
// started before the first scan workgroup there waits, and prep wavefronts
// never wait on anything: every wait ends.
template <typename E, int DK, int DV, int KIND, int BV>
union FusedLds {
    Prep2Lds<E, DK, DV> prep[2];
    ScanLds<E, DK, DV, KIND, BV> scan;
};

template <typename E, int DK, int DV, int KIND, int BV>
__global__ __launch_bounds__(256, 2) void chunk_fused_kernel(const E* __restrict__ q,
                                                             const E* __restrict__ k,
                                                             const E* __restrict__ v,
                                                             const E* __restrict__ beta,
                                                             const E* __restrict__ g,
                                                             char* __restrict__ ws,
                                                             const float* __restrict__ S0,
                                                             E* __restrict__ o,
                                                             float* __restrict__ S_final, int T,
                                                             int nchunks, int BH, int NP, u64 epoch,
                                                             int spin, HeadMap hm) {
    typedef WsLayout<E, DK, DV> Lw;
    constexpr int NV = DV / BV;
    __shared__ FusedLds<E, DK, DV, KIND, BV> lds;
    const int xcd = blockIdx.x & 7, s = blockIdx.x >> 3;
    const int nh = xcd < BH ? (BH - 1 - xcd) / 8 + 1 : 0;   // heads xcd, xcd + 8, ...
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    u64* tags = block_tags<E, DK, DV>(ws, BH, nchunks);
    u64* err = tags + 2L * BH * nchunks;
    const u64 tag = xcc_tag(epoch);
    // the epoch of the latest one-launch call on this workspace, for the
    // status query (the word after the error word)
    if (blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store(err + 1, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    if (s < NP) {
        const int unit = w >> 1, wu = w & 1;
        const long total = (long)nh * nchunks;
        for (long m0 = 2L * s; m0 < total; m0 += 2L * NP) {
            const long m = m0 + unit;
            if (m < total) {
                const int c = (int)(m / nh);
                const long bh = xcd + 8L * (m % nh);
                // a lane index the compiler cannot see to be the same in every
                // iteration, so that it keeps the item's lane-dependent offsets
                // and constants inside the loop instead of holding them in
                // registers across it
                int ln;
                asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
                const int t0 = c * CHUNK;
                prep2_item<E, DK, DV, KIND>(q, k, v, beta, g, ws + (bh * nchunks + c) * Lw::BYTES,
                                            lds.prep[unit], bh * T + t0, hm.key(bh) * T + t0,
                                            min(CHUNK, T - t0), wu, ln);
                publish(tags + 2 * (bh * nchunks + c) + wu, tag, ln);
            } else {
                lds_barrier();   // the item's one barrier, passed with the other unit
            }
            lds_barrier();   // this item's LDS reads are done before the next item writes
        }
        return;
    }
    const int slot = s - NP, vt = slot % NV, i = slot / NV;
    if (i >= nh) return;
    const long bh = xcd + 8L * i;
    const SeqView sv{ws + bh * nchunks * Lw::BYTES, hm.key(bh) * T, bh * T, bh, T, nchunks};
    scan_body<E, DK, DV, KIND, BV, true, 2>(sv, q, S0, o, S_final, vt, w, lane, lds.scan,
                                         tags + 2 * bh * nchunks, tag, err, epoch, spin);
}

// ---------------------------------------------------------------------------
// Fused prefill for KDA: the same hand-off as above, with the four-wavefront
// KDA prep as the prep workgroups.
// ---------------------------------------------------------------------------
// On each XCD the first NP workgroups each take the XCD's (chunk, head)
// items in chunk-major order, one item at a time on all four wavefronts;
// after an item every wavefront waits for its stores, and once all four
// have passed a barrier one of them publishes the block's two tags. The
// workgroups after them scan the XCD's heads exactly as in chunk_fused_kernel.
// KDA's prep is bound by the SIMDs' issue (exponentials), so the prep gets
// every workgroup slot the scan leaves free, and the scan takes wide value
// tiles (fewer scan workgroups). The scan keeps two chunks of operands in
// flight, as in the two-phase form (2-3 % faster than one here; the
// matrix-core accumulators in vector registers leave room for both roles).
// Measured at 2x16x8192: 243 us with every free slot taken by the prep,
// against 260 us with 40 prep workgroups per XCD and 292 us with 32.
template <typename E, int D, int BV>
union FusedKdaLds {
    KdaPrepLds<E, D, D> prep;
    ScanLds<E, D, D, KIND_KDA, BV> scan;
};

template <typename E, int D, int BV>
__global__ __launch_bounds__(256, 2) void chunk_fused_kda_kernel(const E* __restrict__ q,
                                                                 const E* __restrict__ k,
                                                                 const E* __restrict__ v,
                                                                 const E* __restrict__ beta,
                                                                 const E* __restrict__ g,
                                                                 char* __restrict__ ws,
                                                                 const float* __restrict__ S0,
                                                                 E* __restrict__ o,
                                                                 float* __restrict__ S_final, int T,
                                                                 int nchunks, int BH, int NP, u64 epoch,
                                                                 int spin, HeadMap hm) {
    typedef WsLayout<E, D, D> Lw;
    constexpr int NV = D / BV;
    __shared__ FusedKdaLds<E, D, BV> lds;
    const int xcd = blockIdx.x & 7, s = blockIdx.x >> 3;
    const int nh = xcd < BH ? (BH - 1 - xcd) / 8 + 1 : 0;   // heads xcd, xcd + 8, ...
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    u64* tags = block_tags<E, D, D>(ws, BH, nchunks);
    u64* err = tags + 2L * BH * nchunks;
    const u64 tag = xcc_tag(epoch);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store(err + 1, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    if (s < NP) {
        const long total = (long)nh * nchunks;
        for (long m = s; m < total; m += NP) {
            const int c = (int)(m / nh);
            const long bh = xcd + 8L * (m % nh);
            int ln;   // (see chunk_fused_kernel)
            asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
            const int t0 = c * CHUNK;
            kda_prep4_item<E, D, D>(q, k, v, beta, g, ws + (bh * nchunks + c) * Lw::BYTES, lds.prep, bh * T + t0,
                                    hm.key(bh) * T + t0, min(CHUNK, T - t0), w, ln);
            // every wavefront's stores to the block have completed before the
            // barrier; the tags follow it (the barrier also keeps the next
            // item's LDS writes behind this item's reads)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            if (w == 0 && ln == 0) {
                __hip_atomic_store(tags + 2 * (bh * nchunks + c), tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(tags + 2 * (bh * nchunks + c) + 1, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        return;
    }
    const int slot = s - NP, vt = slot % NV, i = slot / NV;
    if (i >= nh) return;
    const long bh = xcd + 8L * i;
    const SeqView sv{ws + bh * nchunks * Lw::BYTES, hm.key(bh) * T, bh * T, bh, T, nchunks};
    scan_body<E, D, D, KIND_KDA, BV, true, 3>(sv, q, S0, o, S_final, vt, w, lane, lds.scan,
                                           tags + 2 * bh * nchunks, tag, err, epoch, spin);
}

// KDA's prep as the recomputation after a one-launch call: it runs only if
// that launch's hand-off failed (its error word holds gval); few workgroups
// take the items in turn.
template <typename E, int D>
__global__ __launch_bounds__(256, 2) void chunk_prep_kda_redo_kernel(const E* __restrict__ q,
                                                                     const E* __restrict__ k,
                                                                     const E* __restrict__ v,
                                                                     const E* __restrict__ beta,
                                                                     const E* __restrict__ g,
                                                                     char* __restrict__ ws, int T, int nchunks,
                                                                     long nitems, HeadMap hm,
                                                                     const unsigned long long* guard,
                                                                     unsigned long long gval) {
    if (__hip_atomic_load(guard, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gval) return;
    __shared__ KdaPrepLds<E, D, D> lds;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (long item = blockIdx.x; item < nitems; item += gridDim.x) {
        const long bh = item / nchunks;
        const int t0 = (int)(item % nchunks) * CHUNK;
        int ln;   // (see chunk_fused_kernel)
        asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
        kda_prep4_item<E, D, D>(q, k, v, beta, g, ws + item * WsLayout<E, D, D>::BYTES, lds, bh * T + t0,
                                hm.key(bh) * T + t0, min(CHUNK, T - t0), w, ln);
        if (item + gridDim.x < nitems) lds_barrier();   // every wavefront is done with the LDS
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Compute units of the current device (queried once per device).
static int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// The chunk blocks, then the words of the one-launch form: two 64-bit
// hand-off tags per block, the error word and the latest epoch (padded to 256
// bytes), then a copy of the start state [BH][D][D] fp32 (the one-launch
// form may overwrite S0 in place before a failed hand-off is recomputed).
template <typename E, int D>
static long long ws_tail_off(long long BH, long long nchunks) {
    return BH * nchunks * WsLayout<E, D, D>::BYTES;
}
template <typename E, int D>
static long long ws_s0copy_off(long long BH, long long nchunks) {
    return ws_tail_off<E, D>(BH, nchunks) + (BH * nchunks * 16 + 16 + 255) / 256 * 256;
}
template <typename E, int D>
static size_t ws_bytes_t(long long BH, long long nchunks) {
    return (size_t)(ws_s0copy_off<E, D>(BH, nchunks) + BH * D * D * 4);
}

size_t chunk_workspace_bytes(long long BH, long long T, int dk, int dv, int dtype) {
    (void)dv;
    const long long nchunks = (T + CHUNK - 1) / CHUNK;
    if (dtype == DT_BF16) return dk == 128 ? ws_bytes_t<bf16, 128>(BH, nchunks) : ws_bytes_t<bf16, 64>(BH, nchunks);
    return dk == 128 ? ws_bytes_t<float, 128>(BH, nchunks) : ws_bytes_t<float, 64>(BH, nchunks);
}

// Value tile width of the scan for BH heads (shared by the scan and the fused launch).
template <int D>
static int scan_bv(int BH) {
    return ((long)BH * (D / 32) >= 256 || D == 64) ? 32 : 16;
}

template <typename E, int D, int KIND>
static hipError_t prep_t(const void* q, const void* k, const void* v, const void* beta,
                         const void* g, void* ws, int BH, int T, hipStream_t st, HeadMap hm) {
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    const int nitems = nchunks * BH;
    if constexpr (KIND == KIND_KDA) {
        return launch_kda_prep<E, D>(q, k, v, beta, g, ws, nitems, T, nchunks, hm, nullptr, st);
    } else if constexpr (sizeof(E) == 2 || D == 64) {
        // two wavefronts per chunk where their fragments fit in 256 registers
        hipLaunchKernelGGL((chunk_prep2_kernel<E, D, D, KIND>), dim3((unsigned)nitems), dim3(128), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g,
                           (char*)ws, T, nchunks, hm);
        return hipGetLastError();
    } else {
        // persistent workgroups: as many as fit on the device at once (LDS bound)
        constexpr long lds = PrepSmem<E, D, D, KIND>::TOTAL + 1024;
        constexpr int per_cu = (int)(163840 / lds) < 1 ? 1 : (int)(163840 / lds);
        const long resident = (long)per_cu * device_cu_count();
        const int grid = (int)(nitems < resident ? nitems : resident);
        hipLaunchKernelGGL((chunk_prep_kernel<E, D, D, KIND>), dim3((unsigned)grid), dim3(256), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g,
                           (char*)ws, T, nchunks, nitems, hm);
        return hipGetLastError();
    }
}

template <typename E, int D, int KIND, bool EMIT>
static hipError_t scan_launch(const void* q, const float* S0, void* o, float* S_final, const void* ws,
                              int BH, int T, float* S_bound, hipStream_t st, HeadMap hm,
                              const u64* guard = nullptr, u64 gval = 0) {
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    const long groups = ((long)BH + 7) / 8;
    // 32-column value tiles unless that leaves most of the 256 CUs idle
    if (scan_bv<D>(BH) == 32) {
        constexpr int BV = 32;
        const long nblk = groups * 8 * (D / BV);
        hipLaunchKernelGGL((chunk_scan_kernel<E, D, D, KIND, BV, EMIT>), dim3((unsigned)nblk), dim3(256), 0,
                           st, (const char*)ws, (const E*)q, S0, (E*)o, S_final, T, nchunks, BH, S_bound, hm,
                           guard, gval);
    } else {
        constexpr int BV = 16;
        const long nblk = groups * 8 * (D / BV);
        hipLaunchKernelGGL((chunk_scan_kernel<E, D, D, KIND, BV, EMIT>), dim3((unsigned)nblk), dim3(256), 0,
                           st, (const char*)ws, (const E*)q, S0, (E*)o, S_final, T, nchunks, BH, S_bound, hm,
                           guard, gval);
    }
    return hipGetLastError();
}

// S_bound: NULL, or the states at every chunk boundary, [BH][nchunks][D][D] fp32
template <typename E, int D, int KIND>
static hipError_t scan_t(const void* q, const float* S0, void* o, float* S_final, const void* ws,
                         int BH, int T, hipStream_t st, HeadMap hm, float* S_bound) {
    if (S_bound) return scan_launch<E, D, KIND, true>(q, S0, o, S_final, ws, BH, T, S_bound, st, hm);
    return scan_launch<E, D, KIND, false>(q, S0, o, S_final, ws, BH, T, nullptr, st, hm);
}

// Polls a hand-off wait makes before it gives up: SPIN_LIMIT, or the value of
// the environment variable DN_HANDOFF_SPIN_LIMIT (a small value forces the
// recomputation path, for testing it).
static int handoff_spin_limit() {
    const char* s = getenv("DN_HANDOFF_SPIN_LIMIT");
    if (!s || !*s) return SPIN_LIMIT;
    char* end = nullptr;
    const long v = strtol(s, &end, 10);
    return (end && *end == 0 && v >= 0 && v <= SPIN_LIMIT) ? (int)v : SPIN_LIMIT;
}

// A new 64-bit epoch per fused launch: a random per-process prefix and a
// launch counter.
static u64 next_epoch() {
    static const u64 salt = [] {
        std::random_device rd;
        return ((u64)rd() << 32) | 1u;
    }();
    static std::atomic<unsigned> counter{0};
    return salt ^ (u64)counter.fetch_add(1, std::memory_order_relaxed);
}

// Fused launch when every XCD's scan workgroups leave room for at least 16
// prep workgroups among the two workgroups per CU that can be resident.
template <typename E, int D, int KIND, int BV>
static hipError_t fused_t(const void* q, const void* k, const void* v, const void* beta,
                          const void* g, const float* S0, void* o, float* S_final, void* ws, int BH,
                          int T, hipStream_t st, HeadMap hm) {
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    const int per_xcd = 2 * device_cu_count() / 8;
    const int ns = (BH + 7) / 8 * (D / BV);   // scan workgroups of the busiest XCD
    const long items = (long)(BH + 7) / 8 * nchunks;
    int np = per_xcd - ns;
    if (np < 16) return hipErrorNotSupported;
    // Seven prep workgroups (fourteen items in flight) per head keep just
    // ahead of the scan at d = 128: the blocks are then read soon after they
    // are written, and the prep traffic is spread thin. With up to two heads
    // per XCD they fit beside the scan workgroups one to a CU (the hardware
    // deals out one workgroup per CU before it doubles up). Measured with 16
    // heads of 65536 tokens: 0.88 ms with 7, against 1.17 ms with 5 and 8 and
    // 1.00 ms with 6 prep workgroups per head.
    np = min(np, 7 * ((BH + 7) / 8));
    if ((long)np > (items + 1) / 2) np = (int)((items + 1) / 2);
    char* wsc = static_cast<char*>(ws);
    const u64* err = reinterpret_cast<const u64*>(wsc + ws_tail_off<E, D>(BH, nchunks)) + 2L * BH * nchunks;
    // the start state as it is now: an in-place call overwrites S0 before a
    // failed hand-off could be recomputed
    float* s0c = nullptr;
    if (S0) {
        s0c = reinterpret_cast<float*>(wsc + ws_s0copy_off<E, D>(BH, nchunks));
        const hipError_t e = launch_state_copy(S0, s0c, (long long)BH * D * D, st);
        if (e != hipSuccess) return e;
    }
    const u64 epoch = next_epoch();
    hipLaunchKernelGGL((chunk_fused_kernel<E, D, D, KIND, BV>), dim3((unsigned)(8 * (np + ns))), dim3(256),
                       0, st, (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g,
                       (char*)ws, S0, (E*)o, S_final, T, nchunks, BH, np, epoch, handoff_spin_limit(), hm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the two phases, which return at once unless this launch's hand-off
    // failed (its error word holds the epoch): then they recompute the call
    const long pitems = (long)BH * nchunks;
    const long pgrid = min(pitems, 4L * device_cu_count());
    hipLaunchKernelGGL((chunk_prep2_redo_kernel<E, D, D, KIND>), dim3((unsigned)pgrid), dim3(128), 0,
                       st, (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g, (char*)ws, T,
                       nchunks, pitems, hm, err, epoch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return scan_launch<E, D, KIND, false>(q, s0c, o, S_final, ws, BH, T, nullptr, st, hm, err, epoch);
}

// KDA's one-launch form: the prep (bound by the SIMDs' issue) takes every
// workgroup slot the scan leaves free, two per CU (its LDS allows no more),
// and the scan takes value tiles of BV columns.
template <typename E, int D, int BV>
static hipError_t fused_kda_t(const void* q, const void* k, const void* v, const void* beta,
                              const void* g, const float* S0, void* o, float* S_final, void* ws, int BH,
                              int T, hipStream_t st, HeadMap hm) {
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    const int per_xcd = 2 * device_cu_count() / 8;
    const int ns = (BH + 7) / 8 * (D / BV);   // scan workgroups of the busiest XCD
    const long items = (long)(BH + 7) / 8 * nchunks;
    int np = per_xcd - ns;
    if (np < 16) return hipErrorNotSupported;
    if ((long)np > items) np = (int)items;
    char* wsc = static_cast<char*>(ws);
    const u64* err = reinterpret_cast<const u64*>(wsc + ws_tail_off<E, D>(BH, nchunks)) + 2L * BH * nchunks;
    float* s0c = nullptr;
    if (S0) {
        s0c = reinterpret_cast<float*>(wsc + ws_s0copy_off<E, D>(BH, nchunks));
        const hipError_t e = launch_state_copy(S0, s0c, (long long)BH * D * D, st);
        if (e != hipSuccess) return e;
    }
    const u64 epoch = next_epoch();
    hipLaunchKernelGGL((chunk_fused_kda_kernel<E, D, BV>), dim3((unsigned)(8 * (np + ns))), dim3(256), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g, (char*)ws, S0, (E*)o,
                       S_final, T, nchunks, BH, np, epoch, handoff_spin_limit(), hm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long pitems = (long)BH * nchunks;
    const long pgrid = min(pitems, 2L * device_cu_count());
    hipLaunchKernelGGL((chunk_prep_kda_redo_kernel<E, D>), dim3((unsigned)pgrid), dim3(256), 0, st, (const E*)q,
                       (const E*)k, (const E*)v, (const E*)beta, (const E*)g, (char*)ws, T, nchunks, pitems, hm, err,
                       epoch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return scan_launch<E, D, KIND_KDA, false>(q, s0c, o, S_final, ws, BH, T, nullptr, st, hm, err, epoch);
}

// Two-phase prefill with chunks of CH tokens (32, 64 or 128): the prep and the
// scan above instantiated for that length (CH = 64 is dn_chunk_fwd's two-phase
// form). Blocks of WsLayout<E, D, D, CH>::BYTES, one per (head, chunk), and
// nothing after them.
template <typename E, int D, int KIND, int CH>
static hipError_t fwd_ch_t(const void* q, const void* k, const void* v, const void* beta,
                           const void* g, const float* S0, void* o, float* S_final, void* ws, int BH,
                           int T, hipStream_t st, HeadMap hm) {
    const int nchunks = (T + CH - 1) / CH;
    hipLaunchKernelGGL((chunk_prep2_kernel<E, D, D, KIND, CH>), dim3((unsigned)((long)BH * nchunks)), dim3(128),
                       0, st, (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g, (char*)ws, T,
                       nchunks, hm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long groups = ((long)BH + 7) / 8;
    // DeltaNet shares the Gated DeltaNet scan (its prep stores a unit decay)
    if (scan_bv<D>(BH) == 32) {
        constexpr int BV = 32;
        hipLaunchKernelGGL((chunk_scan_kernel<E, D, D, KIND_GATED, BV, false, CH>),
                           dim3((unsigned)(groups * 8 * (D / BV))), dim3(4 * CH), 0, st, (const char*)ws,
                           (const E*)q, S0, (E*)o, S_final, T, nchunks, BH, (float*)nullptr, hm,
                           (const u64*)nullptr, 0ull);
    } else {
        constexpr int BV = 16;
        hipLaunchKernelGGL((chunk_scan_kernel<E, D, D, KIND_GATED, BV, false, CH>),
                           dim3((unsigned)(groups * 8 * (D / BV))), dim3(4 * CH), 0, st, (const char*)ws,
                           (const E*)q, S0, (E*)o, S_final, T, nchunks, BH, (float*)nullptr, hm,
                           (const u64*)nullptr, 0ull);
    }
    return hipGetLastError();
}

template <int D, int KIND>
static hipError_t fwd_ch_len(int chunk, const void* q, const void* k, const void* v, const void* beta,
                             const void* g, const float* S0, void* o, float* S_final, void* ws, int BH, int T,
                             hipStream_t st, HeadMap hm) {
    if (chunk == 32) return fwd_ch_t<bf16, D, KIND, 32>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
    if (chunk == 64) return fwd_ch_t<bf16, D, KIND, 64>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
    if constexpr (D == 128) {
        if (chunk == 128) return fwd_ch_t<bf16, D, KIND, 128>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
    }
    return hipErrorNotSupported;
}

bool chunk_len_supported(int chunk, int dk, int dtype) {
    return dtype == DT_BF16 && (chunk == 32 || chunk == 64 || (chunk == 128 && dk == 128));
}

size_t chunk_len_workspace_bytes(long long BH, long long T, int dk, int chunk) {
    const long long nchunks = (T + chunk - 1) / chunk;
    long long blk = 0;
    if (dk == 128) {
        blk = chunk == 32 ? WsLayout<bf16, 128, 128, 32>::BYTES
            : chunk == 64 ? WsLayout<bf16, 128, 128, 64>::BYTES : WsLayout<bf16, 128, 128, 128>::BYTES;
    } else {
        blk = chunk == 32 ? WsLayout<bf16, 64, 64, 32>::BYTES : WsLayout<bf16, 64, 64, 64>::BYTES;
    }
    return (size_t)(BH * nchunks * blk);
}

hipError_t launch_chunk_fwd_len(int kind, int dtype, int chunk, const void* q, const void* k, const void* v,
                                const void* beta, const void* g, const float* S0, void* o, float* S_final,
                                void* ws, int BH, int T, int dk, hipStream_t st) {
    if (!chunk_len_supported(chunk, dk, dtype) || (kind != KIND_GATED && kind != KIND_DELTANET))
        return hipErrorNotSupported;
    const HeadMap hm;
    if (dk == 128)
        return kind == KIND_GATED ? fwd_ch_len<128, KIND_GATED>(chunk, q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm)
                                  : fwd_ch_len<128, KIND_DELTANET>(chunk, q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
    return kind == KIND_GATED ? fwd_ch_len<64, KIND_GATED>(chunk, q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm)
                              : fwd_ch_len<64, KIND_DELTANET>(chunk, q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
}

// Byte offset of the one-launch form's error word (followed by the latest
// epoch) in the workspace.
size_t chunk_handoff_offset(long long BH, long long T, int dk, int dtype) {
    const long long nchunks = (T + CHUNK - 1) / CHUNK;
    long long tail;
    if (dtype == DT_BF16) tail = dk == 128 ? ws_tail_off<bf16, 128>(BH, nchunks) : ws_tail_off<bf16, 64>(BH, nchunks);
    else tail = dk == 128 ? ws_tail_off<float, 128>(BH, nchunks) : ws_tail_off<float, 64>(BH, nchunks);
    return (size_t)(tail + BH * nchunks * 16);
}

template <typename E, int D>
static hipError_t prep_kind(int kind, const void* q, const void* k, const void* v,
                            const void* beta, const void* g, void* ws, int BH, int T,
                            hipStream_t st, HeadMap hm) {
    if (kind == KIND_DELTANET) return prep_t<E, D, KIND_DELTANET>(q, k, v, beta, g, ws, BH, T, st, hm);
    if (kind == KIND_GATED) return prep_t<E, D, KIND_GATED>(q, k, v, beta, g, ws, BH, T, st, hm);
    if (kind == KIND_SSM) return prep_t<E, D, KIND_SSM>(q, k, v, beta, g, ws, BH, T, st, hm);
    return prep_t<E, D, KIND_KDA>(q, k, v, beta, g, ws, BH, T, st, hm);
}

template <typename E, int D>
static hipError_t scan_kind(int kind, const void* q, const float* S0, void* o, float* S_final,
                            const void* ws, int BH, int T, hipStream_t st, HeadMap hm,
                            float* S_bound = nullptr) {
    // DeltaNet and Gated DeltaNet share the scan (a unit decay is stored for
    // DeltaNet); the state-space kind drops its W S product
    if (kind == KIND_KDA) return scan_t<E, D, KIND_KDA>(q, S0, o, S_final, ws, BH, T, st, hm, S_bound);
    if (kind == KIND_SSM) return scan_t<E, D, KIND_SSM>(q, S0, o, S_final, ws, BH, T, st, hm, S_bound);
    return scan_t<E, D, KIND_GATED>(q, S0, o, S_final, ws, BH, T, st, hm, S_bound);
}

hipError_t launch_chunk_prep(int kind, int dtype, const void* q, const void* k, const void* v,
                             const void* beta, const void* g, void* ws, int BH, int T, int dk,
                             int dv, hipStream_t st, HeadMap hm) {
    (void)dv;
    if (dtype == DT_BF16)
        return dk == 128 ? prep_kind<bf16, 128>(kind, q, k, v, beta, g, ws, BH, T, st, hm)
                         : prep_kind<bf16, 64>(kind, q, k, v, beta, g, ws, BH, T, st, hm);
    return dk == 128 ? prep_kind<float, 128>(kind, q, k, v, beta, g, ws, BH, T, st, hm)
                     : prep_kind<float, 64>(kind, q, k, v, beta, g, ws, BH, T, st, hm);
}

hipError_t launch_chunk_scan(int kind, int dtype, const void* q, const float* S0, void* o,
                             float* S_final, const void* ws, int BH, int T, int dk, int dv,
                             hipStream_t st, HeadMap hm) {
    (void)dv;
    if (dtype == DT_BF16)
        return dk == 128 ? scan_kind<bf16, 128>(kind, q, S0, o, S_final, ws, BH, T, st, hm)
                         : scan_kind<bf16, 64>(kind, q, S0, o, S_final, ws, BH, T, st, hm);
    return dk == 128 ? scan_kind<float, 128>(kind, q, S0, o, S_final, ws, BH, T, st, hm)
                     : scan_kind<float, 64>(kind, q, S0, o, S_final, ws, BH, T, st, hm);
}

hipError_t launch_chunk_fwd_states(int kind, int dtype, const void* q, const void* k,
                                   const void* v, const void* beta, const void* g,
                                   const float* S0, void* o, float* S_final, float* S_bound,
                                   void* ws, int BH, int T, int dk, int dv, hipStream_t st,
                                   HeadMap hm) {
    const hipError_t e = launch_chunk_prep(kind, dtype, q, k, v, beta, g, ws, BH, T, dk, dv, st, hm);
    if (e != hipSuccess) return e;
    if (dtype == DT_BF16)
        return dk == 128 ? scan_kind<bf16, 128>(kind, q, S0, o, S_final, ws, BH, T, st, hm, S_bound)
                         : scan_kind<bf16, 64>(kind, q, S0, o, S_final, ws, BH, T, st, hm, S_bound);
    return dk == 128 ? scan_kind<float, 128>(kind, q, S0, o, S_final, ws, BH, T, st, hm, S_bound)
                     : scan_kind<float, 64>(kind, q, S0, o, S_final, ws, BH, T, st, hm, S_bound);
}

// Packed sequences: the chunk blocks [H][NC] with NC = ceil(T/64) + N (every
// sequence boundary can split a chunk), then the chunk offsets cs[0..N] and
// the chunk table ctab[NC] (first token, length).
template <typename E, int D>
static size_t varlen_ws_t(long long N, long long H, long long T) {
    const long long nc = (T + CHUNK - 1) / CHUNK + N;
    return (size_t)(H * nc * WsLayout<E, D, D>::BYTES + (4 * (N + 1) + 255) / 256 * 256 +
                    (8 * nc + 255) / 256 * 256);
}

size_t chunk_varlen_workspace_bytes(long long N, long long H, long long T, int dk, int dv, int dtype) {
    (void)dv;
    if (dtype == DT_BF16) return dk == 128 ? varlen_ws_t<bf16, 128>(N, H, T) : varlen_ws_t<bf16, 64>(N, H, T);
    return dk == 128 ? varlen_ws_t<float, 128>(N, H, T) : varlen_ws_t<float, 64>(N, H, T);
}

template <typename E, int D, int KIND, int BV>
static hipError_t varlen_scan_t(const void* q, const float* S0, void* o, float* S_final,
                                const void* ws, const int* cu, const int* cs, int N, int H, int T,
                                int nc, hipStream_t st) {
    const long rows = (long)N * H;
    const long nblk = (rows + 7) / 8 * 8 * (D / BV);
    hipLaunchKernelGGL((chunk_scan_varlen_kernel<E, D, D, KIND, BV>), dim3((unsigned)nblk), dim3(256), 0,
                       st, (const char*)ws, (const E*)q, S0, (E*)o, S_final, T, nc, N, H, cu, cs);
    return hipGetLastError();
}

template <typename E, int D, int KIND>
static hipError_t varlen_kind_t(const void* q, const void* k, const void* v, const void* beta,
                                const void* g, const float* S0, void* o, float* S_final,
                                const int* cu, int N, int H, int T, void* ws, hipStream_t st) {
    typedef WsLayout<E, D, D> Lw;
    const int nc = (T + CHUNK - 1) / CHUNK + N;
    char* tab = (char*)ws + (long)H * nc * Lw::BYTES;
    int* cs = reinterpret_cast<int*>(tab);
    int2* ctab = reinterpret_cast<int2*>(tab + (4L * (N + 1) + 255) / 256 * 256);
    hipLaunchKernelGGL(varlen_chunks_kernel, dim3(1), dim3(1024), 0, st, cu, N, T, cs);
    hipLaunchKernelGGL(varlen_table_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, st, cu,
                       (const int*)cs, N, T, nc, ctab);
    const long nitems = (long)H * nc;
    if constexpr (KIND == KIND_KDA) {
        const hipError_t e = launch_kda_prep<E, D>(q, k, v, beta, g, ws, nitems, T, nc, HeadMap(), ctab, st);
        if (e != hipSuccess) return e;
    } else if constexpr (KIND != KIND_KDA && (sizeof(E) == 2 || D == 64)) {
        hipLaunchKernelGGL((chunk_prep2_varlen_kernel<E, D, D, KIND>), dim3((unsigned)nitems), dim3(128),
                           0, st, (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g,
                           (char*)ws, T, nc, (const int2*)ctab);
    } else {
        constexpr long lds = PrepSmem<E, D, D, KIND>::TOTAL + 1024;
        constexpr int per_cu = (int)(163840 / lds) < 1 ? 1 : (int)(163840 / lds);
        const long resident = (long)per_cu * device_cu_count();
        const int grid = (int)(nitems < resident ? nitems : resident);
        hipLaunchKernelGGL((chunk_prep_kernel<E, D, D, KIND, true>), dim3((unsigned)grid), dim3(256), 0,
                           st, (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g,
                           (char*)ws, T, nc, (int)nitems, HeadMap(), (const int2*)ctab);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int SK = KIND == KIND_KDA ? KIND_KDA : KIND_GATED;   // DeltaNet shares the scan
    if (scan_bv<D>(N * H) == 32)
        return varlen_scan_t<E, D, SK, 32>(q, S0, o, S_final, ws, cu, cs, N, H, T, nc, st);
    return varlen_scan_t<E, D, SK, 16>(q, S0, o, S_final, ws, cu, cs, N, H, T, nc, st);
}

template <typename E, int D>
static hipError_t varlen_t(int kind, const void* q, const void* k, const void* v, const void* beta,
                           const void* g, const float* S0, void* o, float* S_final, const int* cu,
                           int N, int H, int T, void* ws, hipStream_t st) {
    if (kind == KIND_SSM) return hipErrorNotSupported;
    if (kind == KIND_DELTANET)
        return varlen_kind_t<E, D, KIND_DELTANET>(q, k, v, beta, g, S0, o, S_final, cu, N, H, T, ws, st);
    if (kind == KIND_GATED)
        return varlen_kind_t<E, D, KIND_GATED>(q, k, v, beta, g, S0, o, S_final, cu, N, H, T, ws, st);
    return varlen_kind_t<E, D, KIND_KDA>(q, k, v, beta, g, S0, o, S_final, cu, N, H, T, ws, st);
}

hipError_t launch_chunk_fwd_varlen(int kind, int dtype, const void* q, const void* k,
                                   const void* v, const void* beta, const void* g,
                                   const float* S0, void* o, float* S_final, const int* cu_seqlens,
                                   int N, int H, int T, int dk, int dv, void* ws, hipStream_t st) {
    (void)dv;
    if (dtype == DT_BF16)
        return dk == 128 ? varlen_t<bf16, 128>(kind, q, k, v, beta, g, S0, o, S_final, cu_seqlens, N, H, T, ws, st)
                         : varlen_t<bf16, 64>(kind, q, k, v, beta, g, S0, o, S_final, cu_seqlens, N, H, T, ws, st);
    return dk == 128 ? varlen_t<float, 128>(kind, q, k, v, beta, g, S0, o, S_final, cu_seqlens, N, H, T, ws, st)
                     : varlen_t<float, 64>(kind, q, k, v, beta, g, S0, o, S_final, cu_seqlens, N, H, T, ws, st);
}

// One-launch prefill where it exists: bf16, DeltaNet or Gated DeltaNet, and
// few enough heads that every XCD keeps room for at least 16 prep workgroups.
template <typename E, int D>
static hipError_t fused_kind(int kind, const void* q, const void* k, const void* v, const void* beta,
                             const void* g, const float* S0, void* o, float* S_final, void* ws,
                             int BH, int T, hipStream_t st, HeadMap hm) {
    if constexpr (sizeof(E) != 2) {
        return hipErrorNotSupported;
    } else {
        if (kind == KIND_SSM) return hipErrorNotSupported;
        if (kind == KIND_KDA) {
            // sixteen scan workgroups per XCD where the heads allow it: 16-column
            // tiles for up to two heads per XCD, 32 columns above (measured at
            // d = 128: 1x16x16384 373 us with 16 columns against 405 with 32;
            // 2x16x8192 243 us with 32 columns against 305 with 16 and 290 with 64)
            if ((BH + 7) / 8 * (D / 16) <= 16)
                return fused_kda_t<E, D, 16>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
            return fused_kda_t<E, D, 32>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
        }
        const bool wide = scan_bv<D>(BH) == 32;
        if (kind == KIND_GATED)
            return wide ? fused_t<E, D, KIND_GATED, 32>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm)
                        : fused_t<E, D, KIND_GATED, 16>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
        return wide ? fused_t<E, D, KIND_DELTANET, 32>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm)
                    : fused_t<E, D, KIND_DELTANET, 16>(q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
    }
}

// Where the one-launch form beats the two launches (dn_chunk_fwd and
// dn_kda_chunk_fwd without a choice). It pays about one prep item's latency
// before the scan can start and shares the CUs between the two roles; it saves
// the prep phase's own time and reads the blocks from L2. Measured at d = 128
// (bf16), one launch against two, Gated DeltaNet: 1.04-1.09x at 64 chunks per
// sequence and at 128 chunks with 8 heads, 0.94-0.96x at 128 chunks with 16-32
// heads, 0.72x at 256 chunks with 16 heads, 0.63-0.72x at 1,024 chunks with
// 4-16 heads. KDA (whose prep is bound by the SIMDs' issue): 0.79-0.93x from
// 64 chunks on with 8-32 heads, 1.03x with 64 heads, and 1.08-1.15x at 1,024
// chunks with 4-8 heads (the scan chain, slower beside the prep, then sets
// the time).
static bool fused_preferred(int kind, int BH, int nchunks) {
    if (kind == KIND_KDA) return nchunks >= 64 && BH <= 32 && (nchunks <= 512 || BH >= 16);
    return nchunks >= 512 || (nchunks >= 128 && BH >= 16);
}

template <typename E, int D>
static hipError_t fwd_t(int kind, const void* q, const void* k, const void* v, const void* beta,
                        const void* g, const float* S0, void* o, float* S_final, void* ws, int BH,
                        int T, int mode, hipStream_t st, HeadMap hm) {
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    if (mode == FWD_FUSED || (mode == FWD_AUTO && fused_preferred(kind, BH, nchunks))) {
        const hipError_t e = fused_kind<E, D>(kind, q, k, v, beta, g, S0, o, S_final, ws, BH, T, st, hm);
        if (e != hipErrorNotSupported || mode == FWD_FUSED) return e;
    }
    hipError_t e = prep_kind<E, D>(kind, q, k, v, beta, g, ws, BH, T, st, hm);
    if (e != hipSuccess) return e;
    return scan_kind<E, D>(kind, q, S0, o, S_final, ws, BH, T, st, hm);
}

hipError_t launch_chunk_fwd(int kind, int dtype, const void* q, const void* k, const void* v,
                            const void* beta, const void* g, const float* S0, void* o,
                            float* S_final, void* ws, int BH, int T, int dk, int dv, int mode,
                            hipStream_t st, HeadMap hm) {
    (void)dv;
    if (dtype == DT_BF16)
        return dk == 128 ? fwd_t<bf16, 128>(kind, q, k, v, beta, g, S0, o, S_final, ws, BH, T, mode, st, hm)
                         : fwd_t<bf16, 64>(kind, q, k, v, beta, g, S0, o, S_final, ws, BH, T, mode, st, hm);
    return dk == 128 ? fwd_t<float, 128>(kind, q, k, v, beta, g, S0, o, S_final, ws, BH, T, mode, st, hm)
                     : fwd_t<float, 64>(kind, q, k, v, beta, g, S0, o, S_final, ws, BH, T, mode, st, hm);
}

// The gated layer's prefill between its projections (bf16, d = 128): the prep
// with the prologue in its load stage, the scan (reading the q rows the prep
// stored), the epilogue. Workspace: the prefill's blocks, then the q rows
// [B][Hk][T][128], then the read-out [B][Hv][T][128] (each 256-byte aligned).
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
size_t layer_prefill_workspace_bytes(long long B, long long T, int Hk, int Hv) {
    return align256(chunk_workspace_bytes(B * Hv, T, 128, 128, DT_BF16)) + align256((size_t)(B * Hk * T * 128 * 2)) +
           align256((size_t)(B * Hv * T * 128 * 2));
}

hipError_t launch_layer_prefill(const void* qkv, const void* conv_w, const void* conv_state, void* conv_state_out,
                                const void* b, const void* a, const float* A_log, const float* dt_bias,
                                const void* z, const void* norm_w, float eps, const float* S0, float* S_final,
                                void* out, float bscale, int B, int T, int Hk, int Hv, void* ws, hipStream_t st) {
    const int BH = B * Hv;
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    char* w = static_cast<char*>(ws);
    bf16* qhat = reinterpret_cast<bf16*>(w + align256(chunk_workspace_bytes(BH, T, 128, 128, DT_BF16)));
    bf16* o = reinterpret_cast<bf16*>(reinterpret_cast<char*>(qhat) + align256((size_t)B * Hk * T * 128 * 2));
    LayerIn li{static_cast<const bf16*>(qkv), static_cast<const bf16*>(conv_w), static_cast<const bf16*>(conv_state),
               static_cast<bf16*>(conv_state_out), static_cast<const bf16*>(b), static_cast<const bf16*>(a), A_log,
               dt_bias, qhat, bscale, T, Hk, Hv};
    const unsigned items = (unsigned)((long)BH * nchunks);
    if (a) hipLaunchKernelGGL((chunk_prep2_layer_kernel<KIND_GATED>), dim3(items), dim3(128), 0, st, li, w, nchunks);
    else hipLaunchKernelGGL((chunk_prep2_layer_kernel<KIND_DELTANET>), dim3(items), dim3(128), 0, st, li, w, nchunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    HeadMap hm;
    hm.hv = Hv;
    hm.g = Hv / Hk;
    e = scan_t<bf16, 128, KIND_GATED>(qhat, S0, o, S_final, w, BH, T, st, hm, nullptr);
    if (e != hipSuccess) return e;
    return launch_layer_epilogue(DT_BF16, o, z, norm_w, out, B, Hv, T, 128, eps, st);
}

}  // namespace dn
