/*
 * oracle.c -- plain, slow, fp64 CPU reference for the delta-rule family
 * (DeltaNet, Gated DeltaNet, KDA).
 *
 * THIS IS TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. The product path (the HIP library
 * and its Python binding) never links, loads or calls anything here, and this
 * file shares no code, header, table or helper with it.
 *
 * Everything is fp64, plain loops, no blocking or reordering beyond what the
 * definitions state. Inputs arrive already upcast to double (an exact widening
 * of the bf16 / fp32 values the GPU path received).
 *
 * Layouts (row-major, contiguous):
 *   q, k  [B,H,T,dk]    v [B,H,T,dv]    beta [B,H,T]
 *   g     kind 0 (DeltaNet): unused, may be NULL
 *         kind 1 (Gated DeltaNet): [B,H,T]     one log-decay per token
 *         kind 2 (KDA): [B,H,T,dk]             one log-decay per key channel
 *   S0    [B,H,dk,dv] or NULL (zero start)     o [B,H,T,dv]   S [B,H,dk,dv]
 * The state S is d_k x d_v and is read as S^T k / S^T q, the orientation of
 * the tensor contract on the page "28. Linear attention and Gated DeltaNet"
 * (section "The recurrent form").
 *
 * Return value: 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_DELTANET = 0, ORC_GATED = 1, ORC_KDA = 2 };

static int orc_bad(int kind, const double* q, const double* k, const double* v,
                   const double* beta, const double* g, const double* o,
                   const double* S, long B, long H, long T, long dk, long dv) {
    if (kind < 0 || kind > 2) return 1;
    if (!q || !k || !v || !beta || !o || !S) return 1;
    if (kind != ORC_DELTANET && !g) return 1;
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return 1;
    return 0;
}

static void orc_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int orc_max_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) return nthreads;
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Decay of the state before a token is processed: row i of S (key channel i)
 * is multiplied by exp(g_i). Gated DeltaNet has one g for all rows; KDA has one
 * per key channel ("forget first, then predict", page "A walk through of the
 * DeltaNet family of linear attention variants", Gated DeltaNet and KDA
 * sections; page "28. Linear attention and Gated DeltaNet", eq. for S_t). */
static void orc_decay(int kind, double* S, const double* g_t, long dk, long dv) {
    if (kind == ORC_GATED) {
        double a = exp(g_t[0]);
        for (long i = 0; i < dk * dv; ++i) S[i] *= a;
    } else if (kind == ORC_KDA) {
        for (long i = 0; i < dk; ++i) {
            double a = exp(g_t[i]);
            for (long j = 0; j < dv; ++j) S[i * dv + j] *= a;
        }
    }
}

static const double* orc_g_at(int kind, const double* g, long bh, long t, long T, long dk) {
    if (kind == ORC_GATED) return g + bh * T + t;
    if (kind == ORC_KDA) return g + (bh * T + t) * dk;
    return NULL;
}

/*
 * Error form, one token at a time: decay, predict p = S^T k, scaled error
 * u = beta (v - p), rank-1 write S += k u^T, read o = S^T q.
 * (Page "28. Linear attention and Gated DeltaNet", sections "Correct: the
 * delta rule", "Gated DeltaNet" and "The recurrent form"; page "DeltaNet:
 * Memory That Edits", section "The delta rule"; page "A walk through of the
 * DeltaNet family ...", KDA recurrence.)
 */
int orc_recurrent(int kind, const double* q, const double* k, const double* v,
                  const double* beta, const double* g, const double* S0,
                  double* o, double* S, long B, long H, long T, long dk, long dv,
                  int nthreads) {
    if (orc_bad(kind, q, k, v, beta, g, o, S, B, H, T, dk, dv)) return -1;
    orc_threads(nthreads);
    long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        double* St = S + bh * dk * dv;
        if (S0) memcpy(St, S0 + bh * dk * dv, sizeof(double) * dk * dv);
        else memset(St, 0, sizeof(double) * dk * dv);
        double* p = (double*)malloc(sizeof(double) * dv);
        double* u = (double*)malloc(sizeof(double) * dv);
        for (long t = 0; t < T; ++t) {
            const double* qt = q + (bh * T + t) * dk;
            const double* kt = k + (bh * T + t) * dk;
            const double* vt = v + (bh * T + t) * dv;
            double bt = beta[bh * T + t];
            orc_decay(kind, St, orc_g_at(kind, g, bh, t, T, dk), dk, dv);
            for (long j = 0; j < dv; ++j) p[j] = 0.0;
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j) p[j] += kt[i] * St[i * dv + j];
            for (long j = 0; j < dv; ++j) u[j] = bt * (vt[j] - p[j]);
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j) St[i * dv + j] += kt[i] * u[j];
            double* ot = o + (bh * T + t) * dv;
            for (long j = 0; j < dv; ++j) ot[j] = 0.0;
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j) ot[j] += qt[i] * St[i * dv + j];
        }
        free(p);
        free(u);
    }
    return 0;
}

/*
 * Transition-then-write form: S <- (I - beta k k^T) Diag(alpha) S + beta k v^T,
 * with the d_k x d_k transition formed explicitly and applied as a dense
 * matrix product, then o = S^T q. alpha = 1 (DeltaNet), exp(g) (Gated
 * DeltaNet) or exp(g_i) per key channel (KDA).
 * (Page "DeltaNet: Memory That Edits", section "One rule, two readings" and
 * "Gating: the modern cell"; page "A walk through of the DeltaNet family ...",
 * DPLR transition of KDA.) O(dk^2 dv) per token: small sizes only.
 */
int orc_recurrent_matrix(int kind, const double* q, const double* k, const double* v,
                         const double* beta, const double* g, const double* S0,
                         double* o, double* S, long B, long H, long T, long dk, long dv,
                         int nthreads) {
    if (orc_bad(kind, q, k, v, beta, g, o, S, B, H, T, dk, dv)) return -1;
    orc_threads(nthreads);
    long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        double* St = S + bh * dk * dv;
        if (S0) memcpy(St, S0 + bh * dk * dv, sizeof(double) * dk * dv);
        else memset(St, 0, sizeof(double) * dk * dv);
        double* M = (double*)malloc(sizeof(double) * dk * dk);
        double* Sn = (double*)malloc(sizeof(double) * dk * dv);
        for (long t = 0; t < T; ++t) {
            const double* qt = q + (bh * T + t) * dk;
            const double* kt = k + (bh * T + t) * dk;
            const double* vt = v + (bh * T + t) * dv;
            double bt = beta[bh * T + t];
            const double* gt = orc_g_at(kind, g, bh, t, T, dk);
            /* M = (I - beta k k^T) Diag(alpha) */
            for (long r = 0; r < dk; ++r) {
                for (long c = 0; c < dk; ++c) {
                    double e = (r == c ? 1.0 : 0.0) - bt * kt[r] * kt[c];
                    double a = 1.0;
                    if (kind == ORC_GATED) a = exp(gt[0]);
                    else if (kind == ORC_KDA) a = exp(gt[c]);
                    M[r * dk + c] = e * a;
                }
            }
            /* Sn = M S + beta k v^T */
            for (long r = 0; r < dk; ++r) {
                for (long j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (long c = 0; c < dk; ++c) acc += M[r * dk + c] * St[c * dv + j];
                    Sn[r * dv + j] = acc + bt * kt[r] * vt[j];
                }
            }
            memcpy(St, Sn, sizeof(double) * dk * dv);
            double* ot = o + (bh * T + t) * dv;
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i) acc += qt[i] * St[i * dv + j];
                ot[j] = acc;
            }
        }
        free(M);
        free(Sn);
    }
    return 0;
}

/*
 * Chunkwise form, used only to cross-check the recurrence. For a chunk of L
 * tokens that starts from state S0, with G_i the running sum of the log-decay
 * inside the chunk (per key channel c; a scalar broadcast for Gated DeltaNet,
 * zero for DeltaNet):
 *   A_ij = beta_i sum_c k_ic k_jc exp(G_ic - G_jc)          (i > j)
 *   (I + A) W = beta * exp(G) * K,   (I + A) u = beta * V   (forward substitution)
 *   U   = u - W S0                                          (values actually written)
 *   O_i = sum_c q_ic exp(G_ic) S0[c,:] + sum_{j<=i} (sum_c q_ic k_jc exp(G_ic - G_jc)) U_j
 *   S_end[c,:] = exp(G_{L-1,c}) S0[c,:] + sum_j k_jc exp(G_{L-1,c} - G_jc) U_j
 * This is the system of the page "28. Linear attention and Gated DeltaNet"
 * (section "The chunked form: recurrence as matrix multiplication", its
 * three-line system), written with the decay kept per key channel so that the
 * same routine covers KDA; with one decay per token it is that system verbatim,
 * and with no decay it is the WY system of page "DeltaNet: Memory That Edits"
 * (section "Training it: the WY trick"). The last chunk is simply shorter (no
 * padding). No matrix inverse is formed.
 */
int orc_chunk(int kind, const double* q, const double* k, const double* v,
              const double* beta, const double* g, const double* S0,
              double* o, double* S, long B, long H, long T, long dk, long dv,
              long C, int nthreads) {
    if (orc_bad(kind, q, k, v, beta, g, o, S, B, H, T, dk, dv)) return -1;
    if (C < 1) return -1;
    orc_threads(nthreads);
    long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        double* St = S + bh * dk * dv;
        if (S0) memcpy(St, S0 + bh * dk * dv, sizeof(double) * dk * dv);
        else memset(St, 0, sizeof(double) * dk * dv);
        double* G = (double*)malloc(sizeof(double) * C * dk);
        double* A = (double*)malloc(sizeof(double) * C * C);
        double* W = (double*)malloc(sizeof(double) * C * dk);
        double* u = (double*)malloc(sizeof(double) * C * dv);
        double* U = (double*)malloc(sizeof(double) * C * dv);
        double* Sn = (double*)malloc(sizeof(double) * dk * dv);
        for (long t0 = 0; t0 < T; t0 += C) {
            long L = (T - t0 < C) ? (T - t0) : C;
            const double* Kc = k + (bh * T + t0) * dk;
            const double* Qc = q + (bh * T + t0) * dk;
            const double* Vc = v + (bh * T + t0) * dv;
            const double* bc = beta + bh * T + t0;
            /* G: running sum of the log-decay, per key channel */
            for (long i = 0; i < L; ++i) {
                for (long c = 0; c < dk; ++c) {
                    double gi = 0.0;
                    if (kind == ORC_GATED) gi = g[bh * T + t0 + i];
                    else if (kind == ORC_KDA) gi = g[(bh * T + t0 + i) * dk + c];
                    G[i * dk + c] = (i == 0 ? 0.0 : G[(i - 1) * dk + c]) + gi;
                }
            }
            /* strictly lower A */
            for (long i = 0; i < L; ++i) {
                for (long j = 0; j < L; ++j) {
                    double acc = 0.0;
                    if (i > j)
                        for (long c = 0; c < dk; ++c)
                            acc += Kc[i * dk + c] * Kc[j * dk + c] * exp(G[i * dk + c] - G[j * dk + c]);
                    A[i * C + j] = bc[i] * acc;
                }
            }
            /* forward substitution for W and u: row i = rhs_i - sum_{j<i} A_ij row_j */
            for (long i = 0; i < L; ++i) {
                for (long c = 0; c < dk; ++c) {
                    double acc = bc[i] * exp(G[i * dk + c]) * Kc[i * dk + c];
                    for (long j = 0; j < i; ++j) acc -= A[i * C + j] * W[j * dk + c];
                    W[i * dk + c] = acc;
                }
                for (long c = 0; c < dv; ++c) {
                    double acc = bc[i] * Vc[i * dv + c];
                    for (long j = 0; j < i; ++j) acc -= A[i * C + j] * u[j * dv + c];
                    u[i * dv + c] = acc;
                }
            }
            /* U = u - W S0 */
            for (long i = 0; i < L; ++i) {
                for (long j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (long c = 0; c < dk; ++c) acc += W[i * dk + c] * St[c * dv + j];
                    U[i * dv + j] = u[i * dv + j] - acc;
                }
            }
            /* outputs */
            for (long i = 0; i < L; ++i) {
                double* oi = o + (bh * T + t0 + i) * dv;
                for (long j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (long c = 0; c < dk; ++c)
                        acc += Qc[i * dk + c] * exp(G[i * dk + c]) * St[c * dv + j];
                    oi[j] = acc;
                }
                for (long m = 0; m <= i; ++m) {
                    double a = 0.0;
                    for (long c = 0; c < dk; ++c)
                        a += Qc[i * dk + c] * Kc[m * dk + c] * exp(G[i * dk + c] - G[m * dk + c]);
                    for (long j = 0; j < dv; ++j) oi[j] += a * U[m * dv + j];
                }
            }
            /* end-of-chunk state */
            for (long c = 0; c < dk; ++c) {
                double gl = G[(L - 1) * dk + c];
                for (long j = 0; j < dv; ++j) {
                    double acc = exp(gl) * St[c * dv + j];
                    for (long m = 0; m < L; ++m)
                        acc += Kc[m * dk + c] * exp(gl - G[m * dk + c]) * U[m * dv + j];
                    Sn[c * dv + j] = acc;
                }
            }
            memcpy(St, Sn, sizeof(double) * dk * dv);
        }
        free(G);
        free(A);
        free(W);
        free(u);
        free(U);
        free(Sn);
    }
    return 0;
}
