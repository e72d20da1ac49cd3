"""fp64 CPU oracle of the generalized delta rule (diagonal-plus-low-rank transition).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: the tests and the
benchmark's CPU leg call it; the product package never imports it and it never
imports the product package.

Page "DeltaNet: Memory That Edits", section "The generalized delta rule": the
roles the delta rule ties together are separated,
    S_t = (diag(w_t) - (a_t * kr_t) kr_t^T) S_{t-1} + kw_t v_t^T,
with a per-key-channel decay w_t, a removal key kr_t, a write key kw_t and a
per-channel removal rate a_t; tying them gives DeltaNet. Page "A walk through
of the DeltaNet family of linear attention variants" calls such a key-space
transition (a diagonal minus a rank-one matrix) diagonal-plus-low-rank. The
state is d_k x d_v (rows = key channels) and the read-out o_t = S_t^T q_t, as
for the other kinds here; the decay is carried as its logarithm g = log w.

Plain float64 numpy, token by token.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def recurrent(q, kw, v, kr, a, g, S0=None):
    """q, kw, kr, a, g [B,H,T,dk]; v [B,H,T,dv]; S0 [B,H,dk,dv] or None.
    Returns (o [B,H,T,dv], S_T [B,H,dk,dv]) in float64."""
    q, kw, v, kr, a, g = (_f64(x) for x in (q, kw, v, kr, a, g))
    B, H, T, dk = kw.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        removed = np.einsum("bhk,bhkv->bhv", kr[:, :, t], S)          # kr^T S_{t-1}
        S = (np.exp(g[:, :, t])[..., None] * S
             - (a[:, :, t] * kr[:, :, t])[..., None] * removed[:, :, None, :]
             + kw[:, :, t, :, None] * v[:, :, t, None, :])
        o[:, :, t] = np.einsum("bhkv,bhk->bhv", S, q[:, :, t])
    return o, S


def chunk_maps(kw, v, kr, a, g, q):
    """The affine map of one chunk of the generalized rule (derived here; the
    pages give no chunked form). Inputs of one chunk [L, .] for one head.

    With G_t the running sum of g inside the chunk (G_{-1} = 0) and l = a * kr,
    the removal read-outs z_s = kr_s^T S_{s-1} obey the unit lower-triangular
    system
        z_s + sum_{j<s} M_sj z_j = (kr_s * e^{G_{s-1}})^T S_0 + sum_{j<s} N_sj v_j,
        M_sj = sum_c kr_sc l_jc e^{G_{s-1,c} - G_{j,c}},   N_sj = (same with kw_j),
    so Z = Wz S_0 + uz with Wz = (I + M)^-1 R^, uz = (I + M)^-1 N V. Then
        S_L = P S_0 + Sh,   P = diag(e^{G_L}) - L~^T Wz,   Sh = Kw~^T V - L~^T uz,
        O   = Q' S_0 + Oh,  Q' = Q^ - A_l Wz,           Oh = A_kw V - A_l uz,
    with L~_s = l_s e^{G_L - G_s}, Kw~_s = kw_s e^{G_L - G_s}, Q^_t = q_t e^{G_t}
    and A_x[t, s] = sum_c q_tc x_sc e^{G_t,c - G_s,c} for s <= t. Every exponent
    is <= 0. Returns (P, Sh, Qp, Oh)."""
    kw, v, kr, a, g, q = (_f64(x) for x in (kw, v, kr, a, g, q))
    L, dk = kr.shape
    G = np.cumsum(g, axis=0)                       # [L, dk], G[t] = sum_{s<=t} g_s
    Gm = np.vstack([np.zeros((1, dk)), G[:-1]])    # G_{t-1}
    l = a * kr
    M = np.zeros((L, L))
    N = np.zeros((L, L))
    Akw = np.zeros((L, L))
    Al = np.zeros((L, L))
    for s in range(L):
        for j in range(s):
            e = np.exp(Gm[s] - G[j])
            M[s, j] = np.sum(kr[s] * l[j] * e)
            N[s, j] = np.sum(kr[s] * kw[j] * e)
        for j in range(s + 1):
            e = np.exp(G[s] - G[j])
            Akw[s, j] = np.sum(q[s] * kw[j] * e)
            Al[s, j] = np.sum(q[s] * l[j] * e)
    Tinv = np.linalg.inv(np.eye(L) + M)
    Wz = Tinv @ (kr * np.exp(Gm))
    uz = Tinv @ (N @ v)
    Lt = l * np.exp(G[-1] - G)
    Kwt = kw * np.exp(G[-1] - G)
    P = np.diag(np.exp(G[-1])) - Lt.T @ Wz
    Sh = Kwt.T @ v - Lt.T @ uz
    Qp = q * np.exp(G) - Al @ Wz
    Oh = Akw @ v - Al @ uz
    return P, Sh, Qp, Oh


def chunk(q, kw, v, kr, a, g, S0=None, C=64):
    """Chunked form: every chunk's affine map from chunk_maps, applied in order.
    Same arguments and results as recurrent()."""
    q, kw, v, kr, a, g = (_f64(x) for x in (q, kw, v, kr, a, g))
    B, H, T, dk = kw.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    Sf = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else _f64(S0)[b, h].copy()
            for c0 in range(0, T, C):
                c1 = min(T, c0 + C)
                P, Sh, Qp, Oh = chunk_maps(kw[b, h, c0:c1], v[b, h, c0:c1], kr[b, h, c0:c1],
                                           a[b, h, c0:c1], g[b, h, c0:c1], q[b, h, c0:c1])
                o[b, h, c0:c1] = Qp @ S + Oh
                S = P @ S + Sh
            Sf[b, h] = S
    return o, Sf
