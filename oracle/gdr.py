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
