"""fp64 CPU oracle of the selective state-space recurrence (decayed linear attention).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: the tests and the
benchmark's CPU leg call it; the product package never imports it and it never
imports the product package.

Page "28. Linear attention and Gated DeltaNet", section "Forget: decay": before
each write the state is multiplied by a per-token decay alpha_t in (0, 1),
    S_t = alpha_t S_{t-1} + k_t v_t^T,
the recurrence behind RetNet, GLA and Mamba-2 (page "DeltaNet: Linear
Transformers with the Delta Rule Guide", section "3. The Inadequacy of Static
Decay Rules (Mamba and RetNet)", gives the same form with a fixed decay). The
read-out is o_t = S_t^T q_t, as for the delta rule. Same page 28, section
"Stretch exercises", item 4: with one scalar alpha_t per head this is Gated
DeltaNet with beta's correction term removed. alpha_t = exp(g_t) with the
log-decay g [B,H,T], as the Gated DeltaNet tensor contract carries it.

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


def recurrent(q, k, v, g, S0=None):
    """q, k [B,H,T,dk]; v [B,H,T,dv]; g [B,H,T] log-decay; S0 [B,H,dk,dv] or
    None (zeros). Returns (o [B,H,T,dv], S_T [B,H,dk,dv]) in float64."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        S = np.exp(g[:, :, t])[:, :, None, None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
        o[:, :, t] = np.einsum("bhkv,bhk->bhv", S, q[:, :, t])
    return o, S
