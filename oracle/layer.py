"""fp64 CPU oracle of the gated layer's prologue and epilogue around the rule.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: the tests and the
benchmark's CPU leg call it; the product package never imports it and it never
imports the product package.

Page "28. Linear attention and Gated DeltaNet", section "The full layer": the
layer projects the input to q, k, v in one matrix, runs a depthwise causal
convolution of width 4 over time on those channels (its state: the last 3
inputs) followed by SiLU, splits the channels into key heads (q, k) and value
heads (v), L2-normalises q and k and scales q by d_k^-1/2, and computes the
gates beta = sigmoid(b) and g = -exp(A_log) * softplus(a + dt_bias). After the
rule, each value head's read-out is RMS-normalised (eps 1e-6), multiplied by a
weight vector and by SiLU(z). The L2 norm divides by max(||x||, 1e-12) (page
"DeltaNet: Memory That Edits", section "One rule, two readings", the unit-key
convention).

Everything is plain float64 numpy on the stored input values.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def silu(x):
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    return np.logaddexp(0.0, x)


def causal_conv1d(x, w, state=None):
    """x [B,T,C] token-major; w [C,K]; state [B,C,K-1] (the previous K-1 inputs,
    oldest first) or None for zeros. Output t of channel c is
    SiLU(sum_j w[c,j] * joined[c, t+j]) with joined = state followed by x along
    time. Returns (y [B,T,C], new_state [B,C,K-1]: the last K-1 entries of joined)."""
    x, w = _f64(x), _f64(w)
    B, T, C = x.shape
    K = w.shape[1]
    st = np.zeros((B, C, K - 1)) if state is None else _f64(state)
    joined = np.concatenate([st, np.transpose(x, (0, 2, 1))], axis=2)   # [B,C,K-1+T]
    y = np.zeros((B, C, T))
    for j in range(K):
        y += w[None, :, j:j + 1] * joined[:, :, j:j + T]
    return np.transpose(silu(y), (0, 2, 1)), joined[:, :, T:T + K - 1].copy()


def l2norm(x, eps=1e-12):
    x = _f64(x)
    n = np.sqrt((x * x).sum(-1, keepdims=True))
    return x / np.maximum(n, eps)


def gates(b, a, A_log, dt_bias, allow_neg_eigval=False):
    """b, a [B,T,Hv]; A_log, dt_bias [Hv] -> (beta, g) [B,Hv,T].

    allow_neg_eigval doubles the write strength to 2 sigmoid(b) in (0, 2), so
    that I - beta k k^T can reach eigenvalue 1 - beta < 0 along k (page
    "DeltaNet: Memory That Edits", section "The reflection hiding in the delta
    rule")."""
    b, a, A_log, dt_bias = _f64(b), _f64(a), _f64(A_log), _f64(dt_bias)
    beta = sigmoid(b) * (2.0 if allow_neg_eigval else 1.0)
    g = -np.exp(A_log) * softplus(a + dt_bias)
    return np.transpose(beta, (0, 2, 1)), np.transpose(g, (0, 2, 1))


def prologue(qkv, conv_w, conv_state, b, a, A_log, dt_bias, Hk, Hv, dk, dv,
             allow_neg_eigval=False):
    """Returns q, k [B,Hk,T,dk], v [B,Hv,T,dv], beta, g [B,Hv,T], new conv state."""
    y, st = causal_conv1d(qkv, conv_w, conv_state)
    B, T, _ = y.shape
    ks = Hk * dk
    q = y[:, :, :ks].reshape(B, T, Hk, dk).transpose(0, 2, 1, 3)
    k = y[:, :, ks:2 * ks].reshape(B, T, Hk, dk).transpose(0, 2, 1, 3)
    v = y[:, :, 2 * ks:].reshape(B, T, Hv, dv).transpose(0, 2, 1, 3)
    q = l2norm(q) * dk ** -0.5
    k = l2norm(k)
    beta, g = gates(b, a, A_log, dt_bias, allow_neg_eigval)
    return q, k, v, beta, g, st


def rmsnorm_gated(o, z, w, eps=1e-6):
    """o [B,Hv,T,dv] (head-major read-out), z [B,T,Hv*dv], w [dv] ->
    [B,T,Hv*dv]: w * o / sqrt(mean(o^2) + eps) * SiLU(z), per value head."""
    o, z, w = _f64(o), _f64(z), _f64(w)
    B, Hv, T, dv = o.shape
    normed = o / np.sqrt((o * o).mean(-1, keepdims=True) + eps)
    normed = normed.transpose(0, 2, 1, 3).reshape(B, T, Hv * dv)
    return np.tile(w, Hv)[None, None, :] * normed * silu(z)
