"""Pins of the layer prologue/epilogue oracle (``oracle/layer.py``) against
closed forms, library routines and invariants (page "28. Linear attention and
Gated DeltaNet", section "The full layer")."""
import math

import numpy as np
import pytest

from oracle import layer as L


def _rng(seed):
    return np.random.default_rng(seed)


def test_conv_identity_tap_is_silu_and_keeps_last_inputs():
    r = _rng(1)
    x = r.standard_normal((2, 7, 5))
    w = np.zeros((5, 4))
    w[:, 3] = 1.0                                  # only the current input
    y, st = L.causal_conv1d(x, w)
    assert np.allclose(y, x / (1 + np.exp(-x)), rtol=0, atol=1e-15)
    assert np.array_equal(st, np.transpose(x[:, -3:, :], (0, 2, 1)))


def test_conv_oldest_tap_reads_the_carried_state():
    r = _rng(2)
    x = r.standard_normal((1, 6, 3))
    state = r.standard_normal((1, 3, 3))
    w = np.zeros((3, 4))
    w[:, 0] = 1.0                                  # input t - 3
    y, _ = L.causal_conv1d(x, w, state)
    joined = np.concatenate([state, x.transpose(0, 2, 1)], axis=2)
    expect = joined[:, :, :6].transpose(0, 2, 1)
    assert np.allclose(y, L.silu(expect), rtol=0, atol=1e-15)


def test_conv_matches_numpy_convolve():
    r = _rng(3)
    B, T, C = 2, 9, 4
    x = r.standard_normal((B, T, C))
    w = r.standard_normal((C, 4))
    state = r.standard_normal((B, C, 3))
    y, _ = L.causal_conv1d(x, w, state)
    for b in range(B):
        for c in range(C):
            joined = np.concatenate([state[b, c], x[b, :, c]])
            full = np.convolve(joined, w[c, ::-1], mode="valid")   # correlation with w
            assert np.allclose(L.silu(full), y[b, :, c], rtol=0, atol=1e-12)


def test_conv_state_handoff():
    r = _rng(4)
    x = r.standard_normal((2, 11, 6))
    w = r.standard_normal((6, 4))
    s0 = r.standard_normal((2, 6, 3))
    y, s = L.causal_conv1d(x, w, s0)
    y1, s1 = L.causal_conv1d(x[:, :5], w, s0)
    y2, s2 = L.causal_conv1d(x[:, 5:], w, s1)
    assert np.allclose(np.concatenate([y1, y2], axis=1), y, rtol=0, atol=1e-14)
    assert np.array_equal(s2, s)
    # fewer tokens than the history: the state shifts by T
    y3, s3 = L.causal_conv1d(x[:, :2], w, s0)
    assert np.array_equal(s3, np.concatenate([s0[:, :, 2:], x[:, :2].transpose(0, 2, 1)], axis=2))


def test_silu_sigmoid_softplus_closed_forms():
    assert L.silu(np.array(0.0)) == 0.0
    assert L.sigmoid(np.array(0.0)) == 0.5
    assert abs(L.softplus(np.array(0.0)) - math.log(2.0)) < 1e-16
    assert abs(L.softplus(np.array(50.0)) - 50.0) < 1e-15
    x = np.linspace(-6, 6, 13)
    assert np.allclose(L.silu(x), x * L.sigmoid(x), rtol=0, atol=1e-15)


def test_l2norm_unit_and_zero():
    r = _rng(5)
    x = r.standard_normal((3, 4, 16))
    n = np.linalg.norm(L.l2norm(x), axis=-1)
    assert np.allclose(n, 1.0, rtol=0, atol=1e-14)
    assert np.array_equal(L.l2norm(np.zeros((2, 8))), np.zeros((2, 8)))


def test_gates():
    A_log = np.log(np.array([0.5, 2.0, 8.0]))
    dt_bias = np.array([1.0, -0.5, 0.25])
    b = np.zeros((1, 1, 3))
    a = -dt_bias[None, None, :]                    # softplus(0) = ln 2
    beta, g = L.gates(b, a, A_log, dt_bias)
    assert np.allclose(beta, 0.5) and beta.shape == (1, 3, 1)
    assert np.allclose(g[0, :, 0], -np.exp(A_log) * math.log(2.0), rtol=1e-15, atol=0)
    r = _rng(6)
    _, g2 = L.gates(r.standard_normal((2, 5, 3)), 5 * r.standard_normal((2, 5, 3)), A_log, dt_bias)
    assert (g2 < 0).all()


def test_rmsnorm_gated():
    B, Hv, T, dv = 1, 2, 3, 8
    w = np.linspace(0.5, 2.0, dv)
    o = np.full((B, Hv, T, dv), -3.0)              # constant row: normed = sign * (9 / (9 + eps))^1/2
    z_big = np.full((B, T, Hv * dv), 40.0)          # SiLU(40) = 40 (to 1e-16)
    out = L.rmsnorm_gated(o, z_big, w)
    expect = -math.sqrt(9.0 / (9.0 + 1e-6)) * np.tile(w, Hv) * 40.0
    assert np.allclose(out[0, 0], expect, rtol=1e-12, atol=0)
    assert np.array_equal(L.rmsnorm_gated(o, np.zeros_like(z_big), w), np.zeros_like(z_big))
    # the norm is per value head: scaling one head's row leaves the output unchanged
    r = _rng(7)
    o2 = r.standard_normal((B, Hv, T, dv))
    z2 = r.standard_normal((B, T, Hv * dv))
    o3 = o2.copy()
    o3[:, 1] *= 1e3
    d = np.abs(L.rmsnorm_gated(o2, z2, w, eps=0.0) - L.rmsnorm_gated(o3, z2, w, eps=0.0)).max()
    assert d < 1e-12


def test_prologue_splits_heads():
    r = _rng(8)
    B, T, Hk, Hv, dk, dv = 2, 5, 2, 4, 8, 4
    C = 2 * Hk * dk + Hv * dv
    qkv = r.standard_normal((B, T, C))
    w = np.zeros((C, 4))
    w[:, 3] = 1.0
    b, a = r.standard_normal((B, T, Hv)), r.standard_normal((B, T, Hv))
    q, k, v, beta, g, st = L.prologue(qkv, w, None, b, a, np.zeros(Hv), np.zeros(Hv), Hk, Hv, dk, dv)
    assert q.shape == (B, Hk, T, dk) and k.shape == (B, Hk, T, dk) and v.shape == (B, Hv, T, dv)
    assert np.allclose(np.linalg.norm(q, axis=-1), dk ** -0.5)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0)
    y = L.silu(qkv)
    assert np.allclose(v, y[:, :, 2 * Hk * dk:].reshape(B, T, Hv, dv).transpose(0, 2, 1, 3))
    assert beta.shape == (B, Hv, T) and g.shape == (B, Hv, T) and st.shape == (B, C, 3)


def test_gates_allow_neg_eigval():
    """The flag doubles beta to 2 sigmoid(b) in (0, 2) and leaves g alone; at
    large b the transition I - beta k k^T then has eigenvalue near -1 along k
    (a reflection; page "DeltaNet: Memory That Edits", section "The reflection
    hiding in the delta rule"), where the plain gate stops near 0."""
    r = np.random.default_rng(11)
    b, a = r.standard_normal((2, 7, 3)), r.standard_normal((2, 7, 3))
    A_log, dt_bias = np.log(r.uniform(0.01, 16, 3)), np.ones(3)
    b1, g1 = L.gates(b, a, A_log, dt_bias)
    b2, g2 = L.gates(b, a, A_log, dt_bias, allow_neg_eigval=True)
    assert np.array_equal(b2, 2 * b1) and np.array_equal(g1, g2)
    assert (b2 > 0).all() and (b2 < 2).all()
    k = r.standard_normal(8)
    k /= np.linalg.norm(k)
    big = np.full((1, 1, 1), 30.0)
    for flag, along in ((False, 0.0), (True, -1.0)):
        beta = L.gates(big, big, np.zeros(1), np.zeros(1), allow_neg_eigval=flag)[0][0, 0, 0]
        ev = np.sort(np.linalg.eigvalsh(np.eye(8) - beta * np.outer(k, k)))
        assert abs(ev[0] - along) < 1e-9 and np.allclose(ev[1:], 1.0)
