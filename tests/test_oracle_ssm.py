"""Pins of the selective state-space oracle (oracle/ssm.py) to results fixed
by the mathematics and by an independent implementation, not by itself:
  * the pairwise (attention) form of the same recurrence, brute force;
  * no decay and no start state: causal linear attention, tril(Q K^T) V with
    the library matrix product;
  * a very strong decay leaves only the current token: o_t = (q_t . k_t) v_t;
  * page 28, "Stretch exercises" item 4 (Gated DeltaNet with beta's
    correction removed): with orthonormal keys and beta = 1 the correction
    term of Gated DeltaNet is zero, so the C oracle of Gated DeltaNet must
    give exactly the same outputs and state.
"""
import numpy as np
import pytest

import oracle
from oracle import ssm


def _inputs(B, H, T, dk, dv, seed, decay=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk))
    v = r.standard_normal((B, H, T, dv))
    g = -decay * np.log1p(np.exp(r.standard_normal((B, H, T))))
    S0 = r.standard_normal((B, H, dk, dv))
    return q, k, v, g, S0


def test_pairwise_form_brute_force():
    q, k, v, g, S0 = _inputs(2, 2, 9, 4, 3, seed=1)
    o, S = ssm.recurrent(q, k, v, g, S0)
    B, H, T, _ = q.shape
    for b in range(B):
        for h in range(H):
            G = np.cumsum(g[b, h])
            for t in range(T):
                ref = np.exp(G[t]) * (S0[b, h].T @ q[b, h, t])
                for s in range(t + 1):
                    ref = ref + np.exp(G[t] - G[s]) * np.dot(q[b, h, t], k[b, h, s]) * v[b, h, s]
                assert np.allclose(o[b, h, t], ref, rtol=1e-12, atol=1e-12)
            Sref = np.exp(G[-1]) * S0[b, h]
            for s in range(T):
                Sref = Sref + np.exp(G[-1] - G[s]) * np.outer(k[b, h, s], v[b, h, s])
            assert np.allclose(S[b, h], Sref, rtol=1e-12, atol=1e-12)


def test_no_decay_is_causal_linear_attention():
    q, k, v, _, _ = _inputs(1, 3, 17, 8, 5, seed=2)
    o, S = ssm.recurrent(q, k, v, np.zeros(q.shape[:3]), None)
    for h in range(3):
        A = np.tril(q[0, h] @ k[0, h].T)
        assert np.allclose(o[0, h], A @ v[0, h], rtol=1e-12, atol=1e-12)
        assert np.allclose(S[0, h], k[0, h].T @ v[0, h], rtol=1e-12, atol=1e-12)


def test_strong_decay_keeps_only_the_current_token():
    q, k, v, _, S0 = _inputs(1, 2, 6, 4, 4, seed=3)
    g = np.full(q.shape[:3], -800.0)   # exp(-800) == 0 in float64
    o, S = ssm.recurrent(q, k, v, g, S0)
    ref = np.einsum("bhtk,bhtk->bht", q, k)[..., None] * v
    # (the sum over key channels is taken in another order: equal up to rounding)
    assert np.allclose(o, ref, rtol=1e-13, atol=1e-13)
    assert np.array_equal(S, k[:, :, -1, :, None] * v[:, :, -1, None, :])


@pytest.mark.parametrize("T", [1, 5, 16])
def test_equals_gated_deltanet_without_correction(T):
    d = 16
    r = np.random.default_rng(40 + T)
    B, H = 2, 2
    k = np.empty((B, H, T, d))
    for b in range(B):
        for h in range(H):
            Qm, _ = np.linalg.qr(r.standard_normal((d, d)))
            k[b, h] = Qm[:, :T].T          # orthonormal keys: k_s . k_t = [s == t]
    q = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, d))
    g = -np.log1p(np.exp(r.standard_normal((B, H, T))))
    beta = np.ones((B, H, T))
    o1, S1 = ssm.recurrent(q, k, v, g, None)
    o2, S2 = oracle.recurrent(q, k, v, beta, g, None, kind=oracle.GATED)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(S1, S2, rtol=1e-12, atol=1e-12)
    # with overlapping keys the correction term is not zero: the two differ
    k2 = r.standard_normal((B, H, T, d))
    if T > 1:
        o3, _ = ssm.recurrent(q, k2, v, g, None)
        o4, _ = oracle.recurrent(q, k2, v, beta, g, None, kind=oracle.GATED)
        assert not np.allclose(o3, o4)
