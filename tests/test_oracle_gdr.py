"""Pins of the generalized delta rule oracle (oracle/gdr.py) to the C oracle of
the three tied kinds, an independent implementation of a different form (the
error form u = beta (v - S~^T k)):
  * DeltaNet: w = 1, kr = k, a = beta (every channel), kw = beta k — the tie
    the page "DeltaNet: Memory That Edits" states ("The generalized delta
    rule");
  * Gated DeltaNet: w = alpha (every channel), kr = k, a = alpha beta, kw =
    beta k, since (I - beta k k^T) alpha = alpha I - alpha beta k k^T;
  * KDA: w = alpha (per channel), kr = alpha * k, a = beta / alpha, kw = beta k,
    since (I - beta k k^T) diag(alpha) = diag(alpha) - beta k (alpha * k)^T.
A transposed rank-one term, a dropped decay or a mixed-up key fails one of them.
"""
import numpy as np
import pytest

import oracle
from oracle import gdr


def _base(seed, B=2, H=2, T=13, dk=8, dv=6):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, dv))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, H, T))))
    S0 = r.standard_normal((B, H, dk, dv))
    return r, q, k, v, beta, S0


def test_tied_roles_give_deltanet():
    r, q, k, v, beta, S0 = _base(1)
    ones = np.ones_like(k)
    o1, S1 = gdr.recurrent(q, beta[..., None] * k, v, k, beta[..., None] * ones,
                           np.zeros_like(k), S0)
    o2, S2 = oracle.recurrent(q, k, v, beta, None, S0, kind=oracle.DELTANET)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(S1, S2, rtol=1e-12, atol=1e-12)


def test_scalar_decay_gives_gated_deltanet():
    r, q, k, v, beta, S0 = _base(2)
    g = -np.log1p(np.exp(r.standard_normal(beta.shape)))
    alpha = np.exp(g)[..., None] * np.ones_like(k)
    o1, S1 = gdr.recurrent(q, beta[..., None] * k, v, k, alpha * beta[..., None],
                           np.log(alpha), S0)
    o2, S2 = oracle.recurrent(q, k, v, beta, g, S0, kind=oracle.GATED)
    assert np.allclose(o1, o2, rtol=1e-11, atol=1e-12)
    assert np.allclose(S1, S2, rtol=1e-11, atol=1e-12)


def test_channel_decay_gives_kda():
    r, q, k, v, beta, S0 = _base(3)
    g = -np.log1p(np.exp(r.standard_normal(k.shape)))
    alpha = np.exp(g)
    o1, S1 = gdr.recurrent(q, beta[..., None] * k, v, alpha * k, beta[..., None] / alpha, g, S0)
    o2, S2 = oracle.recurrent(q, k, v, beta, g, S0, kind=oracle.KDA)
    assert np.allclose(o1, o2, rtol=1e-10, atol=1e-11)
    assert np.allclose(S1, S2, rtol=1e-10, atol=1e-11)


def test_separate_keys_differ_from_tied():
    """With a removal key different from the write key the result is not
    DeltaNet's (the roles really are separate)."""
    r, q, k, v, beta, S0 = _base(4)
    kr = r.standard_normal(k.shape)
    kr /= np.linalg.norm(kr, axis=-1, keepdims=True)
    ones = np.ones_like(k)
    o1, _ = gdr.recurrent(q, beta[..., None] * k, v, kr, beta[..., None] * ones, np.zeros_like(k), S0)
    o2, _ = oracle.recurrent(q, k, v, beta, None, S0, kind=oracle.DELTANET)
    assert not np.allclose(o1, o2)


@pytest.mark.parametrize("C", [1, 3, 8, 16, 40])
def test_chunk_form_equals_recurrence(C):
    """The chunked form (its derivation is in oracle/gdr.chunk_maps) against the
    token-by-token recurrence, with separate keys, per-channel decay and rate,
    a start state and a ragged last chunk."""
    r = np.random.default_rng(50 + C)
    B, H, T, dk, dv = 1, 2, 37, 8, 5
    q = r.standard_normal((B, H, T, dk))
    kw = r.standard_normal((B, H, T, dk)) * 0.5
    kr = r.standard_normal((B, H, T, dk))
    kr /= np.linalg.norm(kr, axis=-1, keepdims=True)
    a = 1.0 / (1.0 + np.exp(-r.standard_normal((B, H, T, dk))))
    g = -np.log1p(np.exp(r.standard_normal((B, H, T, dk))))
    v = r.standard_normal((B, H, T, dv))
    S0 = r.standard_normal((B, H, dk, dv))
    o1, S1 = gdr.recurrent(q, kw, v, kr, a, g, S0)
    o2, S2 = gdr.chunk(q, kw, v, kr, a, g, S0, C=C)
    assert np.allclose(o1, o2, rtol=1e-9, atol=1e-10)
    assert np.allclose(S1, S2, rtol=1e-9, atol=1e-10)


def test_chunk_form_strong_decay_is_finite():
    """Decays summing to -1000 inside a chunk: every factor of the chunked form
    has a non-positive exponent, so nothing overflows."""
    r = np.random.default_rng(77)
    B, H, T, d = 1, 1, 20, 4
    q, kw, kr, v = (r.standard_normal((B, H, T, d)) for _ in range(4))
    a = np.full((B, H, T, d), 0.5)
    g = np.full((B, H, T, d), -50.0)
    o1, S1 = gdr.recurrent(q, kw, v, kr, a, g, None)
    o2, S2 = gdr.chunk(q, kw, v, kr, a, g, None, C=16)
    assert np.isfinite(o2).all() and np.allclose(o1, o2, rtol=1e-9, atol=1e-12)
