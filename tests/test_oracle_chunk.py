"""fp64 chunk form of the oracle versus its recurrence (brute force).

Page "28. Linear attention and Gated DeltaNet", section "The chunked form":
chunk sizes that do not divide the length, and a non-zero start state, are
what catch a wrong triangle in the chunk system (the page's own note on its
first version); chunk size 1 alone cannot.
"""
import numpy as np
import pytest

import oracle
from test_oracle_pins import _rand_inputs, _rel

KINDS = [oracle.DELTANET, oracle.GATED, oracle.KDA]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("T", [1, 2, 5, 9, 16])
def test_every_chunk_size_small(kind, T):
    q, k, v, beta, g, S0 = _rand_inputs(1, 2, T, 6, 5, kind, seed=30 + T)
    o_r, S_r = oracle.recurrent(q, k, v, beta, g, S0, kind=kind)
    for C in range(1, T + 1):
        o_c, S_c = oracle.chunk(q, k, v, beta, g, S0, kind=kind, C=C)
        assert _rel(o_c, o_r) < 1e-12, C
        assert _rel(S_c, S_r) < 1e-12, C


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("C", [1, 5, 8, 64])
def test_milestone_t37_nonzero_state(kind, C):
    """Chunk sizes 1, 5, 8 and 64 against the recurrence at T=37 with S0 != 0."""
    q, k, v, beta, g, S0 = _rand_inputs(2, 2, 37, 16, 16, kind, seed=41)
    o_r, S_r = oracle.recurrent(q, k, v, beta, g, S0, kind=kind)
    o_c, S_c = oracle.chunk(q, k, v, beta, g, S0, kind=kind, C=C)
    assert _rel(o_c, o_r) < 1e-12
    assert _rel(S_c, S_r) < 1e-12


@pytest.mark.parametrize("kind", KINDS)
def test_chunk_reflection_range_beta(kind):
    """beta in (0, 2) (the negative-eigenvalue range) is not clamped by either form."""
    q, k, v, beta, g, S0 = _rand_inputs(1, 1, 40, 8, 8, kind, seed=42, beta_scale=2.0)
    o_r, S_r = oracle.recurrent(q, k, v, beta, g, S0, kind=kind)
    o_c, S_c = oracle.chunk(q, k, v, beta, g, S0, kind=kind, C=16)
    assert _rel(o_c, o_r) < 1e-11 and _rel(S_c, S_r) < 1e-11


def test_chunk_deltanet_recipe_d64():
    """DeltaNet, T=512, d=64 at the page's chunk sizes 16, 64, 256."""
    q, k, v, beta, _, _ = _rand_inputs(1, 1, 512, 64, 64, oracle.DELTANET, seed=43, s0=False)
    o_r, S_r = oracle.recurrent(q, k, v, beta)
    for C in (16, 64, 256):
        o_c, S_c = oracle.chunk(q, k, v, beta, C=C)
        assert _rel(o_c, o_r) < 1e-12 and _rel(S_c, S_r) < 1e-12


def test_decode_steps_is_the_recurrence():
    """N single-token steps applied to a state equal the recurrence over N tokens."""
    q, k, v, beta, g, S0 = _rand_inputs(3, 2, 7, 8, 8, oracle.GATED, seed=44)
    o_r, S_r = oracle.recurrent(q, k, v, beta, g, S0)
    mv = lambda x: np.moveaxis(x, 2, 0)
    o_d, S_d = oracle.decode_steps(mv(q), mv(k), mv(v), mv(beta), mv(g), S0)
    assert np.array_equal(np.moveaxis(o_d, 0, 2), o_r) and np.array_equal(S_d, S_r)
