"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU. Each one targets a mistake a plausible
oracle could make (a dropped term, a wrong sign, a transposed state, decay
applied after the prediction, decay on the wrong axis, a wrong triangle in
the chunk system) and would fail on it.
"""
import json
import os

import numpy as np
import pytest

import oracle

rng = np.random.default_rng(1234)


def _unit(x):
    return x / np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), 1e-12)


def _rand_inputs(B, H, T, dk, dv, kind, seed, s0=True, beta_scale=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk))
    k = _unit(r.standard_normal((B, H, T, dk)))
    v = r.standard_normal((B, H, T, dv))
    beta = beta_scale / (1 + np.exp(-r.standard_normal((B, H, T))))
    g = None
    if kind == oracle.GATED:
        g = -np.log1p(np.exp(r.standard_normal((B, H, T))))
    elif kind == oracle.KDA:
        g = -np.log1p(np.exp(r.standard_normal((B, H, T, dk))))
    S0 = r.standard_normal((B, H, dk, dv)) * 0.5 if s0 else None
    return q, k, v, beta, g, S0


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# --------------------------------------------------------------------------
# Worked example: page "28. Linear attention and Gated DeltaNet",
# section "Correct: the delta rule".
# --------------------------------------------------------------------------
def test_worked_example_exact(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    q = np.array(ex["q"]).reshape(1, 1, 1, 2)
    k = np.array(ex["k"]).reshape(1, 1, 1, 2)
    v = np.array(ex["v"]).reshape(1, 1, 1, 2)
    S = np.zeros((1, 1, 2, 2))
    for step in ex["steps"]:
        pred = S[0, 0].T @ k[0, 0, 0]          # what the state returns for k before the write
        assert np.array_equal(pred, step["prediction"])
        o, S = oracle.recurrent(q, k, v, np.array([[[step["beta"]]]]), S0=S)
        assert np.array_equal(S[0, 0, 0], step["state_row0"])      # exact in binary fp
        assert np.array_equal(S[0, 0, 1], [0.0, 0.0])
        assert np.array_equal(o[0, 0, 0], step["output"])
    # The matrix (transition-then-write) form reproduces it as well.
    S = np.zeros((1, 1, 2, 2))
    for step in ex["steps"]:
        o, S = oracle.recurrent_matrix(q, k, v, np.array([[[step["beta"]]]]), S0=S)
        assert np.array_equal(o[0, 0, 0], step["output"])


def test_worked_example_as_one_sequence(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    T = len(ex["steps"])
    q = np.tile(np.array(ex["q"]), (1, 1, T, 1))
    k = np.tile(np.array(ex["k"]), (1, 1, T, 1))
    v = np.tile(np.array(ex["v"]), (1, 1, T, 1))
    beta = np.array([[[s["beta"] for s in ex["steps"]]]])
    for fn in (oracle.recurrent, oracle.recurrent_matrix):
        o, S = fn(q, k, v, beta)
        for t, s in enumerate(ex["steps"]):
            assert np.array_equal(o[0, 0, t], s["output"])
        assert np.array_equal(S[0, 0, 0], ex["steps"][-1]["state_row0"])
    o, S = oracle.chunk(q, k, v, beta, C=2)
    assert np.allclose(o[0, 0, -1], ex["steps"][-1]["output"], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# Error form == transition-then-write form: page "DeltaNet: Memory That
# Edits", section "One rule, two readings" (the page prints 1.38e-06 for its
# fp32 run and asserts < 1e-5; fp64 must be near machine precision).
# --------------------------------------------------------------------------
def test_error_form_equals_matrix_form_on_the_pages_recipe(golden_dir):
    ctx = json.load(open(os.path.join(golden_dir, "fp32_deviation_context.json")))
    T, d = 512, 64
    r = np.random.default_rng(0)
    Q = r.standard_normal((1, 1, T, d))
    K = _unit(r.standard_normal((1, 1, T, d)))
    V = r.standard_normal((1, 1, T, d))
    beta = 1 / (1 + np.exp(-r.standard_normal((1, 1, T))))
    o1, S1 = oracle.recurrent(Q, K, V, beta)
    o2, S2 = oracle.recurrent_matrix(Q, K, V, beta)
    err = _rel(o2, o1)
    assert err < 1e-12
    assert err < ctx["error_form_vs_matrix_form"] / 1e4
    assert _rel(S2, S1) < 1e-12


@pytest.mark.parametrize("kind", [oracle.DELTANET, oracle.GATED, oracle.KDA])
def test_error_form_equals_matrix_form_all_kinds(kind):
    q, k, v, beta, g, S0 = _rand_inputs(2, 2, 16, 8, 6, kind, seed=kind + 10, beta_scale=2.0)
    o1, S1 = oracle.recurrent(q, k, v, beta, g, S0, kind=kind)
    o2, S2 = oracle.recurrent_matrix(q, k, v, beta, g, S0, kind=kind)
    assert _rel(o2, o1) < 1e-13 and _rel(S2, S1) < 1e-13


# --------------------------------------------------------------------------
# beta = 1 and a unit key: reading k afterwards returns v exactly, also with a
# decay, because the write corrects the prediction of the decayed state.
# Page "28. Linear attention and Gated DeltaNet", section "Correct: the delta
# rule"; page "A walk through of the DeltaNet family ...", DeltaNet and Gated
# DeltaNet sections (order: forget, predict, correct, write).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind", [oracle.DELTANET, oracle.GATED, oracle.KDA])
def test_beta_one_unit_key_recalls_value(kind):
    dk, dv, T = 16, 12, 9
    q, k, v, beta, g, S0 = _rand_inputs(1, 3, T, dk, dv, kind, seed=20 + kind)
    beta[..., -1] = 1.0
    q[..., -1, :] = k[..., -1, :]          # read the last token back with its own key
    o, S = oracle.recurrent(q, k, v, beta, g, S0, kind=kind)
    # the read-out of the last step is S_T^T k_T
    assert np.abs(o[..., -1, :] - v[..., -1, :]).max() < 1e-14 * max(1, np.abs(v).max()) * 10
    readback = np.einsum("bhk,bhkv->bhv", k[..., -1, :], S)
    assert np.abs(readback - v[..., -1, :]).max() < 1e-13


# Unit key: the value stored along k moves to (1 - beta) v_old + beta v_new.
# Page "DeltaNet: Memory That Edits", section "The delta rule".
@pytest.mark.parametrize("beta_val", [0.0, 0.25, 0.5, 0.9, 1.0, 1.5])
def test_unit_key_blend(beta_val):
    dk, dv = 8, 5
    r = np.random.default_rng(3)
    kk = _unit(r.standard_normal(dk))
    S0 = r.standard_normal((dk, dv))
    v_old = S0.T @ kk
    v_new = r.standard_normal(dv)
    o, S = oracle.recurrent(kk.reshape(1, 1, 1, dk), kk.reshape(1, 1, 1, dk),
                            v_new.reshape(1, 1, 1, dv), np.array([[[beta_val]]]),
                            S0=S0.reshape(1, 1, dk, dv))
    expect = (1 - beta_val) * v_old + beta_val * v_new
    assert np.abs(S[0, 0].T @ kk - expect).max() < 1e-13
    assert np.abs(o[0, 0, 0] - expect).max() < 1e-13


# Orthogonal directions are untouched by a write (alpha = 1).
# Page "DeltaNet: Linear Transformers with the Delta Rule Guide", section
# "Selective Erasure via Projection Operators"; page "A walk through ...".
def test_orthogonal_directions_untouched():
    dk, dv = 16, 7
    r = np.random.default_rng(4)
    kk = _unit(r.standard_normal(dk))
    S0 = r.standard_normal((dk, dv))
    x = r.standard_normal(dk)
    x -= (x @ kk) * kk
    _, S = oracle.recurrent(kk.reshape(1, 1, 1, dk), kk.reshape(1, 1, 1, dk),
                            r.standard_normal((1, 1, 1, dv)), np.array([[[0.7]]]),
                            S0=S0.reshape(1, 1, dk, dv))
    assert np.abs(S[0, 0].T @ x - S0.T @ x).max() < 1e-13
    # and the component along k did change
    assert np.abs(S[0, 0].T @ kk - S0.T @ kk).max() > 1e-3


# Eigenvalues of the transition: 1 - beta along k, 1 elsewhere.
# Page "DeltaNet: Memory That Edits", section "The reflection hiding in the
# delta rule" (printed list). The transition is read off the oracle by
# applying one step with v = 0 to the identity state.
def test_transition_eigenvalues(golden_dir):
    tab = json.load(open(os.path.join(golden_dir, "householder_eigenvalues.json")))
    d = 6
    r = np.random.default_rng(5)
    kk = _unit(r.standard_normal(d))
    for row in tab["rows"]:
        for fn in (oracle.recurrent, oracle.recurrent_matrix):
            _, S = fn(kk.reshape(1, 1, 1, d), kk.reshape(1, 1, 1, d), np.zeros((1, 1, 1, d)),
                      np.array([[[row["beta"]]]]), S0=np.eye(d).reshape(1, 1, d, d))
            M = S[0, 0]
            assert np.allclose(M, M.T, atol=1e-15)
            ev = np.sort(np.linalg.eigvalsh(M))
            expect = np.sort([row["along_k"]] + [row["elsewhere"]] * (d - 1))
            assert np.abs(ev - expect).max() < 1e-12
            assert abs(kk @ M @ kk - row["along_k"]) < 1e-12


# Overwrite recall: 8 orthonormal keys, R shuffled re-bindings each, the latest
# binding is recalled for every key (delta column = 1.000 for every R).
# Page "DeltaNet: Memory That Edits", section "Overwriting, measured".
def _recall(S, keys, values_per_key, latest):
    hits = 0
    for i, kvec in enumerate(keys):
        read = S.T @ kvec
        cands = values_per_key[i]
        cos = [read @ c / (np.linalg.norm(read) * np.linalg.norm(c) + 1e-300) for c in cands]
        hits += int(np.argmax(cos) == latest[i])
    return hits / len(keys)


def test_overwrite_recall_table(golden_dir):
    tab = json.load(open(os.path.join(golden_dir, "overwrite_recall.json")))
    d = 8
    for R, want_delta in zip(tab["writes_per_key"], tab["delta"]):
        delta_scores, hebb_scores = [], []
        for trial in range(20):
            r = np.random.default_rng(100 * R + trial)
            keys = np.linalg.qr(r.standard_normal((d, d)))[0].T  # orthonormal rows
            vals = r.standard_normal((d, R, d))
            order = [(i, rep) for i in range(d) for rep in range(R)]
            perm = r.permutation(len(order))
            seq = [order[p] for p in perm]
            latest = {}
            for i, rep in seq:
                latest[i] = rep
            K = np.stack([keys[i] for i, _ in seq])[None, None]
            V = np.stack([vals[i, rep] for i, rep in seq])[None, None]
            beta = np.ones((1, 1, len(seq)))
            _, S = oracle.recurrent(K, K, V, beta)
            delta_scores.append(_recall(S[0, 0], keys, vals, latest))
            # Hebbian comparator (additive write), only for the trend
            Sh = np.einsum("tk,tv->kv", K[0, 0], V[0, 0])
            hebb_scores.append(_recall(Sh, keys, vals, latest))
        assert np.mean(delta_scores) == want_delta
        if R >= 2:
            assert np.mean(hebb_scores) < 1.0


# alpha = 1 (g = 0) reduces Gated DeltaNet to DeltaNet bitwise; KDA with all
# channels equal reduces to Gated DeltaNet bitwise.
# Page "DeltaNet: Memory That Edits", section "Gating: the modern cell";
# page "A walk through ...", KDA section (only the decay is promoted to a vector).
def test_special_case_reductions_bitwise():
    B, H, T, dk, dv = 2, 2, 11, 8, 6
    q, k, v, beta, g, S0 = _rand_inputs(B, H, T, dk, dv, oracle.GATED, seed=7)
    o_dn, S_dn = oracle.recurrent(q, k, v, beta, None, S0, kind=oracle.DELTANET)
    o_g0, S_g0 = oracle.recurrent(q, k, v, beta, np.zeros_like(g), S0, kind=oracle.GATED)
    assert np.array_equal(o_dn, o_g0) and np.array_equal(S_dn, S_g0)
    o_g, S_g = oracle.recurrent(q, k, v, beta, g, S0, kind=oracle.GATED)
    g_kda = np.repeat(g[..., None], dk, axis=-1)
    o_k, S_k = oracle.recurrent(q, k, v, beta, g_kda, S0, kind=oracle.KDA)
    assert np.array_equal(o_g, o_k) and np.array_equal(S_g, S_k)
    assert not np.array_equal(o_g, o_dn)


# beta = 0: with alpha = 1 the state is unchanged; with alpha < 1 the state is
# the start state times the product of the decays (page "DeltaNet: Memory That
# Edits", section "Gating: the modern cell": beta = 0 is the pure-decay row).
def test_beta_zero():
    B, H, T, dk, dv = 1, 2, 13, 8, 5
    q, k, v, beta, g, S0 = _rand_inputs(B, H, T, dk, dv, oracle.GATED, seed=8)
    beta = np.zeros_like(beta)
    _, S = oracle.recurrent(q, k, v, beta, None, S0, kind=oracle.DELTANET)
    assert np.array_equal(S, S0)
    _, S = oracle.recurrent(q, k, v, beta, g, S0, kind=oracle.GATED)
    expect = S0 * np.exp(g.sum(-1))[..., None, None]
    assert _rel(S, expect) < 1e-14
    gk = -np.abs(np.random.default_rng(9).standard_normal((B, H, T, dk)))
    _, S = oracle.recurrent(q, k, v, beta, gk, S0, kind=oracle.KDA)
    expect = S0 * np.exp(gk.sum(2))[..., :, None]
    assert _rel(S, expect) < 1e-14


# KDA decays the rows of the d_k x d_v state, i.e. the key channels: a read
# along key channel i sees only alpha_i (page "A walk through ...", KDA
# section; its five-line recurrence scales the d_k axis).
def test_kda_decay_axis():
    dk, dv = 6, 4
    r = np.random.default_rng(11)
    S0 = r.standard_normal((1, 1, dk, dv))
    gk = -np.abs(r.standard_normal((1, 1, 1, dk)))
    for i in range(dk):
        qv = np.zeros((1, 1, 1, dk))
        qv[..., i] = 1.0
        o, _ = oracle.recurrent(qv, _unit(r.standard_normal((1, 1, 1, dk))),
                                r.standard_normal((1, 1, 1, dv)), np.zeros((1, 1, 1)), gk, S0,
                                kind=oracle.KDA)
        assert np.abs(o[0, 0, 0] - np.exp(gk[0, 0, 0, i]) * S0[0, 0, i]).max() < 1e-15


# Zero-padded tokens (k = 0, beta = 0, g = 0) are inert: the state after them
# and every earlier output are unchanged (page "28. Linear attention and Gated
# DeltaNet", section "The chunked form": the listing pads the last chunk).
@pytest.mark.parametrize("kind", [oracle.DELTANET, oracle.GATED, oracle.KDA])
def test_zero_padding_inert(kind):
    B, H, T, dk, dv, P = 1, 2, 10, 8, 6, 5
    q, k, v, beta, g, S0 = _rand_inputs(B, H, T, dk, dv, kind, seed=12)
    o, S = oracle.recurrent(q, k, v, beta, g, S0, kind=kind)

    def pad(x, last_dims):
        if x is None:
            return None
        shape = list(x.shape)
        shape[2] = P
        return np.concatenate([x, np.zeros(shape)], axis=2)

    qp = np.concatenate([q, np.random.default_rng(1).standard_normal((B, H, P, dk))], axis=2)
    vp = np.concatenate([v, np.random.default_rng(2).standard_normal((B, H, P, dv))], axis=2)
    op, Sp = oracle.recurrent(qp, pad(k, 1), vp, pad(beta, 0), pad(g, 0), S0, kind=kind)
    assert np.array_equal(Sp, S)
    assert np.array_equal(op[:, :, :T], o)


# State hand-off: running T1 then T2 from the carried state equals running
# T1 + T2 (the state argument of the contract on page "28. Linear attention
# and Gated DeltaNet", section "The recurrent form").
@pytest.mark.parametrize("kind", [oracle.DELTANET, oracle.GATED, oracle.KDA])
def test_state_handoff(kind):
    B, H, T, dk, dv = 2, 1, 21, 8, 8
    q, k, v, beta, g, S0 = _rand_inputs(B, H, T, dk, dv, kind, seed=13)
    o, S = oracle.recurrent(q, k, v, beta, g, S0, kind=kind)
    T1 = 8
    sl = lambda x, a, b: None if x is None else x[:, :, a:b]
    o1, S1 = oracle.recurrent(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(beta, 0, T1),
                              sl(g, 0, T1), S0, kind=kind)
    o2, S2 = oracle.recurrent(sl(q, T1, T), sl(k, T1, T), sl(v, T1, T), sl(beta, T1, T),
                              sl(g, T1, T), S1, kind=kind)
    assert np.array_equal(np.concatenate([o1, o2], axis=2), o)
    assert np.array_equal(S2, S)


# The matrix-form brute force over a whole sequence: the state equals the
# ordered product of the transitions applied to S0 plus the propagated writes
# (page "DeltaNet: Memory That Edits", "One rule, two readings"), here
# computed with numpy matrices independently of the oracle's own loops.
@pytest.mark.parametrize("kind", [oracle.DELTANET, oracle.GATED, oracle.KDA])
def test_brute_force_product_of_transitions(kind):
    B, H, T, dk, dv = 1, 1, 16, 6, 4
    q, k, v, beta, g, S0 = _rand_inputs(B, H, T, dk, dv, kind, seed=14, beta_scale=2.0)
    _, S = oracle.recurrent(q, k, v, beta, g, S0, kind=kind)
    Sx = S0[0, 0].copy()
    for t in range(T):
        kt = k[0, 0, t]
        if kind == oracle.DELTANET:
            D = np.eye(dk)
        elif kind == oracle.GATED:
            D = np.exp(g[0, 0, t]) * np.eye(dk)
        else:
            D = np.diag(np.exp(g[0, 0, t]))
        Mt = (np.eye(dk) - beta[0, 0, t] * np.outer(kt, kt)) @ D
        Sx = Mt @ Sx + beta[0, 0, t] * np.outer(kt, v[0, 0, t])
    assert _rel(S[0, 0], Sx) < 1e-13
