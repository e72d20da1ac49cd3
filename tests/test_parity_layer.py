"""GPU layer kernels (through the C ABI) versus the fp64 oracle of the gated layer.

The prologue (convolution + SiLU with carried history, head split, L2 norm,
q scale, gates) and the epilogue (gated RMSNorm) are checked element by element
against ``oracle.layer`` on seeded inputs (``synthetic.make_layer``), at sizes
that span several workgroup tiles and a ragged tail (T = 1, 2, 3, 5, 64, 300,
517, 1100), both head sizes, both dtypes, with and without carried
convolution state and decay gate. The new convolution state is a copy of
stored inputs and must match bit for bit. The whole layer between its
projections is then run as prefill followed by single-token decode steps with
the carried states, against the oracle run on the concatenated sequence.
Bound: max|gpu - ref| / max|ref| <= 1e-4 (fp32 inputs), 2e-2 (bf16 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import TOL, rel_err, say, to_dev
from oracle import layer as ol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_amd as dn  # noqa: F401  (loads libdeltanet.so)


def _dn():
    import delta_rule_recurrent_amd as dn
    return dn


def _prologue_ref(x, neg=False):
    return ol.prologue(x["qkv"], x["conv_w"], x["conv_state"], x["b"], x["a"] if x["a"] is not None
                       else torch.zeros_like(x["b"]), x["A_log"] if x["A_log"] is not None
                       else torch.zeros(x["Hv"]), x["dt_bias"] if x["dt_bias"] is not None
                       else torch.zeros(x["Hv"]), x["Hk"], x["Hv"], x["d"], x["d"],
                       allow_neg_eigval=neg)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 64, 300, 517, 1100])
def test_prologue_matches_oracle(dtype, d, T):
    dn = _dn()
    with_state = T % 2 == 1
    gated = T != 64
    neg = T in (1, 5, 517)   # beta = 2 sigmoid(b): the reflection range
    Hk, Hv = (1, 2) if d == 128 else (2, 4)
    say("prologue", dtype, d, T, "state" if with_state else "zeros", "gated" if gated else "ungated")
    x = synthetic.make_layer(2, T, Hk, Hv, d, dtype, seed=T * 3 + d, conv_state=with_state,
                             gated=gated)
    dx = to_dev(x)
    q, k, v, beta, g, cst = dn.layer_prologue(dx["qkv"], dx["conv_w"], dx["b"], dx["a"],
                                              dx["A_log"], dx["dt_bias"], Hk, Hv,
                                              conv_state=dx["conv_state"], allow_neg_eigval=neg)
    torch.cuda.synchronize()
    rq, rk, rv, rbeta, rg, rst = _prologue_ref(x, neg)
    tol = TOL[dtype]
    for name, gpu, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv), ("beta", beta, rbeta)):
        e = rel_err(gpu, ref)
        say("  %s err %.3g" % (name, e))
        assert e <= tol, (name, e)
    if gated:
        e = rel_err(g, rg)
        say("  g err %.3g" % e)
        assert e <= tol, ("g", e)
    else:
        assert g is None
    # the new state is a copy of stored values: exact
    assert np.array_equal(cst.float().cpu().double().numpy(), rst)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [0, 1, 2, 7])
def test_conv_state_in_place(dtype, T):
    """conv_state_out == conv_state: the update reads the old state before
    writing it (short sequences take part of the new state from the old one)."""
    dn = _dn()
    say("conv state in place", dtype, T)
    x = synthetic.make_layer(3, T, 1, 1, 64, dtype, seed=77 + T)
    dx = to_dev(x)
    st = dx["conv_state"].clone()
    _, _, _, _, _, out = dn.layer_prologue(dx["qkv"], dx["conv_w"], dx["b"], dx["a"], dx["A_log"],
                                           dx["dt_bias"], 1, 1, conv_state=st, conv_state_out=st)
    torch.cuda.synchronize()
    assert out is st
    _, ref = ol.causal_conv1d(x["qkv"], x["conv_w"], x["conv_state"])
    assert np.array_equal(st.float().cpu().double().numpy(), ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 63, 200])
def test_epilogue_matches_oracle(dtype, d, T):
    dn = _dn()
    B, Hv = 2, 3
    say("epilogue", dtype, d, T)
    gen = torch.Generator().manual_seed(900 + T + d)
    dt = synthetic.DTYPES[dtype]
    o = (torch.randn(B, Hv, T, d, generator=gen) * 0.3).to(dt)
    x = synthetic.make_layer(B, T, 1, Hv, d, dtype, seed=901 + T)
    out = dn.layer_epilogue(o.cuda(), x["z"].cuda(), x["norm_w"].cuda(), 1e-6)
    torch.cuda.synchronize()
    ref = ol.rmsnorm_gated(o, x["z"], x["norm_w"], 1e-6)
    e = rel_err(out, ref)
    say("  out err %.3g" % e)
    assert e <= TOL[dtype], e


def test_epilogue_zero_rows():
    """A read-out row of zeros gives zeros (rsqrt(eps) times 0), not NaN."""
    dn = _dn()
    o = torch.zeros(1, 2, 5, 64, dtype=torch.float32, device="cuda")
    x = synthetic.make_layer(1, 5, 1, 2, 64, "f32", seed=3)
    out = dn.layer_epilogue(o, x["z"].cuda(), x["norm_w"].cuda(), 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.zeros(1, 5, 128))


def _rule_ref(q, k, v, beta, g, Hk, Hv, S0):
    rep = Hv // Hk
    q = np.repeat(q, rep, axis=1)
    k = np.repeat(k, rep, axis=1)
    kind = oracle.GATED if g is not None else oracle.DELTANET
    return oracle.recurrent(q, k, v, beta, g, S0, kind=kind)


@pytest.mark.parametrize("dtype,d,Hk,Hv,gated", [("f32", 64, 1, 2, True), ("bf16", 128, 2, 4, True),
                                                  ("f32", 128, 1, 1, False)])
def test_layer_prefill_then_decode(dtype, d, Hk, Hv, gated):
    """Prefill of 200 tokens, then three single-token steps with the carried
    convolution and recurrent states, against the oracle on all 203 tokens."""
    dn = _dn()
    B, T0, steps = 2, 200, 3
    say("layer", dtype, d, Hk, Hv, "gated" if gated else "ungated")
    x = synthetic.make_layer(B, T0 + steps, Hk, Hv, d, dtype, seed=4242 + d, conv_state=False,
                             gated=gated)
    dx = to_dev(x)
    sl = lambda t, a, b: t[:, a:b].contiguous()   # noqa: E731  (token slice of [B,T,...])
    outs = []
    out, cst, S = dn.gated_deltanet_layer(sl(dx["qkv"], 0, T0), sl(dx["z"], 0, T0),
                                          sl(dx["b"], 0, T0),
                                          sl(dx["a"], 0, T0) if gated else None, dx["conv_w"],
                                          dx["A_log"], dx["dt_bias"], dx["norm_w"], Hk, Hv)
    outs.append(out)
    for t in range(T0, T0 + steps):
        out, cst, S = dn.gated_deltanet_layer(sl(dx["qkv"], t, t + 1), sl(dx["z"], t, t + 1),
                                              sl(dx["b"], t, t + 1),
                                              sl(dx["a"], t, t + 1) if gated else None,
                                              dx["conv_w"], dx["A_log"], dx["dt_bias"],
                                              dx["norm_w"], Hk, Hv, conv_state=cst, S=S)
        outs.append(out)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=1)

    rx = dict(x)
    rq, rk, rv, rbeta, rg, rst = _prologue_ref(rx)
    o_ref, S_ref = _rule_ref(rq, rk, rv, rbeta, rg if gated else None, Hk, Hv, None)
    ref = ol.rmsnorm_gated(o_ref, x["z"], x["norm_w"], 1e-6)
    e = rel_err(got, ref)
    eS = rel_err(S, S_ref)
    say("  out err %.3g, state err %.3g" % (e, eS))
    assert e <= TOL[dtype], e
    assert eS <= TOL[dtype], eS
    assert np.array_equal(cst.float().cpu().double().numpy(), rst)
