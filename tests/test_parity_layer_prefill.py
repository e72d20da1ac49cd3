"""The gated layer's prefill with its prologue inside the prefill's
chunk-parallel phase (dn_layer_prefill, through the C ABI).

The entry point does the work of dn_layer_prologue, dn_chunk_fwd_gqa and
dn_layer_epilogue, forming q, k, v, beta and g in the prep's load stage with
the prologue kernel's arithmetic. Checked:

  * bitwise against the three separate calls on the same seeded inputs
    (``synthetic.make_layer``): out, the end state and the new convolution
    history, at T in {1, 5, 64, 65, 130, 300} (one chunk, a ragged chunk, chunk
    boundaries, a history that reaches across chunks), with and without the
    carried history, a start state, the decay gate, shared key heads and the
    doubled beta;
  * against the fp64 oracle (its prologue, the token-by-token recurrence, its
    gated RMSNorm) at T in {37, 200}: bound 2e-2 (bf16), history bit for bit;
  * the bench's prefill layer size (B=4, T=2048, 8 + 8 heads of 128) bitwise
    against the three calls, whose full-size oracle parity
    test_parity_layer_full.py checks;
  * T = 0: the history passes through and the state is copied.
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


def _three_calls(dn, x, Hk, Hv, S0, neg):
    q, k, v, beta, g, cst = dn.layer_prologue(x["qkv"], x["conv_w"], x["b"], x["a"], x["A_log"],
                                              x["dt_bias"], Hk, Hv, conv_state=x["conv_state"],
                                              allow_neg_eigval=neg)
    o, S = dn.chunk_fwd_gqa(q, k, v, beta, g, S0)
    return dn.layer_epilogue(o, x["z"], x["norm_w"], 1e-6), cst, S


def _fused(dn, x, Hk, Hv, S0, neg):
    return dn.layer_prefill(x["qkv"], x["z"], x["b"], x["a"], x["conv_w"], x["A_log"], x["dt_bias"],
                            x["norm_w"], Hk, Hv, conv_state=x["conv_state"], S0=S0,
                            allow_neg_eigval=neg)


def _state(B, Hv, d, seed, std=0.05):
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn(B, Hv, d, d, generator=gen) * std).float()


@pytest.mark.parametrize("T,Hk,Hv,gated,neg,hist,s0", [
    (1, 1, 1, True, False, True, False),
    (5, 2, 4, True, True, False, True),
    (64, 1, 2, False, False, True, True),
    (65, 2, 2, True, False, True, False),
    (130, 1, 3, True, False, False, True),
    (300, 2, 2, False, True, True, True),
])
def test_layer_prefill_bitwise_three_calls(T, Hk, Hv, gated, neg, hist, s0):
    dn = _dn()
    B, d = 2, 128
    say("layer prefill", T, Hk, Hv, "gated" if gated else "ungated", "neg" if neg else "",
        "history" if hist else "no history", "S0" if s0 else "zero state")
    x = to_dev(synthetic.make_layer(B, T, Hk, Hv, d, "bf16", seed=5000 + T + 7 * Hv, conv_state=hist,
                                    gated=gated))
    S0 = _state(B, Hv, d, seed=T).cuda() if s0 else None
    out1, cst1, S1 = _fused(dn, x, Hk, Hv, S0, neg)
    out2, cst2, S2 = _three_calls(dn, x, Hk, Hv, S0, neg)
    torch.cuda.synchronize()
    say("  max |out diff| %.3g, max |S diff| %.3g" % ((out1.float() - out2.float()).abs().max().item(),
                                                      (S1 - S2).abs().max().item()))
    assert torch.equal(cst1, cst2)
    assert torch.equal(S1, S2)
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("T,Hk,Hv,gated", [(37, 1, 2, True), (200, 2, 2, False)])
def test_layer_prefill_matches_oracle(T, Hk, Hv, gated):
    dn = _dn()
    B, d = 2, 128
    x = synthetic.make_layer(B, T, Hk, Hv, d, "bf16", seed=6000 + T, conv_state=True, gated=gated)
    S0 = _state(B, Hv, d, seed=61)
    dx = to_dev(x)
    out, cst, S = _fused(dn, dx, Hk, Hv, S0.cuda(), False)
    torch.cuda.synchronize()
    q, k, v, beta, g, st = ol.prologue(
        x["qkv"], x["conv_w"], x["conv_state"], x["b"], x["a"] if gated else torch.zeros_like(x["b"]),
        x["A_log"] if gated else torch.zeros(Hv), x["dt_bias"] if gated else torch.zeros(Hv),
        Hk, Hv, d, d)
    rep = Hv // Hk
    q, k = np.repeat(q, rep, axis=1), np.repeat(k, rep, axis=1)
    o, S_ref = oracle.recurrent(q, k, v, beta, g if gated else None, S0.double().numpy(),
                                kind=oracle.GATED if gated else oracle.DELTANET)
    ref = ol.rmsnorm_gated(o, x["z"], x["norm_w"], 1e-6)
    e, eS = rel_err(out, ref), rel_err(S, S_ref)
    say("layer prefill vs oracle T=%d: out err %.3g, state err %.3g" % (T, e, eS))
    assert e <= TOL["bf16"], e
    assert eS <= TOL["bf16"], eS
    assert np.array_equal(cst.float().cpu().double().numpy(), st)


def test_layer_prefill_full_size_bitwise():
    dn = _dn()
    B, T, H, d = 4, 2048, 8, 128
    say("layer prefill full size", B, T, H, d)
    x = to_dev(synthetic.make_layer(B, T, H, H, d, "bf16", seed=3001))
    out1, cst1, S1 = _fused(dn, x, H, H, None, False)
    out2, cst2, S2 = _three_calls(dn, x, H, H, None, False)
    torch.cuda.synchronize()
    assert torch.equal(cst1, cst2)
    assert torch.equal(S1, S2)
    assert torch.equal(out1, out2)


def test_layer_prefill_no_tokens():
    """T = 0: the history passes through unchanged and the state is copied."""
    dn = _dn()
    B, Hk, Hv, d = 2, 1, 2, 128
    x = to_dev(synthetic.make_layer(B, 1, Hk, Hv, d, "bf16", seed=77, conv_state=True))
    e = lambda t: t[:, :0].contiguous()   # noqa: E731  (no tokens)
    S0 = _state(B, Hv, d, seed=78).cuda()
    out, cst, S = dn.layer_prefill(e(x["qkv"]), e(x["z"]), e(x["b"]), e(x["a"]), x["conv_w"], x["A_log"],
                                   x["dt_bias"], x["norm_w"], Hk, Hv, conv_state=x["conv_state"], S0=S0)
    torch.cuda.synchronize()
    assert out.shape == (B, 0, Hv * d)
    assert torch.equal(cst, x["conv_state"])
    assert torch.equal(S, S0)
