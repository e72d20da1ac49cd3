"""The single-kernel layer step for one token (dn_layer_decode_step, through
the C ABI) against the fp64 oracle of the gated layer.

The kernel does the single-token prologue (convolution with the carried
history, SiLU, head split, L2 norms, q scale, gates), the recurrent step on
the carried state and the gated RMSNorm in one launch. Its reference is the
oracle's prologue (``oracle.layer.prologue``), the token-by-token recurrence
(``oracle.recurrent``) and the oracle's gated RMSNorm, run on the same seeded
inputs (``synthetic.make_layer``):

  * one step at both head sizes and dtypes, with and without decay gate,
    carried convolution history, shared key heads and the reflection range;
  * several steps in a row with the convolution history carried in place (one
    value head per key head) and in two alternating buffers (shared key
    heads), against the oracle on the concatenated tokens;
  * the three separate calls (dn_layer_prologue, dn_decode_step_gqa,
    dn_layer_epilogue) on the same inputs, which compute the same values up to
    the order of the reductions;
  * the decode size bench.py measures (256 sequences x 16 + 16 heads of 128,
    bf16): every new convolution history entry, and outputs and states of
    sampled (sequence, head) pairs.
Bound: max|gpu - ref| / max|ref| <= 1e-4 (fp32 inputs), 2e-2 (bf16 inputs);
the new convolution history is a copy of stored inputs and must match bit
for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, rel_err, say, to_dev
from oracle import layer as ol
import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_recurrent_amd as dn  # noqa: F401  (loads libdeltanet.so)


def _dn():
    import delta_rule_recurrent_amd as dn
    return dn


def _state(B, Hv, d, seed, std=0.05):
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn(B, Hv, d, d, generator=gen) * std).float()


def _reference(x, S0, neg=False):
    """Oracle prologue -> recurrence from S0 -> gated RMSNorm over all of x's
    tokens. Returns (out [B,T,Hv*d], S [B,Hv,d,d], new conv state)."""
    gated = x["a"] is not None
    q, k, v, beta, g, st = ol.prologue(
        x["qkv"], x["conv_w"], x["conv_state"], x["b"],
        x["a"] if gated else torch.zeros_like(x["b"]),
        x["A_log"] if gated else torch.zeros(x["Hv"]),
        x["dt_bias"] if gated else torch.zeros(x["Hv"]), x["Hk"], x["Hv"], x["d"], x["d"],
        allow_neg_eigval=neg)
    rep = x["Hv"] // x["Hk"]
    q, k = np.repeat(q, rep, axis=1), np.repeat(k, rep, axis=1)
    kind = oracle.GATED if gated else oracle.DELTANET
    o, S = oracle.recurrent(q, k, v, beta, g if gated else None,
                            None if S0 is None else S0.double().numpy(), kind=kind)
    return ol.rmsnorm_gated(o, x["z"], x["norm_w"], 1e-6), S, st


def _step(dn, dx, t, S, Hk, Hv, conv_state, conv_state_out=None, neg=False):
    sl = lambda a: a[:, t:t + 1].contiguous()   # noqa: E731  (token t of [B,T,...])
    gated = dx["a"] is not None
    return dn.layer_decode_step(sl(dx["qkv"]), sl(dx["z"]), sl(dx["b"]),
                                sl(dx["a"]) if gated else None, dx["conv_w"], dx["A_log"],
                                dx["dt_bias"], dx["norm_w"], Hk, Hv, S, conv_state=conv_state,
                                conv_state_out=conv_state_out, allow_neg_eigval=neg)


@pytest.mark.parametrize("dtype,d,Hk,Hv,gated,neg,with_state", [
    ("bf16", 128, 1, 1, True, False, True),
    ("bf16", 128, 2, 4, True, True, False),
    ("bf16", 64, 2, 2, False, False, True),
    ("f32", 128, 1, 3, True, False, True),
    ("f32", 64, 1, 1, True, True, False),
    ("f32", 128, 2, 2, False, False, False),
])
def test_layer_decode_step_matches_oracle(dtype, d, Hk, Hv, gated, neg, with_state):
    dn = _dn()
    B = 3
    say("layer decode step", dtype, d, Hk, Hv, "gated" if gated else "ungated", "neg" if neg else "",
        "history" if with_state else "zeros")
    x = synthetic.make_layer(B, 1, Hk, Hv, d, dtype, seed=700 + d + 10 * Hv + Hk, conv_state=with_state,
                             gated=gated)
    S0 = _state(B, Hv, d, seed=71 + d)
    dx = to_dev(x)
    S = S0.cuda()
    out, cst = _step(dn, dx, 0, S, Hk, Hv, dx["conv_state"], neg=neg)
    torch.cuda.synchronize()
    ref, S_ref, st_ref = _reference(x, S0, neg)
    e, eS = rel_err(out, ref), rel_err(S, S_ref)
    say("  out err %.3g, state err %.3g" % (e, eS))
    assert e <= TOL[dtype], e
    assert eS <= TOL[dtype], eS
    assert np.array_equal(cst.float().cpu().double().numpy(), st_ref)


@pytest.mark.parametrize("dtype,Hk,Hv,gated", [("bf16", 2, 2, True), ("f32", 1, 2, True),
                                               ("bf16", 1, 4, False)])
def test_layer_decode_steps_carried(dtype, Hk, Hv, gated):
    """Seven steps in a row; the convolution history in place when every key
    head serves one value head, else in two alternating buffers."""
    dn = _dn()
    B, T, d = 2, 7, 128
    x = synthetic.make_layer(B, T, Hk, Hv, d, dtype, seed=900 + Hv, conv_state=True, gated=gated)
    S0 = _state(B, Hv, d, seed=91)
    dx = to_dev(x)
    S = S0.cuda()
    in_place = Hk == Hv
    say("layer decode steps", dtype, Hk, Hv, "in place" if in_place else "two buffers")
    cst = dx["conv_state"].clone()
    other = torch.empty_like(cst)
    outs = []
    for t in range(T):
        if in_place:
            out, cst = _step(dn, dx, t, S, Hk, Hv, cst, conv_state_out=cst)
        else:
            out, nxt = _step(dn, dx, t, S, Hk, Hv, cst, conv_state_out=other)
            cst, other = nxt, cst
        outs.append(out)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=1)
    ref, S_ref, st_ref = _reference(x, S0)
    e, eS = rel_err(got, ref), rel_err(S, S_ref)
    say("  out err %.3g, state err %.3g" % (e, eS))
    assert e <= TOL[dtype], e
    assert eS <= TOL[dtype], eS
    assert np.array_equal(cst.float().cpu().double().numpy(), st_ref)


@pytest.mark.parametrize("dtype,d,Hk,Hv", [("bf16", 128, 2, 4), ("f32", 64, 1, 1)])
def test_layer_decode_step_matches_three_calls(dtype, d, Hk, Hv):
    """The same inputs through dn_layer_prologue, dn_decode_step_gqa and
    dn_layer_epilogue: the new history is identical, the state and the output
    agree to rounding (the two forms add their reductions in other orders)."""
    dn = _dn()
    B = 5
    x = to_dev(synthetic.make_layer(B, 1, Hk, Hv, d, dtype, seed=1234 + d, conv_state=True))
    S0 = _state(B, Hv, d, seed=12).cuda()
    S1, S2 = S0.clone(), S0.clone()
    out1, cst1 = _step(dn, x, 0, S1, Hk, Hv, x["conv_state"])
    q, k, v, beta, g, cst2 = dn.layer_prologue(x["qkv"], x["conv_w"], x["b"], x["a"], x["A_log"],
                                               x["dt_bias"], Hk, Hv, conv_state=x["conv_state"])
    o = dn.decode_step_gqa(q[:, :, 0], k[:, :, 0], v[:, :, 0], beta[:, :, 0], g[:, :, 0], S2)
    out2 = dn.layer_epilogue(o.unsqueeze(2), x["z"], x["norm_w"], 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(cst1, cst2)
    eS = rel_err(S1, S2.double().cpu().numpy())
    e = rel_err(out1, out2.double().cpu().numpy())
    say("  fused vs three calls: out %.3g, state %.3g" % (e, eS))
    assert eS <= 1e-5, eS
    assert e <= TOL[dtype], e


def test_layer_decode_step_full_size():
    """256 sequences x 16 + 16 heads of 128, bf16: every new history entry,
    and out and S of sampled (sequence, head) pairs (the pairs are
    independent: the oracle runs on those sequences alone)."""
    dn = _dn()
    B, H, d = 256, 16, 128
    x = synthetic.make_layer(B, 1, H, H, d, "bf16", seed=2025, conv_state=True)
    S0 = _state(B, H, d, seed=2026, std=0.02)
    dx = to_dev(x)
    S = S0.cuda()
    say("layer decode step full size", B, H, d)
    out, cst = _step(dn, dx, 0, S, H, H, dx["conv_state"])
    torch.cuda.synchronize()
    # every new history entry: the last three of (old history, this token)
    whole = torch.cat([x["conv_state"].float(), x["qkv"].float().transpose(1, 2)], dim=2)[:, :, -3:]
    assert torch.equal(cst.float().cpu(), whole)
    seqs = [0, 37, 128, 255]
    xs = {kk: (vv[seqs].contiguous() if isinstance(vv, torch.Tensor) and vv.dim() >= 2 and
               vv.shape[0] == B else vv) for kk, vv in x.items()}
    xs["B"] = len(seqs)
    ref, S_ref, _ = _reference(xs, S0[seqs])
    got = out.float().cpu()[seqs]
    e, eS = rel_err(got, ref), rel_err(S.cpu()[seqs], S_ref)
    say("  sampled sequences %s: out err %.3g, state err %.3g" % (seqs, e, eS))
    assert e <= TOL["bf16"], e
    assert eS <= TOL["bf16"], eS
